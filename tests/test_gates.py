"""The parity gates reject the failures they exist to catch (CPU, oracle data only).

A gate that passes a wrong answer proves nothing, so each one is shown to fail on a planted
defect: an all-zero attention output on the production value distribution (where it would
pass the absolute bar alone), a K/V confusion (values read from the wrong dimensions of the
shared row) and a wrong tie-break in the selection.
"""
import numpy as np
import pytest
import torch

from gates import check_attn, check_idx
from gen import inputs as gi
from oracle import dsa_oracle as orc


def _prefill(D_k, D_v, sigma, L=64, top_k=16):
    wl = gi.Workload(name="gate", L=L,
                     idx=gi.IndexerSpec(H_I=2, d_I=16, grid_lo=-3, grid_hi=3, grid_step=0.125,
                                        w_choices=(0.5, 1.0), top_k=top_k),
                     mqa=gi.MqaSpec(H=4, D_k=D_k, D_v=D_v, sigma=sigma, scale=D_k ** -0.5))
    return gi.prefill_inputs(wl)


def test_reference_passes_its_own_gate():
    d = _prefill(576, 512, 576 ** -0.5)
    idx, o, lse = orc.prefill(d)
    check_idx(idx, idx)
    check_attn(torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(lse).float(), o, lse)


def test_zero_output_fails_on_production_distribution():
    # late rows of a long sequence average hundreds of N(0,1)/24 value rows, as in production
    d = _prefill(576, 512, 576 ** -0.5, L=1024, top_k=1024)
    _, o, lse = orc.prefill(d, rows=list(range(896, 1024)))
    assert np.abs(o).max() < 1e-2          # the absolute bar alone would let zeros through
    with pytest.raises(AssertionError, match="normalised"):
        check_attn(torch.zeros(o.shape), None, o, lse)


def test_swapped_key_value_dimensions_fail():
    d = _prefill(96, 64, 1.0)
    idx, o, lse = orc.prefill(d)
    # values taken from the last D_v dimensions of the row instead of the first
    bad = d.copy()
    kv = d["kv"]
    bad["kv"] = torch.cat([kv[:, 96 - 64:], kv[:, :96 - 64]], dim=1)
    _, o_bad, _ = orc.prefill(bad, idx=idx)
    with pytest.raises(AssertionError):
        check_attn(torch.from_numpy(o_bad), None, o, lse)


def test_wrong_tie_break_fails():
    d = _prefill(64, 64, 1.0, L=64, top_k=16)
    d["q_idx"] = torch.zeros_like(d["q_idx"])          # every score 0: all keys tie
    idx = orc.prefill_indexer_topk(d)
    wrong = idx.copy()
    for t in range(idx.shape[0]):                     # highest positions instead of lowest
        n = min(16, t + 1)
        wrong[t, :n] = np.arange(t + 1 - n, t + 1)
    with pytest.raises(AssertionError, match="index rows differ"):
        check_idx(wrong, idx)

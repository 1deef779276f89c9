"""GPU parity of the dense causal MLA/MQA baseline (dsa_dense_mqa_prefill / _decode) through the
C ABI, against the oracle's dense attention (itself pinned to torch's causal SDPA)."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

from gates import check_attn

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


@pytest.mark.parametrize("D_k,D_v,H,L,sharp,n_rows", [
    (64, 64, 8, 300, True, None),          # one split, every row
    (96, 64, 33, 5000, True, 60),          # up to 3 splits, heads ending inside a wave
    (576, 512, 128, 4500, True, 40),       # production shapes, 3 splits
    (576, 512, 128, 4500, False, 40),      # production distribution (N(0,1)/24)
    (576, 512, 128, 20000, True, 12),      # 10 splits: the many-partial combine
])
def test_dense_prefill(D_k, D_v, H, L, sharp, n_rows):
    dsa = _dsa()
    wl = gi.Workload(name="dense", L=L, idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=8),
                     mqa=gi.MqaSpec(H=H, D_k=D_k, D_v=D_v, sigma=1.0 if sharp else D_k ** -0.5,
                                    scale=D_k ** -0.5), seed=91)
    d = gi.prefill_inputs(wl)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    step(f"dense prefill D_k={D_k} H={H} L={L} sharp={sharp}")
    o, lse = dsa.dense_mqa_prefill(g["q"], g["kv"], g["q_pos"], D_v, d["scale"])
    torch.cuda.synchronize()
    rows = list(range(L)) if n_rows is None else \
        sorted(set(np.linspace(0, L - 1, n_rows).astype(int).tolist()) | {2047, 2048, L - 1})
    o_ref, l_ref = orc.dense_prefill(d, rows=rows)
    check_attn(o[rows], lse[rows], o_ref, l_ref, "dense prefill")


def test_dense_decode_paged():
    dsa = _dsa()
    sp = gi.DecodeSpec(B=5, idx=gi.IndexerSpec(top_k=64), mqa=gi.MqaSpec(sigma=1.0),
                       spare_pages=4, seed=92)
    d = gi.decode_inputs(sp, ctx_lens=(9000, 2049, 100, 1, 4096))
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    step("dense decode B=5 ctx up to 9000")
    o, lse = dsa.dense_mqa_decode(g["q"], g["kv_cache"], g["page_table"], g["ctx"], d["D_v"],
                                  d["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = orc.dense_decode(d)
    check_attn(o, lse, o_ref, l_ref, "dense decode")


def test_dense_equals_sparse_with_every_position_selected():
    """For t < 2048 the sparse kernel given every position 0..t attends the same set as the
    dense one: the two agree to bf16 output rounding."""
    dsa = _dsa()
    L, k = 1500, 2048
    wl = gi.Workload(name="eq", L=L, idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=k),
                     mqa=gi.MqaSpec(sigma=1.0), seed=93)
    d = gi.prefill_inputs(wl)
    g = {kk: (v.cuda() if isinstance(v, torch.Tensor) else v) for kk, v in d.items()}
    ar = torch.arange(k, dtype=torch.int32)
    idx = torch.where(ar[None, :] <= torch.arange(L)[:, None], ar[None, :], torch.tensor(-1))
    step("dense vs sparse with full selection")
    o_d, l_d = dsa.dense_mqa_prefill(g["q"], g["kv"], g["q_pos"], d["D_v"], d["scale"])
    o_s, l_s = dsa.sparse_mqa_prefill(g["q"], g["kv"], idx.to(torch.int32).cuda(), g["q_pos"],
                                      d["D_v"], d["scale"])
    torch.cuda.synchronize()
    assert (o_d.float() - o_s.float()).abs().max().item() <= 2e-3
    assert (l_d - l_s).abs().max().item() <= 1e-4

"""GPU parity of batched prefill over paged caches (dsa_indexer_topk_batched +
dsa_sparse_mqa_batched) through the C ABI, against the oracle: variable-length batches,
chunked prefill of a chunk against a cached prefix, rows of many sequences interleaved (so
that one group of 16 rows spans several sequences), and rows without a sequence."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

from gates import check_attn, check_idx
import oracle_pool as op  # noqa: F401

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


def _run(d, q_seq_given=True):
    dsa = _dsa()
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q_seq = g["q_seq"] if q_seq_given else None
    idx = dsa.indexer_topk_batched(g["q_idx"], g["w"], g["k_cache"], g["page_table"], g["q_pos"],
                                   d["top_k"], q_seq=q_seq)
    o = lse = None
    if "q" in d:
        o, lse = dsa.sparse_mqa_batched(g["q"], g["kv_cache"], g["page_table"], g["q_pos"], idx,
                                        d["D_v"], d["scale"], q_seq=q_seq)
    torch.cuda.synchronize()
    return idx, o, lse


@pytest.mark.parametrize("lens,starts,top_k,shuffle", [
    ((300, 1000, 2500, 77, 4096, 1500), None, 512, False),      # variable lengths, from 0
    ((300, 1000, 2500, 77, 4096, 1500), None, 512, True),       # rows interleaved
    ((10000,), (6000,), 2048, False),                          # a chunk against a prefix
    ((5000, 3000, 2049), (4000, 0, 2000), 2048, False),         # chunks and a full prefill
])
def test_batched_prefill_matches_oracle(lens, starts, top_k, shuffle):
    sp = gi.BatchedSpec(seq_lens=lens, q_start=starts, idx=gi.IndexerSpec(top_k=top_k),
                        mqa=gi.MqaSpec(sigma=1.0), spare_pages=3, seed=81)
    n = sum(lens) - (sum(starts) if starts else 0)
    order = torch.randperm(n, generator=torch.Generator().manual_seed(82)) if shuffle else None
    d = gi.batched_inputs(sp, row_order=order)
    step(f"batched prefill lens={lens} starts={starts} k={top_k} shuffle={shuffle} rows={n}")
    idx, o, lse = _run(d)
    rows = sorted(set(range(0, n, max(1, n // 300))) | {n - 1})
    step(f"batched prefill: oracle on {len(rows)} rows")
    i_ref, o_ref, l_ref = orc.batched_prefill(d, rows=rows)
    check_idx(idx[rows], i_ref, "batched idx")
    check_attn(o[rows], lse[rows], o_ref, l_ref, "batched attn")


def test_batched_indexer_all_rows_and_small_shapes():
    """Every row of a variable-length batch at H_I = 4, d_I = 32 (partial MFMA operands),
    page size 16, k = 48; plus rows of a sequence outside the table and negative positions."""
    sp = gi.BatchedSpec(seq_lens=(700, 33, 1200, 16), page_size=16,
                        idx=gi.IndexerSpec(H_I=4, d_I=32, grid_lo=-3, grid_hi=3,
                                           grid_step=0.125, w_choices=(0.25, 0.5, 1.0),
                                           top_k=48),
                        mqa=gi.MqaSpec(H=8, D_k=64, D_v=64, sigma=1.0, scale=0.125), seed=83)
    d = gi.batched_inputs(sp)
    d["q_seq"] = d["q_seq"].clone()
    d["q_pos"] = d["q_pos"].clone()
    d["q_seq"][[3, 900]] = torch.tensor([7, -1], dtype=torch.int32)
    d["q_pos"][[10, 1500]] = torch.tensor([-1, -30], dtype=torch.int32)
    step("batched prefill small shapes, all rows")
    idx, o, lse = _run(d)
    i_ref, o_ref, l_ref = orc.batched_prefill(d)
    check_idx(idx, i_ref, "batched small idx")
    check_attn(o, lse, o_ref, l_ref, "batched small attn")
    for r in (3, 900, 10, 1500):
        assert (idx[r] == -1).all() and (o[r] == 0).all() and torch.isneginf(lse[r]).all()


def test_batched_single_sequence_without_q_seq_equals_contiguous_prefill():
    """q_seq omitted (every row in sequence 0): a 6000-token sequence in random pages gives the
    same indices and outputs as the contiguous prefill kernels on the same rows."""
    dsa = _dsa()
    sp = gi.BatchedSpec(seq_lens=(6000,), idx=gi.IndexerSpec(top_k=2048),
                        mqa=gi.MqaSpec(sigma=1.0), seed=84)
    d = gi.batched_inputs(sp)
    step("batched (no q_seq) vs contiguous prefill, L=6000")
    idx, o, lse = _run(d, q_seq_given=False)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    idx2 = dsa.indexer_topk(g["q_idx"], g["w"], g["k_flat"], g["q_pos"], d["top_k"])
    o2, lse2 = dsa.sparse_mqa_prefill(g["q"], g["kv_flat"], idx2, g["q_pos"], d["D_v"],
                                      d["scale"])
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)

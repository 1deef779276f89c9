"""GPU parity at full size, on the contracted row sets (through the C ABI, against the oracle).

* L=32768 prefill: index rows of ALL 32768 queries bit-exact; attention on 1025 strided rows
  (every 32nd row and the last one).
* L=131072 prefill in 32 query blocks of 4096, launched exactly as the benchmark launches them
  (``bench.Prefill.run``): in every block, the rows of the 1152-row sample (every 128th row,
  plus the first and the last 64 rows) are checked, indices bit-exact and attention to the
  gates.
* Paged decode, batch 64, ctx ~ U[4096, 131072]: all 64 sequences.
* Off the dyadic grid (head weights ~ U[0.1, 1], many keys with every head <= 0): the
  selections of the prefill and decode indexers are top-k sets of scores within the stated
  fp32 error bound of the exact ones.

The GPU work of each workload runs once per module (fixtures); the oracle's rows are split
over several tests so that each one finishes in seconds and reports as it goes.
"""
import os
import sys

import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

from gates import check_attn, check_idx
import oracle_pool as op

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


# ------------------------------------------------------------------------- L = 32768 prefill

@pytest.fixture(scope="module")
def prefill32k():
    dsa = _dsa()
    step("prefill L=32768: generate on device")
    d = gi.prefill_inputs(gi.prefill_workload(32768), device="cuda")
    step("prefill L=32768: indexer + MQA over all rows")
    idx = dsa.indexer_topk(d["q_idx"], d["w"], d["k_idx"], d["q_pos"], d["top_k"])
    o, lse = dsa.sparse_mqa_prefill(d["q"], d["kv"], idx, d["q_pos"], d["D_v"], d["scale"])
    torch.cuda.synchronize()
    res = {"d": d, "idx": idx.cpu().numpy(), "o": o, "lse": lse}
    yield res
    res.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(8))
def test_prefill_L32768_indices_all_rows(prefill32k, part):
    rows = np.arange(part * 4096, (part + 1) * 4096)
    step(f"L=32768 oracle index rows {rows[0]}..{rows[-1]}")
    want = op.prefill_rows(prefill32k["d"], rows)
    check_idx(prefill32k["idx"][rows], want, f"L=32768 rows {rows[0]}..{rows[-1]}")


def test_prefill_L32768_attention_strided_rows(prefill32k):
    rows = list(range(0, 32768, 32)) + [32767]
    step(f"L=32768 oracle attention on {len(rows)} rows")
    i_ref, o_ref, l_ref = op.prefill_rows(prefill32k["d"], rows, with_attn=True)
    check_idx(prefill32k["idx"][rows], i_ref, "L=32768 idx (attention rows)")
    sel = torch.as_tensor(rows, device="cuda")
    check_attn(prefill32k["o"][sel], prefill32k["lse"][sel], o_ref, l_ref, "L=32768 attn")


# ------------------------------------------------------------------------ L = 131072 prefill

SAMPLE_131072 = sorted(set(range(0, 131072, 128)) | set(range(64)) |
                       set(range(131072 - 64, 131072)))


@pytest.fixture(scope="module")
def prefill128k():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from bench import Prefill
    step("prefill L=131072: generate on device (bench inputs)")
    pre = Prefill(dev=torch.device("cuda"))
    got_idx = {}
    rows = torch.as_tensor(SAMPLE_131072, dtype=torch.int64)

    def keep(bi, a, e, idx_blk):
        r = rows[(rows >= a) & (rows < e)]
        if r.numel():
            got = idx_blk[(r - a).to(idx_blk.device)].cpu().numpy()
            for t, row in zip(r.tolist(), got):
                got_idx[t] = row

    step("prefill L=131072: 32 blocks of 4096 as the benchmark runs them")
    pre.run(after_block=keep)
    torch.cuda.synchronize()
    assert len(got_idx) == len(SAMPLE_131072)
    res = {"pre": pre, "idx": got_idx}
    yield res
    res.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_prefill_L131072_sampled_rows_every_block(prefill128k, part):
    pre = prefill128k["pre"]
    rows = SAMPLE_131072[part::4]
    step(f"L=131072 oracle on {len(rows)} sampled rows (part {part})")
    i_ref, o_ref, l_ref = op.prefill_rows(pre.inp, rows, with_attn=True)
    got = np.stack([prefill128k["idx"][t] for t in rows])
    check_idx(got, i_ref, f"L=131072 idx part {part}")
    sel = torch.as_tensor(rows, device="cuda")
    check_attn(pre.out[sel], pre.lse[sel], o_ref, l_ref, f"L=131072 attn part {part}")


# ------------------------------------------------------------------------- decode, B = 64

def test_decode_full_batch64_all_sequences():
    """Paged decode, batch 64, ctx ~ U[4096, 131072], page size 64, random page tables: every
    sequence checked."""
    dsa = _dsa()
    step("decode B=64: generate on device")
    d = gi.decode_inputs(gi.DecodeSpec(), device="cuda")
    step("decode B=64: indexer + MQA")
    idx = dsa.indexer_topk_paged(d["q_idx"], d["w"], d["k_cache"], d["page_table"], d["ctx"],
                                 d["top_k"])
    o, lse = dsa.sparse_mqa_decode(d["q"], d["kv_cache"], d["page_table"], d["ctx"], idx,
                                   d["D_v"], d["scale"])
    torch.cuda.synchronize()
    step("decode B=64: oracle on all 64 sequences")
    i_ref, o_ref, l_ref = orc.decode(d)
    check_idx(idx, i_ref, "B=64 idx")
    check_attn(o, lse, o_ref, l_ref, "B=64 attn")


# ------------------------------------------------------------------------- off the grid

# Error bound of a computed score (fp32, unit roundoff u = 2^-24): |I_hat - I| <= 2^-16 * M with
# M[t, s] = sum_j |w[t,j]| * sum_i |q_I[t,j,i]| * |k_I[s,i]|.  The largest term of the
# derivation is the fp32 accumulation of the 128 exact FP8 products of each head (at most
# 127 u per head) plus, in prefill, the linear half of the ReLU split (the fp32 head sum of the
# queries, 64 u, and the 384-product bf16 accumulation, about 200 u): below 420 u < 2^-16 / 2.
BOUND = 2.0 ** -16


def _check_within_bound(idx, I, M, t, k, what):
    """idx is a top-k of some scores within BOUND * M of the exact scores I (keys 0..t)."""
    n = min(k, t + 1)
    row = np.asarray(idx)
    assert (row[n:] == -1).all(), f"{what}: padding"
    sel = row[:n]
    assert (sel >= 0).all() and (sel <= t).all() and np.unique(sel).size == n, f"{what}: set"
    assert (np.diff(sel) > 0).all(), f"{what}: order"
    if n == t + 1:
        return
    E = BOUND * M
    mask = np.zeros(t + 1, dtype=bool)
    mask[sel] = True
    lo_sel = (I[mask] + E[mask]).min()
    hi_un = (I[~mask] - E[~mask]).max()
    assert lo_sel >= hi_un, f"{what}: selected {lo_sel} < unselected {hi_un}"


def test_indexer_off_grid_weights_and_all_negative_keys():
    """w ~ U[0.1, 1] (not dyadic), queries >= 0 and every even key <= 0 elementwise (so every
    head of such a key is <= 0 and its exact score is 0), odd keys on the {-2..2}/8 grid.  About
    half the keys score above 0, so rows below t ~ 2k take part of their selection from the
    zero-score keys and later rows are decided among positive scores."""
    dsa = _dsa()
    L, H_I, d_I, k = 2500, 64, 128, 256
    q_idx = gi.grid_fp8((L, H_I, d_I), 0, 2, 0.125, 51, 0)
    kn = gi.grid_fp8((L, d_I), -2, 0, 0.125, 51, 1)
    ka = gi.grid_fp8((L, d_I), -2, 2, 0.125, 51, 2)
    k_idx = torch.where((torch.arange(L) % 2 == 0)[:, None], kn, ka).contiguous()
    w = gi.uniform_f32((L, H_I), 0.1, 1.0, 51, 4)
    q_pos = torch.arange(L, dtype=torch.int32)
    rows = list(range(0, 600, 5)) + list(range(600, L, 61)) + [L - 1]
    step(f"off-grid indexer: prefill L={L}, decode {len(rows)} sequences")
    pre = dsa.indexer_topk(q_idx.cuda(), w.cuda(), k_idx.cuda(), q_pos.cuda(), k).cpu().numpy()
    # decode: one sequence per checked row t (ctx = t + 1) sharing the key pages
    P = 64
    n_pages = (L + P - 1) // P
    kc = torch.zeros((n_pages * P, d_I), dtype=torch.uint8)
    kc[:L] = k_idx
    kc = kc.view(n_pages, P, d_I)
    pt = torch.arange(n_pages, dtype=torch.int32).repeat(len(rows), 1)
    ctx = torch.tensor([t + 1 for t in rows], dtype=torch.int32)
    dec = dsa.indexer_topk_paged(q_idx[rows].contiguous().cuda(), w[rows].contiguous().cuda(),
                                 kc.cuda(), pt.cuda(), ctx.cuda(), k).cpu().numpy()
    torch.cuda.synchronize()
    kd = orc.decode_e4m3fn(k_idx)
    qd = orc.decode_e4m3fn(q_idx)
    wd = w.double().numpy()
    n_zero_sel = 0
    for r, t in enumerate(rows):
        I = orc.indexer_scores(qd[t], wd[t], kd[: t + 1])
        M = np.abs(kd[: t + 1]) @ np.abs(qd[t]).T @ np.abs(wd[t])
        _check_within_bound(pre[t], I, M, t, k, f"prefill row {t}")
        _check_within_bound(dec[r], I, M, t, k, f"decode row {t}")
        if t + 1 > k:
            n_zero_sel += int((I[pre[t][: min(k, t + 1)]] == 0).sum())
    assert n_zero_sel > 2000, "the test should exercise zero-score keys at the threshold"

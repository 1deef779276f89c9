"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Indices must match bit-exactly (as the kernels emit ascending positions then -1, rows are
compared as they are).  Attention outputs must satisfy max|o - o_ref| <= 1e-2 and, since the
production distribution has |o| ~ 3e-3 (an all-zero output would pass the absolute bar), also
max|o - o_ref| / max|o_ref| <= 1e-2; lse must match to 1e-3 relative.  A "sharp" variant
(q, kv ~ N(0,1)) gives outputs of order 0.1-1 where the absolute bar has force.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

from gates import ABS_TOL, LSE_REL, REL_TOL, check_attn, check_idx  # noqa: F401

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


def to_dev(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}




def run_indexer(d, top_k=None):
    dsa = _dsa()
    dd = to_dev(d)
    return dsa.indexer_topk(dd["q_idx"], dd["w"], dd["k_idx"], dd["q_pos"],
                            top_k or d["top_k"])


# ------------------------------------------------------------------------------ indexer

def test_indexer_tiny_all_rows():
    d = gi.prefill_inputs(gi.tiny_workload(), with_mqa=False)
    step("indexer tiny L=256 H_I=4 d_I=32 k=32")
    got = run_indexer(d)
    torch.cuda.synchronize()
    check_idx(got, orc.prefill_indexer_topk(d), "tiny")


@pytest.mark.parametrize("L,top_k,n_q0", [(1000, 100, 0), (1000, 2048, 0), (777, 64, 300),
                                          (130, 16, 0), (5000, 1500, 3000)])
def test_indexer_production_heads_ragged(L, top_k, n_q0):
    """H_I=64, d_I=128 on the dyadic grid; ragged tiles and row blocks; small top_k forces the
    candidate lists through many cut-downs."""
    wl = gi.Workload(name="r", L=L, idx=gi.IndexerSpec(top_k=top_k), mqa=None, seed=3)
    d = gi.prefill_inputs(wl, rows=(n_q0, L - n_q0), with_mqa=False)
    step(f"indexer L={L} k={top_k} rows {n_q0}..{L - 1}")
    got = run_indexer(d)
    torch.cuda.synchronize()
    check_idx(got, orc.prefill_indexer_topk(d), f"L={L} k={top_k}")


@pytest.mark.parametrize("L,H_I,d_I,top_k,n_q0", [(700, 7, 48, 64, 5), (1000, 33, 80, 200, 0),
                                                  (389, 64, 112, 100, 77)])
def test_indexer_other_dims(L, H_I, d_I, top_k, n_q0):
    """Key rows of 48, 80 and 112 bytes (partial 128-byte tiles), head counts that leave head
    groups partly or wholly empty, key and row counts off the tile sizes."""
    wl = gi.Workload(name="dims", L=L, idx=gi.IndexerSpec(H_I=H_I, d_I=d_I, top_k=top_k),
                     mqa=None, seed=17)
    d = gi.prefill_inputs(wl, rows=(n_q0, L - n_q0), with_mqa=False)
    step(f"indexer L={L} H_I={H_I} d_I={d_I} k={top_k}")
    got = run_indexer(d)
    torch.cuda.synchronize()
    check_idx(got, orc.prefill_indexer_topk(d), f"H_I={H_I} d_I={d_I}")


def test_indexer_ties_everywhere():
    """Operands in {0, 1/8} with unit weights: scores are small multiples of 2^-6, so nearly
    every row has a large tie at its threshold and the lowest-position rule decides it."""
    wl = gi.Workload(name="ties", L=900,
                     idx=gi.IndexerSpec(H_I=8, d_I=32, grid_lo=0, grid_hi=1, grid_step=0.125,
                                        w_choices=(1.0,), top_k=50), mqa=None, seed=5)
    d = gi.prefill_inputs(wl, with_mqa=False)
    step("indexer tie-heavy L=900 k=50")
    got = run_indexer(d)
    torch.cuda.synchronize()
    check_idx(got, orc.prefill_indexer_topk(d), "ties")


def test_indexer_zero_queries_select_first_positions():
    d = gi.prefill_inputs(gi.Workload(name="z", L=700, idx=gi.IndexerSpec(top_k=200), mqa=None),
                          with_mqa=False)
    d["q_idx"] = torch.zeros_like(d["q_idx"])
    step("indexer q_I = 0 L=700 k=200")
    got = run_indexer(d).cpu().numpy()
    for t in (0, 150, 199, 200, 699):
        n = min(200, t + 1)
        assert got[t, :n].tolist() == list(range(n)) and (got[t, n:] == -1).all()


def test_indexer_negative_weights_and_free_positions():
    """Negative power-of-two weights (exact) and arbitrary, unsorted query positions, including
    one past the last key (clamped) and a negative one (empty row)."""
    wl = gi.Workload(name="neg", L=600,
                     idx=gi.IndexerSpec(w_choices=(-1.0, -0.25, 0.5, 1.0), top_k=96), mqa=None,
                     seed=9)
    d = gi.prefill_inputs(wl, with_mqa=False)
    rows = [599, 3, 0, 300, 95, 96, 97, 451, 12, 598, 200, 201, 202, 17, 560, 433, 101]
    pos = list(rows)
    pos[-2] = 10_000   # clamped to n_keys - 1
    pos[-1] = -1       # selects nothing
    d2 = dict(d, q_idx=d["q_idx"][rows].contiguous(), w=d["w"][rows].contiguous(),
              q_pos=torch.tensor(pos, dtype=torch.int32))
    step("indexer negative w, free positions")
    got = run_indexer(d2).cpu().numpy()
    d3 = dict(d2, q_pos=torch.tensor([min(p, 599) for p in pos[:-1]] + [0], dtype=torch.int32))
    want = orc.prefill_indexer_topk(d3)
    want[-1] = -1
    check_idx(got, want, "negative w")


def test_indexer_repeatable():
    d = gi.prefill_inputs(gi.Workload(name="rep", L=3000, idx=gi.IndexerSpec(top_k=512),
                                      mqa=None), with_mqa=False)
    step("indexer repeatability L=3000")
    a = run_indexer(d)
    b = run_indexer(d)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_indexer_L8192_all_rows():
    """Indexer + top-k only, L=8192, H_I=64, d_I=128, k=2048: every row, bit-exact."""
    d = gi.prefill_inputs(gi.indexer_workload(), with_mqa=False)
    step("indexer L=8192 all rows")
    got = run_indexer(d)
    torch.cuda.synchronize()
    check_idx(got, orc.prefill_indexer_topk(d), "L=8192")


# ------------------------------------------------------------------------------ prefill MQA

def run_mqa(d, idx_dev):
    dsa = _dsa()
    dd = to_dev(d)
    return dsa.sparse_mqa_prefill(dd["q"], dd["kv"], idx_dev, dd["q_pos"], d["D_v"], d["scale"])


def test_prefill_tiny_full_path():
    d = gi.prefill_inputs(gi.tiny_workload())
    step("prefill tiny: indexer + MQA, D_k=D_v=64 (V=K), H=8")
    idx = run_indexer(d)
    o, lse = run_mqa(d, idx)
    torch.cuda.synchronize()
    i_ref, o_ref, l_ref = orc.prefill(d)
    check_idx(idx, i_ref, "tiny idx")
    check_attn(o, lse, o_ref, l_ref, "tiny attn")


@pytest.mark.parametrize("D_k,D_v,H,L,top_k,sharp", [
    (96, 64, 8, 200, 40, True),
    (64, 64, 16, 300, 300, True),
    (576, 512, 128, 300, 64, False),
    (576, 512, 128, 300, 64, True),
    (576, 512, 128, 2100, 2048, True),
    (576, 512, 100, 500, 256, True),
    (64, 64, 1, 100, 50, True),        # a single head: one wave active
    (96, 64, 33, 150, 40, True),       # heads end inside a wave
])
def test_mqa_shapes(D_k, D_v, H, L, top_k, sharp):
    wl = gi.Workload(name="m", L=L,
                     idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=top_k),
                     mqa=gi.MqaSpec(H=H, D_k=D_k, D_v=D_v, sigma=1.0 if sharp else D_k ** -0.5,
                                    scale=D_k ** -0.5), seed=11)
    d = gi.prefill_inputs(wl)
    step(f"mqa D_k={D_k} D_v={D_v} H={H} L={L} k={top_k} sharp={sharp}")
    idx = run_indexer(d)
    o, lse = run_mqa(d, idx)
    torch.cuda.synchronize()
    rows = list(range(0, L, max(1, L // 40))) + [L - 1]
    i_ref, o_ref, l_ref = orc.prefill(d, rows=rows)
    check_idx(idx[rows], i_ref, "idx")
    check_attn(o[rows], lse[rows], o_ref, l_ref, "attn")


def test_mqa_skips_invalid_entries_and_empty_rows():
    wl = gi.Workload(name="inv", L=400, idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=96),
                     mqa=gi.MqaSpec(sigma=1.0), seed=13)
    d = gi.prefill_inputs(wl)
    idx = run_indexer(d).cpu()
    bad = idx.clone()
    bad[50, 3] = -1
    bad[60, :10] = 399          # beyond t = 60: skipped
    bad[70, 5] = -7
    bad[80, :] = -1             # nothing attended: o = 0, lse = -inf
    bad[90, 1] = 100000         # out of the kv range
    # whole 32-entry chunks without a valid entry: in the middle of the list (still computed,
    # valid entries follow), at its end (not gathered), and before the only valid chunk
    bad[95, 32:64] = -1
    bad[96, 41:] = -1
    bad[97, :64] = -1
    step("mqa invalid entries")
    o, lse = run_mqa(d, bad.cuda())
    torch.cuda.synchronize()
    rows = [50, 60, 70, 80, 90, 91, 95, 96, 97]
    _, o_ref, l_ref = orc.prefill(d, rows=rows, idx=bad[rows].numpy())
    check_attn(o[rows], lse[rows], o_ref, l_ref, "invalid")
    assert (o[80] == 0).all() and torch.isneginf(lse[80]).all()


def test_mqa_kv_array_over_2gib():
    """A KV array larger than 2 GiB (rows addressed with 64-bit offsets), rows selected on both
    sides of the 2 GiB mark."""
    dsa = _dsa()
    n_kv, H, D_k, D_v, top_k, n_q = 1_900_000, 128, 576, 512, 96, 3
    g = torch.Generator().manual_seed(21)
    hi0 = (1 << 31) // (2 * D_k) + 1           # first row wholly past 2 GiB
    idx = torch.empty((n_q, top_k), dtype=torch.int32)
    for i in range(n_q):
        lo = torch.randperm(hi0, generator=g)[: top_k // 2]
        hi = hi0 + torch.randperm(n_kv - hi0, generator=g)[: top_k - top_k // 2]
        idx[i] = torch.cat([lo, hi]).to(torch.int32)
    rows = torch.unique(idx.flatten().long())
    vals = torch.randn((rows.numel(), D_k), generator=g).to(torch.bfloat16)
    q = (torch.randn((n_q, H, D_k), generator=g) * 0.3).to(torch.bfloat16)
    step(f"mqa kv over 2 GiB: n_kv={n_kv} rows, D_k={D_k}, k={top_k}")
    kv = torch.zeros((n_kv, D_k), dtype=torch.bfloat16, device="cuda")
    kv[rows.cuda()] = vals.cuda()
    q_pos = torch.full((n_q,), n_kv - 1, dtype=torch.int32)
    scale = D_k ** -0.5
    o, lse = dsa.sparse_mqa_prefill(q.cuda(), kv, idx.cuda(), q_pos.cuda(), D_v, scale)
    torch.cuda.synchronize()
    pos = {int(r): k for k, r in enumerate(rows.tolist())}
    o_ref = np.zeros((n_q, H, D_v))
    l_ref = np.zeros((n_q, H))
    for i in range(n_q):
        sel = vals[[pos[int(r)] for r in idx[i].tolist()]].double().numpy()
        o_ref[i], l_ref[i] = orc.sparse_mqa(q[i].double().numpy(), sel, D_v, scale)
    check_attn(o, lse, o_ref, l_ref, "kv > 2 GiB")
    del kv


def test_prefill_L32768_sharp_sampled():
    wl = gi.prefill_workload(32768, sharp=True)
    step("prefill L=32768 sharp: generate on device")
    d = gi.prefill_inputs(wl, device="cuda", rows=(30000, 300))
    step("prefill L=32768 sharp: indexer + MQA")
    idx = run_indexer(d)
    o, lse = run_mqa(d, idx)
    torch.cuda.synchronize()
    rows = [0, 150, 299]
    i_ref, o_ref, l_ref = orc.prefill(d, rows=rows)
    check_idx(idx[rows], i_ref, "sharp idx")
    err = check_attn(o[rows], lse[rows], o_ref, l_ref, "sharp attn")
    assert np.abs(o_ref).max() > 0.1 and err < 5e-3


# ------------------------------------------------------------------------------ decode

def run_decode(d, n_split=0):
    dsa = _dsa()
    dd = to_dev(d)
    idx = dsa.indexer_topk_paged(dd["q_idx"], dd["w"], dd["k_cache"], dd["page_table"],
                                 dd["ctx"], d["top_k"])
    o, lse = dsa.sparse_mqa_decode(dd["q"], dd["kv_cache"], dd["page_table"], dd["ctx"], idx,
                                   d["D_v"], d["scale"], n_split=n_split)
    return idx, o, lse


@pytest.mark.parametrize("page_size,top_k,ctx,n_split,small_idx", [
    (64, 2048, (4096, 5000, 2100, 9000), 0, False),
    (64, 256, (300, 64, 1, 1000, 777), 0, False),
    (16, 512, (513, 2000, 100), 3, False),
    (64, 2048, (2047, 2048, 2049, 130), 1, False),
    (32, 64, (3000, 65, 700), 0, True),     # H_I = 4, d_I = 32: partial MFMA operands
    (64, 128, (0, 200, 0, 70, 64), 0, False),  # empty rows between scored ones
])
def test_decode_small(page_size, top_k, ctx, n_split, small_idx):
    ix = gi.IndexerSpec(top_k=top_k)
    if small_idx:
        ix = gi.IndexerSpec(H_I=4, d_I=32, grid_lo=-3, grid_hi=3, grid_step=0.125,
                            w_choices=(0.25, 0.5, 1.0), top_k=top_k)
    sp = gi.DecodeSpec(B=len(ctx), page_size=page_size, idx=ix,
                       mqa=gi.MqaSpec(sigma=1.0), spare_pages=5, seed=21)
    d = gi.decode_inputs(sp, ctx_lens=ctx)
    step(f"decode P={page_size} k={top_k} ctx={ctx} split={n_split}")
    idx, o, lse = run_decode(d, n_split)
    torch.cuda.synchronize()
    i_ref, o_ref, l_ref = orc.decode(d)
    check_idx(idx, i_ref, "decode idx")
    check_attn(o, lse, o_ref, l_ref, "decode attn")


@pytest.mark.parametrize("D_k,D_v,H", [(96, 64, 20), (64, 64, 128)])
def test_decode_small_shapes(D_k, D_v, H):
    sp = gi.DecodeSpec(B=3, page_size=64, idx=gi.IndexerSpec(top_k=128),
                       mqa=gi.MqaSpec(H=H, D_k=D_k, D_v=D_v, sigma=1.0, scale=D_k ** -0.5),
                       spare_pages=3, seed=5)
    d = gi.decode_inputs(sp, ctx_lens=(700, 129, 2000))
    step(f"decode shapes D_k={D_k} D_v={D_v} H={H}")
    for n_split in (1, 2):
        idx, o, lse = run_decode(d, n_split)
        torch.cuda.synchronize()
        i_ref, o_ref, l_ref = orc.decode(d)
        check_idx(idx, i_ref, "decode idx")
        check_attn(o, lse, o_ref, l_ref, f"decode attn split={n_split}")


def test_decode_ties_large_candidate_list():
    """All scores of sequence 0 tie (zero query): the threshold bin holds every key, more than
    the selection stages on chip, so the exact tie-break runs over the whole list."""
    sp = gi.DecodeSpec(B=3, idx=gi.IndexerSpec(top_k=2048), mqa=gi.MqaSpec(sigma=1.0), seed=29)
    d = gi.decode_inputs(sp, ctx_lens=(20000, 5000, 13000))
    d["q_idx"][0].zero_()
    d["w"][2] = -d["w"][2]          # all scores <= 0: the selection runs over non-positive keys
    step("decode ties / large candidate list")
    idx, o, lse = run_decode(d)
    torch.cuda.synchronize()
    i_ref, o_ref, l_ref = orc.decode(d)
    assert np.array_equal(i_ref[0], np.arange(2048))
    check_idx(idx, i_ref, "decode ties idx")
    check_attn(o, lse, o_ref, l_ref, "decode ties attn")


def test_decode_equals_prefill_last_row():
    sp = gi.DecodeSpec(B=3, idx=gi.IndexerSpec(top_k=2048), mqa=gi.MqaSpec(sigma=1.0), seed=23)
    d = gi.decode_inputs(sp, ctx_lens=(3000, 4500, 2048))
    step("decode vs prefill last row")
    idx, o, lse = run_decode(d)
    dsa = _dsa()
    P = d["page_size"]
    for b, n in enumerate(d["ctx"].tolist()):
        s = torch.arange(n)
        pages = d["page_table"][b][s // P].long()
        pre = {"q_idx": d["q_idx"][b:b + 1], "w": d["w"][b:b + 1],
               "k_idx": d["k_cache"][pages, s % P].contiguous(),
               "q_pos": torch.tensor([n - 1], dtype=torch.int32), "top_k": 2048,
               "q": d["q"][b:b + 1], "kv": d["kv_cache"][pages, s % P].contiguous(),
               "D_v": d["D_v"], "scale": d["scale"]}
        pi = run_indexer(pre)
        po, pl = run_mqa(pre, pi)
        torch.cuda.synchronize()
        assert torch.equal(pi[0].cpu(), idx[b].cpu())
        assert (po[0].float() - o[b].float()).abs().max().item() <= 2e-3
        assert (pl[0] - lse[b]).abs().max().item() <= 1e-4


def test_decode_row_longer_than_position_bitmap():
    """A row of 270000 keys: more positions than the selection's on-chip bitmap covers
    (2^18), so the selected positions are listed and sorted instead."""
    sp = gi.DecodeSpec(B=2, idx=gi.IndexerSpec(top_k=2048), mqa=gi.MqaSpec(sigma=1.0),
                       spare_pages=2, seed=37)
    d = gi.decode_inputs(sp, ctx_lens=(270000, 3000))
    step("decode: a row beyond the position bitmap (270000 keys)")
    idx, o, lse = run_decode(d)
    torch.cuda.synchronize()
    i_ref, o_ref, l_ref = orc.decode(d)
    check_idx(idx, i_ref, "long row idx")
    check_attn(o, lse, o_ref, l_ref, "long row attn")


def test_decode_page_table_entries_outside_the_pool():
    """Page-table entries outside [0, n_pages) inside a context: the indexer scores their keys
    as zero keys and the attention skips them.  Reference: the same step with those pages
    pointing at an all-zero k_I page (indexer), and those positions dropped (attention)."""
    sp = gi.DecodeSpec(B=3, idx=gi.IndexerSpec(top_k=512), mqa=gi.MqaSpec(sigma=1.0),
                       spare_pages=2, seed=41)
    d = gi.decode_inputs(sp, ctx_lens=(3000, 5000, 1000))
    P, n_pages = d["page_size"], d["n_pages"]
    bad = [(0, 5, -1), (1, 10, n_pages + 3), (1, 11, 1 << 30), (2, 0, -7)]
    pt = d["page_table"].clone()
    for b, j, v in bad:
        pt[b, j] = v
    d_bad = dict(d, page_table=pt)
    step("decode: page-table entries outside the pool")
    idx, o, lse = run_decode(d_bad)
    torch.cuda.synchronize()
    # indexer reference: the bad entries point at an extra all-zero k_I page
    pt_z = pt.clone()
    for b, j, v in bad:
        pt_z[b, j] = n_pages
    kz = torch.cat([d["k_cache"], torch.zeros_like(d["k_cache"][:1])])
    d_z = dict(d, page_table=pt_z, k_cache=kz)
    i_ref, _, _ = orc.decode(d_z)
    check_idx(idx, i_ref, "bad pages idx")
    # attention reference: positions on bad pages are not attended
    drop = np.array(i_ref, copy=True)
    for b, j, v in bad:
        on_bad = (drop[b] >= j * P) & (drop[b] < (j + 1) * P)
        drop[b][on_bad] = -1
    _, o_ref, l_ref = orc.decode(d_bad, idx=drop)
    check_attn(o, lse, o_ref, l_ref, "bad pages attn")


def test_binding_rejects_bad_outputs_before_launch():
    """Caller-supplied outputs of the wrong shape, dtype or device, and a host workspace, are
    refused by the binding before anything is enqueued."""
    dsa = _dsa()
    d = to_dev(gi.prefill_inputs(gi.tiny_workload()))
    k = d["top_k"]
    n_q = d["q_idx"].shape[0]
    bad_outs = [torch.empty((n_q, k + 1), dtype=torch.int32, device="cuda"),
                torch.empty((n_q - 1, k), dtype=torch.int32, device="cuda"),
                torch.empty((n_q, k), dtype=torch.int64, device="cuda"),
                torch.empty((n_q, k), dtype=torch.int32)]
    for out in bad_outs:
        with pytest.raises((ValueError, TypeError)):
            dsa.indexer_topk(d["q_idx"], d["w"], d["k_idx"], d["q_pos"], k, out=out)
    with pytest.raises(ValueError):
        dsa.indexer_topk(d["q_idx"], d["w"], d["k_idx"], d["q_pos"], k,
                         workspace=torch.empty(1 << 20, dtype=torch.uint8))
    idx = dsa.indexer_topk(d["q_idx"], d["w"], d["k_idx"], d["q_pos"], k)
    H, D_v = d["q"].shape[1], d["D_v"]
    for out, lse in [(torch.empty((n_q, H, D_v - 16), dtype=torch.bfloat16, device="cuda"), None),
                     (None, torch.empty((n_q, H - 1), dtype=torch.float32, device="cuda")),
                     (None, torch.empty((n_q, H), dtype=torch.float32))]:
        with pytest.raises((ValueError, TypeError)):
            dsa.sparse_mqa_prefill(d["q"], d["kv"], idx, d["q_pos"], D_v, d["scale"], out=out,
                                   lse=lse)
    torch.cuda.synchronize()

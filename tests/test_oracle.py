"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped ReLU or weight, a wrong
sign, a transposed operand, the wrong tie-break, an off-by-one causal bound, K and V swapped)
fails at least one of them; ``test_planted_mistakes_are_caught`` plants such slips and checks.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import brute
from oracle import dsa_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- number formats

def test_e4m3fn_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = orc.decode_e4m3fn(codes)
    nan_ref, nan_mine = np.isnan(ref), np.isnan(mine)
    assert (nan_ref == nan_mine).all()
    assert nan_mine.sum() == 2                      # 0x7F and 0xFF
    assert np.array_equal(ref[~nan_ref], mine[~nan_mine])
    assert orc.decode_e4m3fn(np.array([0x7E]))[0] == 448.0
    assert orc.decode_e4m3fn(np.array([0x01]))[0] == 2.0 ** -9


def test_e4m3fn_brute_field_decoder_agrees():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert float(brute.e4m3fn_value(c)) == orc.E4M3FN[c]


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(4096, generator=g) * torch.exp(torch.randn(4096, generator=g) * 10)
    xb = x.to(torch.bfloat16)
    ref = xb.to(torch.float64).numpy()
    assert np.array_equal(orc.decode_bf16(xb), ref)
    bits = xb.view(torch.int16).numpy()
    assert all(brute.bf16_value(int(b) & 0xFFFF) == r for b, r in zip(bits[:64], ref[:64]))


# --------------------------------------------------------------------------- step 1: scores

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_scores_handworked_example():
    g = _golden("indexer_handworked.json")
    sc = orc.indexer_scores(np.array(g["q_I"]), np.array(g["w"]), np.array(g["k_I"])[: g["t"] + 1])
    assert sc.tolist() == g["scores"]
    for k, want in g["topk"].items():
        assert orc.topk_select(sc, int(k)).tolist() == want


def _tiny_grid(seed, L=48, H_I=3, d_I=8, lo=-3, hi=3, w=(0.25, 0.5, 1.0, -0.5)):
    q = gi.grid_fp8((H_I, d_I), lo, hi, 0.125, seed, 101)
    k = gi.grid_fp8((L, d_I), lo, hi, 0.125, seed, 102)
    ww = gi.choice_f32((H_I,), w, seed, 103)
    return q, k, ww


@pytest.mark.parametrize("seed", range(6))
def test_scores_equal_exact_rational_brute_force(seed):
    q, k, w = _tiny_grid(seed)
    t = 40
    mine = orc.indexer_scores(orc.decode_e4m3fn(q), w.numpy().astype(np.float64),
                              orc.decode_e4m3fn(k)[: t + 1])
    exact = brute.scores(q.tolist(), w.tolist(), k.tolist(), t)
    assert [float(x) for x in exact] == mine.tolist()      # exact on the dyadic grid


def test_scores_single_head_unit_weight_is_relu_of_matmul():
    q, k, _ = _tiny_grid(11, H_I=1)
    qf = q.view(torch.float8_e4m3fn).to(torch.float64)
    kf = k.view(torch.float8_e4m3fn).to(torch.float64)
    ref = torch.relu(kf @ qf[0]).numpy()
    mine = orc.indexer_scores(orc.decode_e4m3fn(q), np.ones(1), orc.decode_e4m3fn(k))
    assert np.array_equal(mine, ref)


def test_scores_weighted_heads_match_library_einsum():
    q, k, w = _tiny_grid(12, H_I=5, d_I=16)
    qf = q.view(torch.float8_e4m3fn).to(torch.float64)
    kf = k.view(torch.float8_e4m3fn).to(torch.float64)
    ref = (torch.relu(torch.einsum("jd,sd->sj", qf, kf)) * w.to(torch.float64)).sum(1).numpy()
    mine = orc.indexer_scores(orc.decode_e4m3fn(q), w.numpy().astype(np.float64), orc.decode_e4m3fn(k))
    assert np.array_equal(mine, ref)


def test_scores_are_exact_in_fp32_on_production_grid():
    """Dyadic grid {-2..2}/8, w in 2^{-4..0}, d_I=128, H_I=64: every score is a multiple of
    2^-10 of magnitude <= 512, hence fp32-exact in any summation order."""
    wl = gi.indexer_workload()
    d = gi.prefill_inputs(gi.Workload(name="x", L=600, idx=wl.idx, mqa=None))
    qi, ki = orc.decode_e4m3fn(d["q_idx"]), orc.decode_e4m3fn(d["k_idx"])
    w = d["w"].numpy().astype(np.float64)
    for t in (0, 17, 599):
        sc = orc.indexer_scores(qi[t], w[t], ki[: t + 1])
        assert np.all(sc * 1024 == np.round(sc * 1024)) and np.all(np.abs(sc) <= 512)
        assert np.array_equal(sc.astype(np.float32).astype(np.float64), sc)
        # a reversed-order fp32 sum gives the same values
        x = (ki[: t + 1] @ qi[t].T).astype(np.float32)
        acc = np.zeros(t + 1, dtype=np.float32)
        for j in reversed(range(qi.shape[1])):
            acc += np.float32(w[t, j]) * np.maximum(x[:, j], np.float32(0))
        assert np.array_equal(acc.astype(np.float64), sc)


# --------------------------------------------------------------------------- step 2: top-k

@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("k", [1, 3, 7, 20, 64])
def test_topk_equals_counting_definition(seed, k):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    sc = rng.integers(-3, 4, n).astype(np.float64) * 0.5     # many ties
    sc[rng.random(n) < 0.2] = -0.0                           # signed zeros tie with +0
    want = brute.topk(sc.tolist(), k)
    got = orc.topk_select(sc, k)
    assert got[: len(want)].tolist() == want
    assert (got[len(want):] == -1).all()


@pytest.mark.parametrize("seed", range(4))
def test_topk_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    n, k = 500, 37
    sc = rng.integers(0, 30, n).astype(np.float64)
    sel = orc.topk_select(sc, k)
    assert (sel[: min(k, n)] >= 0).all() and len(set(sel.tolist())) == k
    mask = np.zeros(n, bool)
    mask[sel] = True
    assert sc[mask].min() >= sc[~mask].max()
    thr = sc[mask].min()
    tied = np.flatnonzero(sc == thr)
    kept_tied = np.flatnonzero(mask & (sc == thr))
    assert kept_tied.tolist() == tied[: len(kept_tied)].tolist()      # lowest positions win
    # nesting: the top-k is contained in the top-(k+10)
    assert set(sel.tolist()) <= set(orc.topk_select(sc, k + 10).tolist())
    # fewer candidates than k: all of them, then -1
    few = orc.topk_select(sc[:5], k)
    assert few[:5].tolist() == [0, 1, 2, 3, 4] and (few[5:] == -1).all()


def test_zero_query_gives_first_positions():
    """q_I = 0 makes every score 0, so the selection is positions 0..n-1 (closed form)."""
    d = gi.prefill_inputs(gi.tiny_workload(), with_mqa=False)
    d["q_idx"] = torch.zeros_like(d["q_idx"])
    idx = orc.prefill_indexer_topk(d, rows=[0, 5, 31, 32, 255])
    for r, t in enumerate([0, 5, 31, 32, 255]):
        n = min(32, t + 1)
        assert idx[r, :n].tolist() == list(range(n)) and (idx[r, n:] == -1).all()


# --------------------------------------------------------------------------- step 3: attention

def test_attention_handworked_example():
    g = _golden("attention_handworked.json")
    kv = np.array([[4.0, 0.0], [8.0, math.log(3.0)]])
    o, lse = orc.sparse_mqa(np.array(g["q"]), kv, g["d_v"], g["scale"])
    assert abs(o[0, 0] - 7.0) < 1e-12 and abs(lse[0] - math.log(4.0)) < 1e-12


@pytest.mark.parametrize("D_k,D_v", [(64, 64), (96, 64)])
def test_full_selection_equals_dense_causal_sdpa(D_k, D_v):
    """With k >= t + 1 every earlier key is selected, so DSA is dense causal attention."""
    L, H = 40, 3
    wl = gi.Workload(name="t", L=L,
                     idx=gi.IndexerSpec(H_I=2, d_I=16, grid_lo=-3, grid_hi=3, grid_step=0.125,
                                        w_choices=(0.5, 1.0), top_k=L),
                     mqa=gi.MqaSpec(H=H, D_k=D_k, D_v=D_v, sigma=1.0, scale=D_k ** -0.5))
    d = gi.prefill_inputs(wl)
    idx, o, lse = orc.prefill(d)
    assert (idx[np.arange(L), np.arange(L)] == np.arange(L)).all()   # diagonal: s = t kept
    q = d["q"].to(torch.float64).permute(1, 0, 2)                      # [H, L, D_k]
    kv = d["kv"].to(torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, kv[None, :, :].expand(H, L, D_k).contiguous(),
        kv[None, :, :D_v].expand(H, L, D_v).contiguous(), is_causal=True, scale=D_k ** -0.5)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    zz = torch.einsum("hld,sd->hls", q, kv) * D_k ** -0.5
    zz = zz.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), -math.inf)
    assert np.allclose(lse, torch.logsumexp(zz, -1).T.numpy(), rtol=0, atol=1e-12)


def test_sparse_attention_equals_brute_masked_dense_attention():
    wl = gi.tiny_workload()
    wl.L = 80
    d = gi.prefill_inputs(wl)
    rows = [0, 10, 31, 32, 50, 79]
    idx, o, lse = orc.prefill(d, rows=rows)
    qb = d["q"].view(torch.int16).numpy()
    kvb = d["kv"].view(torch.int16).numpy()
    kv_rows = [[brute.bf16_value(int(x)) for x in r] for r in kvb]
    for r, t in enumerate(rows):
        keep = brute.topk(brute.scores(d["q_idx"][t].tolist(), d["w"][t].tolist(),
                                       d["k_idx"].tolist(), t), 32)
        assert idx[r][idx[r] >= 0].tolist() == keep
        qr = [[brute.bf16_value(int(x)) for x in hrow] for hrow in qb[t]]
        bo, bl = brute.masked_attention(qr, kv_rows, t, keep, 64, 1 / 8)
        assert np.allclose(o[r], np.array(bo), rtol=0, atol=1e-12)
        assert np.allclose(lse[r], np.array(bl), rtol=0, atol=1e-12)


def test_attention_invariants():
    rng = np.random.default_rng(3)
    H, m, D_k, D_v = 4, 30, 24, 16
    q = rng.standard_normal((H, D_k))
    kv = rng.standard_normal((m, D_k))
    o, lse = orc.sparse_mqa(q, kv, D_v, 0.3)
    # permutation of the selected rows changes nothing (to rounding)
    perm = rng.permutation(m)
    o2, lse2 = orc.sparse_mqa(q, kv[perm], D_v, 0.3)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)
    # probabilities sum to one: sum_s exp(z_s - lse) == 1
    z = 0.3 * q @ kv.T
    assert np.allclose(np.exp(z - lse[:, None]).sum(1), 1.0, atol=1e-13)
    # constant V rows give that constant
    kvc = kv.copy()
    kvc[:, :D_v] = 2.5
    oc, _ = orc.sparse_mqa(q, kvc, D_v, 0.3)
    assert np.allclose(oc, 2.5, atol=1e-13)
    # one dominant logit picks that row's V
    kvd = kv.copy()
    kvd[7, D_v:] = 200.0 * np.sign(q[0, D_v:])
    od, _ = orc.sparse_mqa(q[:1], kvd, D_v, 1.0)
    assert np.allclose(od[0], kvd[7, :D_v], atol=1e-9)
    # empty selection
    oe, le = orc.sparse_mqa(q, kv[:0], D_v, 0.3)
    assert (oe == 0).all() and np.isneginf(le).all()


def test_invalid_indices_are_skipped():
    d = gi.prefill_inputs(gi.tiny_workload())
    idx, o, lse = orc.prefill(d, rows=[40])
    bad = idx.copy()
    bad[0, 5] = -1            # drop one entry
    bad[0, 6] = 41            # beyond t = 40: ignored
    _, o2, _ = orc.prefill(d, rows=[40], idx=bad)
    keep = [s for s in idx[0].tolist() if s not in (idx[0, 5], idx[0, 6])]
    _, o3, _ = orc.prefill(d, rows=[40], idx=np.array([keep + [-1] * (32 - len(keep))]))
    assert np.allclose(o2, o3, atol=0)


# --------------------------------------------------------------------------- decode

def _tiny_decode(seed, page_size=16, ctx=(37, 100, 64, 1)):
    sp = gi.DecodeSpec(B=len(ctx), page_size=page_size, spare_pages=3,
                       idx=gi.IndexerSpec(H_I=4, d_I=32, grid_lo=-3, grid_hi=3, grid_step=0.125,
                                          w_choices=(0.25, 0.5, 1.0), top_k=32),
                       mqa=gi.MqaSpec(H=8, D_k=96, D_v=64, sigma=1.0, scale=96 ** -0.5))
    return gi.decode_inputs(sp, seed=seed, ctx_lens=ctx)


def test_decode_equals_prefill_last_row():
    d = _tiny_decode(0)
    idx, o, lse = orc.decode(d)
    P = d["page_size"]
    for b, n in enumerate(d["ctx"].tolist()):
        pt = d["page_table"][b]
        s = torch.arange(n)
        k_rows = d["k_cache"][pt[s // P].long(), s % P]
        kv_rows = d["kv_cache"][pt[s // P].long(), s % P]
        pre = {"q_idx": d["q_idx"][b:b + 1], "w": d["w"][b:b + 1], "k_idx": k_rows,
               "q_pos": torch.tensor([n - 1], dtype=torch.int32), "top_k": d["top_k"],
               "q": d["q"][b:b + 1], "kv": kv_rows, "D_v": d["D_v"], "scale": d["scale"]}
        i2, o2, l2 = orc.prefill(pre)
        assert np.array_equal(i2[0], idx[b])
        assert np.allclose(o2[0], o[b], atol=1e-13) and np.allclose(l2[0], lse[b], atol=1e-13)


def test_decode_invariant_under_page_permutation():
    d = _tiny_decode(1)
    idx, o, lse = orc.decode(d)
    ctx = d["ctx"].tolist()
    pt_id, n_used = gi.identity_page_table(ctx, d["page_size"])
    kc = torch.zeros((n_used,) + tuple(d["k_cache"].shape[1:]), dtype=torch.uint8)
    kvc = torch.zeros((n_used,) + tuple(d["kv_cache"].shape[1:]), dtype=torch.bfloat16)
    P = d["page_size"]
    for b, n in enumerate(ctx):
        s = torch.arange(n)
        src = d["page_table"][b][s // P].long()
        kc[pt_id[b][s // P].long(), s % P] = d["k_cache"][src, s % P]
        kvc[pt_id[b][s // P].long(), s % P] = d["kv_cache"][src, s % P]
    d2 = dict(d, page_table=pt_id, k_cache=kc, kv_cache=kvc, n_pages=n_used)
    i2, o2, l2 = orc.decode(d2)
    assert np.array_equal(idx, i2) and np.array_equal(o, o2) and np.array_equal(lse, l2)


# --------------------------------------------------------------------------- cache write

def _all_bf16():
    return torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)


def test_quantize_e4m3fn_matches_torch_cast_on_every_bf16_value():
    """Every bf16 bit pattern: the saturating quantiser equals torch's (round-to-nearest-even)
    e4m3fn cast of the value clamped to [-448, 448]; NaNs give the NaN code with their sign."""
    allb = _all_bf16()
    v = allb.double().numpy()
    q = orc.quantize_e4m3fn(v)
    fin = ~np.isnan(v)
    ref = allb.float().clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[fin], ref[fin])
    assert set(np.unique(q[~fin]).tolist()) == {0x7F, 0xFF}
    assert orc.quantize_e4m3fn(np.array([-0.0]))[0] == 0x80
    assert orc.quantize_e4m3fn(np.array([np.inf, -np.inf, 1e30])).tolist() == [0x7E, 0xFE, 0x7E]


def test_quantize_e4m3fn_equals_exact_nearest_brute_force():
    """Against the exact-distance search over all codes (Fractions): every midpoint between
    neighbouring codes (the ties), points just off them, and a spread of bf16 values."""
    from fractions import Fraction
    vals = [brute.e4m3fn_value(c) for c in range(0x7F)]
    pts = []
    for a, b in zip(vals, vals[1:]):
        mid = (a + b) / 2
        pts += [mid, mid + Fraction(1, 2 ** 20), mid - Fraction(1, 2 ** 20)]
    g = torch.Generator().manual_seed(3)
    pick = torch.randint(0, 65536, (600,), generator=g)
    for b in _all_bf16()[pick].double().numpy():
        if np.isfinite(b):
            pts.append(Fraction(float(b)))
    pts += [-p for p in pts[:50]] + [Fraction(448), Fraction(470), Fraction(480), Fraction(10 ** 6)]
    got = orc.quantize_e4m3fn(np.array([float(p) for p in pts]))
    want = [brute.nearest_e4m3fn(p) for p in pts]
    assert got.tolist() == want


def test_cache_append_writes_the_slots_and_nothing_else():
    """The appended rows come back through the page table as the quantised keys and the exact
    KV rows; every other byte is unchanged; rows with an invalid slot write nothing; the result
    equals a scatter written with torch's indexing (a library data move)."""
    g = torch.Generator().manual_seed(7)
    P, n_pages, d_I, D_k = 8, 12, 16, 24
    kc = torch.randint(0, 256, (n_pages, P, d_I), generator=g, dtype=torch.int32).to(torch.uint8)
    kvc = torch.randn((n_pages, P, D_k), generator=g).to(torch.bfloat16)
    pt = torch.tensor([[3, 7, 1, -1], [0, 11, 5, 40]], dtype=torch.int32)
    seq = torch.tensor([0, 1, 0, 1, 1, 0, 1], dtype=torch.int32)
    pos = torch.tensor([0, 9, 20, 23, 31, -2, 25], dtype=torch.int32)   # last three invalid
    T = pos.shape[0]
    k_new = (torch.randn((T, d_I), generator=g) * 3).to(torch.bfloat16)
    kv_new = torch.randn((T, D_k), generator=g).to(torch.bfloat16)
    kc2, kvc2 = orc.cache_append(kc, kvc, pt, seq, pos, k_new, kv_new)
    ref_k, ref_kv = kc.clone(), kvc.clone()
    q = orc.quantize_e4m3fn(orc.decode_bf16(k_new))
    for r in range(4):
        b, p = int(seq[r]), int(pos[r])
        page = int(pt[b, p // P])
        ref_k[page, p % P] = torch.from_numpy(q[r])
        ref_kv[page, p % P] = kv_new[r]
        assert np.array_equal(orc.paged_gather(kc2, pt[b], [p], P)[0], q[r])
    assert np.array_equal(kc2, ref_k.numpy())
    assert np.array_equal(kvc2, ref_kv.view(torch.int16).numpy())
    assert np.array_equal(orc.decode_e4m3fn(q), orc.decode_e4m3fn(
        k_new.float().clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)))


# --------------------------------------------------------------------------- dense baseline

@pytest.mark.parametrize("D_k,D_v", [(64, 64), (96, 64)])
def test_dense_prefill_equals_causal_sdpa(D_k, D_v):
    """The dense baseline is torch's causal scaled_dot_product_attention (fp64, CPU) with every
    head reading the one shared row (K = the row, V = its first D_v dims)."""
    wl = gi.Workload(name="d", L=90, idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=8),
                     mqa=gi.MqaSpec(H=3, D_k=D_k, D_v=D_v, sigma=1.0, scale=D_k ** -0.5), seed=4)
    d = gi.prefill_inputs(wl)
    o, lse = orc.dense_prefill(d)
    q = d["q"].double().permute(1, 0, 2)                      # [H, L, D_k]
    kv = d["kv"].double()
    k = kv[None].expand(3, -1, -1)
    v = kv[None, :, :D_v].expand(3, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                           scale=D_k ** -0.5)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    z = (q @ k.transpose(1, 2)) * D_k ** -0.5
    z = z.masked_fill(torch.triu(torch.ones(90, 90, dtype=torch.bool), 1), float("-inf"))
    assert np.allclose(lse, torch.logsumexp(z, -1).T.numpy(), rtol=0, atol=1e-12)


def test_dense_decode_equals_dense_prefill_last_row():
    sp = gi.DecodeSpec(B=2, idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=8),
                       mqa=gi.MqaSpec(H=2, D_k=64, D_v=64, sigma=1.0, scale=0.125), seed=6)
    d = gi.decode_inputs(sp, ctx_lens=(150, 77))
    o, lse = orc.dense_decode(d)
    P = d["page_size"]
    for b, n in enumerate(d["ctx"].tolist()):
        s = torch.arange(n)
        pages = d["page_table"][b][s // P].long()
        pre = {"q": d["q"][b:b + 1], "kv": d["kv_cache"][pages, s % P], "D_v": 64,
               "scale": 0.125, "q_pos": torch.tensor([n - 1])}
        o2, l2 = orc.dense_prefill(pre)
        assert np.allclose(o[b], o2[0], rtol=0, atol=1e-13)
        assert np.allclose(lse[b], l2[0], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- indexer KL

def test_kl_matches_torch_kl_div_and_is_zero_at_the_target():
    g = torch.Generator().manual_seed(11)
    sc = torch.randn(300, generator=g, dtype=torch.float64) * 3
    tgt = torch.softmax(torch.randn(300, generator=g, dtype=torch.float64) * 2, 0)
    tgt[:7] = 0
    tgt /= tgt.sum()
    loss, grad = orc.kl_from_scores(sc.numpy(), tgt.numpy())
    ref = torch.nn.functional.kl_div(torch.log_softmax(sc, 0), tgt, reduction="sum")
    assert abs(loss - ref.item()) <= 1e-12 * max(1.0, abs(ref.item()))
    assert loss > 0
    # scores equal to log(target) + c (target > 0 everywhere): the indexer matches, loss 0
    t2 = torch.softmax(sc, 0).numpy()
    l0, g0 = orc.kl_from_scores(np.log(t2) + 4.0, t2)
    assert abs(l0) <= 1e-12 and np.abs(g0).max() <= 1e-12


def test_kl_gradient_equals_finite_differences():
    g = torch.Generator().manual_seed(12)
    sc = (torch.randn(40, generator=g, dtype=torch.float64) * 2).numpy()
    tgt = torch.softmax(torch.randn(40, generator=g, dtype=torch.float64), 0).numpy()
    _, grad = orc.kl_from_scores(sc, tgt)
    h = 1e-6
    num = np.array([(orc.kl_from_scores(sc + h * np.eye(40)[e], tgt)[0] -
                     orc.kl_from_scores(sc - h * np.eye(40)[e], tgt)[0]) / (2 * h)
                    for e in range(40)])
    assert np.abs(num - grad).max() <= 1e-7


def test_indexer_kl_target_is_the_head_mean_of_softmax():
    """The target of a row is the mean over heads of torch's softmax of the scaled logits over
    the listed rows; it sums to 1; entries not in the list (-1, > t) get nothing."""
    wl = gi.Workload(name="kl", L=120, idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=24),
                     mqa=gi.MqaSpec(H=5, D_k=64, D_v=64, sigma=1.0, scale=0.125), seed=8)
    d = gi.prefill_inputs(wl)
    idx = orc.prefill_indexer_topk(d)
    idx[100, 3] = -1
    idx[100, 4] = 119           # beyond t = 100: not in the list
    loss, target, grad = orc.indexer_kl(d, idx, rows=None)
    for t in (5, 30, 100, 119):
        lst = [(e, s) for e, s in enumerate(idx[t]) if 0 <= s <= t]
        s = torch.tensor([x for _, x in lst])
        z = d["q"][t].double() @ d["kv"][s].double().T * 0.125
        ref = torch.softmax(z, dim=1).mean(0).numpy()
        assert np.allclose(target[t, [e for e, _ in lst]], ref, rtol=0, atol=1e-14)
        assert abs(target[t].sum() - 1.0) <= 1e-12
        assert loss[t] >= 0
    assert target[100, 3] == 0 and target[100, 4] == 0 and grad[100, 4] == 0


# --------------------------------------------------------------------------- backward

def test_sparse_backward_equals_torch_autograd():
    """The analytic gradients equal torch autograd (fp64, CPU) of sum(d_out * o) through the
    gathered rows, softmax and value product; rows with -1 and out-of-range entries, and a KV
    row listed by many queries, included."""
    wl = gi.Workload(name="bw", L=80, idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=16),
                     mqa=gi.MqaSpec(H=3, D_k=96, D_v=64, sigma=1.0, scale=96 ** -0.5), seed=21)
    d = gi.prefill_inputs(wl)
    idx = orc.prefill_indexer_topk(d)
    idx[40, 2] = -1
    idx[41, 0] = 79            # beyond t: not attended
    g = torch.Generator().manual_seed(22)
    d_out = torch.randn((80, 3, 64), generator=g).to(torch.bfloat16)
    dq, dkv = orc.sparse_mqa_backward(d, idx, d_out)
    q = d["q"].double().requires_grad_(True)
    kv = d["kv"].double().requires_grad_(True)
    total = 0.0
    for t in range(80):
        sel = torch.tensor([s for s in idx[t] if 0 <= s <= t], dtype=torch.long)
        K = kv[sel]
        z = (q[t] @ K.T) * 96 ** -0.5
        o = torch.softmax(z, dim=1) @ K[:, :64]
        total = total + (o * d_out[t].double()).sum()
    total.backward()
    assert np.allclose(dq, q.grad.numpy(), rtol=0, atol=1e-11)
    assert np.allclose(dkv, kv.grad.numpy(), rtol=0, atol=1e-11)
    assert np.abs(dkv).max() > 0.1 and np.abs(dq).max() > 0.1


# --------------------------------------------------------------------------- batched prefill

def _contiguous_of(d, b, rows):
    """The contiguous single-sequence inputs of sequence b's query rows ``rows`` (data move)."""
    L, off = d["seq_lens"][b], d["seq_off"][b]
    return {"q_idx": d["q_idx"][rows], "w": d["w"][rows], "k_idx": d["k_flat"][off:off + L],
            "q_pos": d["q_pos"][rows], "top_k": d["top_k"], "q": d["q"][rows],
            "kv": d["kv_flat"][off:off + L], "D_v": d["D_v"], "scale": d["scale"]}


@pytest.mark.parametrize("seed", [0, 1])
def test_batched_prefill_equals_each_sequence_prefilled_alone(seed):
    """Variable-length sequences (one prefilled from 0, one as a chunk against a cached
    prefix, one short) in random pages, with the query rows in a shuffled order: every row
    equals the contiguous single-sequence prefill of its own sequence."""
    sp = gi.BatchedSpec(seq_lens=(300, 700, 129), q_start=(0, 500, 0),
                        idx=gi.IndexerSpec(H_I=4, d_I=32, grid_lo=-3, grid_hi=3, grid_step=0.125,
                                           w_choices=(0.25, 0.5, 1.0), top_k=64),
                        mqa=gi.MqaSpec(H=4, D_k=96, D_v=64, sigma=1.0, scale=96 ** -0.5),
                        seed=seed)
    n = 300 + 200 + 129
    order = torch.randperm(n, generator=torch.Generator().manual_seed(seed))
    d = gi.batched_inputs(sp, row_order=order)
    i1, o1, l1 = orc.batched_prefill(d)
    q_seq = d["q_seq"].numpy()
    for b in range(3):
        rows = np.flatnonzero(q_seq == b)
        i2, o2, l2 = orc.prefill(_contiguous_of(d, b, torch.as_tensor(rows)))
        assert np.array_equal(i1[rows], i2)
        assert np.allclose(o1[rows], o2, rtol=0, atol=1e-13)
        assert np.allclose(l1[rows], l2, rtol=0, atol=1e-13)


def test_batched_prefill_rows_without_a_sequence_select_nothing():
    sp = gi.BatchedSpec(seq_lens=(200,), idx=gi.IndexerSpec(H_I=4, d_I=32, top_k=16),
                        mqa=gi.MqaSpec(H=2, D_k=64, D_v=64, sigma=1.0, scale=0.125))
    d = gi.batched_inputs(sp)
    d["q_seq"] = d["q_seq"].clone()
    d["q_seq"][5] = 3
    d["q_seq"][6] = -1
    d["q_pos"] = d["q_pos"].clone()
    d["q_pos"][7] = -4
    idx, o, lse = orc.batched_prefill(d, rows=[5, 6, 7, 8])
    assert (idx[:3] == -1).all() and (o[:3] == 0).all() and np.isneginf(lse[:3]).all()
    assert (idx[3, :9] == np.arange(9)).all()


# --------------------------------------------------------------------------- generators

def test_generators_are_seeded_and_on_grid():
    a = gi.prefill_inputs(gi.tiny_workload())
    b = gi.prefill_inputs(gi.tiny_workload())
    c = gi.prefill_inputs(gi.tiny_workload(), seed=1)
    for key in ("q_idx", "w", "k_idx", "q", "kv"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    vals = orc.decode_e4m3fn(a["q_idx"]) * 8
    assert set(np.unique(vals).tolist()) <= set(range(-3, 4))
    assert set(np.unique(a["w"].numpy()).tolist()) <= {0.25, 0.5, 1.0}
    part = gi.prefill_inputs(gi.tiny_workload(), rows=(100, 7))
    assert torch.equal(part["q_idx"], a["q_idx"][100:107]) and torch.equal(part["q"], a["q"][100:107])


def test_work_model_closed_forms():
    assert orc.causal_pairs(131072) == 8_590_000_128
    assert orc.selected_pairs(131072, 2048) == sum(min(2048, t + 1) for t in range(131072))
    assert orc.selected_pairs(100, 2048) == 5050


# --------------------------------------------------------------------------- planted mistakes

def _pins_pass(monkeypatched):
    """Run a small battery of the pins above; return False if any fails."""
    try:
        test_scores_handworked_example()
        for s in range(2):
            test_scores_equal_exact_rational_brute_force(s)
        for s in range(2):
            test_topk_equals_counting_definition(s, 3)
        test_attention_handworked_example()
        test_full_selection_equals_dense_causal_sdpa(96, 64)
        test_decode_equals_prefill_last_row()
        test_quantize_e4m3fn_matches_torch_cast_on_every_bf16_value()
    except AssertionError:
        return False
    return True


def _wrong_topk_high_index(scores, k):
    n = scores.shape[0]
    order = np.lexsort((-np.arange(n), -scores))
    m = min(k, n)
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = np.sort(order[:m])
    return out


def _wrong_scores_no_relu(q_i, w, k_i):
    return (k_i @ q_i.T) @ w + 0.0


def _wrong_scores_no_weight(q_i, w, k_i):
    return np.maximum(k_i @ q_i.T, 0).sum(1) + 0.0


def _wrong_mqa_v_from_tail(q, kv_sel, d_v, scale):
    if kv_sel.shape[0] == 0:
        return np.zeros((q.shape[0], d_v)), np.full(q.shape[0], -np.inf)
    z = scale * (q @ kv_sel.T)
    p = np.exp(z - z.max(1, keepdims=True))
    den = p.sum(1, keepdims=True)
    return (p @ kv_sel[:, -d_v:]) / den, (z.max(1, keepdims=True) + np.log(den))[:, 0]


def _wrong_valid_off_by_one(idx_row, t):
    return idx_row[(idx_row >= 0) & (idx_row < t)]


def _wrong_quantize_ties_away(x):
    v = np.asarray(x, dtype=np.float64)
    finite = orc.E4M3FN[:127]
    out = np.empty(v.shape, dtype=np.uint8)
    for i, val in enumerate(v.reshape(-1)):
        a = min(abs(val), 448.0) if not np.isnan(val) else val
        if np.isnan(a):
            code = 0x7F
        else:
            hi = int(np.searchsorted(finite, a))
            lo = max(hi - 1, 0)
            code = hi if (finite[hi] - a) <= (a - finite[lo]) else lo
        out.reshape(-1)[i] = code | (0x80 if np.signbit(val) else 0)
    return out


@pytest.mark.parametrize("name,attr,bad", [
    ("FP8 ties rounded away from zero", "quantize_e4m3fn", _wrong_quantize_ties_away),
    ("tie-break to highest index", "topk_select", _wrong_topk_high_index),
    ("ReLU dropped", "indexer_scores", _wrong_scores_no_relu),
    ("head weights dropped", "indexer_scores", _wrong_scores_no_weight),
    ("V taken from the wrong end of the row", "sparse_mqa", _wrong_mqa_v_from_tail),
    ("causal bound off by one", "valid_selected", _wrong_valid_off_by_one),
])
def test_planted_mistakes_are_caught(monkeypatch, name, attr, bad):
    assert _pins_pass(False)
    monkeypatch.setattr(orc, attr, bad)
    assert not _pins_pass(True), f"planted mistake not caught: {name}"

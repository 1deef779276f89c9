"""CPU oracle of the DeepSeek Sparse Attention (DSA) hot path — TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy.  It exists to check the HIP library; only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``sparse_attention_long_gemm_amd``) never imports, calls or links it, and it
shares no code with that path: its FP8/bf16 decoders, scoring, selection and attention are all
written here from the definitions below.

What the path computes (one query row t of a causal sequence; decode is the same with
t = ctx - 1 and keys read through a page table):

1. Lightning-indexer score, for every earlier key s <= t:
       I[t, s] = sum_j  w[t, j] * ReLU( q_I[t, j, :] . k_I[s, :] )
   a ReLU-activated dot product per indexer head, weighted and summed over a handful of
   heads, with FP8 operands.  Sources: jdon.com "DeepSeek-V3.2-Exp" article, paragraph on the
   lightning indexer (ReLU, weight w_I, q_I meeting k_I, few heads H_I, FP8); openi.cn
   "DeepSeek-V3.2" page, section on the technology behind the model (the indexer relates the
   query token to the preceding tokens).  The keys are shared by all indexer heads.
2. Fine-grained token selection: keep the k = 2048 keys of highest score, drop the rest
   (jdon.com article, paragraph on fine-grained token selection; openi.cn page, item on token
   selection).  Ties are broken toward the lower position; with n = min(k, t + 1) candidates
   the selection is unique.  Scores are compared numerically (-0 == +0).
3. Attention in MQA mode over only the selected entries: one shared latent KV row per token
   (K = all D_k dims, V = its first D_v dims) serves every query head (openi.cn page, item on
   MLA in MQA mode; mundobytes.com page, section "How it works: lightning indexer and token
   selection").  o[t, h] = sum_s softmax_s(scale * q[t, h] . kv[s]) * kv[s, :D_v] and
   lse[t, h] = log sum_s exp(scale * q[t, h] . kv[s]) over the selected s.

Readings where the pages are silent (listed with reasons in the design notes): the key at
s = t itself is a candidate; ties go to the lowest index; FP8 is OCP e4m3fn with no scale
factors; the softmax scale is 1/sqrt(D_k); an empty selection gives o = 0 and lse = -inf;
a selected index that is -1 or outside [0, t] contributes nothing.

Exactness: operands on the dyadic grids the tests use make every score exact in fp64 (and in
fp32), so the selection is decided identically on both sides.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------------


def _e4m3fn_table() -> np.ndarray:
    """All 256 OCP e4m3fn codes as fp64: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m/8 * 2^-6); the single NaN pattern per sign is
    exponent 15 with mantissa 7; there are no infinities (largest finite value 448).
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3FN = _e4m3fn_table()


def decode_e4m3fn(codes) -> np.ndarray:
    """FP8 e4m3fn bytes (uint8 array / tensor) -> exact fp64 values."""
    c = _np(codes).astype(np.uint8)
    return E4M3FN[c]


def decode_bf16(x) -> np.ndarray:
    """bf16 values (torch.bfloat16 tensor, or their uint16 bit patterns) -> exact fp64.

    A bf16 number is the upper half of an fp32 bit pattern, so widening is a 16-bit shift.
    """
    u = _np(x).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _np(x) -> np.ndarray:
    """Host NumPy view of an array or tensor; bf16 tensors come back as their uint16 bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            return x.cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x)


# ----------------------------------------------------------------------------------------
# Step 1: lightning-indexer scores
# ----------------------------------------------------------------------------------------


def indexer_scores(q_i: np.ndarray, w: np.ndarray, k_i: np.ndarray) -> np.ndarray:
    """Scores of one query row against the candidate keys.

    q_i: [H_I, d_I] fp64, w: [H_I] fp64, k_i: [n, d_I] fp64 (the keys s = 0..n-1, n = t + 1).
    Returns I: [n] with I[s] = sum_j w[j] * max(q_i[j] . k_i[s], 0).
    (jdon.com article, lightning-indexer paragraph.)
    """
    x = k_i @ q_i.T                      # [n, H_I]: per-head dot products q_I[j] . k_I[s]
    relu = np.maximum(x, 0.0)            # ReLU activation per head
    scores = relu @ w                    # weighted sum over indexer heads
    return scores + 0.0                  # -0 -> +0, so equal scores compare equal


# ----------------------------------------------------------------------------------------
# Step 2: top-k selection
# ----------------------------------------------------------------------------------------


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best keys under (score descending, index ascending); int32 [k].

    n = min(k, len(scores)) indices are returned in ascending order, then -1 padding.
    (jdon.com article, paragraph on fine-grained token selection: keep the 2048 highest.)
    """
    n = scores.shape[0]
    pos = np.arange(n)
    order = np.lexsort((pos, -scores))   # primary key: -score; secondary: position
    m = min(k, n)
    sel = np.sort(order[:m]).astype(np.int32)
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = sel
    return out


# ----------------------------------------------------------------------------------------
# Step 3: sparse MQA attention over the selected shared KV rows
# ----------------------------------------------------------------------------------------


def sparse_mqa(q: np.ndarray, kv_sel: np.ndarray, d_v: int, scale: float):
    """Attention of every head of one query over the selected shared rows.

    q: [H, D_k] fp64; kv_sel: [m, D_k] fp64 (the selected rows; V is the first d_v dims).
    Returns (o [H, d_v], lse [H]); with m == 0, o = 0 and lse = -inf.
    (openi.cn page: MQA mode, one KV entry shared by many queries; only the top-k entries
    are attended.)
    """
    H = q.shape[0]
    if kv_sel.shape[0] == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    z = scale * (q @ kv_sel.T)                       # [H, m] logits
    zmax = z.max(axis=1, keepdims=True)
    p = np.exp(z - zmax)
    den = p.sum(axis=1, keepdims=True)
    o = (p @ kv_sel[:, :d_v]) / den
    lse = (zmax + np.log(den))[:, 0]
    return o, lse


def valid_selected(idx_row: np.ndarray, t: int) -> np.ndarray:
    """The entries of an index row that are attended: in [0, t]; -1 and others are skipped."""
    return idx_row[(idx_row >= 0) & (idx_row <= t)]


# ----------------------------------------------------------------------------------------
# Whole-path drivers (prefill of one contiguous sequence; paged decode)
# ----------------------------------------------------------------------------------------


def prefill_indexer_topk(inp: dict, rows=None) -> np.ndarray:
    """Top-k index rows for the given query rows (local row numbers; default all)."""
    q_codes = _np(inp["q_idx"])               # FP8 bytes; rows decoded one at a time
    k_i = decode_e4m3fn(inp["k_idx"])
    w = _np(inp["w"]).astype(np.float64)
    q_pos = _np(inp["q_pos"]).astype(np.int64)
    k = int(inp["top_k"])
    rows = range(q_pos.shape[0]) if rows is None else rows
    out = np.empty((len(rows), k), dtype=np.int32)
    for r, i in enumerate(rows):
        t = int(q_pos[i])
        if t < 0:
            out[r] = -1
            continue
        sc = indexer_scores(decode_e4m3fn(q_codes[i]), w[i], k_i[: t + 1])
        out[r] = topk_select(sc, k)
    return out


def prefill(inp: dict, rows=None, idx=None):
    """Full path for the given rows: returns (idx [n,k], o [n,H,D_v], lse [n,H]).

    ``idx`` may be passed to run step 3 on a given selection (the selection itself is then
    not recomputed).
    """
    rows = list(range(_np(inp["q_pos"]).shape[0])) if rows is None else list(rows)
    if idx is None:
        idx = prefill_indexer_topk(inp, rows)
    q_pos = _np(inp["q_pos"]).astype(np.int64)
    kv_bits = _np(inp["kv"])                  # raw bf16 bits, decoded per gathered set
    d_v = int(inp["D_v"])
    scale = float(inp["scale"])
    qt = inp["q"]
    H = qt.shape[1]
    o = np.empty((len(rows), H, d_v))
    lse = np.empty((len(rows), H))
    for r, i in enumerate(rows):
        t = int(q_pos[i])
        sel = valid_selected(np.asarray(idx[r]), t)
        q = decode_bf16(qt[i])
        o[r], lse[r] = sparse_mqa(q, decode_bf16(kv_bits[sel]), d_v, scale)
    return idx, o, lse


def paged_gather(cache, page_table_row, positions, page_size: int) -> np.ndarray:
    """Logical rows ``positions`` of one sequence from a paged cache, on the host (bf16 as bits).

    Row s lives at page page_table_row[s // page_size], slot s % page_size.  Paging with
    page size 64 is the serving layout named on the mundobytes.com page (section "Quick guide
    to running locally") and used by the paged indexer kernels it mentions (section "Open
    kernels and ecosystem support").
    """
    pt = _np(page_table_row).astype(np.int64)
    s = np.asarray(positions, dtype=np.int64)
    pages, slots = pt[s // page_size], s % page_size
    return _np(cache)[pages, slots]


def paged_rows(cache, page_table_row, n: int, page_size: int) -> np.ndarray:
    """Logical rows 0..n-1 of one sequence from a paged cache."""
    return paged_gather(cache, page_table_row, np.arange(n), page_size)


def decode(inp: dict, seqs=None, idx=None):
    """One paged decode step: per sequence b, query at t = ctx_b - 1 over keys [0, ctx_b).

    Returns (idx [B,k], o [B,H,D_v], lse [B,H]) for the requested sequences.
    """
    ctx = _np(inp["ctx"]).astype(np.int64)
    pt = _np(inp["page_table"])
    P = int(inp["page_size"])
    k = int(inp["top_k"])
    d_v = int(inp["D_v"])
    scale = float(inp["scale"])
    seqs = list(range(ctx.shape[0])) if seqs is None else list(seqs)
    q_i_all = decode_e4m3fn(inp["q_idx"])
    w_all = _np(inp["w"]).astype(np.float64)
    kc = _np(inp["k_cache"])            # host copies (a device cache is copied over once)
    kvc = _np(inp["kv_cache"])
    H = inp["q"].shape[1]
    out_idx = np.empty((len(seqs), k), dtype=np.int32)
    o = np.empty((len(seqs), H, d_v))
    lse = np.empty((len(seqs), H))
    for r, b in enumerate(seqs):
        n = int(ctx[b])
        t = n - 1
        if idx is None:
            k_i = decode_e4m3fn(paged_rows(kc, pt[b], n, P))
            sc = indexer_scores(q_i_all[b], w_all[b], k_i)
            out_idx[r] = topk_select(sc, k)
        else:
            out_idx[r] = np.asarray(idx[r])
        sel = valid_selected(out_idx[r], t)
        kv_sel = decode_bf16(paged_gather(kvc, pt[b], sel, P)) if len(sel) else \
            np.zeros((0, kvc.shape[-1]))
        q = decode_bf16(inp["q"][b])
        o[r], lse[r] = sparse_mqa(q, kv_sel, d_v, scale)
    return out_idx, o, lse


def kl_from_scores(scores: np.ndarray, target: np.ndarray):
    """(loss, grad) of the indexer's KL loss for one row, over the entries of its list:
    loss = sum_e target[e] (log target[e] - log softmax(scores)[e]) (0 log 0 = 0), and
    grad[e] = d loss / d scores[e] = softmax(scores)[e] - target[e] (target sums to 1).
    Empty list: (0, [])."""
    if scores.shape[0] == 0:
        return 0.0, np.zeros(0)
    m = scores.max()
    log_q = scores - m - np.log(np.exp(scores - m).sum())
    pos = target > 0
    loss = float((target[pos] * (np.log(target[pos]) - log_q[pos])).sum())
    return loss, np.exp(log_q) - target


def indexer_kl(inp: dict, idx, rows=None):
    """The indexer's training signal for the given rows and index lists (one contiguous
    sequence): the main attention's probabilities over the row's list, summed over heads and
    divided by H, are the target; the indexer's distribution is the softmax of its scores over
    the same list; the loss is their KL divergence, target first.  The indexer learns to
    reproduce the main attention with a KL loss (jdon.com article, paragraph on the indexer's
    warm-up; its sparse-training paragraph keeps that loss separate from the model's).
    Returns (loss [n], target [n, k], grad [n, k]); entries outside [0, t] or -1 are not in the
    list (target and grad 0 there).
    """
    q_pos = _np(inp["q_pos"]).astype(np.int64)
    rows = list(range(q_pos.shape[0])) if rows is None else list(rows)
    idx = np.asarray(idx)
    k = idx.shape[1]
    kv = _np(inp["kv"])
    k_i = decode_e4m3fn(inp["k_idx"])
    q_codes = _np(inp["q_idx"])
    w = _np(inp["w"]).astype(np.float64)
    scale = float(inp["scale"])
    loss = np.zeros(len(rows))
    target = np.zeros((len(rows), k))
    grad = np.zeros((len(rows), k))
    for r, i in enumerate(rows):
        t = min(int(q_pos[i]), kv.shape[0] - 1)
        listed = np.flatnonzero((idx[r] >= 0) & (idx[r] <= t))
        if listed.size == 0:
            continue
        s = idx[r][listed]
        z = scale * (decode_bf16(inp["q"][i]) @ decode_bf16(kv[s]).T)       # [H, m] logits
        a = np.exp(z - z.max(axis=1, keepdims=True))
        a /= a.sum(axis=1, keepdims=True)                                   # per-head softmax
        p = a.mean(axis=0)                                                  # heads summed / H
        sc = indexer_scores(decode_e4m3fn(q_codes[i]), w[i], k_i)[s]
        loss[r], g = kl_from_scores(sc, p)
        target[r, listed] = p
        grad[r, listed] = g
    return loss, target, grad


def sparse_mqa_backward(inp: dict, idx, d_out):
    """Gradients of sum(d_out * o) with respect to q and the KV rows, o the sparse MQA output of
    every query row over its index list (the selection itself is not differentiated).  In the
    sparse training stage the model's loss reaches the attention through the selected entries
    only (jdon.com article, sparse-training paragraph).  Per row, over the listed rows K (V =
    their first D_v dims):  P = softmax(scale q K^T),  o = P V,  dP = dO V^T,
    dS = P (dP - rowsum(dO o)),  dq = scale dS K,  dK = scale dS^T q,  dV = P^T dO, the last
    two added into the listed KV rows (a row listed several times collects each share).
    Returns (dq [n, H, D_k], dkv [n_kv, D_k]).
    """
    q_pos = _np(inp["q_pos"]).astype(np.int64)
    kv = decode_bf16(inp["kv"])
    d_v, scale = int(inp["D_v"]), float(inp["scale"])
    idx = np.asarray(idx)
    n, H = q_pos.shape[0], inp["q"].shape[1]
    dq = np.zeros((n, H, kv.shape[1]))
    dkv = np.zeros_like(kv)
    for i in range(n):
        t = min(int(q_pos[i]), kv.shape[0] - 1)
        sel = valid_selected(idx[i], t)
        if sel.size == 0:
            continue
        q = decode_bf16(inp["q"][i])
        K = kv[sel]
        V = K[:, :d_v]
        z = scale * (q @ K.T)
        P = np.exp(z - z.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        o = P @ V
        dO = decode_bf16(d_out[i])
        dS = P * (dO @ V.T - (dO * o).sum(axis=1, keepdims=True))
        dq[i] = scale * (dS @ K)
        dK = scale * (dS.T @ q)
        dK[:, :d_v] += P.T @ dO
        np.add.at(dkv, sel, dK)
    return dq, dkv


def dense_prefill(inp: dict, rows=None):
    """Dense causal attention, the baseline DSA replaces: row t attends every position 0..t
    (t = q_pos, clamped to the KV rows; t < 0 attends nothing).  Returns (o [n,H,D_v],
    lse [n,H]).  (jdon.com article: core attention goes from O(L^2) to O(L k); its
    inference-cost paragraph compares the two per token position.)
    """
    q_pos = _np(inp["q_pos"]).astype(np.int64)
    rows = list(range(q_pos.shape[0])) if rows is None else list(rows)
    kv = _np(inp["kv"])
    d_v, scale = int(inp["D_v"]), float(inp["scale"])
    H = inp["q"].shape[1]
    o = np.empty((len(rows), H, d_v))
    lse = np.empty((len(rows), H))
    for r, i in enumerate(rows):
        t = min(int(q_pos[i]), kv.shape[0] - 1)
        kv_all = decode_bf16(kv[: t + 1]) if t >= 0 else np.zeros((0, kv.shape[1]))
        o[r], lse[r] = sparse_mqa(decode_bf16(inp["q"][i]), kv_all, d_v, scale)
    return o, lse


def dense_decode(inp: dict, seqs=None):
    """Dense attention of each sequence's new query (t = ctx - 1) over its positions [0, ctx),
    read through the page table.  Returns (o [B,H,D_v], lse [B,H])."""
    ctx = _np(inp["ctx"]).astype(np.int64)
    pt = _np(inp["page_table"])
    P = int(inp["page_size"])
    seqs = list(range(ctx.shape[0])) if seqs is None else list(seqs)
    kvc = _np(inp["kv_cache"])
    d_v, scale = int(inp["D_v"]), float(inp["scale"])
    H = inp["q"].shape[1]
    o = np.empty((len(seqs), H, d_v))
    lse = np.empty((len(seqs), H))
    for r, b in enumerate(seqs):
        n = int(ctx[b])
        kv_all = decode_bf16(paged_rows(kvc, pt[b], n, P)) if n > 0 else \
            np.zeros((0, kvc.shape[-1]))
        o[r], lse[r] = sparse_mqa(decode_bf16(inp["q"][b]), kv_all, d_v, scale)
    return o, lse


def batched_prefill(inp: dict, rows=None, idx=None):
    """Prefill of many sequences whose keys and KV rows sit in paged caches: query row i is
    position t = q_pos[i] of sequence b = q_seq[i] (all 0 when q_seq is absent) and reads that
    sequence's rows 0..t through page_table[b].  Variable-length batches and chunked prefill
    (queries of a chunk against the prefix already cached) are both this.  Returns
    (idx [n,k], o [n,H,D_v], lse [n,H]) for the requested rows; ``idx`` may be given to run the
    attention alone.  A row of a sequence outside the page table, or with t < 0, selects
    nothing.  (Paging: mundobytes.com page, "Quick guide to running locally".)
    """
    pt = _np(inp["page_table"])
    P = int(inp["page_size"])
    q_pos = _np(inp["q_pos"]).astype(np.int64)
    n = q_pos.shape[0]
    q_seq = np.zeros(n, dtype=np.int64) if inp.get("q_seq") is None else \
        _np(inp["q_seq"]).astype(np.int64)
    rows = list(range(n)) if rows is None else list(rows)
    k = int(inp["top_k"])
    d_v = int(inp["D_v"]) if "D_v" in inp else 0
    with_attn = "q" in inp and inp.get("q") is not None
    kc = _np(inp["k_cache"])
    kvc = _np(inp["kv_cache"]) if with_attn else None
    q_codes = _np(inp["q_idx"])
    w = _np(inp["w"]).astype(np.float64)
    t_cap = pt.shape[1] * P - 1
    out_idx = np.empty((len(rows), k), dtype=np.int32)
    H = inp["q"].shape[1] if with_attn else 0
    o = np.empty((len(rows), H, d_v))
    lse = np.empty((len(rows), H))
    for r, i in enumerate(rows):
        b = int(q_seq[i])
        t = min(int(q_pos[i]), t_cap)
        if b < 0 or b >= pt.shape[0] or t < 0:
            t = -1
        if idx is not None:
            out_idx[r] = np.asarray(idx[r])
        elif t < 0:
            out_idx[r] = -1
        else:
            keys = decode_e4m3fn(paged_rows(kc, pt[b], t + 1, P))
            out_idx[r] = topk_select(indexer_scores(decode_e4m3fn(q_codes[i]), w[i], keys), k)
        if with_attn:
            sel = valid_selected(out_idx[r], t)
            kv_sel = decode_bf16(paged_gather(kvc, pt[b], sel, P)) if len(sel) else \
                np.zeros((0, kvc.shape[-1]))
            o[r], lse[r] = sparse_mqa(decode_bf16(inp["q"][i]), kv_sel, d_v,
                                      float(inp["scale"]))
    return out_idx, o, lse


# ----------------------------------------------------------------------------------------
# Cache write: FP8 quantisation of new indexer keys and the paged append
# ----------------------------------------------------------------------------------------


def quantize_e4m3fn(x) -> np.ndarray:
    """Nearest e4m3fn code of each value (uint8), from the format's value set.

    The indexer keeps its keys in FP8 (jdon.com article, lightning-indexer paragraph).  Reading
    (the pages give no conversion rule): round to the nearest representable value, a tie going
    to the even code (the codes of two neighbouring values differ by one); finite values and
    infinities past the largest magnitude, 448, saturate to +-448; NaN gives the NaN code 0x7f
    with the sign bit of the input; the sign of zero is kept.
    """
    v = np.asarray(x, dtype=np.float64)
    finite = E4M3FN[:127]                        # codes 0x00..0x7e: 0 .. 448, increasing
    out = np.empty(v.shape, dtype=np.uint8)
    flat_v, flat_o = v.reshape(-1), out.reshape(-1)
    for i, val in enumerate(flat_v):
        neg = np.signbit(val)
        a = abs(val)
        if np.isnan(val):
            code = 0x7F
        elif a >= 448.0:
            code = 0x7E
        else:
            hi = int(np.searchsorted(finite, a, side="left"))   # finite[hi] >= a
            if finite[hi] == a:
                code = hi
            else:
                lo = hi - 1
                d_lo, d_hi = a - finite[lo], finite[hi] - a
                code = lo if d_lo < d_hi else hi if d_hi < d_lo else (lo if lo % 2 == 0 else hi)
        flat_o[i] = code | (0x80 if neg else 0)
    return out


def cache_append(k_cache, kv_cache, page_table, seq, pos, k_new, kv_new):
    """The caches after writing the new rows: row r of sequence seq[r] (r if seq is None) at
    logical position pos[r] goes to page page_table[seq[r], pos[r] // P], slot pos[r] % P, its
    k_I quantised to e4m3fn and its KV row copied; a row with a negative position, a page index
    past the table or a page-table entry outside [0, n_pages) writes nothing.  Returns new host
    arrays (FP8 codes, bf16 as bits); either cache may be None when its rows are not given.
    (mundobytes.com page, "Quick guide to running locally": 64-token pages.)
    """
    pt = _np(page_table).astype(np.int64)
    pos = _np(pos).astype(np.int64)
    T = pos.shape[0]
    seq = np.arange(T) if seq is None else _np(seq).astype(np.int64)
    kc = None if k_cache is None else _np(k_cache).copy()
    kvc = None if kv_cache is None else _np(kv_cache).copy()
    geo = (kc if kc is not None else kvc).shape
    n_pages, P = geo[0], geo[1]
    kq = None if k_new is None else quantize_e4m3fn(decode_bf16(k_new))
    kvb = None if kv_new is None else _np(kv_new)
    for r in range(T):
        b, p = int(seq[r]), int(pos[r])
        if b < 0 or p < 0 or p // P >= pt.shape[1]:
            continue
        page = int(pt[b, p // P])
        if page < 0 or page >= n_pages:
            continue
        if kq is not None:
            kc[page, p % P] = kq[r]
        if kvb is not None:
            kvc[page, p % P] = kvb[r]
    return kc, kvc


# ----------------------------------------------------------------------------------------
# Work model used to extrapolate sampled oracle timings
# ----------------------------------------------------------------------------------------


def row_work(t: int, H_I: int, d_I: int, H: int, D_k: int, D_v: int, k: int) -> float:
    """Multiply-adds x2 that one prefill row t costs: indexer over t+1 keys + MQA over min(k,t+1)."""
    return (t + 1) * 2.0 * H_I * d_I + min(k, t + 1) * 2.0 * H * (D_k + D_v)


def causal_pairs(L: int) -> int:
    return L * (L + 1) // 2


def selected_pairs(L: int, k: int) -> int:
    """Sum over t < L of min(k, t + 1)."""
    m = min(k, L)
    return m * (m + 1) // 2 + max(0, L - k) * k


__all__ = [
    "E4M3FN", "decode_e4m3fn", "decode_bf16", "indexer_scores", "topk_select", "sparse_mqa",
    "valid_selected", "prefill_indexer_topk", "prefill", "paged_gather", "paged_rows", "decode",
    "batched_prefill", "dense_prefill", "dense_decode", "kl_from_scores", "indexer_kl",
    "sparse_mqa_backward",
    "quantize_e4m3fn", "cache_append",
    "row_work",
    "causal_pairs", "selected_pairs",
]

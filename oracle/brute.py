"""Loop-only brute force of the DSA hot path for tiny inputs — TEST INFRASTRUCTURE ONLY.

A second, independent statement of the same definitions as ``dsa_oracle`` (which it does not
import), used to pin that oracle.  Scores are computed in exact rational arithmetic
(``fractions.Fraction``) from FP8 bit fields decoded here, selection is the counting
definition of "top-k" (a key is kept when fewer than k keys beat it), and attention is dense
causal attention whose mask is the selected set.  Pure Python: only for L of a few hundred.

Definitions followed: jdon.com "DeepSeek-V3.2-Exp" article (lightning-indexer paragraph:
ReLU-activated per-head dot products, weighted and summed; token-selection paragraph: keep the
2048 best keys per query), openi.cn "DeepSeek-V3.2" page (MQA mode: one shared KV entry per
token serves all query heads).
"""
from __future__ import annotations

import math
from fractions import Fraction


def e4m3fn_value(code: int) -> Fraction:
    """Exact value of an OCP e4m3fn code from its bit fields (NaN codes are rejected)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        raise ValueError("NaN code")
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def nearest_e4m3fn(x: Fraction) -> int:
    """Saturating round-to-nearest e4m3fn code of an exact value, by trying every code: the
    finite code at the smallest exact distance, a tie going to the even code, magnitudes at or
    past 448 to the largest finite code; the sign is carried over (also for zero results)."""
    neg = x < 0
    a = -x if neg else x
    if a >= 448:
        best = 0x7E
    else:
        best, best_d = None, None
        for code in range(0x7F):                  # 0x00 .. 0x7e: every finite magnitude
            d = abs(e4m3fn_value(code) - a)
            if best_d is None or d < best_d or (d == best_d and code % 2 == 0):
                best, best_d = code, d
    return best | (0x80 if neg else 0)


def bf16_value(bits: int) -> float:
    """bf16 bit pattern (uint16) -> float, by building the fp32 pattern bits << 16."""
    import struct
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def scores(q_i, w, k_i, t: int):
    """Exact scores I[s] for s = 0..t.  q_i: [H_I][d_I] codes, w: [H_I] floats, k_i: [L][d_I] codes."""
    qf = [[e4m3fn_value(c) for c in row] for row in q_i]
    wf = [Fraction(x) for x in w]
    out = []
    for s in range(t + 1):
        kf = [e4m3fn_value(c) for c in k_i[s]]
        tot = Fraction(0)
        for j in range(len(qf)):
            x = sum((a * b for a, b in zip(qf[j], kf)), Fraction(0))
            if x > 0:
                tot += wf[j] * x
        out.append(tot)
    return out


def topk(sc, k: int):
    """Kept positions: s is kept iff fewer than k positions beat it (higher score, or equal
    score and lower position).  Returned ascending."""
    n = len(sc)
    kept = []
    for s in range(n):
        beaten_by = sum(1 for u in range(n) if sc[u] > sc[s] or (sc[u] == sc[s] and u < s))
        if beaten_by < k:
            kept.append(s)
    return kept


def masked_attention(q_rows, kv_rows, t: int, keep, d_v: int, scale: float):
    """Dense causal attention of one query over keys 0..t with mask = ``keep``.

    q_rows: [H][D_k] floats; kv_rows: [L][D_k] floats.  Returns (o [H][d_v], lse [H]).
    """
    keep = set(keep)
    H = len(q_rows)
    o, lse = [], []
    for h in range(H):
        logits = []
        for s in range(t + 1):
            if s in keep:
                logits.append((s, scale * math.fsum(a * b for a, b in zip(q_rows[h], kv_rows[s]))))
        if not logits:
            o.append([0.0] * d_v)
            lse.append(-math.inf)
            continue
        mx = max(z for _, z in logits)
        ps = [(s, math.exp(z - mx)) for s, z in logits]
        den = math.fsum(p for _, p in ps)
        o.append([math.fsum(p * kv_rows[s][d] for s, p in ps) / den for d in range(d_v)])
        lse.append(mx + math.log(den))
    return o, lse

"""Seeded synthetic inputs for the DSA hot path (shared by the oracle side and the HIP side).

This module only *draws* values: it holds none of the method's arithmetic (no scores, no
selection, no attention).  Both the CPU oracle (``oracle/``) and the HIP path receive the
exact same tensors from here, so that parity is checked on identical bytes.

Encodings handed out:
  * FP8 operands are OCP e4m3fn bytes in ``torch.uint8`` tensors.  The indexer runs in FP8
    (jdon.com DeepSeek-V3.2-Exp article, paragraph on the lightning indexer).
  * bf16 operands are ``torch.bfloat16`` tensors (round-to-nearest-even of an fp32 draw).
  * weights ``w`` are fp32, indices / positions / page tables are int32.

Value recipes (workload shapes of the pages' 128K-context prefill and paged decode):
  * dyadic FP8 grid: integers drawn uniformly in [lo, hi] times a power of two, so every
    indexer score is exactly representable in fp32 in any summation order;
  * w: a power of two drawn uniformly from a small set (or any given list of values);
  * q, kv: N(0, sigma^2) rounded to bf16;
  * decode: context lengths uniform in [ctx_lo, ctx_hi], one shared page table for the FP8
    key cache and the bf16 KV cache, physical pages taken from a random permutation.

Every tensor draws from its own generator seeded by (seed, tensor id), so a tensor's values
do not depend on which other tensors were requested.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Tensor ids: one independent random stream per tensor.
_T_QIDX, _T_W, _T_KIDX, _T_Q, _T_KV, _T_CTX, _T_PERM = range(7)

# Large normal tensors are filled in slices of this many rows, so the device never holds an
# fp32 copy of the whole tensor.  Fixed, so that the draw is a function of the seed only.
_FILL_ROWS = 4096


def _gen(seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed((int(seed) * 1_000_003 + 7919 * tensor_id + 17) % (2**62))
    return g


def grid_fp8(shape, lo: int, hi: int, step: float, seed: int, tensor_id: int, device="cpu"):
    """Integers uniform in [lo, hi] times ``step`` (a power of two), as e4m3fn bytes."""
    g = _gen(seed, tensor_id, device)
    ints = torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int32)
    vals = ints.to(torch.float32) * step
    return vals.to(torch.float8_e4m3fn).view(torch.uint8)


def choice_f32(shape, choices, seed: int, tensor_id: int, device="cpu"):
    """Values drawn uniformly from ``choices`` (fp32)."""
    g = _gen(seed, tensor_id, device)
    table = torch.tensor([float(c) for c in choices], dtype=torch.float32, device=device)
    pick = torch.randint(0, len(choices), tuple(shape), generator=g, device=device)
    return table[pick]


def uniform_f32(shape, lo: float, hi: float, seed: int, tensor_id: int, device="cpu"):
    """Values uniform in [lo, hi) (fp32): weights off the dyadic grid."""
    g = _gen(seed, tensor_id, device)
    u = torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return u * (hi - lo) + lo


def normal_bf16(shape, sigma: float, seed: int, tensor_id: int, device="cpu"):
    """N(0, sigma^2) rounded to bf16, filled slice by slice along dim 0."""
    g = _gen(seed, tensor_id, device)
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    rows = shape[0]
    for r0 in range(0, rows, _FILL_ROWS):
        r1 = min(rows, r0 + _FILL_ROWS)
        blk = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        if sigma != 1.0:
            blk.mul_(sigma)
        out[r0:r1] = blk.to(torch.bfloat16)
    return out


@dataclass
class IndexerSpec:
    H_I: int = 64
    d_I: int = 128
    grid_lo: int = -2
    grid_hi: int = 2
    grid_step: float = 2.0 ** -3
    w_choices: tuple = (2.0 ** -4, 2.0 ** -3, 2.0 ** -2, 2.0 ** -1, 1.0)
    top_k: int = 2048


@dataclass
class MqaSpec:
    H: int = 128
    D_k: int = 576
    D_v: int = 512
    sigma: float = 1.0 / 24.0          # N(0,1)/sqrt(576)
    scale: float = 1.0 / 24.0          # 1/sqrt(576)


@dataclass
class Workload:
    """Named shapes of the five workloads the library is measured and tested on."""
    name: str
    L: int
    idx: IndexerSpec = field(default_factory=IndexerSpec)
    mqa: MqaSpec | None = field(default_factory=MqaSpec)
    block: int | None = None        # query block for streamed prefill
    seed: int = 0


def tiny_workload() -> Workload:
    """L=256 causal, H_I=4, d_I=32, grid {-3..3}/8, w in {1/4,1/2,1}, k=32, H=8, D=64 (V=K)."""
    return Workload(
        name="tiny_L256", L=256,
        idx=IndexerSpec(H_I=4, d_I=32, grid_lo=-3, grid_hi=3, grid_step=0.125,
                        w_choices=(0.25, 0.5, 1.0), top_k=32),
        mqa=MqaSpec(H=8, D_k=64, D_v=64, sigma=1.0, scale=1.0 / 8.0))


def indexer_workload() -> Workload:
    """Indexer + top-k only, L=8192 causal, H_I=64, d_I=128, k=2048."""
    return Workload(name="indexer_L8192", L=8192, mqa=None)


def prefill_workload(L: int = 32768, block: int | None = None, sharp: bool = False) -> Workload:
    """Full DSA prefill: indexer as above + sparse MQA, 128 heads of 576 (512 latent + 64 rope)."""
    mqa = MqaSpec(sigma=1.0 if sharp else 1.0 / 24.0)
    nm = f"prefill_L{L}" + ("_sharp" if sharp else "") + (f"_blk{block}" if block else "")
    return Workload(name=nm, L=L, mqa=mqa, block=block)


def prefill_inputs(wl: Workload, device="cpu", seed: int | None = None, rows=None,
                   with_mqa: bool = True):
    """Inputs of a causal prefill of one sequence of length ``wl.L``.

    ``rows``: optional (q_start, n_q) restricting the query rows drawn (the key side is always
    the whole sequence).  Query tensors are drawn for all L rows and then sliced, so a row's
    values never depend on ``rows``.
    """
    seed = wl.seed if seed is None else seed
    L, ix = wl.L, wl.idx
    q0, nq = (0, L) if rows is None else rows
    d = {}
    q_idx = grid_fp8((L, ix.H_I, ix.d_I), ix.grid_lo, ix.grid_hi, ix.grid_step, seed, _T_QIDX, device)
    d["q_idx"] = q_idx[q0:q0 + nq].contiguous()
    del q_idx
    d["w"] = choice_f32((L, ix.H_I), ix.w_choices, seed, _T_W, device)[q0:q0 + nq].contiguous()
    d["k_idx"] = grid_fp8((L, ix.d_I), ix.grid_lo, ix.grid_hi, ix.grid_step, seed, _T_KIDX, device)
    d["q_pos"] = torch.arange(q0, q0 + nq, dtype=torch.int32, device=device)
    d["top_k"] = ix.top_k
    if with_mqa and wl.mqa is not None:
        m = wl.mqa
        if rows is None:
            d["q"] = normal_bf16((L, m.H, m.D_k), m.sigma, seed, _T_Q, device)
        else:
            full = normal_bf16((L, m.H, m.D_k), m.sigma, seed, _T_Q, device)
            d["q"] = full[q0:q0 + nq].contiguous()
            del full
        d["kv"] = normal_bf16((L, m.D_k), m.sigma, seed, _T_KV, device)
        d["D_v"] = m.D_v
        d["scale"] = m.scale
    return d


@dataclass
class DecodeSpec:
    B: int = 64
    ctx_lo: int = 4096
    ctx_hi: int = 131072
    page_size: int = 64
    idx: IndexerSpec = field(default_factory=IndexerSpec)
    mqa: MqaSpec = field(default_factory=MqaSpec)
    spare_pages: int = 0
    seed: int = 0


def decode_inputs(sp: DecodeSpec, device="cpu", seed: int | None = None, ctx_lens=None):
    """Inputs of one paged decode step: one new query per sequence, t = ctx_b - 1.

    The key cache (FP8 k_I rows) and the KV cache (bf16 576-wide rows) share one page table.
    Physical pages are a random permutation of the pool; unused page-table slots hold -1.
    """
    seed = sp.seed if seed is None else seed
    B, P = sp.B, sp.page_size
    if ctx_lens is None:
        g = _gen(seed, _T_CTX, "cpu")
        ctx = torch.randint(sp.ctx_lo, sp.ctx_hi + 1, (B,), generator=g, dtype=torch.int64)
    else:
        ctx = torch.as_tensor(ctx_lens, dtype=torch.int64)
    pages_per = [(int(c) + P - 1) // P for c in ctx.tolist()]
    n_pages = sum(pages_per) + sp.spare_pages
    max_pages = max(pages_per)
    g = _gen(seed, _T_PERM, "cpu")
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    pt = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, npg in enumerate(pages_per):
        pt[b, :npg] = perm[off:off + npg]
        off += npg
    ix, m = sp.idx, sp.mqa
    d = {
        "ctx": ctx.to(torch.int32).to(device),
        "page_table": pt.to(device),
        "page_size": P,
        "n_pages": n_pages,
        "max_pages": max_pages,
        "q_idx": grid_fp8((B, ix.H_I, ix.d_I), ix.grid_lo, ix.grid_hi, ix.grid_step, seed, _T_QIDX, device),
        "w": choice_f32((B, ix.H_I), ix.w_choices, seed, _T_W, device),
        "k_cache": grid_fp8((n_pages, P, ix.d_I), ix.grid_lo, ix.grid_hi, ix.grid_step, seed, _T_KIDX, device),
        "q": normal_bf16((B, m.H, m.D_k), m.sigma, seed, _T_Q, device),
        "kv_cache": normal_bf16((n_pages, P, m.D_k), m.sigma, seed, _T_KV, device),
        "top_k": ix.top_k,
        "D_v": m.D_v,
        "scale": m.scale,
    }
    return d


@dataclass
class BatchedSpec:
    """Many sequences in paged caches, prefilled in one call: sequence b holds seq_lens[b]
    tokens, of which positions q_start[b] .. seq_lens[b]-1 are queried (q_start > 0: a chunk
    against a cached prefix)."""
    seq_lens: tuple = (1000, 3000)
    q_start: tuple | None = None
    page_size: int = 64
    idx: IndexerSpec = field(default_factory=IndexerSpec)
    mqa: MqaSpec | None = field(default_factory=MqaSpec)
    spare_pages: int = 0
    seed: int = 0


def batched_inputs(sp: BatchedSpec, device="cpu", seed: int | None = None, row_order=None):
    """Inputs of a batched prefill over paged caches.

    The keys and KV rows of all sequences are drawn as one contiguous run of rows
    (``k_flat`` / ``kv_flat``, sequence b at rows seq_off[b] ..), then laid into pages of a
    random permutation of the pool (one page table for both caches).  Query rows are listed
    sequence by sequence (``q_seq`` non-decreasing) unless ``row_order`` permutes them.
    """
    seed = sp.seed if seed is None else seed
    P, ix, m = sp.page_size, sp.idx, sp.mqa
    lens = [int(x) for x in sp.seq_lens]
    starts = [0] * len(lens) if sp.q_start is None else [int(x) for x in sp.q_start]
    B = len(lens)
    off = [0]
    for n in lens:
        off.append(off[-1] + n)
    total = off[-1]
    pages_per = [(n + P - 1) // P for n in lens]
    n_pages = sum(pages_per) + sp.spare_pages
    max_pages = max(pages_per)
    g = _gen(seed, _T_PERM, "cpu")
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    pt = torch.full((B, max_pages), -1, dtype=torch.int32)
    o = 0
    for b, npg in enumerate(pages_per):
        pt[b, :npg] = perm[o:o + npg]
        o += npg
    k_flat = grid_fp8((total, ix.d_I), ix.grid_lo, ix.grid_hi, ix.grid_step, seed, _T_KIDX, device)
    k_cache = torch.zeros((n_pages, P, ix.d_I), dtype=torch.uint8, device=device)
    kv_flat = kv_cache = None
    if m is not None:
        kv_flat = normal_bf16((total, m.D_k), m.sigma, seed, _T_KV, device)
        kv_cache = torch.zeros((n_pages, P, m.D_k), dtype=torch.bfloat16, device=device)
    for b in range(B):
        contiguous_to_pages(k_flat[off[b]:off[b + 1]], pt, b, n_pages, P, k_cache)
        if m is not None:
            contiguous_to_pages(kv_flat[off[b]:off[b + 1]], pt, b, n_pages, P, kv_cache)
    q_seq = torch.cat([torch.full((lens[b] - starts[b],), b, dtype=torch.int32) for b in range(B)])
    q_pos = torch.cat([torch.arange(starts[b], lens[b], dtype=torch.int32) for b in range(B)])
    # query-side draws are made for every token of every sequence, then the queried rows taken
    flat_rows = torch.cat([torch.arange(off[b] + starts[b], off[b + 1]) for b in range(B)])
    if row_order is not None:
        ro = torch.as_tensor(row_order, dtype=torch.int64)
        q_seq, q_pos, flat_rows = q_seq[ro], q_pos[ro], flat_rows[ro]
    fr = flat_rows.to(device)
    d = {
        "seq_lens": lens, "q_start": starts, "seq_off": off,
        "page_table": pt.to(device), "page_size": P, "n_pages": n_pages, "max_pages": max_pages,
        "k_flat": k_flat, "k_cache": k_cache,
        "q_seq": q_seq.to(device), "q_pos": q_pos.to(device),
        "q_idx": grid_fp8((total, ix.H_I, ix.d_I), ix.grid_lo, ix.grid_hi, ix.grid_step, seed,
                          _T_QIDX, device)[fr].contiguous(),
        "w": choice_f32((total, ix.H_I), ix.w_choices, seed, _T_W, device)[fr].contiguous(),
        "top_k": ix.top_k,
    }
    if m is not None:
        d["kv_flat"], d["kv_cache"] = kv_flat, kv_cache
        d["q"] = normal_bf16((total, m.H, m.D_k), m.sigma, seed, _T_Q, device)[fr].contiguous()
        d["D_v"], d["scale"] = m.D_v, m.scale
    return d


def identity_page_table(ctx_lens, page_size: int):
    """Page table that lays each sequence's pages out back to back in order (no permutation)."""
    pages_per = [(int(c) + page_size - 1) // page_size for c in ctx_lens]
    max_pages = max(pages_per)
    pt = torch.full((len(pages_per), max_pages), -1, dtype=torch.int32)
    off = 0
    for b, npg in enumerate(pages_per):
        pt[b, :npg] = torch.arange(off, off + npg, dtype=torch.int32)
        off += npg
    return pt, off


def contiguous_to_pages(rows: torch.Tensor, page_table: torch.Tensor, b: int, n_pages: int,
                        page_size: int, cache: torch.Tensor | None = None):
    """Scatter one sequence's contiguous rows [ctx, ...] into a paged cache [n_pages, P, ...].

    Pure data movement (used to build paged copies of a prefill's inputs).
    """
    ctx = rows.shape[0]
    if cache is None:
        cache = torch.zeros((n_pages, page_size) + tuple(rows.shape[1:]), dtype=rows.dtype,
                            device=rows.device)
    for p in range(math.ceil(ctx / page_size)):
        s0, s1 = p * page_size, min(ctx, (p + 1) * page_size)
        cache[int(page_table[b, p]), : s1 - s0] = rows[s0:s1]
    return cache

"""Benchmark of the DSA hot path on one MI355X.

One step = the whole path on one batch of synthetic input:
  * prefill of one L=131072 sequence in 32 query blocks of 4096 rows; per block the FP8
    indexer + exact top-2048 (dsa_indexer_topk over keys [0, block end)) and the sparse MQA
    over the selected rows (dsa_sparse_mqa_prefill), H=128, D_k=576, D_v=512;
  * one paged decode step, B=64, ctx ~ U[4096, 131072], page size 64
    (dsa_indexer_topk_paged + dsa_sparse_mqa_decode).
``value`` is prefill tokens/s (131072 / prefill time); decode us/token is reported next to it.
Inputs are generated on the device before the timed region.  Kernel durations come from HIP
events recorded on the stream the kernels run on (torch's current stream, which the binding
passes to the library).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

from gen import inputs as gi  # noqa: E402

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
CSRC = os.path.join(ROOT, "sparse_attention_long_gemm_amd", "csrc")
# sources whose text fixes each kernel's code: a recorded HBM traffic figure is used only while
# their digest matches the one stored with it
KERNEL_SOURCES = {
    "indexer_topk_prefill_kernel": ["indexer_topk.hip", "dsa_select.hpp", "dsa_common.hpp"],
    "sparse_mqa_kernel<576,512>": ["sparse_mqa.hip", "dsa_common.hpp"],
    "decode_step": ["indexer_topk.hip", "dsa_select.hpp", "sparse_mqa.hip", "dsa_common.hpp"],
}

PEAK_FP8 = 5.0e15      # dense FP8 MFMA, FLOP/s (MI355X published)
PEAK_BF16 = 2.5e15     # dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12      # HBM3E, B/s
# fp32 FMA on the vector units without packed math (256 CUs x 4 SIMDs x 16 lanes x 2 flop x
# 2.4 GHz); the packed-math figure of 157.3 TFLOP/s does not apply: packed fp32 is not used
PEAK_VALU_FP32 = 78.6e12


def causal_pairs_range(q0, q1):
    """Sum over t in [q0, q1) of (t + 1): (query, key) pairs the indexer scores."""
    return (q1 * (q1 + 1) - q0 * (q0 + 1)) // 2


def scored_pairs_range(q0, q1, k):
    """Sum over t in [q0, q1) with t + 1 > k of (t + 1): the (query, key) pairs whose scores
    the selection depends on (a row with at most k candidates keeps all of them)."""
    lo = max(q0, k)
    return causal_pairs_range(lo, q1) if q1 > lo else 0


def selected_pairs_range(q0, q1, k):
    return sum(min(k, t + 1) for t in range(q0, q1))


class Prefill:
    def __init__(self, L=131072, block=4096, dev="cuda"):
        import sparse_attention_long_gemm_amd as dsa
        self.dsa = dsa
        self.L, self.block = L, block
        wl = gi.prefill_workload(L, block=block)
        self.wl = wl
        self.inp = gi.prefill_inputs(wl, device=dev)
        self.top_k = wl.idx.top_k
        d = self.inp
        self.out = torch.empty((L, wl.mqa.H, wl.mqa.D_v), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((L, wl.mqa.H), dtype=torch.float32, device=dev)
        self.idx = torch.empty((block, self.top_k), dtype=torch.int32, device=dev)
        self.ws = torch.empty(dsa.indexer_topk_workspace_size(block, self.top_k),
                              dtype=torch.uint8, device=dev)
        self.nblk = (L + block - 1) // block
        self.blocks = [(b * block, min(L, (b + 1) * block)) for b in range(self.nblk)]
        self.flops_idx = [2.0 * wl.idx.H_I * wl.idx.d_I * scored_pairs_range(a, e, self.top_k)
                          for a, e in self.blocks]
        self.flops_mqa = [2.0 * wl.mqa.H * (wl.mqa.D_k + wl.mqa.D_v) *
                          selected_pairs_range(a, e, self.top_k) for a, e in self.blocks]
        del d

    def run(self, events=None, after_block=None):
        """All blocks, in order.  ``after_block(bi, a, e, idx)`` (tests) is called after each
        block's two launches with that block's index rows (overwritten by the next block)."""
        d, dsa = self.inp, self.dsa
        for bi, (a, e) in enumerate(self.blocks):
            if events is not None:
                events[bi][0].record()
            dsa.indexer_topk(d["q_idx"][a:e], d["w"][a:e], d["k_idx"][:e], d["q_pos"][a:e],
                             self.top_k, out=self.idx[: e - a], workspace=self.ws)
            if events is not None:
                events[bi][1].record()
            dsa.sparse_mqa_prefill(d["q"][a:e], d["kv"][:e], self.idx[: e - a], d["q_pos"][a:e],
                                   self.wl.mqa.D_v, self.wl.mqa.scale, out=self.out[a:e],
                                   lse=self.lse[a:e])
            if events is not None:
                events[bi][2].record()
            if after_block is not None:
                after_block(bi, a, e, self.idx[: e - a])


class Decode:
    def __init__(self, dev="cuda", seed=0):
        import sparse_attention_long_gemm_amd as dsa
        self.dsa = dsa
        self.sp = gi.DecodeSpec(seed=seed)
        self.inp = gi.decode_inputs(self.sp, device=dev)
        d = self.inp
        B, m = self.sp.B, self.sp.mqa
        self.idx = torch.empty((B, d["top_k"]), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, m.H, m.D_v), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, m.H), dtype=torch.float32, device=dev)
        self.ws_idx = torch.empty(dsa.indexer_topk_paged_workspace_size(B, d["max_pages"],
                                                                         d["page_size"]),
                                  dtype=torch.uint8, device=dev)
        nb = dsa.sparse_mqa_decode_workspace_size(B, m.H, m.D_v, d["top_k"])
        self.ws_mqa = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        ctx = d["ctx"].cpu().tolist()
        self.ctx = ctx
        kk = d["top_k"]
        ix = self.sp.idx
        # algorithmic HBM bytes of one step: the indexer reads each sequence's FP8 keys (d_I
        # bytes per token) plus q_I and w; the MQA gathers the selected 576-wide bf16 rows and
        # reads q / writes o.  Intermediates (logits, partial outputs, the index round trip)
        # are not counted.
        self.bytes_idx = sum(ix.d_I * c for c in ctx) + B * (ix.H_I * ix.d_I + ix.H_I * 4)
        self.bytes_mqa = sum(min(kk, c) for c in ctx) * m.D_k * 2 + B * m.H * (m.D_k + m.D_v) * 2
        self.flops_idx = sum(2.0 * 64 * 128 * c for c in ctx if c > kk)
        self.flops_mqa = sum(2.0 * m.H * (m.D_k + m.D_v) * min(kk, c) for c in ctx)

    def setup_append(self):
        """The new token of each sequence (position ctx-1) as it leaves its projections: the
        indexer key in bf16 (values on the FP8 grid, so the cached key is unchanged) and the
        latent KV row (the cached one), written back by dsa_cache_append."""
        d = self.inp
        P = d["page_size"]
        pos = (d["ctx"] - 1).long()
        pages = d["page_table"][torch.arange(self.sp.B, device=pos.device), pos // P].long()
        self.app_pos = pos.to(torch.int32)
        self.app_k = d["k_cache"][pages, pos % P].view(torch.float8_e4m3fn).to(torch.bfloat16)
        self.app_kv = d["kv_cache"][pages, pos % P].contiguous()
        m, ix = self.sp.mqa, self.sp.idx
        # bytes per token: bf16 key + KV row read, FP8 key + KV row written, position and the
        # page-table entry read
        self.bytes_append = self.sp.B * (2 * ix.d_I + 2 * m.D_k + ix.d_I + 2 * m.D_k + 8)

    def run_append(self):
        d = self.inp
        self.dsa.cache_append(d["page_table"], self.app_pos, k_cache=d["k_cache"],
                              kv_cache=d["kv_cache"], k_new=self.app_k, kv_new=self.app_kv)

    def run(self, events=None):
        d, dsa = self.inp, self.dsa
        if events is not None:
            events[0].record()
        dsa.indexer_topk_paged(d["q_idx"], d["w"], d["k_cache"], d["page_table"], d["ctx"],
                               d["top_k"], out=self.idx, workspace=self.ws_idx)
        if events is not None:
            events[1].record()
        dsa.sparse_mqa_decode(d["q"], d["kv_cache"], d["page_table"], d["ctx"], self.idx,
                              d["D_v"], d["scale"], out=self.out, lse=self.lse,
                              workspace=self.ws_mqa)
        if events is not None:
            events[2].record()


class ChunkedPaged:
    """The same L=131072 prefill, chunk by chunk (4096 queries per call) against the growing
    prefix held in 64-token pages (random page order): dsa_indexer_topk_batched +
    dsa_sparse_mqa_batched.  Same rows, same work as ``Prefill``; the difference is the paging."""

    def __init__(self, pre: Prefill, dev, seed=0, page_size=64):
        self.pre, self.dsa = pre, pre.dsa
        d = pre.inp
        L, P = pre.L, page_size
        n_pages = (L + P - 1) // P
        g = torch.Generator().manual_seed(seed + 77)
        perm = torch.randperm(n_pages, generator=g).to(torch.int32)
        self.pt = perm[None, :].to(dev)
        self.k_cache = torch.zeros((n_pages, P, d["k_idx"].shape[1]), dtype=torch.uint8,
                                   device=dev)
        self.kv_cache = torch.zeros((n_pages, P, d["kv"].shape[1]), dtype=torch.bfloat16,
                                    device=dev)
        gi.contiguous_to_pages(d["k_idx"], self.pt.cpu(), 0, n_pages, P, self.k_cache)
        gi.contiguous_to_pages(d["kv"], self.pt.cpu(), 0, n_pages, P, self.kv_cache)
        self.out = torch.empty_like(pre.out)
        self.lse = torch.empty_like(pre.lse)

    def run(self, events=None):
        d, dsa, pre = self.pre.inp, self.dsa, self.pre
        if events is not None:
            events[0].record()
        for a, e in pre.blocks:
            dsa.indexer_topk_batched(d["q_idx"][a:e], d["w"][a:e], self.k_cache, self.pt,
                                     d["q_pos"][a:e], pre.top_k, out=pre.idx[: e - a],
                                     workspace=pre.ws)
            dsa.sparse_mqa_batched(d["q"][a:e], self.kv_cache, self.pt, d["q_pos"][a:e],
                                   pre.idx[: e - a], pre.wl.mqa.D_v, pre.wl.mqa.scale,
                                   out=self.out[a:e], lse=self.lse[a:e])
        if events is not None:
            events[1].record()


class Varlen:
    """A variable-length batch prefilled in one call pair: 32 sequences, lengths uniform in
    [1024, 8192] (seeded), keys and KV rows in 64-token pages."""

    def __init__(self, dev, seed=0, n_seq=32):
        import sparse_attention_long_gemm_amd as dsa
        self.dsa = dsa
        g = torch.Generator().manual_seed(seed + 5)
        lens = torch.randint(1024, 8193, (n_seq,), generator=g).tolist()
        self.sp = gi.BatchedSpec(seq_lens=tuple(lens), seed=seed)
        self.inp = gi.batched_inputs(self.sp, device=dev)
        d = self.inp
        n_q = d["q_pos"].shape[0]
        k = d["top_k"]
        self.idx = torch.empty((n_q, k), dtype=torch.int32, device=dev)
        self.out = torch.empty((n_q, self.sp.mqa.H, self.sp.mqa.D_v), dtype=torch.bfloat16,
                               device=dev)
        self.lse = torch.empty((n_q, self.sp.mqa.H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(dsa.indexer_topk_workspace_size(n_q, k), dtype=torch.uint8,
                              device=dev)
        self.tokens = n_q
        ix, m = self.sp.idx, self.sp.mqa
        self.flops_idx = sum(2.0 * ix.H_I * ix.d_I * scored_pairs_range(0, n, k) for n in lens)
        self.flops_mqa = sum(2.0 * m.H * (m.D_k + m.D_v) * selected_pairs_range(0, n, k)
                             for n in lens)
        self.lens = lens

    def run(self, events=None):
        d, dsa = self.inp, self.dsa
        if events is not None:
            events[0].record()
        dsa.indexer_topk_batched(d["q_idx"], d["w"], d["k_cache"], d["page_table"], d["q_pos"],
                                 d["top_k"], q_seq=d["q_seq"], out=self.idx, workspace=self.ws)
        if events is not None:
            events[1].record()
        dsa.sparse_mqa_batched(d["q"], d["kv_cache"], d["page_table"], d["q_pos"], self.idx,
                               self.sp.mqa.D_v, self.sp.mqa.scale, q_seq=d["q_seq"],
                               out=self.out, lse=self.lse)
        if events is not None:
            events[2].record()


def _ev():
    return torch.cuda.Event(enable_timing=True)


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str):
    """HBM bytes per launch (per decode step for "decode_step") from the FETCH_SIZE and
    WRITE_SIZE counter runs stored under profiles/, scaled by the copy-kernel calibration; None
    when nothing is stored or the kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec["bytes_per_launch"]


def recorded_decode_traffic():
    """Per-kernel HBM bytes of one decode step and each kernel's L2 hit rate, from the same
    counter runs (only while the sources match); {} otherwise."""
    try:
        with open(TRAFFIC_FILE) as fh:
            recs = json.load(fh)["decode_kernels"]
    except (OSError, KeyError, ValueError):
        return {}
    dig = source_digest("decode_step")
    return {k: {"bytes": v["bytes_per_launch"], "l2_hit_rate": v["l2_hit_rate"]}
            for k, v in recs.items() if v.get("source_sha256") == dig}


def copy_calibration(dev, nbytes=1 << 30, reps=3):
    """A plain elementwise copy of known size (fp32 negation: reads nbytes, writes nbytes) for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch.neg fp32", "read_bytes": nbytes,
                                           "write_bytes": nbytes, "launches": reps}}), flush=True)


def measured_ceilings(dsa, dev, reps: int = 3):
    """What this GPU sustains: MFMA loops on register operands (the bf16 and FP8 instruction
    shapes of the path) and a 4 GiB streaming read with 16-byte non-temporal loads; best of
    `reps` launches each, timed with HIP events on the current stream."""
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    n_wg = 4 * n_cu
    sink = torch.empty(n_wg * 512, dtype=torch.float32, device=dev)
    out = {}
    for kind, name in ((0, "bf16_mfma_tflops"), (1, "fp8_mfma_tflops")):
        best = 0.0
        for _ in range(reps):
            e0, e1 = _ev(), _ev()
            e0.record()
            fl = dsa.ceiling_mfma(kind, n_wg, 20000, sink)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out[name] = best
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev)   # 4 GiB
    src.fill_(1.0)
    best = 0.0
    for _ in range(reps):
        e0, e1 = _ev(), _ev()
        e0.record()
        nb = dsa.ceiling_read(src, 2 * n_wg, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nb / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    out["hbm_read_gbps"] = best
    del src
    # the shader clock these MFMA rates imply: a SIMD retires 1024 bf16 or 2048 FP8 flop per
    # cycle on these shapes (32x32x16 bf16 in 32 cycles, 16x16x128 FP8 in 32 cycles)
    simds = 4 * n_cu
    out["implied_mfma_clock_ghz"] = {
        "bf16": out["bf16_mfma_tflops"] * 1e12 / (simds * 1024) / 1e9,
        "fp8": out["fp8_mfma_tflops"] * 1e12 / (simds * 2048) / 1e9}
    out["kernels"] = ("dsa_ceiling_mfma (32x32x16 bf16 / 16x16x128 FP8 chains, "
                      f"{n_wg} workgroups x 8 waves) and dsa_ceiling_read (4 GiB, nt loads)")
    return out


def gather_ceilings(dsa, pre: Prefill, dev, reps: int = 3):
    """Random-row gather rates on the attention's own rows: the prefill's KV pool and the
    last 4096-row block's selected rows (4096 x 2048 rows of 1152 bytes, ascending positions;
    called after the timed steps, which leave that block's rows in pre.idx),
    moved by workgroups of 8 waves, one per CU, as in the attention: through the LDS DMA
    (the attention's path) and through loads into registers; best of `reps` launches each."""
    d = pre.inp
    a, e = pre.blocks[-1]
    idx = pre.idx[: e - a]   # the last block's index rows, left there by the block loop
    n_wg = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(n_wg * 512, dtype=torch.float32, device=dev)
    kv = d["kv"][:e]
    out = {}
    for kind, name in ((0, "gather_lds_dma_tbps"), (1, "gather_registers_tbps")):
        best = 0.0
        for _ in range(reps):
            e0, e1 = _ev(), _ev()
            e0.record()
            nb = dsa.ceiling_gather(kind, kv, idx, n_wg, sink)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, nb / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out[name] = best
    out["gather_kernel"] = ("dsa_ceiling_gather over the last block's index rows "
                            f"({e - a} x {pre.top_k} rows of 1152 bytes), {n_wg} workgroups x 8 waves")
    return out


def cpu_baseline(prefill: Prefill, budget_s: float = 20.0):
    """The fp64 oracle (as it stands) on a strided sample of the 128K prefill's rows, timed on
    this host; extrapolated to all rows by the exact per-row work model."""
    from oracle import dsa_oracle as orc
    # the cores this process may run on; the BLAS pools are pinned to that many threads so the
    # reported count is the one the oracle actually used
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover
        limiter = None
    d = prefill.inp
    wl = prefill.wl
    host = {"q_idx": d["q_idx"].cpu(), "w": d["w"].cpu(), "k_idx": d["k_idx"].cpu(),
            "q_pos": d["q_pos"].cpu(), "top_k": d["top_k"], "kv": d["kv"].cpu(),
            "D_v": d["D_v"], "scale": d["scale"], "q": d["q"]}
    L = prefill.L
    work = lambda t: orc.row_work(t, wl.idx.H_I, wl.idx.d_I, wl.mqa.H, wl.mqa.D_k, wl.mqa.D_v,
                                  prefill.top_k)
    stride = 128
    rows = list(range(stride - 1, L, stride))          # 1024 rows spread over the sequence
    n_grp = len(rows) // 32
    done, t_used, w_done = [], 0.0, 0.0
    t0 = time.perf_counter()
    for g in range(n_grp):
        grp = rows[g::n_grp]          # each group of 32 rows spans the whole sequence
        orc.prefill(host, rows=grp)
        done += grp
        w_done += sum(work(r) for r in grp)
        t_used = time.perf_counter() - t0
        if t_used > budget_s:
            break
    if limiter is not None:
        limiter.unregister()
    w_full = sum(work(t) for t in range(L))
    t_full = t_used * w_full / w_done
    return {"value": L / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 NumPy oracle on {len(done)} prefill rows of the L=131072 sequence "
                      f"(from every {stride}th row, t={min(done)}..{max(done)}), {t_used:.1f}s, "
                      f"extrapolated to all rows by per-row work (t+1)*2*H_I*d_I + "
                      f"min(k,t+1)*2*H*(D_k+D_v)"}


def extra_legs(pre: Prefill, dec: Decode, dev, reps: int):
    """The next rows of the path, each timed on its own (not part of the step above):
    the 128K prefill chunk by chunk through paged caches, a variable-length batch, and the
    decode step's cache append."""
    out = {}
    ch = ChunkedPaged(pre, dev)
    ch.run()
    t = _time(ch.run, reps) * 1e-3
    F_idx, F_mqa = sum(pre.flops_idx), sum(pre.flops_mqa)
    roof = F_idx / PEAK_FP8 + F_mqa / PEAK_BF16
    out["chunked_paged_prefill"] = {
        "workload": "L=131072 in 32 chunks of 4096 against 64-token pages (random order)",
        "ms": t * 1e3, "tokens_per_s": pre.L / t, "frac_of_roofline": roof / t}
    del ch
    torch.cuda.empty_cache()
    vl = Varlen(dev)
    vl.run()
    ev = [[_ev(), _ev(), _ev()] for _ in range(reps)]
    for e in ev:
        vl.run(e)
    torch.cuda.synchronize()
    t_i = sum(e[0].elapsed_time(e[1]) for e in ev) / reps * 1e-3
    t_m = sum(e[1].elapsed_time(e[2]) for e in ev) / reps * 1e-3
    out["varlen_prefill"] = {
        "workload": f"{len(vl.lens)} sequences, lengths U[1024, 8192] (sum {sum(vl.lens)}), "
                    "one batched call pair over 64-token pages",
        "ms": (t_i + t_m) * 1e3, "tokens_per_s": vl.tokens / (t_i + t_m),
        "indexer_frac": vl.flops_idx / t_i / PEAK_FP8, "mqa_frac": vl.flops_mqa / t_m / PEAK_BF16,
        "frac_of_roofline": (vl.flops_idx / PEAK_FP8 + vl.flops_mqa / PEAK_BF16) / (t_i + t_m)}
    del vl
    torch.cuda.empty_cache()
    # training-side rows on the last 4096-row block of the prefill (its indices are the last
    # ones the block loop left in pre.idx; out and lse hold every row)
    a, e = pre.blocks[-1]
    d, m, ix = pre.inp, pre.wl.mqa, pre.wl.idx
    n = e - a
    idx_b = pre.idx[:n]
    dsa = pre.dsa

    def kl():
        dsa.indexer_kl(d["q"][a:e], d["kv"][:e], idx_b, d["q_pos"][a:e], pre.lse[a:e], m.scale,
                       d["q_idx"][a:e], d["w"][a:e], d["k_idx"][:e])
    kl()
    t = _time(kl, reps) * 1e-3
    pairs = selected_pairs_range(a, e, pre.top_k)
    f_bf16, f_fp8 = 2.0 * m.H * m.D_k * pairs, 2.0 * ix.H_I * ix.d_I * pairs
    out["indexer_kl"] = {
        "workload": f"rows {a}..{e - 1} of the L=131072 prefill, their 2048 selected keys",
        "ms": t * 1e3, "frac_of_roofline": (f_bf16 / PEAK_BF16 + f_fp8 / PEAK_FP8) / t,
        "algorithmic": "per selected pair 2*H*D_k bf16 (logits) + 2*H_I*d_I FP8 (rescoring)"}
    g = torch.Generator(device=dev).manual_seed(3)
    d_out = torch.randn((n, m.H, m.D_v), generator=g, device=dev).to(torch.bfloat16)
    d_kv = torch.zeros((e, m.D_k), dtype=torch.float32, device=dev)
    ws_b = torch.empty(int(dsa.load_library().dsa_sparse_mqa_backward_workspace_size(
        n, m.H, pre.top_k)), dtype=torch.uint8, device=dev)

    def bwd():
        dsa.sparse_mqa_backward(d["q"][a:e], d["kv"][:e], idx_b, d["q_pos"][a:e], pre.out[a:e],
                                pre.lse[a:e], d_out, m.scale, d_kv=d_kv, workspace=ws_b)
    bwd()
    t = _time(bwd, reps) * 1e-3
    f_mfma = 2.0 * m.H * (3 * m.D_k + 2 * m.D_v) * pairs   # logits, dP, dQ, dKV
    out["sparse_backward"] = {
        "workload": f"rows {a}..{e - 1} of the L=131072 prefill (dQ, dKV)",
        "ms": t * 1e3,
        "achieved_tflops": f_mfma / t / 1e12,
        "frac_of_roofline": f_mfma / PEAK_BF16 / t,
        "algorithmic": "per selected pair 2*H*(3*D_k+2*D_v) bf16 MFMA flop (logits, dP, dQ, "
                       "dKV) against 2.5 PFLOP/s"}
    del d_out, d_kv, ws_b
    torch.cuda.empty_cache()
    dec.setup_append()
    dec.run_append()
    t = _time(dec.run_append, max(reps, 5)) * 1e-3
    out["cache_append"] = {"workload": f"decode step's new tokens, B={dec.sp.B}",
                           "us": t * 1e6, "bytes": dec.bytes_append,
                           "achieved_gbps": dec.bytes_append / t / 1e9}
    return out


_BUSY = {}


def _time(fn, reps):
    """Mean milliseconds of fn() over reps launches, HIP events on the current stream.  A
    millisecond of unrelated GPU work is queued first, so that the host has enqueued the timed
    launches before the GPU reaches them (the events then see GPU time, not launch latency)."""
    dev = torch.cuda.current_device()
    if dev not in _BUSY:
        _BUSY[dev] = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    _BUSY[dev].add_(1.0)
    evs = [(_ev(), _ev()) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


USD_PER_GPU_HOUR = 2.0   # the pricing unit of the pages' cost-per-token figures


def curves(dev, reps: int = 3, block: int = 256):
    """Cost per token against token position, DSA next to dense causal attention, on the same
    shapes (H=128, D_k=576, D_v=512; H_I=64, d_I=128, k=2048):
      prefill: a block of `block` query rows ending at position p (keys [0, p)): DSA = indexer +
               top-k + sparse MQA, dense = dense MQA over all earlier positions;
      decode:  a step of B=64 sequences all at context length p: DSA = paged indexer + top-k +
               sparse MQA, dense = dense MQA over the whole context.
    Reported as microseconds per token and as dollars per million tokens at $2 per GPU-hour."""
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library()
    L = 131072
    points = [4096, 8192, 16384, 32768, 65536, 98304, 131072]
    pre = Prefill(L=L, block=block, dev=dev)
    d, wl = pre.inp, pre.wl
    m = wl.mqa
    H, D_v, k = m.H, m.D_v, pre.top_k
    o = torch.empty((block, H, D_v), dtype=torch.bfloat16, device=dev)
    ls = torch.empty((block, H), dtype=torch.float32, device=dev)
    ws_dense = torch.empty(max(1, dsa.dense_mqa_workspace_size(block, H, D_v, L)),
                           dtype=torch.uint8, device=dev)
    rows = []
    for p in points:
        a, e = p - block, p
        def dsa_block():
            dsa.indexer_topk(d["q_idx"][a:e], d["w"][a:e], d["k_idx"][:e], d["q_pos"][a:e], k,
                             out=pre.idx[:block], workspace=pre.ws)
            dsa.sparse_mqa_prefill(d["q"][a:e], d["kv"][:e], pre.idx[:block], d["q_pos"][a:e],
                                   D_v, m.scale, out=o, lse=ls)

        def dense_block():
            dsa.dense_mqa_prefill(d["q"][a:e], d["kv"][:e], d["q_pos"][a:e], D_v, m.scale,
                                  out=o, lse=ls, workspace=ws_dense)
        dsa_block(), dense_block()
        t_dsa, t_dense = _time(dsa_block, reps), _time(dense_block, reps)
        f_dense = 2.0 * H * (576 + D_v) * causal_pairs_range(a, e)
        rows.append({"phase": "prefill", "position": p, "dsa_us_per_token": t_dsa * 1e3 / block,
                     "dense_us_per_token": t_dense * 1e3 / block,
                     "dense_mfma_frac": f_dense / (t_dense * 1e-3) / PEAK_BF16})
        print(f"[curves] prefill p={p}: dsa {t_dsa:.3f} ms dense {t_dense:.3f} ms",
              file=sys.stderr, flush=True)
    del pre, ws_dense
    torch.cuda.empty_cache()
    B = 64
    sp = gi.DecodeSpec(B=B, ctx_lo=L, ctx_hi=L)
    dd = gi.decode_inputs(sp, device=dev, ctx_lens=[L] * B)
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    od = torch.empty((B, H, D_v), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws_i = torch.empty(dsa.indexer_topk_paged_workspace_size(B, dd["max_pages"], 64),
                       dtype=torch.uint8, device=dev)
    ws_m = torch.empty(max(1, dsa.sparse_mqa_decode_workspace_size(B, H, D_v, k)),
                       dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, dsa.dense_mqa_workspace_size(B, H, D_v, dd["max_pages"] * 64)),
                       dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB: evicts the MALL
    for p in points:
        ctx = torch.full((B,), p, dtype=torch.int32, device=dev)
        # the page table as wide as this context (the dense split count and the indexer's
        # score rows follow the table's width; the host does not read the context lengths)
        pt = dd["page_table"][:, : (p + 63) // 64].contiguous()

        def dsa_step():
            flush.add_(1.0)
            dsa.indexer_topk_paged(dd["q_idx"], dd["w"], dd["k_cache"], pt, ctx, k,
                                   out=idx, workspace=ws_i)
            dsa.sparse_mqa_decode(dd["q"], dd["kv_cache"], pt, ctx, idx, D_v,
                                  m.scale, out=od, lse=ld, workspace=ws_m)

        def dense_step():
            flush.add_(1.0)
            dsa.dense_mqa_decode(dd["q"], dd["kv_cache"], pt, ctx, D_v, m.scale,
                                 out=od, lse=ld, workspace=ws_d)

        def flush_only():
            flush.add_(1.0)
        dsa_step(), dense_step()
        t_f = _time(flush_only, reps)
        t_dsa = _time(dsa_step, reps) - t_f
        t_dense = _time(dense_step, reps) - t_f
        rows.append({"phase": "decode", "position": p, "batch": B,
                     "dsa_us_per_token": t_dsa * 1e3 / B, "dense_us_per_token": t_dense * 1e3 / B,
                     "dense_hbm_frac": B * p * 1152 / (t_dense * 1e-3) / PEAK_HBM})
        print(f"[curves] decode ctx={p}: dsa {t_dsa:.3f} ms dense {t_dense:.3f} ms",
              file=sys.stderr, flush=True)
    for r in rows:
        r["dsa_usd_per_mtok"] = r["dsa_us_per_token"] * USD_PER_GPU_HOUR / 3600.0
        r["dense_usd_per_mtok"] = r["dense_us_per_token"] * USD_PER_GPU_HOUR / 3600.0
        r["dense_over_dsa"] = r["dense_us_per_token"] / r["dsa_us_per_token"]
    return {"curves": rows, "prefill_block": block, "decode_batch": B,
            "usd_per_gpu_hour": USD_PER_GPU_HOUR, "reps": reps}


def curves_markdown(res) -> str:
    lines = ["| phase | position | DSA µs/token | dense µs/token | dense / DSA | DSA $/Mtok | "
             "dense $/Mtok | dense kernel roofline frac |", "|---|---|---|---|---|---|---|---|"]
    for r in res["curves"]:
        fr = r.get("dense_mfma_frac", r.get("dense_hbm_frac"))
        kind = "MFMA" if "dense_mfma_frac" in r else "HBM"
        lines.append(f"| {r['phase']} | {r['position']} | {r['dsa_us_per_token']:.3f} | "
                     f"{r['dense_us_per_token']:.3f} | {r['dense_over_dsa']:.2f} | "
                     f"{r['dsa_usd_per_mtok']:.5f} | {r['dense_usd_per_mtok']:.5f} | "
                     f"{fr:.2f} ({kind}) |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB copy kernel used to scale the HBM byte counters")
    ap.add_argument("--curves", action="store_true",
                    help="only measure cost per token against position, DSA and dense")
    ap.add_argument("--curves-md", default=None, help="also write the curves as a markdown table")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the chunked, variable-length and cache-append legs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DSA path here is a single-GPU build "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(dev)
        return
    if args.curves:
        res = curves(dev)
        if args.curves_md:
            with open(args.curves_md, "w") as fh:
                fh.write(curves_markdown(res))
        print(json.dumps(res), flush=True)
        return
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library()
    print("[bench] generating inputs on device", file=sys.stderr, flush=True)
    pre = Prefill(dev=dev)
    dec = Decode(dev=dev)
    torch.cuda.synchronize()

    for w in range(args.warmup):
        pre.run()
        dec.run()
        torch.cuda.synchronize()
        print(f"[bench] warmup {w + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    ev_pre = [[[_ev(), _ev(), _ev()] for _ in pre.blocks] for _ in range(args.steps)]
    ev_dec = [[_ev(), _ev(), _ev()] for _ in range(args.steps)]
    ev_step = [[_ev(), _ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev_step[s][0].record()
        pre.run(ev_pre[s])
        ev_step[s][1].record()
        dec.run(ev_dec[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {args.steps} timed steps done in {wall:.2f}s", file=sys.stderr, flush=True)

    t_idx = sum(e[0].elapsed_time(e[1]) for st in ev_pre for e in st) / args.steps / 1e3
    t_mqa = sum(e[1].elapsed_time(e[2]) for st in ev_pre for e in st) / args.steps / 1e3
    t_pre = sum(st[0].elapsed_time(st[1]) for st in ev_step) / args.steps / 1e3
    t_didx = sum(e[0].elapsed_time(e[1]) for e in ev_dec) / args.steps / 1e3
    t_dmqa = sum(e[1].elapsed_time(e[2]) for e in ev_dec) / args.steps / 1e3
    t_dec = t_didx + t_dmqa
    F_idx, F_mqa = sum(pre.flops_idx), sum(pre.flops_mqa)
    n_launch = len(pre.blocks)

    roof_idx = {"bound": "mfma", "kernel": "indexer_topk_prefill_kernel",
                "achieved": F_idx / t_idx / 1e12, "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s",
                "frac": F_idx / t_idx / PEAK_FP8,
                "traffic": recorded_traffic("indexer_topk_prefill_kernel"),
                "avg_launch_ms": t_idx / n_launch * 1e3,
                "algorithmic": "2*H_I*d_I = 16384 FP8 flop per causal (t,s) pair of rows with t+1 > top_k; "
                               f"{F_idx / n_launch:.4g} flop per launch on average"}
    roof_mqa = {"bound": "mfma", "kernel": "sparse_mqa_kernel<576,512>",
                "achieved": F_mqa / t_mqa / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": F_mqa / t_mqa / PEAK_BF16,
                "traffic": recorded_traffic("sparse_mqa_kernel<576,512>"),
                "avg_launch_ms": t_mqa / n_launch * 1e3,
                "algorithmic": "2*H*(D_k+D_v) = 278528 bf16 flop per selected (t,s) pair; "
                               f"{F_mqa / n_launch:.4g} flop per launch on average"}
    dominant = roof_idx if t_idx >= t_mqa else roof_mqa
    roof_time = F_idx / PEAK_FP8 + F_mqa / PEAK_BF16
    dec_bytes = dec.bytes_idx + dec.bytes_mqa
    decode = {
        "us_per_token": t_dec / dec.sp.B * 1e6, "us_per_step": t_dec * 1e6, "batch": dec.sp.B,
        "indexer_us": t_didx * 1e6, "mqa_us": t_dmqa * 1e6,
        "roofline": {"bound": "hbm", "achieved": dec_bytes / t_dec / 1e9, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": dec_bytes / t_dec / PEAK_HBM,
                     "traffic": recorded_traffic("decode_step"),
                     "algorithmic_bytes_per_step": dec_bytes,
                     "traffic_per_kernel": recorded_decode_traffic()},
    }
    res = {
        "metric": "DSA prefill tokens/s at 128K (decode us/token alongside), % of MFMA/HBM roofline",
        "value": pre.L / t_pre,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16 (fp32 accumulate)",
        "data": "synthetic (seeded; dyadic FP8 grid indexer operands, N(0,1)/24 bf16 q/kv)",
        "config": {"workload": "prefill L=131072 in 4096-row blocks + paged decode B=64",
                   "seq_len": pre.L, "block": pre.block, "top_k": pre.top_k, "H_I": 64,
                   "d_I": 128, "H": 128, "D_k": 576, "D_v": 512, "decode_batch": dec.sp.B,
                   "page_size": dec.sp.page_size, "parallelism": "single GPU"},
        "prefill": {"ms": t_pre * 1e3, "indexer_ms": t_idx * 1e3, "mqa_ms": t_mqa * 1e3,
                    "roofline_ms": roof_time * 1e3, "frac_of_roofline": roof_time / t_pre,
                    "indexer": roof_idx, "mqa": roof_mqa},
        "decode": decode,
        "roofline": dominant,
    }
    if not args.no_extra:
        res["extra"] = extra_legs(pre, dec, dev, max(1, args.steps))
    ceil = measured_ceilings(dsa, dev)
    ceil.update(gather_ceilings(dsa, pre, dev))
    res["ceilings"] = ceil
    # the attention's row gathers: 1152 bytes per selected (t, s) pair
    gathered = F_mqa / (2.0 * pre.wl.mqa.H * (pre.wl.mqa.D_k + pre.wl.mqa.D_v)) * (2 * pre.wl.mqa.D_k)
    roof_mqa["gather"] = {"bytes": gathered, "achieved_tbps": gathered / t_mqa / 1e12,
                          "frac_of_lds_dma_ceiling": gathered / t_mqa / 1e12
                          / ceil["gather_lds_dma_tbps"]}
    roof_idx["frac_of_measured"] = roof_idx["achieved"] / ceil["fp8_mfma_tflops"]
    roof_mqa["frac_of_measured"] = roof_mqa["achieved"] / ceil["bf16_mfma_tflops"]
    decode["roofline"]["frac_of_measured"] = decode["roofline"]["achieved"] / ceil["hbm_read_gbps"]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(pre, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

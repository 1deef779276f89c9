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


def causal_pairs_range(q0, q1):
    """Sum over t in [q0, q1) of (t + 1): (query, key) pairs the indexer scores."""
    return (q1 * (q1 + 1) - q0 * (q0 + 1)) // 2


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
        self.flops_idx = [2.0 * wl.idx.H_I * wl.idx.d_I * causal_pairs_range(a, e) for a, e in self.blocks]
        self.flops_mqa = [2.0 * wl.mqa.H * (wl.mqa.D_k + wl.mqa.D_v) *
                          selected_pairs_range(a, e, self.top_k) for a, e in self.blocks]
        del d

    def run(self, events=None):
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
        self.flops_idx = sum(2.0 * 64 * 128 * c for c in ctx)
        self.flops_mqa = sum(2.0 * m.H * (m.D_k + m.D_v) * min(kk, c) for c in ctx)

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


def cpu_baseline(prefill: Prefill, budget_s: float = 20.0):
    """The fp64 oracle (as it stands) on a strided sample of the 128K prefill's rows, timed on
    this host; extrapolated to all rows by the exact per-row work model."""
    from oracle import dsa_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
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
    w_full = sum(work(t) for t in range(L))
    t_full = t_used * w_full / w_done
    return {"value": L / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 NumPy oracle on {len(done)} prefill rows of the L=131072 sequence "
                      f"(from every {stride}th row, t={min(done)}..{max(done)}), {t_used:.1f}s, "
                      f"extrapolated to all rows by per-row work (t+1)*2*H_I*d_I + "
                      f"min(k,t+1)*2*H*(D_k+D_v)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB copy kernel used to scale the HBM byte counters")
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
                "algorithmic": "2*H_I*d_I = 16384 FP8 flop per causal (t,s) pair; "
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
                     "algorithmic_bytes_per_step": dec_bytes},
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
    ceil = measured_ceilings(dsa, dev)
    res["ceilings"] = ceil
    roof_idx["frac_of_measured"] = roof_idx["achieved"] / ceil["fp8_mfma_tflops"]
    roof_mqa["frac_of_measured"] = roof_mqa["achieved"] / ceil["bf16_mfma_tflops"]
    decode["roofline"]["frac_of_measured"] = decode["roofline"]["achieved"] / ceil["hbm_read_gbps"]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(pre, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

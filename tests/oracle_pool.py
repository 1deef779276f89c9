"""Run the CPU oracle over many prefill rows on every host core (test infrastructure only).

The full-size parity tests compare tens of thousands of index rows, which the fp64 oracle
computes one row at a time.  This module runs those rows on a pool of threads, each calling
the oracle on its own slice of rows, with the BLAS pools pinned to one thread per call: the
oracle's time goes to NumPy matrix products, elementwise passes and sorts, which run without
Python's global lock, so the threads use the cores in parallel.  Threads (not processes) keep
everything in one process: nothing is spawned, nothing can be left behind.  Nothing here
computes any part of the method: every value comes from ``oracle.dsa_oracle``.  Index rows are
identical to the serial call's; fp64 attention values can differ from it in the last bits,
because single-threaded BLAS sums the products in another order.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

_PER_ROW = ("q_idx", "w", "q_pos", "q")


def n_workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _host(x):
    """Host NumPy copy of a tensor or array; bf16 tensors as their 16-bit patterns."""
    if isinstance(x, torch.Tensor):
        x = x.detach()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        return x.cpu().numpy()
    return x


def prefill_rows(inp: dict, rows, with_attn: bool = False, workers: int | None = None):
    """``oracle.prefill_indexer_topk(inp, rows)`` (or ``oracle.prefill(inp, rows)`` when
    ``with_attn``), computed on a thread pool."""
    from oracle import dsa_oracle as orc
    workers = workers or n_workers()
    rows = np.asarray(list(rows), dtype=np.int64)
    per_row = [k for k in _PER_ROW if k in inp and (with_attn or k != "q")]
    shared = {k: _host(v) for k, v in inp.items() if k not in _PER_ROW}
    # interleaved slices (rows i, i + n, i + 2n, ...): the cost of a row grows with its
    # position, so every slice gets a like share of short and long rows
    n_task = max(1, min(len(rows), workers))
    slices = [np.arange(i, len(rows), n_task) for i in range(n_task)]
    tasks = []
    for sl in slices:
        c = rows[sl]
        local = dict(shared)
        for k in per_row:
            local[k] = _host(inp[k][torch.as_tensor(c).to(inp[k].device)])
        tasks.append(local)

    def run(local):
        n = local["q_pos"].shape[0]
        if with_attn:
            return orc.prefill(local, rows=range(n))
        return orc.prefill_indexer_topk(local, rows=range(n))

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            parts = list(ex.map(run, tasks))
    finally:
        if limiter is not None:
            limiter.unregister()

    def gather(arrs):
        out = np.empty((len(rows),) + arrs[0].shape[1:], dtype=arrs[0].dtype)
        for sl, a in zip(slices, arrs):
            out[sl] = a
        return out

    if not with_attn:
        return gather(parts)
    return tuple(gather([p[j] for p in parts]) for j in range(3))

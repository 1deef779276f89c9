"""Python binding of libdsa.so, the MI355X DSA hot-path library (argument marshalling only).

Every step of the path runs in the HIP kernels behind the C ABI declared in ``include/dsa.h``;
this module checks tensor dtypes/shapes/devices, allocates outputs and workspaces with
PyTorch, and passes raw device pointers plus the current HIP stream.  There is no fallback:
if the library is missing or cannot be loaded the calls raise.

    idx  = indexer_topk(q_idx, w, k_idx, q_pos, top_k)               # prefill, one sequence
    idx  = indexer_topk_paged(q_idx, w, k_cache, page_table, ctx, top_k)
    o, lse = sparse_mqa_prefill(q, kv, idx, q_pos, d_v, scale)
    o, lse = sparse_mqa_decode(q, kv_cache, page_table, ctx, idx, d_v, scale)

FP8 tensors are ``torch.uint8`` (e4m3fn bytes) or ``torch.float8_e4m3fn``; bf16 tensors are
``torch.bfloat16``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_OK = 0
_STATUS = {0: "DSA_OK", -1: "DSA_ERR_INVALID_ARG", -2: "DSA_ERR_UNSUPPORTED_SHAPE",
           -3: "DSA_ERR_WORKSPACE_TOO_SMALL", -4: "DSA_ERR_HIP", -5: "DSA_ERR_SCRATCH_LIMIT"}

# Every exported symbol of include/dsa.h, with its ctypes signature.
_P, _I, _Z, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "dsa_abi_version": (ctypes.c_int, []),
    "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dsa_indexer_topk_workspace_size": (_Z, [_I, _I]),
    "dsa_indexer_topk": (ctypes.c_int, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "dsa_indexer_topk_paged_workspace_size": (_Z, [_I, _I, _I]),
    "dsa_indexer_topk_paged": (ctypes.c_int,
                               [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "dsa_sparse_mqa_prefill": (ctypes.c_int,
                               [_P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "dsa_sparse_mqa_decode_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "dsa_sparse_mqa_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                             _F, _I, _P, _P, _P, _Z, _P]),
    "dsa_indexer_topk_batched": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _I,
                                                _I, _I, _P, _P, _Z, _P]),
    "dsa_sparse_mqa_batched": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I, _I, _I,
                                              _I, _I, _F, _P, _P, _P]),
    "dsa_dense_mqa_workspace_size": (_Z, [_I, _I, _I, _I]),
    "dsa_dense_mqa_prefill": (ctypes.c_int, [_P, _P, _I, _P, _I, _I, _I, _I, _F, _P, _P, _P, _Z,
                                             _P]),
    "dsa_dense_mqa_decode": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P,
                                            _P, _P, _Z, _P]),
    "dsa_indexer_kl": (ctypes.c_int, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _I,
                                      _I, _P, _P, _P, _P]),
    "dsa_sparse_mqa_backward_workspace_size": (_Z, [_I, _I, _I]),
    "dsa_sparse_mqa_backward": (ctypes.c_int, [_P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                               _F, _P, _P, _P, _Z, _P]),
    "dsa_cache_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "dsa_sparse_mqa_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                                     _I, _I, _I, _F, _I, _P, _P, _P]),
    "dsa_ceiling_mfma": (ctypes.c_int, [_I, _I, _I, _P, _P, _P]),
    "dsa_ceiling_read": (ctypes.c_int, [_P, _Z, _I, _P, _P]),
    "dsa_ceiling_gather": (ctypes.c_int, [_I, _P, ctypes.c_int64, _I, _P, _I, _I, _I, _P, _P]),
}

_lib = None


class DSAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


def load_library(path: str | None = None, build_if_missing: bool = True):
    """Load libdsa.so (building it with hipcc first if it is absent); raise if impossible."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        if not build_if_missing:
            raise RuntimeError(f"DSA HIP library not found at {p}")
        from .build import build_library
        build_library()
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(code: int) -> str:
    try:
        return load_library().dsa_status_string(int(code)).decode()
    except Exception:  # pragma: no cover - used while reporting another error
        return _STATUS.get(int(code), "unknown")


def _check(code: int, where: str):
    if code != DSA_OK:
        raise DSAError(code, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, ndim: int, device=None, shape=None):
    """Check a tensor argument: type, dtype, rank, device memory, contiguity, and (for caller
    supplied outputs) the exact shape the kernels will write."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


_FP8 = (torch.uint8, torch.float8_e4m3fn)
_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    else:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace must be a torch.Tensor")
        if not workspace.is_cuda or workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, expected {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace of {workspace.numel() * workspace.element_size()} "
                             f"bytes < required {nbytes}")
    return workspace, workspace.numel() * workspace.element_size()


def indexer_topk_workspace_size(n_q: int, top_k: int) -> int:
    return int(load_library().dsa_indexer_topk_workspace_size(n_q, top_k))


def indexer_topk(q_idx, w, k_idx, q_pos, top_k: int, out=None, workspace=None):
    """Prefill indexer + top-k.  q_idx [n_q,H_I,d_I] fp8, w [n_q,H_I] fp32, k_idx [L,d_I] fp8,
    q_pos [n_q] int32 -> int32 [n_q, top_k] (ascending positions, then -1)."""
    lib = load_library()
    _need(q_idx, "q_idx", _FP8, 3)
    dev = q_idx.device
    _need(w, "w", _F32, 2, dev)
    _need(k_idx, "k_idx", _FP8, 2, dev)
    _need(q_pos, "q_pos", _I32, 1, dev)
    n_q, H_I, d_I = q_idx.shape
    if tuple(w.shape) != (n_q, H_I) or k_idx.shape[1] != d_I or q_pos.shape[0] != n_q:
        raise ValueError("inconsistent indexer shapes")
    if out is None:
        out = torch.empty((n_q, top_k), dtype=torch.int32, device=dev)
    _need(out, "out", _I32, 2, dev, shape=(n_q, top_k))
    ws, nb = _workspace(indexer_topk_workspace_size(n_q, top_k), dev, workspace)
    _check(lib.dsa_indexer_topk(_ptr(q_idx), _ptr(w), _ptr(k_idx), k_idx.shape[0], _ptr(q_pos),
                                n_q, H_I, d_I, top_k, _ptr(out), _ptr(ws), nb, _stream(dev)),
           "dsa_indexer_topk")
    return out


def indexer_topk_paged_workspace_size(B: int, max_pages: int, page_size: int) -> int:
    return int(load_library().dsa_indexer_topk_paged_workspace_size(B, max_pages, page_size))


def indexer_topk_paged(q_idx, w, k_cache, page_table, ctx_lens, top_k: int, out=None,
                       workspace=None):
    """Decode indexer + top-k over a paged FP8 key cache [n_pages, page_size, d_I]."""
    lib = load_library()
    _need(q_idx, "q_idx", _FP8, 3)
    dev = q_idx.device
    _need(w, "w", _F32, 2, dev)
    _need(k_cache, "k_cache", _FP8, 3, dev)
    _need(page_table, "page_table", _I32, 2, dev)
    _need(ctx_lens, "ctx_lens", _I32, 1, dev)
    B, H_I, d_I = q_idx.shape
    n_pages, page_size, dk = k_cache.shape
    max_pages = page_table.shape[1]
    if tuple(w.shape) != (B, H_I) or dk != d_I or page_table.shape[0] != B or ctx_lens.shape[0] != B:
        raise ValueError("inconsistent paged indexer shapes")
    if out is None:
        out = torch.empty((B, top_k), dtype=torch.int32, device=dev)
    _need(out, "out", _I32, 2, dev, shape=(B, top_k))
    ws, nb = _workspace(indexer_topk_paged_workspace_size(B, max_pages, page_size), dev, workspace)
    _check(lib.dsa_indexer_topk_paged(_ptr(q_idx), _ptr(w), _ptr(k_cache), _ptr(page_table),
                                      _ptr(ctx_lens), B, max_pages, n_pages, page_size, H_I, d_I,
                                      top_k, _ptr(out), _ptr(ws), nb, _stream(dev)),
           "dsa_indexer_topk_paged")
    return out


def sparse_mqa_prefill(q, kv, idx, q_pos, d_v: int, scale: float, out=None, lse=None,
                       want_lse: bool = True):
    """Sparse MQA prefill.  q [n_q,H,D_k] bf16, kv [n_kv,D_k] bf16, idx [n_q,top_k] int32,
    q_pos [n_q] int32 -> (out [n_q,H,d_v] bf16, lse [n_q,H] fp32 or None)."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    _need(kv, "kv", _BF16, 2, dev)
    _need(idx, "idx", _I32, 2, dev)
    _need(q_pos, "q_pos", _I32, 1, dev)
    n_q, H, D_k = q.shape
    if kv.shape[1] != D_k or idx.shape[0] != n_q or q_pos.shape[0] != n_q:
        raise ValueError("inconsistent MQA shapes")
    if out is None:
        out = torch.empty((n_q, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((n_q, H), dtype=torch.float32, device=dev)
    _need(out, "out", _BF16, 3, dev, shape=(n_q, H, d_v))
    if lse is not None:
        _need(lse, "lse", _F32, 2, dev, shape=(n_q, H))
    _check(lib.dsa_sparse_mqa_prefill(_ptr(q), _ptr(kv), kv.shape[0], _ptr(idx), _ptr(q_pos),
                                      n_q, H, D_k, d_v, idx.shape[1], float(scale), _ptr(out),
                                      _ptr(lse), _stream(dev)),
           "dsa_sparse_mqa_prefill")
    return out, lse


def sparse_mqa_decode_workspace_size(B: int, H: int, d_v: int, top_k: int, n_split: int = 0) -> int:
    return int(load_library().dsa_sparse_mqa_decode_workspace_size(B, H, d_v, top_k, n_split))


def sparse_mqa_decode(q, kv_cache, page_table, ctx_lens, idx, d_v: int, scale: float,
                      n_split: int = 0, out=None, lse=None, want_lse: bool = True,
                      workspace=None):
    """Sparse MQA decode over a paged bf16 KV cache [n_pages, page_size, D_k]."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    _need(kv_cache, "kv_cache", _BF16, 3, dev)
    _need(page_table, "page_table", _I32, 2, dev)
    _need(ctx_lens, "ctx_lens", _I32, 1, dev)
    _need(idx, "idx", _I32, 2, dev)
    B, H, D_k = q.shape
    n_pages, page_size, dk = kv_cache.shape
    top_k = idx.shape[1]
    if dk != D_k or page_table.shape[0] != B or ctx_lens.shape[0] != B or idx.shape[0] != B:
        raise ValueError("inconsistent decode shapes")
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _need(out, "out", _BF16, 3, dev, shape=(B, H, d_v))
    if lse is not None:
        _need(lse, "lse", _F32, 2, dev, shape=(B, H))
    ws, nb = _workspace(sparse_mqa_decode_workspace_size(B, H, d_v, top_k, n_split), dev,
                        workspace)
    _check(lib.dsa_sparse_mqa_decode(_ptr(q), _ptr(kv_cache), _ptr(page_table), _ptr(ctx_lens),
                                     _ptr(idx), B, page_table.shape[1], n_pages, page_size, H,
                                     D_k, d_v, top_k, float(scale), n_split, _ptr(out), _ptr(lse),
                                     _ptr(ws), nb, _stream(dev)),
           "dsa_sparse_mqa_decode")
    return out, lse


def indexer_topk_batched(q_idx, w, k_cache, page_table, q_pos, top_k: int, q_seq=None,
                         out=None, workspace=None):
    """Batched prefill indexer + top-k over a paged FP8 key cache (dsa_indexer_topk_batched):
    query row i of sequence q_seq[i] (default 0) at position q_pos[i]."""
    lib = load_library()
    _need(q_idx, "q_idx", _FP8, 3)
    dev = q_idx.device
    n_q, H_I, d_I = q_idx.shape
    _need(w, "w", _F32, 2, dev, shape=(n_q, H_I))
    _need(k_cache, "k_cache", _FP8, 3, dev)
    _need(page_table, "page_table", _I32, 2, dev)
    _need(q_pos, "q_pos", _I32, 1, dev, shape=(n_q,))
    if q_seq is not None:
        _need(q_seq, "q_seq", _I32, 1, dev, shape=(n_q,))
    n_pages, page_size, dk = k_cache.shape
    if dk != d_I:
        raise ValueError("k_cache rows do not match q_idx")
    if out is None:
        out = torch.empty((n_q, top_k), dtype=torch.int32, device=dev)
    _need(out, "out", _I32, 2, dev, shape=(n_q, top_k))
    ws, nb = _workspace(indexer_topk_workspace_size(n_q, top_k), dev, workspace)
    _check(lib.dsa_indexer_topk_batched(_ptr(q_idx), _ptr(w), _ptr(k_cache), _ptr(page_table),
                                        page_table.shape[0], page_table.shape[1], n_pages,
                                        page_size, _ptr(q_seq), _ptr(q_pos), n_q, H_I, d_I, top_k,
                                        _ptr(out), _ptr(ws), nb, _stream(dev)),
           "dsa_indexer_topk_batched")
    return out


def sparse_mqa_batched(q, kv_cache, page_table, q_pos, idx, d_v: int, scale: float, q_seq=None,
                       out=None, lse=None, want_lse: bool = True):
    """Batched sparse MQA over a paged bf16 KV cache (dsa_sparse_mqa_batched)."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    n_q, H, D_k = q.shape
    _need(kv_cache, "kv_cache", _BF16, 3, dev)
    _need(page_table, "page_table", _I32, 2, dev)
    _need(q_pos, "q_pos", _I32, 1, dev, shape=(n_q,))
    _need(idx, "idx", _I32, 2, dev)
    if q_seq is not None:
        _need(q_seq, "q_seq", _I32, 1, dev, shape=(n_q,))
    n_pages, page_size, dk = kv_cache.shape
    if dk != D_k or idx.shape[0] != n_q:
        raise ValueError("inconsistent batched MQA shapes")
    if out is None:
        out = torch.empty((n_q, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((n_q, H), dtype=torch.float32, device=dev)
    _need(out, "out", _BF16, 3, dev, shape=(n_q, H, d_v))
    if lse is not None:
        _need(lse, "lse", _F32, 2, dev, shape=(n_q, H))
    _check(lib.dsa_sparse_mqa_batched(_ptr(q), _ptr(kv_cache), _ptr(page_table),
                                      page_table.shape[0], page_table.shape[1], n_pages,
                                      page_size, _ptr(q_seq), _ptr(q_pos), _ptr(idx), n_q, H, D_k,
                                      d_v, idx.shape[1], float(scale), _ptr(out), _ptr(lse),
                                      _stream(dev)),
           "dsa_sparse_mqa_batched")
    return out, lse


def dense_mqa_workspace_size(n_q: int, H: int, d_v: int, max_len: int) -> int:
    return int(load_library().dsa_dense_mqa_workspace_size(n_q, H, d_v, max_len))


def dense_mqa_prefill(q, kv, q_pos, d_v: int, scale: float, out=None, lse=None,
                      want_lse: bool = True, workspace=None):
    """Dense causal attention of every query row over positions 0..t (the baseline)."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    n_q, H, D_k = q.shape
    _need(kv, "kv", _BF16, 2, dev)
    _need(q_pos, "q_pos", _I32, 1, dev, shape=(n_q,))
    if kv.shape[1] != D_k:
        raise ValueError("kv rows do not match q")
    if out is None:
        out = torch.empty((n_q, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((n_q, H), dtype=torch.float32, device=dev)
    _need(out, "out", _BF16, 3, dev, shape=(n_q, H, d_v))
    if lse is not None:
        _need(lse, "lse", _F32, 2, dev, shape=(n_q, H))
    ws, nb = _workspace(dense_mqa_workspace_size(n_q, H, d_v, kv.shape[0]), dev, workspace)
    _check(lib.dsa_dense_mqa_prefill(_ptr(q), _ptr(kv), kv.shape[0], _ptr(q_pos), n_q, H, D_k,
                                     d_v, float(scale), _ptr(out), _ptr(lse), _ptr(ws), nb,
                                     _stream(dev)),
           "dsa_dense_mqa_prefill")
    return out, lse


def dense_mqa_decode(q, kv_cache, page_table, ctx_lens, d_v: int, scale: float, out=None,
                     lse=None, want_lse: bool = True, workspace=None):
    """Dense attention of one query per sequence over its positions [0, ctx) (the baseline)."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    B, H, D_k = q.shape
    _need(kv_cache, "kv_cache", _BF16, 3, dev)
    _need(page_table, "page_table", _I32, 2, dev)
    _need(ctx_lens, "ctx_lens", _I32, 1, dev, shape=(B,))
    n_pages, page_size, dk = kv_cache.shape
    if dk != D_k or page_table.shape[0] != B:
        raise ValueError("inconsistent dense decode shapes")
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _need(out, "out", _BF16, 3, dev, shape=(B, H, d_v))
    if lse is not None:
        _need(lse, "lse", _F32, 2, dev, shape=(B, H))
    max_len = page_table.shape[1] * page_size
    ws, nb = _workspace(dense_mqa_workspace_size(B, H, d_v, max_len), dev, workspace)
    _check(lib.dsa_dense_mqa_decode(_ptr(q), _ptr(kv_cache), _ptr(page_table), _ptr(ctx_lens), B,
                                    page_table.shape[1], n_pages, page_size, H, D_k, d_v,
                                    float(scale), _ptr(out), _ptr(lse), _ptr(ws), nb,
                                    _stream(dev)),
           "dsa_dense_mqa_decode")
    return out, lse


def indexer_kl(q, kv, idx, q_pos, lse, scale: float, q_idx, w, k_idx, want_grad: bool = True):
    """The indexer's training signal (dsa_indexer_kl): returns (loss [n_q], target [n_q, top_k],
    grad [n_q, top_k] or None) for the index lists idx, given the forward's lse."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    n_q, H, D_k = q.shape
    top_k = idx.shape[1] if isinstance(idx, torch.Tensor) else 0
    _need(kv, "kv", _BF16, 2, dev)
    _need(idx, "idx", _I32, 2, dev, shape=(n_q, top_k))
    _need(q_pos, "q_pos", _I32, 1, dev, shape=(n_q,))
    _need(lse, "lse", _F32, 2, dev, shape=(n_q, H))
    _need(q_idx, "q_idx", _FP8, 3, dev)
    H_I, d_I = q_idx.shape[1], q_idx.shape[2]
    _need(q_idx, "q_idx", _FP8, 3, dev, shape=(n_q, H_I, d_I))
    _need(w, "w", _F32, 2, dev, shape=(n_q, H_I))
    _need(k_idx, "k_idx", _FP8, 2, dev, shape=(kv.shape[0], d_I))
    if kv.shape[1] != D_k:
        raise ValueError("kv rows do not match q")
    target = torch.empty((n_q, top_k), dtype=torch.float32, device=dev)
    loss = torch.empty((n_q,), dtype=torch.float32, device=dev)
    grad = torch.empty((n_q, top_k), dtype=torch.float32, device=dev) if want_grad else None
    _check(lib.dsa_indexer_kl(_ptr(q), _ptr(kv), kv.shape[0], _ptr(idx), _ptr(q_pos), _ptr(lse),
                              n_q, H, D_k, top_k, float(scale), _ptr(q_idx), _ptr(w), _ptr(k_idx),
                              H_I, d_I, _ptr(target), _ptr(loss), _ptr(grad), _stream(dev)),
           "dsa_indexer_kl")
    return loss, target, grad


def sparse_mqa_backward(q, kv, idx, q_pos, out, lse, d_out, scale: float, d_kv=None,
                        workspace=None):
    """Gradients of sum(d_out * out) for dsa_sparse_mqa_prefill's attention
    (dsa_sparse_mqa_backward): returns (d_q fp32 [n_q, H, D_k], d_kv fp32 [n_kv, D_k]).  A given
    d_kv is accumulated into (a new one starts at zero)."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    n_q, H, D_k = q.shape
    _need(kv, "kv", _BF16, 2, dev)
    n_kv = kv.shape[0]
    _need(idx, "idx", _I32, 2, dev)
    top_k = idx.shape[1]
    _need(idx, "idx", _I32, 2, dev, shape=(n_q, top_k))
    _need(q_pos, "q_pos", _I32, 1, dev, shape=(n_q,))
    _need(out, "out", _BF16, 3, dev)
    d_v = out.shape[2]
    _need(out, "out", _BF16, 3, dev, shape=(n_q, H, d_v))
    _need(lse, "lse", _F32, 2, dev, shape=(n_q, H))
    _need(d_out, "d_out", _BF16, 3, dev, shape=(n_q, H, d_v))
    if kv.shape[1] != D_k:
        raise ValueError("kv rows do not match q")
    d_q = torch.empty((n_q, H, D_k), dtype=torch.float32, device=dev)
    if d_kv is None:
        d_kv = torch.zeros((n_kv, D_k), dtype=torch.float32, device=dev)
    _need(d_kv, "d_kv", _F32, 2, dev, shape=(n_kv, D_k))
    nbytes = int(lib.dsa_sparse_mqa_backward_workspace_size(n_q, H, top_k))
    ws, nb = _workspace(nbytes, dev, workspace)
    _check(lib.dsa_sparse_mqa_backward(_ptr(q), _ptr(kv), n_kv, _ptr(idx), _ptr(q_pos), _ptr(out),
                                       _ptr(lse), _ptr(d_out), n_q, H, D_k, d_v, top_k,
                                       float(scale), _ptr(d_q), _ptr(d_kv), _ptr(ws), nb,
                                       _stream(dev)),
           "dsa_sparse_mqa_backward")
    return d_q, d_kv


def cache_append(page_table, pos, k_cache=None, kv_cache=None, k_new=None, kv_new=None,
                 seq=None):
    """Append new tokens to the paged caches (dsa_cache_append): k_new [T, d_I] bf16 is
    quantised to e4m3fn into k_cache [n_pages, page_size, d_I] (uint8 / float8_e4m3fn) and
    kv_new [T, D_k] bf16 copied into kv_cache [n_pages, page_size, D_k] at logical position
    pos[r] of sequence seq[r] (default: r).  The caches are updated in place."""
    lib = load_library()
    _need(page_table, "page_table", _I32, 2)
    dev = page_table.device
    _need(pos, "pos", _I32, 1, dev)
    T = pos.shape[0]
    if seq is not None:
        _need(seq, "seq", _I32, 1, dev, shape=(T,))
    if k_new is None and kv_new is None:
        raise ValueError("nothing to append: give k_new and/or kv_new")
    d_I = D_k = 0
    geo = None
    if k_new is not None:
        _need(k_new, "k_new", _BF16, 2, dev)
        d_I = k_new.shape[1]
        _need(k_new, "k_new", _BF16, 2, dev, shape=(T, d_I))
        if k_cache is None:
            raise ValueError("k_new given without k_cache")
        _need(k_cache, "k_cache", _FP8, 3, dev)
        if k_cache.shape[2] != d_I:
            raise ValueError("k_cache rows do not match k_new")
        geo = tuple(k_cache.shape[:2])
    if kv_new is not None:
        _need(kv_new, "kv_new", _BF16, 2, dev)
        D_k = kv_new.shape[1]
        _need(kv_new, "kv_new", _BF16, 2, dev, shape=(T, D_k))
        if kv_cache is None:
            raise ValueError("kv_new given without kv_cache")
        _need(kv_cache, "kv_cache", _BF16, 3, dev)
        if kv_cache.shape[2] != D_k or (geo is not None and tuple(kv_cache.shape[:2]) != geo):
            raise ValueError("kv_cache does not match kv_new or k_cache")
        geo = tuple(kv_cache.shape[:2])
    n_pages, page_size = geo
    _check(lib.dsa_cache_append(_ptr(k_new), _ptr(kv_new), _ptr(seq), _ptr(pos),
                                _ptr(page_table), T, page_table.shape[1], n_pages, page_size,
                                d_I, D_k, _ptr(k_cache if k_new is not None else None),
                                _ptr(kv_cache if kv_new is not None else None), _stream(dev)),
           "dsa_cache_append")
    return k_cache, kv_cache


def sparse_mqa_decode_noalloc(q, kv_cache, page_table, ctx_lens, idx, d_v: int, scale: float,
                              n_split: int = 0, out=None, lse=None, want_lse: bool = True):
    """dsa_sparse_mqa_decode_noalloc: as sparse_mqa_decode, with the split partials in the
    library's static per-device scratch array instead of a workspace (outputs are still
    allocated here unless given)."""
    lib = load_library()
    _need(q, "q", _BF16, 3)
    dev = q.device
    _need(kv_cache, "kv_cache", _BF16, 3, dev)
    _need(page_table, "page_table", _I32, 2, dev)
    _need(ctx_lens, "ctx_lens", _I32, 1, dev)
    _need(idx, "idx", _I32, 2, dev)
    B, H, D_k = q.shape
    n_pages, page_size, dk = kv_cache.shape
    top_k = idx.shape[1]
    if dk != D_k or page_table.shape[0] != B or ctx_lens.shape[0] != B or idx.shape[0] != B:
        raise ValueError("inconsistent decode shapes")
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _need(out, "out", _BF16, 3, dev, shape=(B, H, d_v))
    if lse is not None:
        _need(lse, "lse", _F32, 2, dev, shape=(B, H))
    _check(lib.dsa_sparse_mqa_decode_noalloc(_ptr(q), _ptr(kv_cache), _ptr(page_table),
                                             _ptr(ctx_lens), _ptr(idx), B, page_table.shape[1],
                                             n_pages, page_size, H, D_k, d_v, top_k,
                                             float(scale), n_split, _ptr(out), _ptr(lse),
                                             _stream(dev)),
           "dsa_sparse_mqa_decode_noalloc")
    return out, lse


__all__ = ["load_library", "DSAError", "indexer_topk", "indexer_topk_paged",
           "sparse_mqa_prefill", "sparse_mqa_decode", "sparse_mqa_decode_noalloc", "cache_append",
           "indexer_topk_batched", "sparse_mqa_batched", "dense_mqa_prefill",
           "dense_mqa_decode", "dense_mqa_workspace_size", "indexer_kl", "sparse_mqa_backward",
           "indexer_topk_workspace_size",
           "indexer_topk_paged_workspace_size", "sparse_mqa_decode_workspace_size",
           "SIGNATURES", "LIB_PATH"]


def ceiling_mfma(kind: int, n_wg: int, iters: int, sink: torch.Tensor) -> float:
    """Launch the MFMA ceiling loop (kind 0: bf16 32x32x16, kind 1: FP8 16x16x128) on the
    current stream; returns the launch's flop count.  sink: float32 [n_wg * 512] on the GPU."""
    _need(sink, "sink", (torch.float32,), 1)
    if sink.numel() < n_wg * 512:
        raise ValueError("sink too small")
    flops = ctypes.c_double(0.0)
    _check(load_library().dsa_ceiling_mfma(kind, n_wg, iters, _ptr(sink), ctypes.byref(flops),
                                           _stream(sink.device)), "dsa_ceiling_mfma")
    return flops.value


def ceiling_read(src: torch.Tensor, n_wg: int, sink: torch.Tensor) -> int:
    """Launch the streaming-read ceiling kernel over src's bytes on the current stream;
    returns the byte count.  sink: float32 [n_wg * 256] on the GPU."""
    _need(sink, "sink", (torch.float32,), 1)
    if sink.numel() < n_wg * 256 or not src.is_contiguous():
        raise ValueError("sink too small or src not contiguous")
    nbytes = src.numel() * src.element_size() // 16 * 16
    _check(load_library().dsa_ceiling_read(_ptr(src), nbytes, n_wg, _ptr(sink),
                                           _stream(sink.device)), "dsa_ceiling_read")
    return nbytes


def ceiling_gather(kind: int, pool: torch.Tensor, idx: torch.Tensor, n_wg: int,
                   sink: torch.Tensor) -> int:
    """Launch the random-row gather ceiling kernel (kind 0: LDS DMA, kind 1: register loads)
    over the rows of pool [n_rows, ...] listed in idx [n_q, top_k] int32, on the current
    stream; returns the bytes gathered.  sink: float32 [n_wg * 512] on the GPU."""
    _need(sink, "sink", (torch.float32,), 1)
    _need(idx, "idx", (torch.int32,), 2)
    if sink.numel() < n_wg * 512 or not pool.is_contiguous():
        raise ValueError("sink too small or pool not contiguous")
    row_bytes = pool[0].numel() * pool.element_size()
    n_q, top_k = idx.shape
    _check(load_library().dsa_ceiling_gather(kind, _ptr(pool), pool.shape[0], row_bytes,
                                             _ptr(idx), n_q, top_k, n_wg, _ptr(sink),
                                             _stream(sink.device)), "dsa_ceiling_gather")
    return n_q * top_k * row_bytes

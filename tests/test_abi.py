"""The C-ABI library builds, loads and exports every declared symbol; host-side argument checks.

CPU only: no call here reaches a kernel launch (each returns a status from the host checks
before anything is enqueued), so these run on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

import sparse_attention_long_gemm_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("dsa_indexer_topk", "dsa_indexer_topk_paged", "dsa_sparse_mqa_prefill",
              "dsa_sparse_mqa_decode", "dsa_sparse_mqa_decode_noalloc", "dsa_status_string",
              "dsa_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = dsa.load_library()
    for n in _declared_functions():
        assert hasattr(lib, n), f"missing export {n}"
        assert n in dsa.SIGNATURES, f"binding lacks a signature for {n}"
    assert set(dsa.SIGNATURES) == set(_declared_functions())


def test_abi_version_and_status_strings():
    lib = dsa.load_library()
    assert lib.dsa_abi_version() == 1
    for code, name in [(0, b"DSA_OK"), (-1, b"DSA_ERR_INVALID_ARG"),
                       (-2, b"DSA_ERR_UNSUPPORTED_SHAPE"), (-3, b"DSA_ERR_WORKSPACE_TOO_SMALL"),
                       (-4, b"DSA_ERR_HIP"), (-5, b"DSA_ERR_SCRATCH_LIMIT")]:
        assert lib.dsa_status_string(code).startswith(name)
    assert lib.dsa_status_string(12345) == b"unknown dsa_status"


def test_ceiling_helpers_reject_bad_arguments():
    lib = dsa.load_library()
    flops = ctypes.c_double(0.0)
    fake = ctypes.c_void_p(16)   # never dereferenced: every call below fails its host checks
    assert lib.dsa_ceiling_mfma(2, 1, 1, fake, ctypes.byref(flops), None) == -1
    assert lib.dsa_ceiling_mfma(0, 0, 1, fake, ctypes.byref(flops), None) == -1
    assert lib.dsa_ceiling_mfma(0, 1, 1, fake, None, None) == -1
    assert lib.dsa_ceiling_read(fake, 24, 1, fake, None) == -1
    assert lib.dsa_ceiling_read(fake, 0, 1, fake, None) == -1
    assert lib.dsa_ceiling_read(None, 32, 1, fake, None) == -1
    # gather: kind, row size (multiple of 16, at most 2048 bytes), index rows of whole chunks
    assert lib.dsa_ceiling_gather(2, fake, 10, 1152, fake, 1, 32, 1, fake, None) == -1
    assert lib.dsa_ceiling_gather(0, fake, 10, 1160, fake, 1, 32, 1, fake, None) == -1
    assert lib.dsa_ceiling_gather(0, fake, 10, 2064, fake, 1, 32, 1, fake, None) == -1
    assert lib.dsa_ceiling_gather(0, fake, 10, 1152, fake, 1, 48, 1, fake, None) == -1
    assert lib.dsa_ceiling_gather(0, fake, 10, 1152, fake, 1, 0, 1, fake, None) == -1
    assert lib.dsa_ceiling_gather(0, fake, 0, 1152, fake, 1, 32, 1, fake, None) == -1
    assert lib.dsa_ceiling_gather(1, fake, 10, 1152, None, 1, 32, 1, fake, None) == -1
    assert lib.dsa_ceiling_gather(1, fake, 10, 1152, fake, 1, 32, 0, fake, None) == -1


def test_workspace_sizes():
    lib = dsa.load_library()
    # candidate lists of (score, position) pairs per row: room for top_k kept items plus two
    # 128-key tiles of appends: 3*top_k + 128, at least top_k + 256, rounded up to 128 entries
    assert lib.dsa_indexer_topk_workspace_size(4096, 2048) == 4096 * 6272 * 8
    assert lib.dsa_indexer_topk_workspace_size(16, 32) == 16 * 384 * 8
    assert lib.dsa_indexer_topk_workspace_size(-1, 32) == 0
    # paged: per key slot an fp32 score and a candidate (order key, position); per row a
    # 4096-bin histogram, 4 counters and a 2048-entry list (each part 256-byte aligned)
    rs = 2048 * 64
    assert lib.dsa_indexer_topk_paged_workspace_size(64, 2048, 64) == \
        3 * 64 * rs * 4 + 64 * 4096 * 4 + 1024 + 64 * 2048 * 4
    # B=64, top_k=2048 -> 4 splits of 512 rows: partial o (bf16) + (max, sum) in fp32 per head
    assert lib.dsa_sparse_mqa_decode_workspace_size(64, 128, 512, 2048, 0) == 64 * 4 * 128 * (512 * 2 + 8)
    assert lib.dsa_sparse_mqa_decode_workspace_size(64, 128, 512, 2048, 1) == 0
    assert lib.dsa_sparse_mqa_decode_workspace_size(64, 128, 512, 32, 0) == 0


P = ctypes.c_void_p
FAKE = P(0x1000)   # never dereferenced: every call below fails the host checks first

# The calls below pass made-up device addresses; each is meant to fail the host checks, but
# they are kept off any machine where a mistake in a case could reach a real launch.
try:
    import torch as _torch
    _GPU = _torch.cuda.is_available()
except Exception:  # pragma: no cover
    _GPU = False
host_only = pytest.mark.skipif(_GPU, reason="fake-pointer host checks run only without a GPU")


@pytest.mark.parametrize("args,code", [
    # (q_idx, w, k_idx, n_keys, q_pos, n_q, H_I, d_I, top_k, out, ws, ws_bytes, stream)
    ((None, None, None, 10, None, 5, 4, 32, 32, None, None, 0, None), -1),      # nulls
    ((FAKE, FAKE, FAKE, 10, FAKE, 5, 4, 33, 32, FAKE, FAKE, 1 << 30, None), -2),  # d_I % 16
    ((FAKE, FAKE, FAKE, 10, FAKE, 5, 65, 32, 32, FAKE, FAKE, 1 << 30, None), -2),  # H_I > 64
    ((FAKE, FAKE, FAKE, 10, FAKE, 5, 4, 32, 2049, FAKE, FAKE, 1 << 30, None), -2),  # k > 2048
    ((FAKE, FAKE, FAKE, 10, FAKE, 5, 4, 32, 0, FAKE, FAKE, 1 << 30, None), -2),     # k = 0
    ((FAKE, FAKE, FAKE, 10, FAKE, 5, 4, 32, 32, FAKE, FAKE, 100, None), -3),        # ws small
    ((FAKE, FAKE, FAKE, -1, FAKE, 5, 4, 32, 32, FAKE, FAKE, 1 << 30, None), -1),    # n_keys<0
    ((None, None, None, 10, None, 0, 4, 32, 32, None, None, 0, None), 0),           # n_q = 0
])
@host_only
def test_indexer_host_checks(args, code):
    assert dsa.load_library().dsa_indexer_topk(*args) == code


@host_only
def test_paged_indexer_host_checks():
    f = dsa.load_library().dsa_indexer_topk_paged
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 10, 40, 64, 64, 128, 2048, FAKE, FAKE, 1 << 40, None]
    for pos, val, code in [(8, 0, -1), (6, 0, -1), (7, 0, -1), (10, 33, -2), (9, 65, -2),
                           (11, 4096, -2), (14, 100, -3),
                           (3, None, -1), (13, 0, -1)]:
        a = list(ok)
        a[pos] = val
        if pos == 13:
            a[13] = None                 # workspace pointer
        assert f(*a) == code, (pos, val)


@host_only
def test_mqa_host_checks():
    lib = dsa.load_library()
    f = lib.dsa_sparse_mqa_prefill
    ok = [FAKE, FAKE, 100, FAKE, FAKE, 3, 128, 576, 512, 2048, 0.0416, FAKE, None, None]
    for pos, val, code in [(6, 129, -2), (7, 512, -2), (8, 256, -2), (2, 0, -1),
                           (10, float("inf"), -1), (0, None, -1), (11, None, -1), (9, 4096, -2)]:
        a = list(ok)
        a[pos] = val
        assert f(*a) == code, (pos, val)
    g = lib.dsa_sparse_mqa_decode
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 2048, 70000, 64, 128, 576, 512, 2048, 0.04, 0,
          FAKE, None, FAKE, 1 << 40, None]
    for pos, val, code in [(14, 17, -1), (8, 0, -1), (18, 10, -3), (17, None, -3),
                           (2, None, -1), (10, 100, -2)]:
        a = list(ok)
        a[pos] = val
        assert g(*a) == code, (pos, val)


@host_only
def test_noalloc_decode_host_checks():
    """The allocation-free decode applies the workspace variant's checks, and refuses a call
    whose partials exceed its static scratch array, before anything is launched."""
    g = dsa.load_library().dsa_sparse_mqa_decode_noalloc
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 2048, 70000, 64, 128, 576, 512, 2048, 0.04, 0,
          FAKE, None, None]
    for change, code in [({13: float("nan")}, -1), ({14: 17}, -1), ({8: 0}, -1),
                         ({2: None}, -1), ({10: 100}, -2), ({9: 129}, -2),
                         ({5: 600, 14: 4}, -5),   # 600 x 4 splits x 128 heads x 1032 B > 64 MiB
                         ({5: 0}, 0)]:            # nothing to do
        a = list(ok)
        for pos, val in change.items():
            a[pos] = val
        assert g(*a) == code, change


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((4, 4, 32), dtype=torch.uint8)
    with pytest.raises(ValueError):
        dsa.indexer_topk(x, torch.zeros((4, 4)), torch.zeros((8, 32), dtype=torch.uint8),
                         torch.zeros(4, dtype=torch.int32), 8)


def test_binding_output_and_workspace_checks():
    """The binding's argument checks (run on host tensors, no GPU needed): an output of the
    wrong shape and a workspace that is not device memory are refused."""
    import torch
    from sparse_attention_long_gemm_amd import _need, _workspace
    out = torch.empty((3, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="expected shape"):
        _need(out, "out", (torch.int32,), 2, shape=(3, 5))
    with pytest.raises(TypeError):
        _need(out, "out", (torch.float32,), 2, shape=(3, 4))
    with pytest.raises(ValueError, match="device"):
        _need(out, "out", (torch.int32,), 2, shape=(3, 4))       # host tensor
    with pytest.raises(ValueError, match="expected cuda"):
        _workspace(64, torch.device("cuda", 0), torch.empty(128, dtype=torch.uint8))
    with pytest.raises(TypeError):
        _workspace(64, torch.device("cuda", 0), bytearray(128))

"""The allocation-free decode attention (dsa_sparse_mqa_decode_noalloc) against the workspace
entry point (dsa_sparse_mqa_decode), through the C ABI: same kernels and split, so the outputs
must be identical, on two calls in a row (the second with a smaller batch, fewer splits and
shorter rows, so anything left over from the first call would show), plus the oracle gate and
the refusal of a call whose partials exceed the static scratch array."""
import ctypes

import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

from gates import check_attn, check_idx

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


def _case(spec, ctx, n_split):
    dsa = _dsa()
    d = gi.decode_inputs(spec, ctx_lens=ctx)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    idx = dsa.indexer_topk_paged(g["q_idx"], g["w"], g["k_cache"], g["page_table"], g["ctx"],
                                 d["top_k"])
    o_na, l_na = dsa.sparse_mqa_decode_noalloc(g["q"], g["kv_cache"], g["page_table"], g["ctx"],
                                               idx, d["D_v"], d["scale"], n_split=n_split)
    o_ws, l_ws = dsa.sparse_mqa_decode(g["q"], g["kv_cache"], g["page_table"], g["ctx"], idx,
                                       d["D_v"], d["scale"], n_split=n_split)
    torch.cuda.synchronize()
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
    assert torch.equal(l_na, l_ws)
    i_ref, o_ref, l_ref = orc.decode(d)
    check_idx(idx, i_ref, "noalloc idx")
    check_attn(o_na, l_na, o_ref, l_ref, "noalloc attn")


def test_noalloc_decode_matches_workspace_entry_point_twice():
    dsa = _dsa()
    assert dsa.sparse_mqa_decode_workspace_size(64, 128, 512, 2048, 0) <= (64 << 20)
    step("noalloc decode: B=64, k=2048, library split (4), ctx 2100..9000")
    ctx1 = tuple(int(c) for c in np.linspace(2100, 9000, 64))
    _case(gi.DecodeSpec(B=64, idx=gi.IndexerSpec(top_k=2048), mqa=gi.MqaSpec(sigma=1.0),
                        seed=61), ctx1, 0)
    step("noalloc decode: B=5, k=512, 3 splits, shorter rows (second call)")
    _case(gi.DecodeSpec(B=5, idx=gi.IndexerSpec(top_k=512), mqa=gi.MqaSpec(sigma=1.0),
                        seed=62), (600, 513, 2000, 100, 1), 3)


def test_noalloc_decode_refuses_calls_beyond_the_scratch_array():
    """B * n_split * H * (2 D_v + 8) bytes of partials beyond DSA_NOALLOC_SCRATCH_BYTES: the
    call returns DSA_ERR_SCRATCH_LIMIT and enqueues nothing (real, zero-context tensors, so
    that nothing could be read out of bounds even if it did)."""
    dsa = _dsa()
    lib = dsa.load_library()
    B, H, D_k, D_v, k, P = 600, 128, 576, 512, 2048, 64
    need = dsa.sparse_mqa_decode_workspace_size(B, H, D_v, k, 4)
    assert need > (64 << 20)
    q = torch.zeros((B, H, D_k), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((4, P, D_k), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    ctx = torch.zeros(B, dtype=torch.int32, device="cuda")
    idx = torch.full((B, k), -1, dtype=torch.int32, device="cuda")
    out = torch.full((B, H, D_v), 7.0, dtype=torch.bfloat16, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.dsa_sparse_mqa_decode_noalloc(p(q), p(kv), p(pt), p(ctx), p(idx), B, 1, 4, P, H,
                                           D_k, D_v, k, 0.04, 4, p(out), None,
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == -5
    assert lib.dsa_status_string(rc).startswith(b"DSA_ERR_SCRATCH_LIMIT")
    assert (out.float() == 7.0).all()          # nothing was written
    with pytest.raises(dsa.DSAError):
        dsa.sparse_mqa_decode_noalloc(q, kv, pt, ctx, idx, D_v, 0.04, n_split=4)

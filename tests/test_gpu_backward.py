"""GPU parity of the sparse MQA backward (dsa_sparse_mqa_backward) through the C ABI, against
the oracle's analytic gradients (themselves pinned to torch autograd in fp64).

Gates: max |g - g_ref| / max |g_ref| <= 1e-2 for d_q and d_kv, the attention gate's form.  P
and dS enter the dQ / dKV products in bf16 (8 significant bits, like the forward's P), and the
forward's bf16 output enters rowsum(dO o); the errors this leaves are a few 1e-3 of the largest
gradient at most.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

pytestmark = pytest.mark.gpu

REL = 1e-2


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


def _grads(D_k, D_v, H, L, top_k, sharp, seed, bad_entries=False):
    dsa = _dsa()
    wl = gi.Workload(name="bw", L=L, idx=gi.IndexerSpec(top_k=top_k),
                     mqa=gi.MqaSpec(H=H, D_k=D_k, D_v=D_v, sigma=1.0 if sharp else D_k ** -0.5,
                                    scale=D_k ** -0.5), seed=seed)
    d = gi.prefill_inputs(wl)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    idx = dsa.indexer_topk(g["q_idx"], g["w"], g["k_idx"], g["q_pos"], top_k)
    if bad_entries:
        idx[L // 2, 1] = -1
        idx[L // 2 + 1, 0] = L - 1      # beyond t: skipped
    o, lse = dsa.sparse_mqa_prefill(g["q"], g["kv"], idx, g["q_pos"], D_v, d["scale"])
    gen = torch.Generator().manual_seed(seed + 1)
    d_out = torch.randn((L, H, D_v), generator=gen).to(torch.bfloat16)
    d_q, d_kv = dsa.sparse_mqa_backward(g["q"], g["kv"], idx, g["q_pos"], o, lse, d_out.cuda(),
                                        d["scale"])
    torch.cuda.synchronize()
    dq_ref, dkv_ref = orc.sparse_mqa_backward(d, idx.cpu().numpy(), d_out)
    return d_q.cpu().numpy(), d_kv.cpu().numpy(), dq_ref, dkv_ref, (d, g, idx, o, lse, d_out)


@pytest.mark.parametrize("D_k,D_v,H,L,top_k,sharp,bad", [
    (96, 64, 16, 600, 128, True, True),
    (64, 64, 5, 300, 300, True, False),     # every position listed (dense rows)
    (576, 512, 128, 700, 256, True, True),
    (576, 512, 128, 700, 256, False, False),
])
def test_sparse_backward_matches_oracle(D_k, D_v, H, L, top_k, sharp, bad):
    step(f"backward D_k={D_k} H={H} L={L} k={top_k} sharp={sharp}")
    dq, dkv, dq_ref, dkv_ref, _ = _grads(D_k, D_v, H, L, top_k, sharp, 111, bad)
    e_q = np.abs(dq - dq_ref).max() / np.abs(dq_ref).max()
    e_kv = np.abs(dkv - dkv_ref).max() / np.abs(dkv_ref).max()
    print(f"d_q err {e_q:.2e}, d_kv err {e_kv:.2e}", flush=True)
    assert e_q <= REL and e_kv <= REL, (e_q, e_kv)


def test_sparse_backward_accumulates_into_d_kv():
    """A given d_kv is added to: two calls give twice the gradient, up to the fp32 rounding of
    atomic additions in another order (gated against the largest gradient)."""
    dsa = _dsa()
    step("backward accumulation")
    dq, dkv, _, _, (d, g, idx, o, lse, d_out) = _grads(96, 64, 16, 400, 64, True, 113)
    acc = torch.zeros((400, 96), dtype=torch.float32, device="cuda")
    for _ in range(2):
        dsa.sparse_mqa_backward(g["q"], g["kv"], idx, g["q_pos"], o, lse, d_out.cuda(),
                                d["scale"], d_kv=acc)
    torch.cuda.synchronize()
    err = np.abs(acc.cpu().numpy() - 2 * dkv).max() / np.abs(dkv).max()
    print(f"accumulation err {err:.2e}", flush=True)
    assert err <= 1e-4

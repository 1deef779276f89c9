"""GPU parity of the indexer's training signal (dsa_indexer_kl) through the C ABI, against the
oracle: the head-averaged main-attention target over each row's selected list, the KL loss to
the indexer's softmax over the same list, and its gradient with respect to the scores.

Tolerances (fp32 GPU against fp64 oracle, bf16 inputs shared): the logits are fp32 sums of
exact bf16 products and the forward's lse is fp32, so each target probability carries a
relative error of a few 1e-6; gates: target and gradient within 1e-4 of the largest target
magnitude, loss within 1e-4 relative (plus 1e-6 absolute).
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


@pytest.mark.parametrize("D_k,D_v,H,L,top_k,sharp", [
    (576, 512, 128, 3000, 2048, True),
    (576, 512, 128, 3000, 256, False),
    (96, 64, 33, 700, 100, True),
    (64, 64, 8, 300, 300, True),        # every position listed: the dense warm-up form
])
def test_indexer_kl_matches_oracle(D_k, D_v, H, L, top_k, sharp):
    dsa = _dsa()
    wl = gi.Workload(name="kl", L=L, idx=gi.IndexerSpec(top_k=top_k),
                     mqa=gi.MqaSpec(H=H, D_k=D_k, D_v=D_v, sigma=1.0 if sharp else D_k ** -0.5,
                                    scale=D_k ** -0.5), seed=101)
    d = gi.prefill_inputs(wl)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    step(f"indexer KL D_k={D_k} H={H} L={L} k={top_k} sharp={sharp}")
    idx = dsa.indexer_topk(g["q_idx"], g["w"], g["k_idx"], g["q_pos"], top_k)
    _, lse = dsa.sparse_mqa_prefill(g["q"], g["kv"], idx, g["q_pos"], D_v, d["scale"])
    loss, target, grad = dsa.indexer_kl(g["q"], g["kv"], idx, g["q_pos"], lse, d["scale"],
                                        g["q_idx"], g["w"], g["k_idx"])
    torch.cuda.synchronize()
    rows = sorted(set(np.linspace(0, L - 1, 40).astype(int).tolist()) | {0, L - 1})
    l_ref, t_ref, g_ref = orc.indexer_kl(d, idx[rows].cpu().numpy(), rows=rows)
    tg, gg, lg = target[rows].cpu().numpy(), grad[rows].cpu().numpy(), loss[rows].cpu().numpy()
    scale_t = np.abs(t_ref).max()
    err_t = np.abs(tg - t_ref).max() / scale_t
    err_g = np.abs(gg - g_ref).max() / scale_t
    err_l = (np.abs(lg - l_ref) / (np.abs(l_ref) + 1e-2)).max()
    print(f"target err {err_t:.2e}, grad err {err_g:.2e}, loss rel err {err_l:.2e}", flush=True)
    assert err_t <= 1e-4, f"target err {err_t}"
    assert err_g <= 1e-4, f"grad err {err_g}"
    assert (np.abs(lg - l_ref) <= 1e-4 * np.abs(l_ref) + 1e-6).all(), f"loss err {err_l}"
    assert np.allclose(tg.sum(1), 1.0, atol=1e-4)

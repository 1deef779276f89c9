"""Parity gates shared by the GPU parity tests and their CPU self-test.

Indices must match bit-exactly.  Attention outputs must satisfy max|o - o_ref| <= 1e-2 and,
since the production distribution has |o| ~ 3e-3 (an all-zero output would pass the absolute
bar), also max|o - o_ref| / max|o_ref| <= 1e-2; lse must match to 1e-3 relative.
"""
import numpy as np
import torch

ABS_TOL = 1e-2
REL_TOL = 1e-2
LSE_REL = 1e-3


def check_idx(got, want, what=""):
    got = got.cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, what
    bad = np.flatnonzero((got != want).any(axis=1))
    assert bad.size == 0, f"{what}: {bad.size} index rows differ, first {bad[:5].tolist()}"


def check_attn(o, lse, o_ref, lse_ref, what=""):
    og = o.float().cpu().numpy()
    err = np.abs(og - o_ref).max() if og.size else 0.0
    ref_scale = np.abs(o_ref).max() if og.size else 0.0
    assert err <= ABS_TOL, f"{what}: max abs err {err}"
    if ref_scale > 0:
        assert err / ref_scale <= REL_TOL, f"{what}: normalised err {err / ref_scale}"
    if lse is not None:
        lg = lse.cpu().numpy().astype(np.float64)
        inf_ref = np.isneginf(lse_ref)
        assert (np.isneginf(lg) == inf_ref).all(), f"{what}: -inf lse mismatch"
        fin = ~inf_ref
        if fin.any():
            rel = np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
            assert rel.max() <= LSE_REL, f"{what}: lse rel err {rel.max()}"
    return err

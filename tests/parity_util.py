"""Helpers shared by the GPU parity tests (inputs in, numpy results out)."""

from __future__ import annotations

import numpy as np

# Tolerances: |O_gpu - O_ref| <= 1e-2 everywhere, mean |O_gpu - O_ref| <= 1e-3,
# |LSE_gpu - LSE_ref| <= 1e-3 (absolute), no NaN or Inf.
MAX_ABS_O = 1e-2
MEAN_ABS_O = 1e-3
MAX_ABS_LSE = 1e-3


def to_dev(*arrays, device="cuda:0"):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).to(device) for a in arrays]


def gpu_attention(q, k, v, scale, causal, device="cuda:0", **kw):
    """Run the HIP path on numpy fp16 inputs; returns (O fp16 ndarray, LSE fp32 ndarray)."""
    import torch

    import exact_attention_121_amd as ea
    tq, tk, tv = to_dev(q, k, v, device=device)
    o, lse = ea.attn_fwd(tq, tk, tv, scale=scale, causal=causal, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


def assert_parity(o_gpu, lse_gpu, O_ref, L_ref, what="", max_abs=MAX_ABS_O, mean_abs=MEAN_ABS_O,
                  lse_abs=MAX_ABS_LSE):
    o = np.asarray(o_gpu, dtype=np.float64)
    assert o.shape == O_ref.shape, f"{what}: O shape {o.shape} vs {O_ref.shape}"
    assert np.isfinite(o).all(), f"{what}: non-finite O"
    err = np.abs(o - O_ref)
    worst = np.unravel_index(int(err.argmax()), err.shape) if err.size else None
    assert err.max(initial=0.0) <= max_abs, f"{what}: max |dO| {err.max():.3e} at {worst}"
    assert (err.mean() if err.size else 0.0) <= mean_abs, f"{what}: mean |dO| {err.mean():.3e}"
    if lse_gpu is not None:
        lse = np.asarray(lse_gpu, dtype=np.float64)
        assert np.isfinite(lse).all(), f"{what}: non-finite LSE"
        lerr = np.abs(lse - L_ref)
        assert lerr.max(initial=0.0) <= lse_abs, f"{what}: max |dLSE| {lerr.max():.3e}"
    return float(err.max(initial=0.0)), float(err.mean() if err.size else 0.0)


def gather_rows(x, rows):
    """x [B, H, N, ...] and rows [B, H, R] -> x at those rows, [B, H, R, ...]."""
    B, H, R = rows.shape
    out = np.empty((B, H, R) + x.shape[3:], dtype=x.dtype)
    for b in range(B):
        for h in range(H):
            out[b, h] = x[b, h, rows[b, h]]
    return out


def convex_hull_ok(o, v, Hq, slack=2e-3):
    """Every output row is a convex combination of value rows, so each column
    of O lies within that column's range over the head's values (any size)."""
    B, Hkv = v.shape[:2]
    G = Hq // Hkv
    vf = v.astype(np.float32)
    lo = vf.min(axis=2)  # [B, Hkv, d]
    hi = vf.max(axis=2)
    of = o.astype(np.float32)
    for h in range(Hq):
        g = h // G
        tol = slack * np.maximum(1.0, np.abs(hi[:, g]))[:, None, :]
        if (of[:, h] < lo[:, g][:, None, :] - tol).any() or (of[:, h] > hi[:, g][:, None, :] + tol).any():
            return False
    return True

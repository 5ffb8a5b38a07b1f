"""Shared helpers of the GPU parity tests (test infrastructure only)."""
import numpy as np
import torch

import indexer_routed_block_amd as irb

DEV = "cuda"


def to_dev(x, dtype=None):
    """Upload a NumPy array, converting on the device (bf16 inputs are exactly representable)."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if dtype is not None:
        t = t.to(dtype)
    return t


def act_dtype(wl_dtype):
    return torch.bfloat16 if wl_dtype == "bf16" else torch.float32


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.detach().cpu().numpy()


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)


BF16_REL = 2.0 ** -7   # two bf16 half-ulps: result storage + bf16 P / dS operands


def attn_tol_check(got, want, dtype, what):
    """Attention outputs / gradients against the FP64 oracle.

    bf16: mean-abs <= 5e-3, and per element |err| <= 2e-2 + 2^-7 |ref|: the
    2e-2 max-abs bound (stated for unit-scale results) on top of two bf16
    half-ulps of the value itself -- one for storing the result in bf16 (a
    value in [8, 16) cannot be stored closer than 0.031) and one for the bf16
    rounding of the softmax probabilities / score gradients that feed the
    FP32-accumulated products.  The plain max-abs is printed as well.
    fp32 inputs: max-abs <= 1e-4.
    """
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    scale = float(np.abs(want).max(initial=0.0))
    if dtype == torch.bfloat16:
        excess = float((err - BF16_REL * np.abs(want)).max(initial=0.0))
        ok = excess <= 2e-2 and mean <= 5e-3
    else:
        excess = mx
        ok = mx <= 1e-4
    print(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} max|ref| {scale:.3f}")
    assert ok, f"{what}: max-abs {mx:.3e} (beyond 2^-7|ref| {excess:.3e}) mean-abs {mean:.3e} (max |ref| {scale:.3f})"
    return mx, mean


def score_bound(qI, w, kc, scale):
    """M[b, t, j] = scale * sum_h |w[t,h]| * sum_d |q[t,h,d] k[j,d]|.

    The "1e-3 relative" score tolerance is taken against this magnitude: it
    bounds the cancellation inside each dot product as well as across the
    signed head weights, so it is the scale FP32-class rounding error lives
    on.  (relu(q.k) alone is not: a dot product that cancels to ~0 still
    carries rounding error of order sum_d |q_d k_d| * 2^-17.)
    """
    dots = np.abs(qI.astype(np.float64)) @ np.abs(np.asarray(kc, dtype=np.float64)).swapaxes(-1, -2)[:, None]
    return scale * (np.abs(w.astype(np.float64))[..., None, :] @ dots)[..., 0, :]

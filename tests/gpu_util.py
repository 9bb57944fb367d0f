"""Helpers for the GPU parity tests: device copies, runs through the C ABI,
comparison against the oracle with the stated tolerances."""

from __future__ import annotations

import math
import sys

import numpy as np

# Tolerances against the fp64 oracle.
#   bf16 storage, fp32 accumulation: max |dO| <= 2e-2, mean |dO| <= 2e-3
#   float32 throughout:              max |dO| <= 1e-4
#   log-sum-exp (both):              max |d lse| <= 1e-3
TOL_BF16 = {"max_abs": 2e-2, "mean_abs": 2e-3, "lse": 1e-3}
TOL_F32 = {"max_abs": 1e-4, "mean_abs": 1e-4, "lse": 1e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_f32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def dev_i32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


def prefill_device(inp):
    if inp["dtype"] == "bf16":
        return tuple(dev_bf16(inp[n + "_bits"]) for n in ("q", "k", "v"))
    return tuple(dev_f32(inp[n]) for n in ("q", "k", "v"))


def run_prefill(inp, causal, window, scale=None, dev=None):
    import torch
    import io_aware_exact_fa_amd as fa
    q, k, v = dev if dev is not None else prefill_device(inp)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def compare(o, lse, o_ref, lse_ref, tol, label):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    assert np.isfinite(lse).all(), f"{label}: non-finite lse"
    d = np.abs(o - o_ref)
    dl = np.abs(lse - lse_ref)
    rel = np.linalg.norm(o - o_ref, axis=-1) / np.maximum(np.linalg.norm(o_ref, axis=-1), 1e-30)
    say(f"  {label}: max|dO|={d.max():.3e} mean|dO|={d.mean():.3e} "
        f"max|dlse|={dl.max():.3e} max row rel={rel.max():.3e}")
    assert d.max() <= tol["max_abs"], f"{label}: max |dO| {d.max()}"
    assert d.mean() <= tol["mean_abs"], f"{label}: mean |dO| {d.mean()}"
    assert dl.max() <= tol["lse"], f"{label}: max |dlse| {dl.max()}"

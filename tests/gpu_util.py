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
# Backward, per gradient tensor against the fp64 oracle: elementwise
# |d| <= 2^-7 M + 1e-6 with M the rounding bound of tests/bwd_bounds.py, and
# ||d||_F / ||ref||_F <= 8e-3 (about 2u, u = 2^-8 the bf16 unit roundoff) on
# whole gradients;
# a gradient that is zero by the mathematics: max |d| <= 1e-4.
TOL_BWD = {"rel_fro": 8e-3, "zero_abs": 1e-4, "abs_floor": 1e-6}


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


def rows_seeing(keys, n, causal, window):
    """A contiguous range of query rows containing every row that sees one of
    ``keys`` (causal: rows at or after the key, at most ``window`` later;
    band: rows within ``window`` on either side; full: all rows)."""
    keys = np.asarray(keys)
    lo = keys.min() if causal else (keys.min() - window if window >= 0 else 0)
    hi = keys.max() + window if window >= 0 else n - 1
    return np.arange(max(int(lo), 0), min(int(hi), n - 1) + 1)


def compare_grad(got, ref, bound, label, tol=TOL_BWD, fro=True):
    """Check one gradient tensor against the oracle's, with its bound M.
    ``fro=False`` skips the relative Frobenius criterion (for values that are
    small differences of large terms, where it measures the cancellation)."""
    from tests.bwd_bounds import BOUND_FACTOR
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape == bound.shape, f"{label}: shapes {got.shape} {ref.shape}"
    assert np.isfinite(got).all(), f"{label}: non-finite gradient"
    diff = np.abs(got - ref)
    ratio = diff / (BOUND_FACTOR * bound + tol["abs_floor"])
    rel_fro = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape)
    say(f"  {label}: relF={rel_fro:.3e} max|d|={diff.max():.3e} "
        f"max |d|/(2^-7 M)={ratio.max():.3f} at {tuple(int(x) for x in worst)} "
        f"(max|ref|={np.abs(ref).max():.3e})")
    if np.abs(ref).max() < 1e-9:
        # Analytically zero gradient (every row sees only itself): what is left
        # is fp32 summation-order noise in dP - D, far below any bf16 rounding.
        assert diff.max() <= tol["zero_abs"], f"{label}: expected zeros, max |d| {diff.max()}"
        return
    assert ratio.max() <= 1.0, f"{label}: error above the rounding bound at {worst}"
    # The Frobenius criterion is statistical (random rounding signs): it is
    # applied to whole gradients, not to a handful of sampled rows, where one
    # row with cancellation dominates it.
    if fro and got.size // got.shape[-1] >= 256:
        assert rel_fro <= tol["rel_fro"], f"{label}: relative Frobenius error {rel_fro}"



def decode_oracle_all(meta, scale, fp8: bool = False, batches=None):
    """The decode oracle over every sequence (or ``batches``), one sequence at
    a time: each call gets that sequence's own pages (converted from the
    stored bf16 bits or E4M3 bytes) and an identity table over them, so the
    whole cache is never widened to float at once."""
    from oracle import decode_fwd
    from oracle.fp8 import decode_fwd_fp8
    from io_aware_exact_fa_amd.inputs import bf16_bits_to_f32
    sl = np.asarray(meta["seqlens"])
    B, H, d = meta["q"].shape
    o = np.zeros((B, H, d))
    lse = np.zeros((B, H))
    ps = meta["page_size"]
    for b in (range(B) if batches is None else batches):
        L = int(sl[b])
        pb = (L + ps - 1) // ps
        phys = meta["page_table"][b, :pb]
        table = np.arange(pb, dtype=np.int32)[None, :]
        if fp8:
            ob, lb = decode_fwd_fp8(meta["q"][b:b + 1], meta["kcache8"][phys],
                                    meta["vcache8"][phys], meta["k_scale"], meta["v_scale"],
                                    table, sl[b:b + 1], scale)
        else:
            ob, lb = decode_fwd(meta["q"][b:b + 1], bf16_bits_to_f32(meta["kcache_bits"][phys]),
                                bf16_bits_to_f32(meta["vcache_bits"][phys]), table,
                                sl[b:b + 1], scale)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def oracle_workers() -> int:
    """Host processes for the oracle in the GPU tests: the cores this process
    may use, at most 16."""
    from oracle.attention import default_workers
    return max(1, min(16, default_workers()))


_ROWS_FN = None


def _rows_task(chunk):
    return _ROWS_FN(chunk)


def oracle_rows_parallel(fn, rows, chunk: int = 256):
    """fn(rows_subset) -> (o [..., R, d], lse [..., R]) evaluated over ``rows``
    in chunks on forked worker processes (the oracle's own arithmetic, only
    spread over cores); results concatenated along the row axis."""
    import multiprocessing as mp
    global _ROWS_FN
    rows = np.asarray(rows)
    chunks = [rows[i:i + chunk] for i in range(0, rows.size, chunk)]
    _ROWS_FN = fn
    try:
        from oracle.attention import _worker_init  # one BLAS thread per worker process
        pool = mp.get_context("fork").Pool(min(oracle_workers(), len(chunks)),
                                           initializer=_worker_init)
        try:
            res = pool.map(_rows_task, chunks, chunksize=1)
        finally:
            pool.close()
            pool.join()
    finally:
        _ROWS_FN = None
    return (np.concatenate([r[0] for r in res], axis=-2),
            np.concatenate([r[1] for r in res], axis=-1))


def stratified_rows(n: int, block: int, seed: int, extra=()):
    """One seeded row from every ``block``-row block of [0, n), plus ``extra``."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, n, block)
    picks = starts + rng.integers(0, block, size=starts.size)
    rows = set(int(r) for r in picks if r < n)
    rows.update(int(r) for r in extra if 0 <= r < n)
    return np.array(sorted(rows))

"""GPU parity of the prefill kernels (fa_fwd through the C ABI) against the oracle.

Small shapes are compared element by element over every output.  At full
size the causal B4 H16 n4096 workload is compared over every output; the
band and long causal workloads over two whole heads and, in every head, one
row of every 256-row query block plus the band and tile edges.
"""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import prefill_inputs
from oracle import attention_fwd
from tests.gpu_util import (TOL_BF16, TOL_F32, compare, oracle_workers, prefill_device,
                             run_prefill, say, stratified_rows)

pytestmark = pytest.mark.gpu

# (B, H, Hkv, n, d, causal, window, dtype)
SMALL = [
    (1, 1, 1, 256, 64, 0, -1, "f32"),      # the single-head fp32 workload, exactly
    (2, 4, 2, 100, 128, 1, -1, "f32"),
    (1, 2, 1, 77, 64, 0, 10, "f32"),
    (1, 2, 2, 300, 128, 1, 50, "f32"),
    # The fp32 kernel splits a block's key tiles over its waves: more tiles
    # than waves, fewer (idle waves), band edges inside a wave's tiles.
    (1, 1, 1, 1, 64, 0, -1, "f32"),
    (2, 4, 1, 1000, 64, 1, -1, "f32"),
    (1, 2, 1, 700, 128, 0, 0, "f32"),
    (1, 2, 2, 513, 64, 1, 37, "f32"),
    (1, 2, 1, 1500, 128, 0, 200, "f32"),
    (1, 1, 1, 1, 128, 0, -1, "bf16"),
    (1, 2, 2, 7, 128, 1, -1, "bf16"),
    (1, 2, 1, 256, 128, 0, -1, "bf16"),
    (2, 4, 2, 129, 64, 0, -1, "bf16"),
    (2, 4, 1, 1000, 128, 1, -1, "bf16"),
    (1, 2, 2, 300, 64, 1, -1, "bf16"),
    (1, 3, 3, 513, 128, 1, -1, "bf16"),
    (1, 2, 1, 700, 128, 0, 0, "bf16"),
    (1, 2, 1, 700, 128, 0, 1, "bf16"),
    (1, 2, 1, 700, 128, 0, 37, "bf16"),
    (1, 2, 1, 700, 128, 0, 64, "bf16"),
    (1, 2, 1, 700, 128, 0, 100, "bf16"),
    (1, 2, 1, 700, 128, 0, 128, "bf16"),
    (1, 2, 1, 700, 128, 0, 255, "bf16"),
    (1, 2, 1, 700, 128, 0, 4096, "bf16"),
    (1, 2, 1, 600, 128, 1, 0, "bf16"),
    (1, 2, 1, 600, 128, 1, 37, "bf16"),
    (1, 2, 1, 600, 128, 1, 128, "bf16"),
    (1, 2, 1, 600, 128, 1, 300, "bf16"),
    (1, 2, 2, 333, 64, 0, 50, "bf16"),
    (1, 4, 4, 2049, 128, 0, 200, "bf16"),
]


def _id(c):
    B, H, Hkv, n, d, causal, w, dt = c
    return f"B{B}H{H}kv{Hkv}n{n}d{d}{'c' if causal else 'b'}w{w}{dt}"


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_prefill_small(case):
    B, H, Hkv, n, d, causal, window, dt = case
    say(f"case {_id(case)}")
    inp = prefill_inputs(B, H, Hkv, n, d, seed=1000 + n + d + window, dtype=dt)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_prefill(inp, causal, window, scale)
    o_ref, lse_ref = attention_fwd(inp["q"], inp["k"], inp["v"], causal, window, scale)
    compare(o, lse, o_ref, lse_ref, TOL_F32 if dt == "f32" else TOL_BF16, _id(case))


def test_prefill_deterministic():
    inp = prefill_inputs(2, 4, 2, 777, 128, seed=9)
    dev = prefill_device(inp)
    a = run_prefill(inp, 1, -1, dev=dev)
    b = run_prefill(inp, 1, -1, dev=dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [0, 1], ids=["full", "causal"])
def test_eight_and_four_wave_workgroups_agree_bitwise(causal):
    """Without a window the dense forward runs 8-wave workgroups (256 query
    rows), with a window 4-wave ones (128 rows).  A window of n - 1 leaves the
    visible set unchanged and each wave visits the same key tiles in the same
    order either way, so the two launches must agree bit for bit."""
    n = 1111
    inp = prefill_inputs(2, 4, 2, n, 128, seed=77 + causal)
    dev = prefill_device(inp)
    a = run_prefill(inp, causal, -1, dev=dev)
    b = run_prefill(inp, causal, n - 1, dev=dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# Windows wide enough for the 8-wave (256-row) workgroups: a band of 8192
# (16385 keys per row) and a causal window of 16383, with masked band edges
# inside those workgroups; sampled rows around the edges and the ends.
WIDE_WINDOWS = [(0, 8192), (1, 16383)]


@pytest.mark.parametrize("causal,window", WIDE_WINDOWS,
                         ids=[f"{'c' if c else 'b'}w{w}" for c, w in WIDE_WINDOWS])
def test_wide_window_sampled(causal, window):
    n, H, Hkv, d = 20000, 4, 2, 128
    say(f"wide window causal={causal} w={window} n={n}")
    inp = prefill_inputs(1, H, Hkv, n, d, seed=90 + causal)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_prefill(inp, causal, window, scale)
    edges = [0, 1, 255, 256, window - 1, window, window + 1, n - window - 1, n - window,
             n // 2, n - 257, n - 256, n - 1]
    rows = _sample_rows(n, edges, seed=window, count=16)
    o_ref, lse_ref = attention_fwd(inp["q"], inp["k"], inp["v"], causal, window, scale, rows=rows)
    compare(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, TOL_BF16, f"wide c{causal} w{window}")


def _sample_rows(n, extra, seed, count=24):
    rng = np.random.default_rng(seed)
    rows = set(r for r in extra if 0 <= r < n)
    rows.update(rng.integers(0, n, size=count).tolist())
    return np.array(sorted(rows))


# The workloads at full size, in the launch configuration the benchmark times.
# causal B4 H16 n4096: every output.  band n32768 and causal GQA n65536: two
# whole heads (from different key/value heads), plus, in every head, one row
# of every 256-row query block and the rows at the band and tile edges.  Each
# set is held to the max, mean and lse tolerances on its own.
FULL = {
    "causal_B4_H16_n4096": dict(B=4, H=16, Hkv=16, n=4096, d=128, causal=1, window=-1,
                                seed=2, scale_draws=1.0, whole="all", edges=[]),
    "band_w2048_H32_n32768": dict(B=1, H=32, Hkv=32, n=32768, d=128, causal=0, window=2048,
                                  seed=3, scale_draws=1.0, whole=(0, 31),
                                  edges=[0, 1, 2047, 2048, 2049, 4095, 4096, 16383, 16384,
                                         30719, 30720, 32766, 32767]),
    "causal_gqa_H32_kv8_n65536": dict(B=1, H=32, Hkv=8, n=65536, d=128, causal=1, window=-1,
                                      seed=4, scale_draws=0.5, whole=(0, 31),
                                      edges=[0, 1, 127, 128, 255, 256, 32767, 32768, 65534,
                                             65535]),
}


@pytest.mark.parametrize("name", list(FULL))
def test_prefill_full_size(name):
    c = FULL[name]
    say(f"case {name}")
    inp = prefill_inputs(c["B"], c["H"], c["Hkv"], c["n"], c["d"], seed=c["seed"],
                         draw_scale=c["scale_draws"])
    scale = 1.0 / math.sqrt(c["d"])
    o, lse = run_prefill(inp, c["causal"], c["window"], scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    W = oracle_workers()
    if c["whole"] == "all":
        o_ref, lse_ref = attention_fwd(inp["q"], inp["k"], inp["v"], c["causal"], c["window"],
                                       scale, workers=W)
        compare(o, lse, o_ref, lse_ref, TOL_BF16, f"{name} (every output)")
        return
    G = c["H"] // c["Hkv"]
    for h in c["whole"]:
        g = h // G
        o_ref, lse_ref = attention_fwd(inp["q"][:, h:h + 1], inp["k"][:, g:g + 1],
                                       inp["v"][:, g:g + 1], c["causal"], c["window"], scale,
                                       workers=W)
        compare(o[:, h:h + 1], lse[:, h:h + 1], o_ref, lse_ref, TOL_BF16,
                f"{name} head {h} (every row)")
    rows = stratified_rows(c["n"], 256, seed=c["seed"], extra=c["edges"])
    o_ref, lse_ref = attention_fwd(inp["q"], inp["k"], inp["v"], c["causal"], c["window"],
                                   scale, rows=rows, workers=W)
    compare(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, TOL_BF16,
            f"{name} all heads, {rows.size} rows (one per 256-row block + edges)")


# Points of the length x window x batch matrix (bidirectional band) the bench
# sweeps: one whole head, and in every (batch, head) one row per 256-row block
# plus the band edges.
SWEEP_POINTS = [(4096, 512, 2), (4096, -1, 2), (8192, 1024, 1), (16384, 2048, 1),
                (32768, 512, 1), (32768, -1, 1)]


@pytest.mark.parametrize("n,window,B", SWEEP_POINTS,
                         ids=[f"n{n}w{w}b{b}" for n, w, b in SWEEP_POINTS])
def test_sweep_points(n, window, B):
    say(f"sweep point n={n} w={window} B={B}")
    H, d = 32, 128
    inp = prefill_inputs(B, H, H, n, d, seed=14 + n + B)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_prefill(inp, 0, window, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    W = oracle_workers()
    h = H - 1
    o_ref, lse_ref = attention_fwd(inp["q"][B - 1:B, h:h + 1], inp["k"][B - 1:B, h:h + 1],
                                   inp["v"][B - 1:B, h:h + 1], False, window, scale, workers=W)
    compare(o[B - 1:B, h:h + 1], lse[B - 1:B, h:h + 1], o_ref, lse_ref, TOL_BF16,
            f"sweep n{n} w{window} b{B - 1} h{h} (every row)")
    rows = stratified_rows(n, 256, seed=n + B,
                           extra=[0, 1, window - 1, window, window + 1, n // 2, n - 1])
    o_ref, lse_ref = attention_fwd(inp["q"], inp["k"], inp["v"], False, window, scale, rows=rows,
                                   workers=W)
    compare(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, TOL_BF16,
            f"sweep n{n} w{window} all heads, {rows.size} rows")

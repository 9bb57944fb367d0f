"""Host logic of the benchmark (CPU only): the visible-pair counts that set the
in-band FLOP numerators, and the clock sampler's filtering of GPU metrics."""

import sys
import types

import numpy as np
import pytest

import bench


def brute_pairs(n, causal, window):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = np.ones((n, n), dtype=bool)
    if causal:
        vis &= j <= i
    if window >= 0:
        vis &= np.abs(i - j) <= window
    return int(vis.sum())


@pytest.mark.parametrize("n", [1, 2, 7, 64, 131])
@pytest.mark.parametrize("causal", [False, True])
def test_inband_pairs_matches_explicit_mask(n, causal):
    for w in sorted({-1, 0, 1, 3, n // 2, n - 2, n - 1, n, n + 5}):
        if w < -1:
            continue
        assert bench.inband_pairs(n, causal, w) == brute_pairs(n, causal, w), (n, causal, w)


def test_inband_pairs_workload_sizes():
    # Causal n = 65536: n(n+1)/2 pairs per head.
    assert bench.inband_pairs(65536, True, -1) == 65536 * 65537 // 2
    # Band |i - j| <= 2048 over n = 32768: about 1/8 of n^2 (2w+1 of n per row).
    p = bench.inband_pairs(32768, False, 2048)
    assert p == 32768 * 4097 - 2048 * 2049
    assert 0.12 < p / 32768 ** 2 < 0.126


def brute_blocksparse(layout, n, bq, bk):
    total = 0
    for lay in layout:
        vis = np.zeros((n, n), dtype=bool)
        for a, c in zip(*np.nonzero(lay)):
            vis[a * bq:(a + 1) * bq, c * bk:(c + 1) * bk] = True
        vis &= np.tril(np.ones((n, n), dtype=bool))
        total += int(vis.sum())
    return total


@pytest.mark.parametrize("n", [128, 300, 511])
def test_blocksparse_pairs_matches_explicit_mask(n):
    rng = np.random.default_rng(n)
    bq, bk = 128, 64
    layout = rng.random((3, -(-n // bq), -(-n // bk))) < 0.4
    layout[0, :, 0] = True
    assert bench.blocksparse_causal_pairs(layout, n, bq, bk) == brute_blocksparse(layout, n, bq, bk)


class _FakeTorch:
    class cuda:
        @staticmethod
        def synchronize():
            pass

        @staticmethod
        def get_device_properties(_):
            return types.SimpleNamespace(pci_bus_id=3)


def _fake_smi(metrics):
    """An amdsmi stand-in whose metrics table returns successive entries."""
    it = iter(metrics)
    last = {}

    def get_metrics(_h):
        nonlocal last
        last = next(it, last)
        return last

    return types.SimpleNamespace(
        amdsmi_init=lambda: None,
        amdsmi_get_processor_handles=lambda: ["gpu0"],
        amdsmi_get_gpu_metrics_info=get_metrics,
        amdsmi_get_gpu_device_bdf=lambda h: "0000:03:00.0")


def test_sustained_clock_averages_settled_samples(monkeypatch):
    m = {"current_gfxclk": 1800, "current_gfxclks": [1750, 1850], "current_socket_power": 1300}
    monkeypatch.setitem(sys.modules, "amdsmi", _fake_smi([m] * 10000))
    r = bench.sustained_clock(_FakeTorch, lambda: None, seconds=0.15, settle=0.05)
    assert r["mhz"] == 1800 and r["xcd0_mhz"] == 1800
    assert r["xcd_mhz_range"] == [1750, 1850]
    assert r["xcd_mhz_mean"] == [1750, 1850]
    assert r["socket_power_w"] == 1300
    assert r["samples"] >= 1 and r["launches"] >= 1


def test_sustained_clock_reports_missing_metrics(monkeypatch):
    m = {"current_gfxclk": "N/A", "current_gfxclks": "N/A", "current_socket_power": "N/A"}
    monkeypatch.setitem(sys.modules, "amdsmi", _fake_smi([m] * 10000))
    r = bench.sustained_clock(_FakeTorch, lambda: None, seconds=0.1, settle=0.0)
    assert r["mhz"] is None and "N/A" in r["why"]


def test_sustained_clock_without_amdsmi(monkeypatch):
    def boom():
        raise RuntimeError("no driver")
    monkeypatch.setitem(sys.modules, "amdsmi", types.SimpleNamespace(amdsmi_init=boom))
    r = bench.sustained_clock(_FakeTorch, lambda: None, seconds=0.1)
    assert r["mhz"] is None and "no driver" in r["why"]


def test_source_hash_ignores_comments_only():
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n"
    same = "/* header\n   text */\nint f(int a)   {\n  return a + 1;\n}  // done\n"
    other = "int f(int a) {\n  return a + 2;  // one more\n}\n"
    assert bench.canonical_source(code) == bench.canonical_source(same)
    assert bench.canonical_source(code) != bench.canonical_source(other)


def test_step_record_schema_and_arithmetic():
    pre = [30.0, 31.0, 29.0, 30.0]
    dec = [0.74, 0.73, 0.75, 0.74]
    rec = bench.step_record(4, 3, pre, dec, wall_s=0.124, kv_bytes=4_302_426_112,
                            pre_traffic=5_500_000_000, dec_traffic=None)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 4 and rec["warmup"] == 3
    assert rec["higher_is_better"] is True and rec["vs_baseline"] is None
    assert "workload" in rec["config"] and "model" not in rec["config"]
    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    # value: in-band FLOPs of the causal n = 65536, H = 32, d = 128 workload
    # over the average prefill duration (30 ms)
    flops = 4 * 128 * 32 * 65536 * 65537 // 2
    assert roof["algorithmic_flops_per_launch"] == flops
    assert abs(rec["value"] - flops / 30e-3 / 1e12) < 0.01
    assert roof["achieved"] == rec["value"] and roof["peak"] == 2500.0
    assert abs(roof["frac"] - rec["value"] / 2500.0) < 1e-4
    assert roof["traffic"] == 5_500_000_000
    assert rec["prefill_ms_median"] == 30.0 and rec["prefill_ms_range"] == [29.0, 31.0]
    assert rec["ms_per_step"] == 31.0
    dr = rec["decode"]["roofline"]
    assert dr["bound"] == "hbm" and dr["traffic"] is None
    assert abs(rec["decode"]["value"] - 4_302_426_112 / 0.74e-3 / 1e9) < 0.1
    assert abs(dr["frac"] - rec["decode"]["value"] / 8000.0) < 1e-4


def test_sustained_clock_uses_the_mean_over_xcds(monkeypatch):
    m = {"current_gfxclk": 1900, "current_gfxclks": [1900, 1700, 2000, 1800],
         "current_socket_power": 1300}
    monkeypatch.setitem(sys.modules, "amdsmi", _fake_smi([m] * 10000))
    r = bench.sustained_clock(_FakeTorch, lambda: None, seconds=0.1, settle=0.0)
    assert r["mhz"] == 1850 and r["xcd0_mhz"] == 1900
    assert r["xcd_mhz_mean"] == [1900, 1700, 2000, 1800]


def test_host_cpu_model_is_a_string():
    m = bench.host_cpu_model()
    assert isinstance(m, str) and m


def brute_tiles(n, causal, window, nw):
    """(visited (wave, tile) pairs, staged (workgroup, tile) pairs) by explicit
    enumeration: a wave visits a 64-key tile when one of its 32 rows sees a
    key in it; a workgroup of nw waves stages the tiles any of its rows sees."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = np.ones((n, n), dtype=bool)
    if causal:
        vis &= j <= i
    if window >= 0:
        vis &= (j >= i - window) if causal else (np.abs(i - j) <= window)
    nt = -(-n // 64)
    tile_hit = np.zeros((n, nt), dtype=bool)
    for t in range(nt):
        tile_hit[:, t] = vis[:, t * 64:(t + 1) * 64].any(axis=1)
    visited = sum(int(tile_hit[r:r + 32].any(axis=0).sum()) for r in range(0, n, 32))
    staged = sum(int(tile_hit[r:r + 32 * nw].any(axis=0).sum()) for r in range(0, n, 32 * nw))
    return visited, staged


@pytest.mark.parametrize("n", [1, 63, 64, 65, 300, 700])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_schedule_matches_enumeration(n, causal):
    for w in sorted({-1, 0, 1, 37, 64, 100, n - 1, n}):
        if w < -1:
            continue
        s = bench.tile_schedule(n, causal, w, B=2, H=3)
        v, st = brute_tiles(n, causal, w, s["waves_per_workgroup"])
        assert s["visited_wave_tiles"] == 6 * v, (n, causal, w)
        assert s["staged_tiles"] == 6 * st, (n, causal, w)
        assert s["inband_pairs"] == 6 * brute_pairs(n, causal, w)
        assert s["visited_pairs"] >= s["inband_pairs"]


def test_tile_schedule_workloads():
    # Long causal: 8-wave workgroups; each wave's last tile straddles the
    # diagonal, so the matrix cores evaluate a little more than n(n+1)/2.
    s = bench.tile_schedule(65536, True, -1, H=32)
    assert s["waves_per_workgroup"] == 8
    assert s["inband_pairs"] == 32 * 65536 * 65537 // 2
    assert 0.998 < s["inband_over_visited"] < 1.0
    # Band w = 2048: 4-wave workgroups; an interior wave's 32 rows see a
    # 4128-key union, 65 tiles of 64 keys, for 4097 visible keys per row.
    s = bench.tile_schedule(32768, False, 2048, H=32)
    assert s["waves_per_workgroup"] == 4
    assert 0.98 < s["inband_over_visited"] < 0.99
    # A large window on the 8-wave rule's edge.
    assert bench.tile_schedule(40000, True, 16383)["waves_per_workgroup"] == 8
    assert bench.tile_schedule(40000, True, 16382)["waves_per_workgroup"] == 4


def _counter_csv(path, counter, rows):
    import csv
    cols = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
            "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for i, (grid, name, value) in enumerate(rows):
            w.writerow([i, i, grid, name, counter, value])


def test_traffic_from_counters_calibrates_on_the_largest_copy(tmp_path):
    """The counters are scaled by the bench's 256 MiB copy (the largest copy
    of the run), whatever other small copies the run made."""
    pre = "void fa::prefill_bf16_kernel<128, 8, 64, 0, false>(fa::PrefillArgs)"
    cnt = "void fa::prefill_bf16_kernel<128, 8, 64, 0, true>(fa::PrefillArgs)"
    dec = ["void fa::decode_split_kernel<128, 4, false>(fa::DecodeArgs)",
           "void fa::decode_combine_kernel<128>(fa::DecodeArgs)"]
    bwd = ["void fa::bwd_delta_kernel<128>(fa::BwdArgs)", "void fa::bwd_dkdv_kernel<128>(fa::BwdArgs)",
           "void fa::bwd_dq_kernel<128, 8>(fa::BwdArgs)"]
    copy = "__amd_rocclr_copyBuffer"
    fetch = [(512, copy, 2.6), (131072, copy, 131072.0), (65536, copy, 523.5), (4096, copy, 44.5),
             (8192, pre, 1000.0), (8192, pre, 1002.0), (8192, cnt, 5000.0),
             (512, dec[0], 10.0), (64, dec[1], 1.0)] + [(8, b, 7.0) for b in bwd]
    write = [(131072, copy, 262144.0), (65536, copy, 1000.0), (8192, pre, 100.0), (8192, cnt, 900.0),
             (512, dec[0], 2.0), (64, dec[1], 3.0)] + [(8, b, 5.0) for b in bwd]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fp, "FETCH_SIZE", fetch)
    _counter_csv(wp, "WRITE_SIZE", write)
    rec = bench.traffic_from_counters(str(fp), str(wp))
    assert rec["scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    # prefill: mean of its two (uncounted) dispatches, scaled
    assert rec["prefill_bf16"]["fetch_size_bytes"] == int(1001.0 * 1024 * 2.0)
    assert rec["prefill_bf16"]["write_size_bytes"] == int(100.0 * 1024)
    # decode: split + merge per launch
    assert rec["decode"]["bytes_per_launch"] == int(11.0 * 1024 * 2.0 + 5.0 * 1024)
    assert rec["backward"]["bytes_per_launch"] == int(21.0 * 1024 * 2.0 + 15.0 * 1024)

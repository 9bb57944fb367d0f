"""Benchmark of the attention forward hot path on one MI355X.

One step = one pass over both halves of the forward path on one batch of
synthetic input already resident in HBM:
  * prefill: causal self-attention with grouped-query heads, B=1, H=32,
    Hkv=8, n=65536, d=128, bf16 (draws x0.5), fp32 lse;
  * decode: paged flash-decoding, 64 sequences, 32 query / 8 KV heads, d=128,
    bf16, lengths uniform in [1024, 32768], 16-token pages behind a permuted
    page table (split kernel + log-sum-exp merge kernel).

Printed: ONE JSON line.  ``value`` is the prefill's useful (in-band) TFLOP/s:
4*d FLOPs per visible (query, key) pair, divided by the prefill kernel's
average duration from HIP events on the stream it runs on (the median and the
range of the per-step durations are printed beside the averages).  The decode's KV
GB/s (bytes of K and V that the sequences' lengths make visible, divided by
split+merge duration) is reported beside it.  ``cpu_baseline`` times the fp64
oracle on a bounded sample of the same prefill workload on the host cores.
``backward`` times fa_bwd (the gradients) on the same prefill workload after
the timed steps, outside the step.  ``roofline.clock`` is the GFX clock the
part sustains under back-to-back prefill launches (the part is power limited
there), with the bf16 peak scaled to that clock and the fraction of it.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--bwd-steps N]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published

PREFILL = dict(B=1, H=32, Hkv=8, n=65536, d=128, causal=1, window=-1, seed=4, draw_scale=0.5)
DECODE = dict(B=64, H=32, Hkv=8, d=128, page_size=16, min_len=1024, max_len=32768, seed=5)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def inband_pairs(n: int, causal: bool, window: int) -> int:
    """Number of visible (query, key) pairs of one head (closed forms)."""
    if window >= n - 1 or window < 0:
        return n * (n + 1) // 2 if causal else n * n
    w = window
    if causal:
        return (w + 1) * n - w * (w + 1) // 2
    return n * (2 * w + 1) - w * (w + 1)


def tile_schedule(n: int, causal: bool, window: int, B: int = 1, H: int = 1) -> dict:
    """Host replica of the dense forward's key-tile schedule (fa_fwd, bf16).

    The launch uses workgroups of NW waves (8 when every row sees 16384 keys
    or more, else 4), each wave owning 32 query rows; key tiles are 64 keys.
    A workgroup stages the tiles [kt_lo, kt_hi] meeting its rows' band, and a
    wave computes a staged tile only when one of its rows sees a key in it.
    Returns, for B*H heads: ``visited_wave_tiles`` ((wave, tile) pairs whose
    products are computed), ``staged_tiles`` (tiles brought on chip),
    ``visited_pairs`` (visited_wave_tiles * 32 * 64: the (query, key) pairs
    the matrix cores evaluate, masked ones included), ``inband_pairs`` and
    their ratio.  The device counts the same quantities in fa_fwd_tile_count
    (xxqk.cn sliding-window prefill article §9.1: computed blocks and the
    KV blocks actually read)."""
    import numpy as np
    if window < 0:
        window = -1
    window = min(window, n)
    kpr = (1 << 62) if window < 0 else (window + 1 if causal else 2 * window + 1)
    nw = 8 if kpr >= 16384 else 4
    br, bc = 32 * nw, 64

    def lo(i):
        return i - window if window >= 0 else np.zeros_like(i)

    def hi(i):
        h = i if causal else (i + window if window >= 0 else np.full_like(i, n - 1))
        return np.minimum(h, n - 1)

    q0 = np.arange(0, n, br, dtype=np.int64)               # workgroup first rows
    qlast = np.minimum(q0 + br, n) - 1
    kt_lo = np.maximum(lo(q0), 0) // bc
    kt_hi = hi(qlast) // bc
    staged = int(np.maximum(kt_hi - kt_lo + 1, 0).sum())
    wq0 = (q0[:, None] + 32 * np.arange(nw)[None, :]).ravel()   # wave first rows
    tlo = np.repeat(kt_lo, nw)
    thi = np.repeat(kt_hi, nw)
    ok = wq0 < n
    wq0 = wq0[ok]
    wr1 = np.minimum(wq0 + 32, n) - 1
    # active tile kt: kt*64 + 63 >= lo(first row) and kt*64 <= hi(last row)
    a_lo = np.maximum(tlo[ok], -(-(lo(wq0) - (bc - 1)) // bc))
    a_hi = np.minimum(thi[ok], hi(wr1) // bc)
    visited = int(np.maximum(a_hi - a_lo + 1, 0).sum())
    inband = inband_pairs(n, causal, window)
    heads = B * H
    return {"waves_per_workgroup": nw, "visited_wave_tiles": visited * heads,
            "staged_tiles": staged * heads, "visited_pairs": visited * heads * 32 * bc,
            "inband_pairs": inband * heads,
            "inband_over_visited": round(inband / (visited * 32 * bc), 6)}


def canonical_source(text: str) -> str:
    """C++/HIP source with comments removed and whitespace collapsed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(*names) -> str:
    """Key of the recorded HBM counters: a hash of the kernel sources without
    their comments, so comment edits keep the record valid and code edits
    void it."""
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "io_aware_exact_fa_amd", "csrc", nm)) as f:
            h.update(canonical_source(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


KERNEL_KEYS = {  # traffic.json key -> (kernel-name patterns, sources)
    # The dense prefill and the dQ kernel are instantiated per wave count.
    # The dense prefill kernel without its counting variant (template flag false).
    "prefill_bf16": ((r"prefill_bf16_kernel<128, \d+, 64, 0, false>",),
                     ("prefill_bf16.hip", "common.hpp")),
    "decode": ((r"decode_split_kernel<128, 4, false>", r"decode_combine_kernel"),
               ("decode.hip", "common.hpp")),
    "backward": ((r"bwd_delta_kernel<128>", r"bwd_dkdv_kernel<128>", r"bwd_dq_kernel<128(, \d+)?>"),
                 ("backward.hip", "common.hpp")),
}
CALIBRATION_COPY_BYTES = 256 << 20


def traffic_from_counters(fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes per launch from two rocprofv3 --pmc CSVs (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch).  Each counter is scaled by the ratio of the
    known size of the 256 MiB calibration copy to what the counter read for
    that copy.  Multi-kernel entries (decode) sum their kernels per launch."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        copies = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name:
                copies.append((int(r["Grid_Size"]), v))
            vals[name].append(v)
        # The calibration copy is the largest device copy of the run (the other
        # copies move a few KiB to a few MiB of results and counters).
        top = max((g for g, _ in copies), default=None)
        calib = [v for g, v in copies if g == top]
        return vals, calib

    out = {"_about": "HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                     "(KiB per dispatch), each scaled by known/measured bytes of a 256 MiB "
                     "device copy in the same run; valid only for the recorded source hash."}
    scale = {}
    vals = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        v, calib = per_kernel(path, counter)
        if not calib:
            raise SystemExit(f"no calibration copy in {path}")
        scale[counter] = CALIBRATION_COPY_BYTES / (1024.0 * (sum(calib) / len(calib)))
        vals[counter] = v
    out["scale"] = {k: round(x, 5) for k, x in scale.items()}
    for key, (frags, srcs) in KERNEL_KEYS.items():
        rec = {"source_hash": source_hash(*srcs)}
        total = 0.0
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            kib = 0.0
            for frag in frags:
                hits = [x for name, xs in vals[counter].items() if re.search(frag, name)
                        for x in xs]
                if not hits:
                    raise SystemExit(f"{frag} not in the {counter} run")
                kib += sum(hits) / len(hits)
            rec[counter.lower() + "_kib_raw"] = round(kib, 1)
            rec[counter.lower() + "_bytes"] = int(kib * 1024 * scale[counter])
            total += kib * 1024 * scale[counter]
        rec["bytes_per_launch"] = int(total)
        out[key] = rec
    return out


def host_cpu_model() -> str:
    """The host processor's model name (from /proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, rows_per_head: int, heads: list[int]):
    """The oracle, as it is, on a bounded sample: `rows_per_head` evenly
    spread rows of the given heads of the prefill workload.  Returns the
    record and the oracle's outputs for those rows (o [1, heads, R, d], lse
    [1, heads, R]) with the row indices, for the consistency check.  Runs
    before the GPU is touched: its worker processes are forked from a process
    with no GPU state."""
    import numpy as np
    from oracle import attention_fwd
    from oracle.attention import default_workers

    n, d = PREFILL["n"], PREFILL["d"]
    workers = min(16, default_workers())
    rows = np.linspace(0, n - 1, rows_per_head).astype(np.int64)
    q = inp["q"][:, heads]
    group = PREFILL["H"] // PREFILL["Hkv"]
    kv_heads = sorted(set(h // group for h in heads))
    # query head h reads key/value head h // group: pass that head along with it
    k = inp["k"][:, [h // group for h in heads]]
    v = inp["v"][:, [h // group for h in heads]]
    t0 = time.perf_counter()
    o_ref, lse_ref = attention_fwd(q, k, v, True, -1, 1.0 / math.sqrt(d), rows=rows,
                                   workers=workers)
    dt = time.perf_counter() - t0
    inband = sum(int(r) + 1 for r in rows) * len(heads)
    flops = 4 * d * inband
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
           "cpu_model": host_cpu_model(), "cpus_available": len(os.sched_getaffinity(0)),
           "kind": "oracle",
           "sample": f"{rows_per_head} evenly spaced query rows x {len(heads)} heads "
                     f"(KV heads {kv_heads}) of the n=65536 causal prefill, fp64, "
                     f"{dt:.1f} s wall; in-band FLOPs of those rows only"}
    return rec, (rows, heads, o_ref, lse_ref)


# Tolerances of the parity gate against the fp64 oracle (bf16 I/O with fp32
# accumulation; float32 throughout), the same as the test suite's.
TOL = {"bf16": {"max_abs": 2e-2, "mean_abs": 2e-3, "lse": 1e-3},
       "f32": {"max_abs": 1e-4, "mean_abs": 1e-4, "lse": 1e-3}}


def consistency(o, lse, o_ref, lse_ref, dtype: str, what: str) -> dict:
    """max / mean |dO| and max |d lse| of a sample against the oracle, and
    whether they pass the parity tolerances (xxqk.cn sliding-window prefill
    article §8.3 compares the two outputs by their largest absolute error;
    §9.2 records whether the consistency check passed)."""
    import numpy as np
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    d = np.abs(o - o_ref)
    dl = np.abs(lse - lse_ref)
    tol = TOL[dtype]
    rec = {"sample": what, "max_abs": float(d.max()), "mean_abs": float(d.mean()),
           "lse_max_abs": float(dl.max()), "finite": bool(np.isfinite(o).all() and
                                                         np.isfinite(lse).all())}
    rec["pass"] = bool(rec["finite"] and rec["max_abs"] <= tol["max_abs"] and
                       rec["mean_abs"] <= tol["mean_abs"] and rec["lse_max_abs"] <= tol["lse"])
    return {k2: (float(f"{x:.4g}") if isinstance(x, float) else x) for k2, x in rec.items()}


def decode_oracle_sample(din, seqs, scale):
    """The decode oracle for the sequences ``seqs`` of a decode workload held
    as bf16 bits: each sequence's own pages are widened and passed with an
    identity table.  Returns (o [len(seqs), H, d], lse [len(seqs), H])."""
    import numpy as np
    from oracle import decode_fwd
    from io_aware_exact_fa_amd.inputs import bf16_bits_to_f32
    ps = din["page_size"]
    outs, lses = [], []
    for b in seqs:
        L = int(din["seqlens"][b])
        pb = (L + ps - 1) // ps
        phys = din["page_table"][b, :pb]
        ob, lb = decode_fwd(din["q"][b:b + 1], bf16_bits_to_f32(din["kcache_bits"][phys]),
                            bf16_bits_to_f32(din["vcache_bits"][phys]),
                            np.arange(pb, dtype=np.int32)[None, :], din["seqlens"][b:b + 1],
                            scale)
        outs.append(ob[0])
        lses.append(lb[0])
    return np.stack(outs), np.stack(lses)


def decode_sample_seqs(seqlens, count: int = 8):
    """Shortest, longest and evenly spread sequences of a decode batch."""
    import numpy as np
    B = len(seqlens)
    pick = {int(np.argmin(seqlens)), int(np.argmax(seqlens))}
    pick.update(int(x) for x in np.linspace(0, B - 1, count - 2).round())
    return sorted(pick)


def stratified_rows(n: int, block: int, seed: int):
    """One seeded row of every ``block``-row block of [0, n), plus the ends."""
    import numpy as np
    rng = np.random.default_rng(seed)
    starts = np.arange(0, n, block)
    rows = set((starts + rng.integers(0, block, size=starts.size)).tolist()) | {0, n - 1}
    return np.array(sorted(r for r in rows if r < n))


OTHER_WORKLOADS = [  # name, B, H, Hkv, n, d, causal, window, dtype, seed
    ("single-head fp32 full n256 d64", 1, 1, 1, 256, 64, 0, -1, "f32", 1),
    ("causal MHA B4 H16 n4096 d128 bf16", 4, 16, 16, 4096, 128, 1, -1, "bf16", 2),
    ("band |i-j|<=2048 B1 H32 n32768 d128 bf16", 1, 32, 32, 32768, 128, 0, 2048, "bf16", 3),
]


def dense_consistency(torch, inp_or_dev, o, lse, causal, window, scale, dtype, picks,
                      rows, rows_block: int = 256):
    """Consistency of a dense prefill output on the (batch, head) pairs
    ``picks`` and query ``rows``, against the oracle run serially on the
    host.  ``inp_or_dev`` holds q, k, v as numpy arrays ("q", "k", "v") or
    device tensors (copied back per head)."""
    import numpy as np
    from oracle import attention_fwd
    H, Hkv = o.shape[1], (inp_or_dev["k"].shape[1])
    G = H // Hkv
    rows_t = torch.from_numpy(rows).to(o.device)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, h in picks:
        g = h // G
        sel = [inp_or_dev[x][b:b + 1, hh:hh + 1] for x, hh in (("q", h), ("k", g), ("v", g))]
        if not isinstance(sel[0], np.ndarray):
            sel = [t.float().cpu().numpy() for t in sel]
        ro, rl = attention_fwd(*sel, causal, window, scale, rows=rows)
        ref_o.append(ro[0, 0])
        ref_l.append(rl[0, 0])
        got_o.append(o[b, h].index_select(0, rows_t).float().cpu().numpy())
        got_l.append(lse[b, h].index_select(0, rows_t).cpu().numpy())
    return consistency(np.stack(got_o), np.stack(got_l), np.stack(ref_o), np.stack(ref_l), dtype,
                       f"{len(rows)} rows (one per block of {rows_block} and the ends) of "
                       f"(batch, head) {list(picks)}")


def time_other_workloads(fa, torch, np, bf, stream, reps: int = 20):
    """Average kernel time (HIP events) of the other prefill workloads, with
    the consistency of a sample of each output against the oracle."""
    from io_aware_exact_fa_amd.inputs import prefill_inputs
    res = []
    for name, B, H, Hkv, n, d, causal, window, dt, seed in OTHER_WORKLOADS:
        inp = prefill_inputs(B, H, Hkv, n, d, seed=seed, dtype=dt)
        if dt == "bf16":
            q, k, v = bf(inp["q_bits"]), bf(inp["k_bits"]), bf(inp["v_bits"])
            dtype = fa.FA_BF16
        else:
            q, k, v = (torch.from_numpy(inp[x]).cuda() for x in ("q", "k", "v"))
            dtype = fa.FA_F32
        o = torch.empty_like(q)
        lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
        f = lambda: fa.fa_fwd(q, k, v, o, lse, B, H, Hkv, n, d, causal, window,
                              1.0 / math.sqrt(d), dtype, stream)
        ms = _time(torch, stream, f, reps)
        flops = 4 * d * inband_pairs(n, bool(causal), window) * B * H
        tf = flops / (ms * 1e-3) / 1e12
        rec = {"workload": name, "ms": round(ms, 4), "TFLOP/s": round(tf, 2)}
        if dt == "bf16":
            rec["frac_of_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
            rec["tiles"] = tile_schedule(n, bool(causal), window, B=B, H=H)
        rows = np.arange(n) if n <= 256 else stratified_rows(n, 256, seed=seed)
        rec["consistency"] = dense_consistency(
            torch, inp, o, lse, bool(causal), window, 1.0 / math.sqrt(d), dt,
            [(0, 0), (B - 1, H - 1)], rows, 1 if n <= 256 else 256)
        log(f"{name}: {ms:.4f} ms  {tf:.1f} TFLOP/s in-band  "
            f"max|dO| {rec['consistency']['max_abs']:.2e} pass={rec['consistency']['pass']}")
        res.append(rec)
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return res


VARLEN = dict(B=16, H=32, Hkv=8, d=128, min_len=1024, max_len=16384, seed=11)
PAGED = dict(B=16, H=32, Hkv=8, d=128, prefix=(1024, 32768), chunk=(2048, 2048), seed=12)
BLOCKSPARSE = {"H": 32, "Hkv": 8, "n": 32768, "d": 128, "density": 0.1, "local": 2,
               "global": 1, "seed": 13}


def _smi_handle(torch):
    """The amdsmi handle of cuda:0 (matched by PCI bus id when several GPUs
    are listed), or None with the reason."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        hs = amdsmi.amdsmi_get_processor_handles()
    except Exception as e:  # library or driver interface missing
        return None, f"amdsmi unavailable: {e}"
    if len(hs) == 1:
        return hs[0], None
    bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
    for h in hs:
        try:
            if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                return h, None
        except Exception:
            pass
    return None, f"{len(hs)} GPUs listed and none matched cuda:0"


def sustained_clock(torch, run, seconds: float, settle: float = 1.0):
    """Mean GFX clock and socket power while ``run`` is launched back to back.

    The GPU metrics table refreshes about once a second, so the run lasts
    ``seconds`` and only samples taken after the first ``settle`` seconds are
    kept.  Returns the mean of the reported current clock (MHz), its per-XCD
    spread and the mean socket power (W)."""
    import threading
    h, why = _smi_handle(torch)
    if h is None:
        return {"mhz": None, "why": why}
    import amdsmi
    samples, stop = [], threading.Event()
    t0 = time.perf_counter()

    def poll():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            except Exception:
                return
            if time.perf_counter() - t0 >= settle:
                samples.append((m.get("current_gfxclk"), m.get("current_gfxclks"),
                                m.get("current_socket_power")))
            stop.wait(0.02)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    launched = 0
    while time.perf_counter() - t0 < seconds:
        run()
        launched += 1
        if launched % 4 == 0:  # keep the queue short so the run ends on time
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    num = lambda x: isinstance(x, (int, float))
    clk = [c for c, _, _ in samples if num(c)]
    if not clk:
        return {"mhz": None, "why": "no clock samples (metrics reported N/A)"}
    xcds = [[x for x in v if num(x)] for _, v, _ in samples if isinstance(v, list)]
    xcds = [v for v in xcds if v]
    pw = [p for _, _, p in samples if num(p)]
    # Per-XCD means: work is dealt to the XCDs statically, so a lasting gap
    # between them shows up as idle time on the faster ones at the end.
    per_xcd = None
    if xcds and len({len(v) for v in xcds}) == 1:
        per_xcd = [round(sum(v[i] for v in xcds) / len(xcds), 1) for i in range(len(xcds[0]))]
    # current_gfxclk is the first XCD's clock; the mean over the XCDs is the
    # clock the whole part sustains.
    mhz = sum(per_xcd) / len(per_xcd) if per_xcd else sum(clk) / len(clk)
    return {"mhz": round(mhz, 1),
            "xcd0_mhz": round(sum(clk) / len(clk), 1),
            "xcd_mhz_range": ([min(min(v) for v in xcds), max(max(v) for v in xcds)]
                              if xcds else None),
            "xcd_mhz_mean": per_xcd,
            "socket_power_w": round(sum(pw) / len(pw), 1) if pw else None,
            "samples": len(clk), "launches": launched,
            "source": f"amdsmi GPU metrics (per-XCD current_gfxclks, mean over the XCDs) "
                      f"sampled every 20 ms after the first {settle:g} s of {seconds:g} s of "
                      f"back-to-back launches"}


def _warm(torch, f, launches: int = 3, seconds: float = 0.5):
    """At least ``launches`` calls and, after host-side input generation has
    left the GPU idle, ``seconds`` of back-to-back calls: the clock takes a
    few hundred milliseconds to ramp (a sub-millisecond kernel timed after 3
    calls read ~20 % slow)."""
    t0 = time.perf_counter()
    done = 0
    while done < launches or time.perf_counter() - t0 < seconds:
        f()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _time(torch, stream, f, reps, warm_seconds: float = 0.5):
    _warm(torch, f, seconds=warm_seconds)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_ragged_workloads(fa, torch, np, bf, stream, reps: int = 20):
    """Ragged-batch causal prefill and chunked prefill over paged histories."""
    from io_aware_exact_fa_amd.inputs import paged_prefill_inputs, varlen_inputs

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(stream.device)

    res = []
    c = VARLEN
    inp = varlen_inputs(c["H"], c["Hkv"], c["d"], seed=c["seed"], B=c["B"],
                        min_len=c["min_len"], max_len=c["max_len"])
    q, k, v = bf(inp["q_bits"]), bf(inp["k_bits"]), bf(inp["v_bits"])
    cu = i32(inp["cu_seqlens"])
    T, L = int(inp["cu_seqlens"][-1]), inp["lengths"].astype(np.int64)
    o = torch.empty_like(q)
    lse = torch.empty((c["H"], T), dtype=torch.float32, device=q.device)
    ms = _time(torch, stream, lambda: fa.fa_fwd_varlen(
        q, k, v, o, lse, cu, c["B"], c["H"], c["Hkv"], T, int(L.max()), c["d"], 1, -1,
        1.0 / math.sqrt(c["d"]), fa.FA_BF16, stream), reps)
    pairs = int((L * (L + 1) // 2).sum()) * c["H"]
    tf = 4 * c["d"] * pairs / (ms * 1e-3) / 1e12
    # Consistency: the shortest and the longest sequence, two heads, one row
    # per 256-row block of each (the oracle's per-row definition over that
    # sequence's keys).
    from oracle import attention_rows
    G = c["H"] // c["Hkv"]
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b in (int(np.argmin(L)), int(np.argmax(L))):
        s0, Lb = int(inp["cu_seqlens"][b]), int(L[b])
        rows = stratified_rows(Lb, 256, seed=b)
        for h in (0, c["H"] - 1):
            g = h // G
            ro, rl = attention_rows(inp["q"][h, s0 + rows], inp["k"][g, s0:s0 + Lb],
                                    inp["v"][g, s0:s0 + Lb], rows, True, -1,
                                    1.0 / math.sqrt(c["d"]))
            idx = torch.from_numpy(s0 + rows).to(o.device)
            got_o.append(o[h].index_select(0, idx).float().cpu().numpy())
            got_l.append(lse[h].index_select(0, idx).cpu().numpy())
            ref_o.append(ro)
            ref_l.append(rl)
    cons = consistency(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o),
                       np.concatenate(ref_l), "bf16",
                       "shortest and longest sequence x heads 0, 31: one row per 256-row block "
                       "and the ends")
    res.append({"workload": f"ragged causal prefill B{c['B']} H{c['H']}/Hkv{c['Hkv']} d{c['d']} "
                            f"L~U[{c['min_len']},{c['max_len']}] (T={T})",
                "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
                "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "consistency": cons})
    log(f"{res[-1]['workload']}: {ms:.4f} ms  {tf:.1f} TFLOP/s in-band  pass={cons['pass']}")
    del q, k, v, o, lse

    c = PAGED
    inp = paged_prefill_inputs(c["B"], c["H"], c["Hkv"], c["d"], 16, c["prefix"][0],
                               c["prefix"][1], c["chunk"][0], c["chunk"][1], seed=c["seed"],
                               with_values=False)
    q, kc, vc = bf(inp["q_bits"]), bf(inp["kcache_bits"]), bf(inp["vcache_bits"])
    pt, cuq, sk = i32(inp["page_table"]), i32(inp["cu_seqlens_q"]), i32(inp["seqlens_k"])
    Tq = int(inp["cu_seqlens_q"][-1])
    C, P = inp["chunk"].astype(np.int64), inp["prefix"].astype(np.int64)
    o = torch.empty_like(q)
    lse = torch.empty((c["H"], Tq), dtype=torch.float32, device=q.device)
    ms = _time(torch, stream, lambda: fa.fa_fwd_paged(
        q, kc, vc, pt, cuq, sk, o, lse, c["B"], c["H"], c["Hkv"], c["d"], Tq, int(C.max()),
        kc.shape[0], 16, pt.shape[1], 1, -1, 1.0 / math.sqrt(c["d"]), fa.FA_BF16, stream), reps)
    pairs = int((C * P + C * (C + 1) // 2).sum()) * c["H"]
    tf = 4 * c["d"] * pairs / (ms * 1e-3) / 1e12
    # Consistency: the chunks over the shortest and the longest prefix, two
    # heads, one row per 256 of each chunk; the oracle reads that sequence's
    # pages (widened from the stored bits) through an identity table.
    from oracle import gather_paged_kv
    from io_aware_exact_fa_amd.inputs import bf16_bits_to_f32
    G = c["H"] // c["Hkv"]
    Lk = inp["seqlens_k"].astype(np.int64)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b in (int(np.argmin(P)), int(np.argmax(P))):
        s0, Cb, Lb = int(inp["cu_seqlens_q"][b]), int(C[b]), int(Lk[b])
        pb = (Lb + 15) // 16
        phys = inp["page_table"][b, :pb]
        kb, vb = gather_paged_kv(bf16_bits_to_f32(inp["kcache_bits"][phys]),
                                 bf16_bits_to_f32(inp["vcache_bits"][phys]),
                                 np.arange(pb, dtype=np.int32)[None, :], Lb, 0)
        rows = stratified_rows(Cb, 256, seed=b)
        for h in (0, c["H"] - 1):
            g = h // G
            ro, rl = attention_rows(inp["q"][h, s0 + rows], kb[g], vb[g], Lb - Cb + rows, True,
                                    -1, 1.0 / math.sqrt(c["d"]))
            idx = torch.from_numpy(s0 + rows).to(o.device)
            got_o.append(o[h].index_select(0, idx).float().cpu().numpy())
            got_l.append(lse[h].index_select(0, idx).cpu().numpy())
            ref_o.append(ro)
            ref_l.append(rl)
    cons = consistency(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o),
                       np.concatenate(ref_l), "bf16",
                       "chunks over the shortest and longest prefix x heads 0, 31: one row per "
                       "256 and the ends")
    res.append({"workload": f"chunked causal prefill over 16-token pages B{c['B']} "
                            f"H{c['H']}/Hkv{c['Hkv']} d{c['d']} prefix~U[{c['prefix'][0]},"
                            f"{c['prefix'][1]}] chunk {c['chunk'][0]}",
                "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
                "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "consistency": cons})
    log(f"{res[-1]['workload']}: {ms:.4f} ms  {tf:.1f} TFLOP/s in-band  pass={cons['pass']}")
    del q, kc, vc, o, lse
    torch.cuda.empty_cache()

    from io_aware_exact_fa_amd.inputs import block_layout, prefill_inputs
    c = BLOCKSPARSE
    inp = prefill_inputs(1, c["H"], c["Hkv"], c["n"], c["d"], seed=c["seed"])
    q, k, v = bf(inp["q_bits"]), bf(inp["k_bits"]), bf(inp["v_bits"])
    lay_np = block_layout(c["H"], c["n"], 128, 64, seed=c["seed"], density=c["density"],
                          local=c["local"], global_cols=c["global"])
    lay = torch.from_numpy(lay_np).to(q.device)
    o = torch.empty_like(q)
    lse = torch.empty((1, c["H"], c["n"]), dtype=torch.float32, device=q.device)
    ms = _time(torch, stream, lambda: fa.fa_fwd_blocksparse(
        q, k, v, o, lse, lay, c["H"], 1, c["H"], c["Hkv"], c["n"], c["d"], 128, 64, 1, -1,
        1.0 / math.sqrt(c["d"]), fa.FA_BF16, stream), reps)
    pairs = blocksparse_causal_pairs(lay_np, c["n"], 128, 64)
    tf = 4 * c["d"] * pairs / (ms * 1e-3) / 1e12
    kept = float(lay_np.mean())
    from oracle import attention_block_sparse
    rows = stratified_rows(c["n"], 256, seed=c["seed"])
    idx = torch.from_numpy(rows).to(o.device)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for h in (0, c["H"] - 1):
        g = h // (c["H"] // c["Hkv"])
        ro, rl = attention_block_sparse(inp["q"][:, h:h + 1], inp["k"][:, g:g + 1],
                                        inp["v"][:, g:g + 1], lay_np[h:h + 1], 128, 64, True, -1,
                                        1.0 / math.sqrt(c["d"]), rows=rows)
        got_o.append(o[0, h].index_select(0, idx).float().cpu().numpy())
        got_l.append(lse[0, h].index_select(0, idx).cpu().numpy())
        ref_o.append(ro[0, 0])
        ref_l.append(rl[0, 0])
    cons = consistency(np.stack(got_o), np.stack(got_l), np.stack(ref_o), np.stack(ref_l),
                       "bf16", f"{rows.size} rows (one per 256-row block and the ends) of heads "
                               f"0, {c['H'] - 1}")
    res.append({"workload": f"block-sparse causal prefill n{c['n']} H{c['H']}/Hkv{c['Hkv']} "
                            f"d{c['d']}, 128x64 blocks: local +-{c['local']}, first "
                            f"{c['global']} column, {c['density']:.0%} random "
                            f"({kept:.1%} of blocks kept)",
                "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
                "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "consistency": cons})
    log(f"{res[-1]['workload']}: {ms:.4f} ms  {tf:.1f} TFLOP/s in-band  pass={cons['pass']}")
    del q, k, v, o, lse, lay
    torch.cuda.empty_cache()
    return res


def time_decode_fp8(fa, torch, np, bf, stream, reps: int = 20):
    """The paged decode workload with an E4M3 cache (per-head scales)."""
    from io_aware_exact_fa_amd.inputs import decode_fp8_inputs
    Dc = DECODE
    meta = decode_fp8_inputs(Dc["B"], Dc["H"], Dc["Hkv"], Dc["d"], Dc["page_size"],
                             Dc["min_len"], Dc["max_len"], seed=Dc["seed"])
    dev = torch.device("cuda")
    q = bf(meta["q_bits"])
    kc = torch.from_numpy(meta["kcache8"]).to(dev)
    vc = torch.from_numpy(meta["vcache8"]).to(dev)
    ks = torch.from_numpy(meta["k_scale"]).to(dev)
    vs = torch.from_numpy(meta["v_scale"]).to(dev)
    pt = torch.from_numpy(meta["page_table"]).to(dev)
    sl = torch.from_numpy(meta["seqlens"]).to(dev)
    k8, v8 = meta.pop("kcache8"), meta.pop("vcache8")
    o = torch.empty_like(q)
    lse = torch.empty((Dc["B"], Dc["H"]), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_decode_workspace_bytes(Dc["B"], Dc["H"], Dc["max_len"], Dc["d"])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ms = _time(torch, stream, lambda: fa.fa_decode_fp8(
        q, kc, vc, ks, vs, pt, sl, o, lse, Dc["B"], Dc["H"], Dc["Hkv"], Dc["d"], kc.shape[0],
        Dc["page_size"], pt.shape[1], Dc["max_len"], 1.0 / math.sqrt(Dc["d"]), ws, ws_bytes,
        stream), reps)
    kv_bytes = int(np.sum(meta["seqlens"].astype(np.int64))) * Dc["Hkv"] * Dc["d"] * 2
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    from oracle.fp8 import decode_fwd_fp8
    seqs = decode_sample_seqs(meta["seqlens"])
    ref_o, ref_l = [], []
    for b in seqs:
        pb = (int(meta["seqlens"][b]) + 15) // 16
        phys = meta["page_table"][b, :pb]
        ro, rl = decode_fwd_fp8(meta["q"][b:b + 1], k8[phys], v8[phys], meta["k_scale"],
                                meta["v_scale"], np.arange(pb, dtype=np.int32)[None, :],
                                meta["seqlens"][b:b + 1], 1.0 / math.sqrt(Dc["d"]))
        ref_o.append(ro[0])
        ref_l.append(rl[0])
    cons = consistency(o.float().cpu().numpy()[seqs], lse.cpu().numpy()[seqs], np.stack(ref_o),
                       np.stack(ref_l), "bf16", f"sequences {seqs}, every head")
    rec = {"workload": "paged decode B64 H32/Hkv8 d128 L~U[1024,32768] page16, E4M3 K/V "
                       "cache with per-head scales",
           "ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "kv_bytes": kv_bytes, "consistency": cons}
    log(f"{rec['workload']}: {ms:.4f} ms  {gbs:.0f} GB/s of KV  pass={cons['pass']}")
    del q, kc, vc, o, lse, ws
    torch.cuda.empty_cache()
    return [rec]


# The experiment matrix of the xxqk.cn sliding-window prefill article §9.2:
# sequence length x window (or full attention) x batch, bidirectional band.
SWEEP = dict(n=(4096, 8192, 16384, 32768), window=(512, 1024, 2048, -1), batch=(1, 2, 4, 8),
             H=32, Hkv=32, d=128, seed=14)


def run_sweep(fa, torch, stream, reps: int = 5):
    """Time fa_fwd over the sweep; returns one record per (n, window, batch)."""
    c = SWEEP
    res = []
    for n in c["n"]:
        for B in c["batch"]:
            g = torch.Generator(device="cuda").manual_seed(c["seed"] + n + B)
            shp_q, shp_kv = (B, c["H"], n, c["d"]), (B, c["Hkv"], n, c["d"])
            q = torch.randn(shp_q, generator=g, device="cuda").to(torch.bfloat16)
            k = torch.randn(shp_kv, generator=g, device="cuda").to(torch.bfloat16)
            v = torch.randn(shp_kv, generator=g, device="cuda").to(torch.bfloat16)
            o = torch.empty_like(q)
            lse = torch.empty((B, c["H"], n), dtype=torch.float32, device="cuda")
            full_ms = None
            for w in sorted(c["window"], key=lambda x: x < 0, reverse=True):  # full first
                ms = _time(torch, stream, lambda: fa.fa_fwd(
                    q, k, v, o, lse, B, c["H"], c["Hkv"], n, c["d"], 0, w,
                    1.0 / math.sqrt(c["d"]), fa.FA_BF16, stream), reps, warm_seconds=0.25)
                pairs = inband_pairs(n, False, w) * B * c["H"]
                tf = 4 * c["d"] * pairs / (ms * 1e-3) / 1e12
                if w < 0:
                    full_ms = ms
                rec = {"n": n, "window": w, "batch": B, "ms": round(ms, 4),
                       "TFLOP/s": round(tf, 2), "speedup_vs_full": round(full_ms / ms, 2),
                       "pair_ratio_full_over_band": round(inband_pairs(n, False, -1) /
                                                          inband_pairs(n, False, w), 2)}
                sched = tile_schedule(n, False, w, B=B, H=c["H"])
                rec["visited_pairs_full_over_band"] = round(
                    tile_schedule(n, False, -1, B=B, H=c["H"])["visited_pairs"] /
                    sched["visited_pairs"], 2)
                rec["inband_over_visited"] = sched["inband_over_visited"]
                rec["consistency"] = dense_consistency(
                    torch, {"q": q, "k": k, "v": v}, o, lse, False, w, 1.0 / math.sqrt(c["d"]),
                    "bf16", [(B - 1, c["H"] - 1)], stratified_rows(n, 512, seed=n + w), 512)
                res.append(rec)
                log(f"sweep n={n} w={w} B={B}: {ms:.3f} ms {tf:.1f} TFLOP/s "
                    f"x{rec['speedup_vs_full']} vs full (pairs x{rec['pair_ratio_full_over_band']}, "
                    f"visited x{rec['visited_pairs_full_over_band']}) "
                    f"pass={rec['consistency']['pass']}")
            del q, k, v, o, lse
            torch.cuda.empty_cache()
    return res


def blocksparse_causal_pairs(layout, n: int, block_q: int, block_k: int) -> int:
    """Visible (query, key) pairs of a block layout under a causal mask."""
    import numpy as np
    total = 0
    t = np.arange(block_q)
    for lay in layout:
        a, c = np.nonzero(lay)
        r0 = a * block_q
        k0 = c * block_k
        rows = r0[:, None] + t[None, :]                     # [blocks, block_q]
        kend = np.minimum(k0 + block_k, n)[:, None]         # exclusive
        cnt = np.clip(np.minimum(rows + 1, kend) - k0[:, None], 0, None)
        cnt[rows >= n] = 0
        total += int(cnt.sum())
    return total


def time_backward(fa, torch, bf, stream, q, k, v, o, lse, scale, steps: int):
    """fa_bwd on the prefill workload (o, lse from its forward), HIP events.

    Useful FLOPs: 10*d per visible pair (the five products of the chain rule:
    S = Q K^T recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q).
    """
    from io_aware_exact_fa_amd.inputs import grad_output
    P = PREFILL
    B, H, Hkv, n, d = P["B"], P["H"], P["Hkv"], P["n"], P["d"]
    log("generating the output gradient")
    _, do_bits = grad_output(B, H, n, d, seed=P["seed"], draw_scale=P["draw_scale"])
    dout = bf(do_bits)
    del do_bits
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = (torch.empty((B, h, n, d), **f32) for h in (H, Hkv, Hkv))
    ws_bytes = fa.fa_bwd_workspace_bytes(B, H, n, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)

    def bwd():
        fa.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, n, d, P["causal"], P["window"],
                  scale, fa.FA_BF16, ws, ws_bytes, stream)

    bwd()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = inband_pairs(n, bool(P["causal"]), P["window"]) * B * H
    flops = 10 * d * pairs
    tf = flops / (ms * 1e-3) / 1e12
    log(f"backward {ms:.3f} ms  {tf:.1f} TFLOP/s (10*d per in-band pair)")
    traffic = measured_traffic("backward", source_hash("backward.hip", "common.hpp"))
    del dout, dq, dk, dv, ws
    return {
        "workload": "backward of the prefill workload (same q, k, v; o and lse from fa_fwd; "
                    "dO drawn like q)",
        "value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4), "steps": steps,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "one fa_bwd call: bwd_delta + bwd_dkdv + bwd_dq kernels",
                     "algorithmic_flops_per_launch": flops},
    }


def step_record(steps: int, warmup: int, pre_ms_each, dec_ms_each, wall_s: float,
                kv_bytes: int, pre_traffic, dec_traffic) -> dict:
    """The JSON record of the timed steps: per-step prefill and decode
    durations (ms, HIP events), the wall time of the timed loop (s), the
    decode's visible K/V bytes, and the measured HBM bytes per launch (or
    None).  ``value`` and ``roofline.achieved`` use the average prefill
    duration; medians and ranges are printed beside it."""
    P, Dc = PREFILL, DECODE
    pre_each, dec_each = sorted(pre_ms_each), sorted(dec_ms_each)
    pre_ms = sum(pre_each) / steps
    dec_ms = sum(dec_each) / steps
    median = lambda xs: (xs[(len(xs) - 1) // 2] + xs[len(xs) // 2]) / 2
    pairs = inband_pairs(P["n"], bool(P["causal"]), P["window"]) * P["B"] * P["H"]
    flops = 4 * P["d"] * pairs
    tflops = flops / (pre_ms * 1e-3) / 1e12
    gbs = kv_bytes / (dec_ms * 1e-3) / 1e9
    return {
        "metric": "prefill attention TFLOP/s (in-band) & % MFMA peak; decode KV GB/s & % HBM peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall_s * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) draws rounded to bf16)",
        "config": {
            "workload": "causal GQA prefill B1 H32/Hkv8 n65536 d128 (draws x0.5) + paged "
                        "decode B64 H32/Hkv8 d128 L~U[1024,32768] page16",
            "prefill": {k2: P[k2] for k2 in ("B", "H", "Hkv", "n", "d", "causal", "window")},
            "decode": {k2: Dc[k2] for k2 in ("B", "H", "Hkv", "d", "page_size", "min_len",
                                             "max_len")},
        },
        "prefill_ms": round(pre_ms, 4),
        "decode_ms": round(dec_ms, 4),
        "prefill_ms_median": round(median(pre_each), 4),
        "prefill_ms_range": [round(pre_each[0], 4), round(pre_each[-1], 4)],
        "decode_ms_median": round(median(dec_each), 4),
        "decode_ms_range": [round(dec_each[0], 4), round(dec_each[-1], 4)],
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": pre_traffic, "kernel": "prefill_bf16_kernel",
            "algorithmic_flops_per_launch": flops,
        },
        "decode": {
            "value": round(gbs, 1), "unit": "GB/s", "kv_bytes": kv_bytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": dec_traffic,
                         "kernel": "decode_split_kernel + decode_combine_kernel"},
        },
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="query rows per sampled head for the oracle baseline (>= 1)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit "
                         "(no GPU needed)")
    ap.add_argument("--bwd-steps", type=int, default=5,
                    help="timed fa_bwd calls on the prefill workload (0: skip the backward)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the length x window x batch matrix of bidirectional band "
                         "prefill (n 4K-32K, w 512/1024/2048/full, batch 1-8) into 'sweep'")
    ap.add_argument("--clock-seconds", type=float, default=2.5,
                    help="seconds of back-to-back prefill launches after the timed steps while "
                         "the GFX clock is sampled, for the clock-adjusted peak (0: skip)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="also time every workload (fp32 n=256, causal n=4096, band n=32768, "
                         "ragged batch, chunked prefill over pages, block-sparse, FP8 decode) "
                         "and print one line each to stderr")
    args = ap.parse_args()
    if args.traffic_from:
        rec = traffic_from_counters(*args.traffic_from)
        path = os.path.join(ROOT, "profiles", "traffic.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=2)
            f.write("\n")
        print(json.dumps(rec, indent=2))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this build "
              "has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import io_aware_exact_fa_amd as fa
    from io_aware_exact_fa_amd.inputs import decode_inputs, prefill_inputs

    P, Dc = PREFILL, DECODE
    scale = 1.0 / math.sqrt(P["d"])
    log("generating prefill inputs")
    pin = prefill_inputs(P["B"], P["H"], P["Hkv"], P["n"], P["d"], seed=P["seed"],
                         draw_scale=P["draw_scale"])
    log("generating decode inputs")
    din = decode_inputs(Dc["B"], Dc["H"], Dc["Hkv"], Dc["d"], Dc["page_size"], Dc["min_len"],
                        Dc["max_len"], seed=Dc["seed"], with_values=False)
    # The oracle runs first, before anything touches the GPU: its worker
    # processes are forked from a process without GPU state (under a profiler
    # they would otherwise inherit its handlers).  Its outputs are kept for the
    # consistency check after the timed steps.
    log("timing the oracle on a bounded sample")
    cpu_rec, cpu_ref = cpu_baseline(pin, max(1, args.cpu_rows),
                                    heads=[0, 5, 10, 15, 16, 21, 26, 31])
    dec_seqs = decode_sample_seqs(din["seqlens"])
    log(f"decode oracle on sequences {dec_seqs}")
    dec_ref = decode_oracle_sample(din, dec_seqs, 1.0 / math.sqrt(Dc["d"]))

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    q, k, v = bf(pin["q_bits"]), bf(pin["k_bits"]), bf(pin["v_bits"])
    o = torch.empty_like(q)
    lse = torch.empty((P["B"], P["H"], P["n"]), dtype=torch.float32, device=dev)
    dq, dk, dv = bf(din["q_bits"]), bf(din["kcache_bits"]), bf(din["vcache_bits"])
    dpt, dsl = i32(din["page_table"]), i32(din["seqlens"])
    do = torch.empty_like(dq)
    dlse = torch.empty((Dc["B"], Dc["H"]), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_decode_workspace_bytes(Dc["B"], Dc["H"], Dc["max_len"], Dc["d"])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    del din["kcache_bits"], din["vcache_bits"]

    # A plain copy of known size: the reference for HBM counter scaling.
    cal_src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    stream = torch.cuda.current_stream()

    def prefill():
        fa.fa_fwd(q, k, v, o, lse, P["B"], P["H"], P["Hkv"], P["n"], P["d"], P["causal"],
                  P["window"], scale, fa.FA_BF16, stream)

    def decode():
        fa.fa_decode(dq, dk, dv, dpt, dsl, do, dlse, Dc["B"], Dc["H"], Dc["Hkv"], Dc["d"],
                     dk.shape[0], Dc["page_size"], dpt.shape[1], Dc["max_len"], scale, ws,
                     ws_bytes, stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        decode()
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kv_bytes = int(np.sum(din["seqlens"].astype(np.int64))) * Dc["Hkv"] * Dc["d"] * 2 * 2
    out = step_record(args.steps, args.warmup,
                      [e[0].elapsed_time(e[1]) for e in evs],
                      [e[1].elapsed_time(e[2]) for e in evs], wall, kv_bytes,
                      measured_traffic("prefill_bf16", source_hash("prefill_bf16.hip", "common.hpp")),
                      measured_traffic("decode", source_hash("decode.hip", "common.hpp")))
    tflops = out["value"]
    log(f"prefill {out['prefill_ms']:.3f} ms  {tflops:.1f} TFLOP/s   decode "
        f"{out['decode_ms']:.3f} ms  {out['decode']['value']:.0f} GB/s")

    # Consistency of the last timed step's outputs with the oracle.
    rows, heads, o_ref, lse_ref = cpu_ref
    idx = torch.from_numpy(rows).to(dev)
    got_o = o[0, heads].index_select(1, idx).float().cpu().numpy()
    got_l = lse[0, heads].index_select(1, idx).cpu().numpy()
    out["consistency"] = {
        "prefill": consistency(got_o, got_l, o_ref[0], lse_ref[0], "bf16",
                               f"{rows.size} evenly spaced rows x heads {heads} (the cpu "
                               f"baseline's sample)"),
        "decode": consistency(do.float().cpu().numpy()[dec_seqs], dlse.cpu().numpy()[dec_seqs],
                              dec_ref[0], dec_ref[1], "bf16",
                              f"sequences {dec_seqs}, every head"),
    }
    log(f"consistency: prefill {out['consistency']['prefill']}  decode "
        f"{out['consistency']['decode']}")

    # The block skip observed on the device: one counting launch (not timed)
    # against the host replica of the schedule.
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    fa.fa_fwd_tile_count(q, k, v, o2, lse2, P["B"], P["H"], P["Hkv"], P["n"], P["d"],
                         P["causal"], P["window"], scale, cnt, stream)
    torch.cuda.synchronize()
    sched = tile_schedule(P["n"], bool(P["causal"]), P["window"], B=P["B"], H=P["H"])
    got = cnt.cpu().tolist()
    sched["device_visited_wave_tiles"] = int(got[0])
    sched["device_staged_tiles"] = int(got[1])
    sched["device_matches_schedule"] = (got[0] == sched["visited_wave_tiles"] and
                                        got[1] == sched["staged_tiles"])
    sched["outputs_equal_fa_fwd"] = bool(torch.equal(o, o2) and torch.equal(lse, lse2))
    out["tiles"] = sched
    log(f"tiles: {sched}")
    del o2, lse2
    if args.clock_seconds > 0:
        log(f"sampling the GFX clock over {args.clock_seconds:g} s of prefill launches")
        clk = sustained_clock(torch, prefill, args.clock_seconds)
        if clk.get("mhz"):
            # The published peak assumes the 2400 MHz top clock; at the
            # sustained clock the same matrix cores deliver proportionally less.
            at = PEAK_BF16_TFLOPS * clk["mhz"] / 2400.0
            clk["peak_at_clock"] = round(at, 1)
            clk["frac_at_clock"] = round(tflops / at, 4)
        out["roofline"]["clock"] = clk
    del dq, dk, dv
    if args.bwd_steps > 0:
        out["backward"] = time_backward(fa, torch, bf, stream, q, k, v, o, lse, scale,
                                        args.bwd_steps)
    del q, k, v, o
    torch.cuda.empty_cache()
    if args.all_workloads:
        out["other_workloads"] = (time_other_workloads(fa, torch, np, bf, stream) +
                                  time_ragged_workloads(fa, torch, np, bf, stream) +
                                  time_decode_fp8(fa, torch, np, bf, stream))
    if args.sweep:
        out["sweep"] = run_sweep(fa, torch, stream)
    out["cpu_baseline"] = cpu_rec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

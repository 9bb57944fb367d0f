"""The block skip observed on the device: fa_fwd_tile_count counts the
(wave, key tile) pairs whose products the kernel computes and the key/value
tiles it stages (xxqk.cn sliding-window prefill article §9.1, §9.3: check
which KV blocks the kernel really visits).  The counts must equal the host
replica of the schedule (bench.tile_schedule, itself checked against an
explicit enumeration on the CPU), and the outputs must be fa_fwd's bits."""

import math

import numpy as np
import pytest

import bench
from io_aware_exact_fa_amd.inputs import prefill_inputs
from tests.gpu_util import prefill_device, say

pytestmark = pytest.mark.gpu

# (B, H, Hkv, n, d, causal, window)
CASES = [
    (1, 2, 1, 1000, 128, 1, -1),     # 8-wave workgroups, causal
    (2, 4, 2, 700, 128, 0, 37),      # 4-wave, band
    (1, 2, 2, 3000, 64, 1, 100),     # causal window
    (1, 2, 1, 1111, 128, 0, -1),     # full
    (1, 2, 1, 20000, 128, 0, 8192),  # band wide enough for 8-wave workgroups
    (1, 4, 1, 4096, 128, 0, 2048),   # the band workload's window at n = 4096
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_device_tile_counts_match_schedule(case):
    import torch
    import io_aware_exact_fa_amd as fa
    B, H, Hkv, n, d, causal, window = case
    say(f"tile count {case}")
    inp = prefill_inputs(B, H, Hkv, n, d, seed=300 + n)
    q, k, v = prefill_device(inp)
    scale = 1.0 / math.sqrt(d)
    o1, l1 = fa.flash_attn_fwd(q, k, v, causal=bool(causal), window=window, scale=scale)
    o2 = torch.empty_like(q)
    l2 = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    cnt = torch.zeros(2, dtype=torch.int64, device=q.device)
    fa.fa_fwd_tile_count(q, k, v, o2, l2, B, H, Hkv, n, d, causal, window, scale, cnt)
    torch.cuda.synchronize()
    got = cnt.cpu().numpy()
    want = bench.tile_schedule(n, bool(causal), window, B=B, H=H)
    say(f"  device visited={got[0]} staged={got[1]}  host visited="
        f"{want['visited_wave_tiles']} staged={want['staged_tiles']}")
    assert got[0] == want["visited_wave_tiles"]
    assert got[1] == want["staged_tiles"]
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

"""GPU parity of the backward pass (fa_bwd through the C ABI) against the oracle.

The HIP path runs its own forward (fa_fwd) for o and lse and then fa_bwd; the
oracle recomputes everything in fp64 from the same bf16 q, k, v and dO.
Small shapes are compared over every gradient element; the full workload
shapes are compared on sampled query rows (dq) and sampled keys (dk, dv),
which the oracle evaluates one by one.
"""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import grad_output, prefill_inputs
from oracle import attention_bwd, attention_bwd_keys, attention_bwd_rows
from tests.bwd_bounds import bwd_bounds
from tests.gpu_util import compare_grad, dev_bf16, prefill_device, rows_seeing, say

pytestmark = pytest.mark.gpu

# (B, H, Hkv, n, d, causal, window)
SMALL = [
    (1, 1, 1, 1, 128, 0, -1),
    (1, 2, 2, 7, 128, 1, -1),
    (1, 2, 1, 256, 128, 0, -1),
    (2, 4, 2, 129, 64, 0, -1),
    (2, 4, 1, 300, 128, 1, -1),
    (1, 2, 2, 333, 64, 1, -1),
    (1, 3, 3, 513, 128, 1, -1),
    (1, 2, 1, 700, 128, 0, 0),
    (1, 2, 1, 700, 128, 0, 1),
    (1, 2, 1, 700, 128, 0, 37),
    (1, 2, 1, 700, 128, 0, 128),
    (1, 2, 1, 700, 128, 0, 4096),
    (1, 2, 1, 600, 128, 1, 0),
    (1, 2, 1, 600, 128, 1, 37),
    (1, 2, 1, 600, 128, 1, 300),
    (1, 2, 2, 333, 64, 0, 50),
    (1, 8, 2, 1000, 128, 1, -1),
]


def _id(c):
    B, H, Hkv, n, d, causal, w = c
    return f"B{B}H{H}kv{Hkv}n{n}d{d}{'c' if causal else 'b'}w{w}"


def run_fwd_bwd(inp, do_bits, causal, window, scale):
    """fa_fwd then fa_bwd on the device; returns the device gradients."""
    import torch
    import io_aware_exact_fa_amd as fa
    q, k, v = prefill_device(inp)
    do = dev_bf16(do_bits)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=causal, window=window, scale=scale)
    dq, dk, dv = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=causal, window=window,
                                   scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_backward_small(case):
    B, H, Hkv, n, d, causal, window = case
    say(f"case {_id(case)}")
    seed = 2000 + n + d + window
    inp = prefill_inputs(B, H, Hkv, n, d, seed=seed)
    do, do_bits = grad_output(B, H, n, d, seed=seed)
    scale = 1.0 / math.sqrt(d)
    got = [t.cpu().numpy() for t in run_fwd_bwd(inp, do_bits, causal, window, scale)]
    ref = attention_bwd(inp["q"], inp["k"], inp["v"], do, causal, window, scale)
    for b in range(B):
        bounds = bwd_bounds(inp["q"][b], inp["k"][b], inp["v"][b], do[b], causal, window, scale)
        for name, g, r, m in zip(("dq", "dk", "dv"), got, ref, bounds):
            compare_grad(g[b], r[b], m, f"{_id(case)} b{b} {name}")


def test_backward_deterministic():
    inp = prefill_inputs(2, 4, 2, 777, 128, seed=9)
    _, do_bits = grad_output(2, 4, 777, 128, seed=9)
    a = [t.cpu().numpy() for t in run_fwd_bwd(inp, do_bits, 1, -1, 0.1)]
    b = [t.cpu().numpy() for t in run_fwd_bwd(inp, do_bits, 1, -1, 0.1)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# The workloads at full size.  dq is checked on sampled rows of two query
# heads; dk/dv on groups of sampled keys of two key/value heads, summed over
# the query heads of each group.  Each key group is evaluated over the rows
# that see it, so groups are kept narrow.  Keys of the long causal workload are
# taken from the tail only: a key near the start is seen by every later row,
# which the oracle cannot evaluate one by one in the time a test has.
FULL = {
    "causal_B4_H16_n4096": dict(B=4, H=16, Hkv=16, n=4096, d=128, causal=1, window=-1,
                                seed=2, scale_draws=1.0, heads=[(0, 0), (3, 15)],
                                rows=[0, 1, 31, 32, 127, 128, 2047, 2048, 4064, 4095],
                                key_groups=[[0, 1, 31, 32, 127, 128, 2047, 2048, 4064, 4095]]),
    "band_w2048_H32_n32768": dict(B=1, H=32, Hkv=32, n=32768, d=128, causal=0, window=2048,
                                  seed=3, scale_draws=1.0, heads=[(0, 0), (0, 31)],
                                  rows=[0, 1, 2047, 2048, 2049, 16384, 30720, 32767],
                                  key_groups=[[0, 1, 2048, 2049], [16383, 16384],
                                              [30719, 32766, 32767]]),
    "causal_gqa_H32_kv8_n65536": dict(B=1, H=32, Hkv=8, n=65536, d=128, causal=1, window=-1,
                                      seed=4, scale_draws=0.5, heads=[(0, 0), (0, 7)],
                                      rows=[0, 1, 127, 128, 32767, 32768, 65534, 65535],
                                      key_groups=[[65280, 65407, 65408, 65500, 65534, 65535]]),
}


@pytest.mark.parametrize("name", list(FULL))
def test_backward_full_size_sampled(name):
    import torch
    c = FULL[name]
    say(f"case {name}")
    B, H, Hkv, n, d = c["B"], c["H"], c["Hkv"], c["n"], c["d"]
    causal, window = c["causal"], c["window"]
    inp = prefill_inputs(B, H, Hkv, n, d, seed=c["seed"], draw_scale=c["scale_draws"])
    do, do_bits = grad_output(B, H, n, d, seed=c["seed"], draw_scale=c["scale_draws"])
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = run_fwd_bwd(inp, do_bits, causal, window, scale)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    G = H // Hkv
    rng = np.random.default_rng(c["seed"])
    rows = np.unique(np.concatenate([c["rows"], rng.integers(0, n, 8)]))
    for b, h in c["heads"]:
        g = h // G
        # dq of query head h: the oracle gets that head with its key/value head.
        ref = attention_bwd_rows(inp["q"][b, h:h + 1], inp["k"][b, g:g + 1],
                                 inp["v"][b, g:g + 1], do[b, h:h + 1], rows, causal,
                                 window, scale)
        m_dq, _, _ = bwd_bounds(inp["q"][b, h:h + 1], inp["k"][b, g:g + 1],
                                inp["v"][b, g:g + 1], do[b, h:h + 1], causal, window, scale,
                                rows=rows, keys=np.zeros(0, dtype=np.int64),
                                key_rows=np.zeros(0, dtype=np.int64))
        got = dq[b, h, torch.from_numpy(rows).to(dq.device)].cpu().numpy()
        compare_grad(got, ref[0], m_dq[0], f"{name} dq b{b} h{h}")
        # dk/dv of key/value head g: every query head of its group.
        hs = slice(g * G, (g + 1) * G)
        for keys in c["key_groups"]:
            keys = np.array(keys)
            r_dk, r_dv = attention_bwd_keys(inp["q"][b, hs], inp["k"][b, g:g + 1],
                                            inp["v"][b, g:g + 1], do[b, hs], keys,
                                            rows_seeing(keys, n, causal, window), causal,
                                            window, scale)
            _, m_dk, m_dv = bwd_bounds(inp["q"][b, hs], inp["k"][b, g:g + 1],
                                       inp["v"][b, g:g + 1], do[b, hs], causal, window, scale,
                                       rows=np.zeros(0, dtype=np.int64), keys=keys,
                                       key_rows=rows_seeing(keys, n, causal, window))
            kidx = torch.from_numpy(keys).to(dk.device)
            tag = f"{name} b{b} g{g} keys {keys.min()}..{keys.max()}"
            compare_grad(dk[b, g, kidx].cpu().numpy(), r_dk[0], m_dk[0], f"{tag} dk")
            compare_grad(dv[b, g, kidx].cpu().numpy(), r_dv[0], m_dv[0], f"{tag} dv")

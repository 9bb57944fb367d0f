"""Tensors of more than 2^31 elements: every kernel's offsets are 64-bit.

A bidirectional band (w = 64) over 17 heads of 2^20 tokens (2.28e9 elements
per tensor) runs through the forward, the backward and the ragged-batch
forward; bf16 and FP8 decode run over caches of 140 000 pages (2.29e9
elements).  The oracle checks segments at the start and at the far end of the
first and last heads, where offsets pass 2^31 elements.

These inputs are too large for the host-side generator: they are drawn on the
device from torch's generator seeded with a fixed value (float32 N(0, 1)
rounded to bf16, or encoded to E4M3), and only the slices the oracle needs are
copied to the host.
"""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import fp8_scales
from oracle import attention_bwd, attention_fwd, decode_fwd
from oracle.fp8 import decode_fwd_fp8
from tests.bwd_bounds import bwd_bounds
from tests.gpu_util import TOL_BF16, compare, compare_grad, say

pytestmark = pytest.mark.gpu


def _draw(shape, gen):
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_band_forward_backward_past_2g_elements():
    import torch
    import io_aware_exact_fa_amd as fa
    H, n, d, w, L = 17, 1 << 20, 128, 64, 1024
    assert H * n * d > 2 ** 31
    say(f"large band H{H} n{n} w{w}")
    g = torch.Generator(device="cuda").manual_seed(4242)
    q, k, v, do = (_draw((1, H, n, d), g) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=False, window=w, scale=scale)
    dq, dk, dv = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=False, window=w, scale=scale)
    # Ragged batch over the same rows: two sequences, the second from n/2.
    cu = torch.tensor([0, n // 2, n], dtype=torch.int32, device="cuda")
    ov, lv = fa.flash_attn_varlen(q[0], k[0], v[0], cu, n // 2, causal=False, window=w,
                                  scale=scale)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        for s0 in (0, n - L):
            seg = slice(s0, s0 + L)
            # rows and keys whose whole band lies inside the segment
            lo = w if s0 > 0 else 0
            hi = L - w if s0 + L < n else L
            label = f"large h{h} rows {s0 + lo}..{s0 + hi - 1}"
            qs, ks, vs, dos = (_host(t[0, h, seg])[None, None] for t in (q, k, v, do))
            o_ref, lse_ref = attention_fwd(qs, ks, vs, False, w, scale)
            compare(_host(o[0, h, seg])[lo:hi], lse[0, h, seg].cpu().numpy()[lo:hi],
                    o_ref[0, 0, lo:hi], lse_ref[0, 0, lo:hi], TOL_BF16, label)
            compare(_host(ov[h, seg])[lo:hi], lv[h, seg].cpu().numpy()[lo:hi],
                    o_ref[0, 0, lo:hi], lse_ref[0, 0, lo:hi], TOL_BF16, label + " varlen")
            ref = attention_bwd(qs, ks, vs, dos, False, w, scale)
            bounds = bwd_bounds(qs[0], ks[0], vs[0], dos[0], False, w, scale)
            # dK, dV of key j sum over the queries within w of it, each of
            # which needs its own keys within w: a margin of 2w.
            klo = 2 * w if s0 > 0 else 0
            khi = L - 2 * w if s0 + L < n else L
            for name, got, r, m in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, bounds):
                a, z = (lo, hi) if name == "dq" else (klo, khi)
                compare_grad(got[0, h, seg].cpu().numpy()[a:z], r[0, 0, a:z], m[0, a:z],
                             f"{label} {name}")


def _big_cache_table(P, lens, seed):
    """Page tables over a cache of P pages: sequence 0 takes the top pages in
    reverse order, the others random pages over the whole cache."""
    rng = np.random.default_rng(seed)
    npg = [(x + 15) // 16 for x in lens]
    table = -np.ones((len(lens), max(npg)), dtype=np.int32)
    table[0, :npg[0]] = np.arange(P - 1, P - 1 - npg[0], -1)
    rest = rng.choice(P - npg[0], size=sum(npg[1:]), replace=False)
    off = 0
    for b in range(1, len(lens)):
        table[b, :npg[b]] = rest[off:off + npg[b]]
        off += npg[b]
    return table


def _compact(table, *caches):
    """Copy the pages a table uses to the host; the table renumbered to them."""
    import torch
    used = np.unique(table[table >= 0])
    idx = torch.from_numpy(used.astype(np.int64)).to("cuda")
    remap = -np.ones(int(used.max()) + 1, dtype=np.int64)
    remap[used] = np.arange(len(used))
    t2 = np.where(table >= 0, remap[np.maximum(table, 0)], -1)
    return t2, [c.index_select(0, idx).cpu() for c in caches]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_decode_cache_past_2g_elements(fp8):
    import torch
    import io_aware_exact_fa_amd as fa
    P, Hkv, H, d = 140000, 8, 32, 128
    assert P * Hkv * 16 * d > 2 ** 31
    lens = [3000, 1, 7777, 1536]
    say(f"large decode fp8={fp8} P={P}")
    g = torch.Generator(device="cuda").manual_seed(4343)
    q = _draw((len(lens), H, d), g)
    table = _big_cache_table(P, lens, seed=4344)
    dt, ds = (torch.from_numpy(table).to("cuda"),
              torch.tensor(lens, dtype=torch.int32, device="cuda"))
    scale = 1.0 / math.sqrt(d)
    if fp8:
        ks, vs = fp8_scales(Hkv)
        kc, vc = ((torch.randn((P, Hkv, 16, d), generator=g, device="cuda") * 8).clamp(-448, 448)
                  .to(torch.float8_e4m3fn).view(torch.uint8) for _ in range(2))
        o, lse = fa.flash_decode_fp8(q, kc, vc, torch.from_numpy(ks).to("cuda"),
                                     torch.from_numpy(vs).to("cuda"), dt, ds, max(lens),
                                     scale=scale)
    else:
        kc, vc = _draw((P, Hkv, 16, d), g), _draw((P, Hkv, 16, d), g)
        o, lse = fa.flash_decode(q, kc, vc, dt, ds, max_seqlen=max(lens), scale=scale)
    torch.cuda.synchronize()
    t2, (kh, vh) = _compact(table, kc, vc)
    qh = _host(q)
    if fp8:
        o_ref, lse_ref = decode_fwd_fp8(qh, kh.numpy(), vh.numpy(), ks, vs, t2, np.array(lens),
                                        scale)
    else:
        o_ref, lse_ref = decode_fwd(qh, kh.float().numpy().astype(np.float64),
                                    vh.float().numpy().astype(np.float64), t2, np.array(lens),
                                    scale)
    compare(_host(o), lse.cpu().numpy(), o_ref, lse_ref, TOL_BF16, f"large decode fp8={fp8}")

"""Pins of the FP8 (E4M3) decode oracle (CPU).

The byte decoder against torch's float8_e4m3fn conversion for all 256 codes and
against hand-computed code points; the decode against decode_fwd over caches
dequantised by torch; the meaning of the two scales (a key scale is a score
scale, a value scale scales the output and leaves lse alone).
"""

import numpy as np
import torch

from oracle import decode_fwd
from oracle.fp8 import decode_fwd_fp8, e4m3_to_float


def test_all_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_to_float(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_code_points_by_hand():
    v = e4m3_to_float(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0x80, 0xB8, 0x00, 0x3C],
                               dtype=np.uint8))
    assert list(v[:5]) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9]
    assert v[5] == 0.0 and np.signbit(v[5])
    assert v[6] == -1.0 and v[7] == 0.0 and v[8] == 1.5
    assert np.isnan(e4m3_to_float(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def _cache(rng, P, Hkv, ps, d):
    x = rng.standard_normal((P, Hkv, ps, d)).astype(np.float32)
    return torch.from_numpy(np.clip(x * 8, -448, 448)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_matches_torch_dequantised_cache():
    rng = np.random.default_rng(90)
    B, H, Hkv, d, ps = 3, 8, 2, 16, 4
    lens = np.array([5, 16, 23])
    P = int(((lens + ps - 1) // ps).sum())
    kb, vb = _cache(rng, P, Hkv, ps, d), _cache(rng, P, Hkv, ps, d)
    table = -np.ones((B, 6), dtype=np.int64)
    perm = rng.permutation(P)
    off = 0
    for b in range(B):
        n = (lens[b] + ps - 1) // ps
        table[b, :n] = perm[off:off + n]
        off += n
    q = rng.standard_normal((B, H, d))
    ks, vs = np.array([0.125, 0.3]), np.array([0.5, 0.07])
    o, lse = decode_fwd_fp8(q, kb, vb, ks, vs, table, lens, 0.25)
    kf = torch.from_numpy(kb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vf = torch.from_numpy(vb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    o2, l2 = decode_fwd(q, kf * ks[None, :, None, None], vf * vs[None, :, None, None], table,
                        lens, 0.25)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-14)
    # key scale acts as a score scale; value scale scales o and leaves lse
    o3, l3 = decode_fwd_fp8(q, kb, vb, 2 * ks, 3 * vs, table, lens, 0.125)
    np.testing.assert_allclose(o3, 3 * o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3, lse, rtol=0, atol=1e-13)

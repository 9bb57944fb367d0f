"""fp64 reference for decode over an FP8 (E4M3) key/value cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Product code never
imports this module.

Sources: the charles2530 blog "算子与编译器：FlashAttention 与长上下文" §9
names quantised KV among the systems the IO-first principle extends to, and
the ruiowl.com deep-dive §四 names FP8 as the data type of FlashAttention-3.
The pages fix no format or scaling, so the plainest reading is taken:

  * each cached key/value element is one byte in the OCP 8-bit floating-point
    format E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent 0 holds subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN);
  * one float32 scale per key/value head dequantises it: k = byte * k_scale[g],
    v = byte * v_scale[g];
  * attention is then exactly the decode of attention.py over those values
    (the gathered rows of each sequence are dequantised and fed to
    attention_rows, as decode_fwd does).
"""

from __future__ import annotations

import numpy as np

from .attention import attention_rows, gather_paged_kv

__all__ = ["e4m3_to_float", "decode_fwd_fp8"]


def e4m3_to_float(bits) -> np.ndarray:
    """Value of E4M3 bytes (uint8 array) as float64, from the format's fields."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    man = (b & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    val = sign * np.where(exp == 0, subnormal, normal)
    return np.where((exp == 0xF) & ((b & 0x7) == 0x7), np.nan, val)


def decode_fwd_fp8(q, kcache_bits, vcache_bits, k_scale, v_scale, page_table, seqlens,
                   scale: float | None = None, batches=None):
    """Decode over E4M3 caches [num_pages, Hkv, page_size, d] (uint8) with
    per-head float32 scales [Hkv]; otherwise as ``decode_fwd``.  Each
    sequence's pages are gathered as bytes and dequantised on their own."""
    q = np.asarray(q)
    B, H, d = q.shape
    Hkv = np.asarray(kcache_bits).shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    ks = np.asarray(k_scale, dtype=np.float64)[:, None, None]
    vs = np.asarray(v_scale, dtype=np.float64)[:, None, None]
    o = np.zeros((B, H, d), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for b in (range(B) if batches is None else batches):
        L = int(seqlens[b])
        kb8, vb8 = gather_paged_kv(kcache_bits, vcache_bits, page_table, L, b)
        kb = e4m3_to_float(kb8) * ks          # [Hkv, L, d]
        vb = e4m3_to_float(vb8) * vs
        for h in range(H):
            g = h // group
            ob, lb = attention_rows(q[b, h][None, :], kb[g], vb[g], [L - 1], causal=False,
                                    window=-1, scale=scale)
            o[b, h] = ob[0]
            lse[b, h] = lb[0]
    return o, lse

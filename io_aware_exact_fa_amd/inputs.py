"""Seeded synthetic inputs shared by the HIP path, its tests and the oracle.

This module draws random numbers, rounds them to the storage type and builds
paged-cache bookkeeping.  It holds none of the attention arithmetic: no
scores, no softmax, no reductions over keys.

Recipe (fixed so every consumer sees bit-identical inputs):
  * generator: numpy ``default_rng(seed)`` (PCG64); draws are float32
    standard normals, ``Generator.standard_normal(dtype=float32)``;
  * prefill: Q, then K, then V are drawn in that order, each in [B, heads, n, d]
    C order; an optional ``draw_scale`` multiplies each float32 draw before
    rounding (0.5 is exact in binary floating point);
  * backward: the output gradient dO [B, H, n, d] is drawn from
    ``default_rng([seed, 3])`` (same draw_scale rule), so Q, K and V do not
    move when it is added;
  * ragged batch: lengths from ``default_rng([seed, 4])`` (discrete uniform,
    inclusive) unless given; then Q [H, T, d], K, V [Hkv, T, d] (T = sum of
    lengths, sequences packed in order) drawn from ``default_rng(seed)`` in
    that order;
  * chunked prefill over pages: from ``default_rng([seed, 6])`` the cached
    prefix lengths, the chunk lengths (both discrete uniform, inclusive) and a
    permutation of the P = sum ceil((prefix + chunk) / page_size) physical
    pages (sequence b takes its consecutive slice in logical order, as in
    decode); the chunks' queries Q [H, total_q, d] from
    ``default_rng([seed, 7])``; sequence b's K and V pages (prefix and chunk)
    from ``default_rng([seed, 1, b])`` and ``default_rng([seed, 2, b])`` like
    decode;
  * block-sparse layouts: [heads, nqb, nkb] uint8 from
    ``default_rng([seed, 8])``: each block kept with probability ``density``,
    plus (optionally) a local band of ``local`` key blocks on each side of the
    diagonal (block indices scaled by block_q / block_k) and the first
    ``global_cols`` key-block columns;
  * FP8 decode: lengths, q and page table as decode; sequence b's K and V
    draws come from the same generators as decode, divided by the per-head
    scale (k_scale[g] = (1 + g/16)/8, v_scale[g] = (1 + g/32)/8) and rounded to
    the nearest OCP E4M3 byte (ties to even, clipped to +-448);
  * score-stress inputs (``stress_inputs``, ``decode_stress``): standard
    draws (prefill from ``default_rng([seed, 9])``, Q then K then V) shaped
    before rounding: "rising" sets q[..., 0] = 4 and adds 849 * j / n to
    k[..., j, 0] (a ramp over key position j), "falling" subtracts that
    ramp, "large" multiplies q and k by 8, "flat" sets q = 0;
  * bf16 storage: round-to-nearest-even of the float32 draw to bfloat16;
    the returned float32 arrays hold exactly the rounded values;
  * decode: from ``default_rng(seed)``: the sequence lengths (discrete uniform
    on [min_len, max_len], inclusive), then q [B, H, d], then a random
    permutation of the P physical pages, P = sum_b ceil(L_b / page_size).
    Sequence b owns logical pages 0..ceil(L_b/ps)-1, mapped in order onto its
    consecutive slice of that permutation.  Its K and V values come from the
    generators ``default_rng([seed, 1, b])`` and ``default_rng([seed, 2, b])``
    as [pages_b, Hkv, page_size, d] draws in logical page order, so one
    sequence can be regenerated without the others.  Slots past L_b in the last
    page hold draws too (never visible).  Unused page-table entries are -1.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits_to_f32",
    "prefill_inputs",
    "grad_output",
    "varlen_inputs",
    "paged_prefill_inputs",
    "block_layout",
    "fp8_scales",
    "decode_fp8_inputs",
    "decode_lengths_and_table",
    "decode_sequence_kv",
    "decode_inputs",
    "STRESS_KINDS",
    "stress_inputs",
    "decode_stress",
]


def bf16_round(x: np.ndarray):
    """Round float32 values to bfloat16, ties to even.

    Returns (values as float32 holding the rounded numbers, raw uint16 bits).
    Inputs are finite standard-normal draws; NaN handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    bits = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    return bf16_bits_to_f32(bits), bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _draw(rng, shape, draw_scale: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if draw_scale != 1.0:
        x *= np.float32(draw_scale)
    return x


def prefill_inputs(B: int, H: int, Hkv: int, n: int, d: int, seed: int,
                   dtype: str = "bf16", draw_scale: float = 1.0) -> dict:
    """Q [B,H,n,d], K and V [B,Hkv,n,d] drawn from ``default_rng(seed)``.

    dtype "bf16": values are rounded to bfloat16 (RNE); the dict holds the
    float32 views ``q, k, v`` (exact bf16 values) and the raw bits
    ``q_bits, k_bits, v_bits`` (uint16).  dtype "f32": float32 draws only.
    """
    rng = np.random.default_rng(seed)
    out = {"dtype": dtype, "seed": seed, "shape": (B, H, Hkv, n, d)}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv)):
        x = _draw(rng, (B, heads, n, d), draw_scale)
        if dtype == "bf16":
            vals, bits = bf16_round(x)
            out[name] = vals
            out[name + "_bits"] = bits
        elif dtype == "f32":
            out[name] = x
        else:
            raise ValueError(f"unknown dtype {dtype!r}")
    return out


def grad_output(B: int, H: int, n: int, d: int, seed: int,
                draw_scale: float = 1.0):
    """Output gradient dO [B,H,n,d] for the backward pass, rounded to bf16.

    Returns (float32 values holding the bf16 numbers, raw uint16 bits).
    """
    return bf16_round(_draw(np.random.default_rng([seed, 3]), (B, H, n, d), draw_scale))


def varlen_inputs(H: int, Hkv: int, d: int, seed: int, lengths=None, B: int = 0,
                  min_len: int = 1, max_len: int = 1, draw_scale: float = 1.0) -> dict:
    """Ragged batch packed per head: q [H, T, d], k, v [Hkv, T, d] (bf16-exact
    float32 values and ``*_bits``), ``cu_seqlens`` [B+1] int32, ``lengths``."""
    if lengths is None:
        lengths = np.random.default_rng([seed, 4]).integers(min_len, max_len + 1, size=B)
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    rng = np.random.default_rng(seed)
    out = {"lengths": lengths.astype(np.int32),
           "cu_seqlens": np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv)):
        vals, bits = bf16_round(_draw(rng, (heads, T, d), draw_scale))
        out[name] = vals
        out[name + "_bits"] = bits
    return out


def paged_prefill_inputs(B: int, H: int, Hkv: int, d: int, page_size: int,
                         prefix_min: int, prefix_max: int, chunk_min: int, chunk_max: int,
                         seed: int, with_values: bool = True) -> dict:
    """Chunks of new queries over paged histories (see the module recipe).

    Returns seqlens_k [B] (prefix + chunk), chunk lengths, cu_seqlens_q [B+1],
    q / q_bits [H, total_q, d], page_table [B, max_pages] (-1 where unused),
    kcache_bits / vcache_bits [P, Hkv, page_size, d] (and float32 values when
    ``with_values``), num_pages, max_pages.
    """
    rng = np.random.default_rng([seed, 6])
    prefix = rng.integers(prefix_min, prefix_max + 1, size=B)
    chunk = rng.integers(chunk_min, chunk_max + 1, size=B)
    seqlens = (prefix + chunk).astype(np.int64)
    pages = (seqlens + page_size - 1) // page_size
    P = int(pages.sum())
    perm = rng.permutation(P).astype(np.int32)
    max_pages = int((prefix_max + chunk_max + page_size - 1) // page_size)
    table = np.full((B, max(max_pages, 1)), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    cu_q = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_vals, q_bits = bf16_round(_draw(np.random.default_rng([seed, 7]),
                                      (H, int(cu_q[-1]), d), 1.0))
    k_bits = np.empty((max(P, 1), Hkv, page_size, d), dtype=np.uint16)
    v_bits = np.empty_like(k_bits)

    def fill(b):
        _, kb, _, vb = decode_sequence_kv(seed, b, int(pages[b]), Hkv, page_size, d)
        phys = table[b, :pages[b]]
        k_bits[phys] = kb
        v_bits[phys] = vb

    with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(B)))
    out = {"seqlens_k": seqlens.astype(np.int32), "chunk": chunk.astype(np.int32),
           "prefix": prefix.astype(np.int32), "cu_seqlens_q": cu_q, "q": q_vals,
           "q_bits": q_bits, "page_table": table, "num_pages": P, "max_pages": table.shape[1],
           "page_size": page_size, "kcache_bits": k_bits, "vcache_bits": v_bits}
    if with_values:
        out["kcache"] = bf16_bits_to_f32(k_bits)
        out["vcache"] = bf16_bits_to_f32(v_bits)
    return out


def block_layout(heads: int, n: int, block_q: int, block_k: int, seed: int,
                 density: float = 0.5, local: int = -1, global_cols: int = 0) -> np.ndarray:
    """Block layout [heads, ceil(n/block_q), ceil(n/block_k)] uint8 (see recipe)."""
    nq, nk = -(-n // block_q), -(-n // block_k)
    rng = np.random.default_rng([seed, 8])
    lay = (rng.random((heads, nq, nk)) < density).astype(np.uint8)
    if local >= 0:
        a = np.arange(nq)[:, None] * block_q // block_k   # key block on the diagonal
        c = np.arange(nk)[None, :]
        lay |= (np.abs(c - a) <= local).astype(np.uint8)[None]
    if global_cols > 0:
        lay[:, :, :global_cols] = 1
    return lay


def decode_lengths_and_table(B: int, H: int, d: int, page_size: int,
                             min_len: int, max_len: int, seed: int,
                             seqlens=None) -> dict:
    """Sequence lengths, q and the permuted page table (no KV values).

    ``seqlens`` (optional, each in [min_len, max_len]) replaces the drawn
    lengths; the length draw is still made so the later draws do not move.

    Returns seqlens [B] int32, q (float32 bf16-exact) and q_bits [B,H,d],
    page_table [B, max_pages] int32 (-1 where unused), num_pages, max_pages,
    and first_page [B] (offset of each sequence's slice in the permutation).
    """
    rng = np.random.default_rng(seed)
    drawn = rng.integers(min_len, max_len + 1, size=B).astype(np.int32)
    if seqlens is None:
        seqlens = drawn
    else:
        seqlens = np.asarray(seqlens, dtype=np.int32).reshape(B)
        if seqlens.min() < min_len or seqlens.max() > max_len:
            raise ValueError("seqlens outside [min_len, max_len]")
    q_vals, q_bits = bf16_round(_draw(rng, (B, H, d), 1.0))
    pages = (seqlens.astype(np.int64) + page_size - 1) // page_size
    num_pages = int(pages.sum())
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = int((max_len + page_size - 1) // page_size)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    first = np.zeros(B, dtype=np.int64)
    off = 0
    for b in range(B):
        first[b] = off
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    return {"seqlens": seqlens, "q": q_vals, "q_bits": q_bits,
            "page_table": table, "num_pages": num_pages,
            "max_pages": max_pages, "pages": pages, "first_page": first,
            "page_size": page_size, "seed": seed}


def decode_sequence_kv(seed: int, b: int, pages_b: int, Hkv: int,
                       page_size: int, d: int):
    """K and V pages of sequence b in logical order: (k_vals, k_bits, v_vals, v_bits),
    each [pages_b, Hkv, page_size, d]."""
    kx = _draw(np.random.default_rng([seed, 1, b]), (pages_b, Hkv, page_size, d), 1.0)
    vx = _draw(np.random.default_rng([seed, 2, b]), (pages_b, Hkv, page_size, d), 1.0)
    kv, kb = bf16_round(kx)
    vv, vb = bf16_round(vx)
    return kv, kb, vv, vb


def decode_inputs(B: int, H: int, Hkv: int, d: int, page_size: int,
                  min_len: int, max_len: int, seed: int,
                  with_values: bool = True, seqlens=None) -> dict:
    """Full paged-decode workload: lengths, table, q and the whole KV cache.

    kcache/vcache are [num_pages, Hkv, page_size, d]; ``*_bits`` are the
    bfloat16 bit patterns, and (when ``with_values``) ``kcache``/``vcache``
    hold the same numbers as float32.
    """
    meta = decode_lengths_and_table(B, H, d, page_size, min_len, max_len, seed,
                                    seqlens=seqlens)
    P = meta["num_pages"]
    k_bits = np.empty((P, Hkv, page_size, d), dtype=np.uint16)
    v_bits = np.empty((P, Hkv, page_size, d), dtype=np.uint16)

    def fill(b):
        pb = int(meta["pages"][b])
        _, kb, _, vb = decode_sequence_kv(seed, b, pb, Hkv, page_size, d)
        phys = meta["page_table"][b, :pb]
        k_bits[phys] = kb
        v_bits[phys] = vb

    # Sequences use independent generators and disjoint pages, so they can be
    # filled concurrently (numpy releases the GIL while drawing).
    with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(B)))
    meta["kcache_bits"] = k_bits
    meta["vcache_bits"] = v_bits
    if with_values:
        meta["kcache"] = bf16_bits_to_f32(k_bits)
        meta["vcache"] = bf16_bits_to_f32(v_bits)
    return meta


def fp8_scales(Hkv: int):
    """Per key/value head FP8 scales (k_scale, v_scale), float32 [Hkv]."""
    g = np.arange(Hkv, dtype=np.float64)
    return ((1 + g / 16) / 8).astype(np.float32), ((1 + g / 32) / 8).astype(np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3 byte of float32 values (ties to even, clipped to +-448)."""
    import torch
    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def decode_fp8_inputs(B: int, H: int, Hkv: int, d: int, page_size: int,
                      min_len: int, max_len: int, seed: int, seqlens=None) -> dict:
    """Paged decode workload with E4M3 caches: as ``decode_inputs`` (lengths,
    q, table) plus ``kcache8``/``vcache8`` [P, Hkv, page_size, d] uint8 and
    ``k_scale``/``v_scale`` [Hkv] float32."""
    meta = decode_lengths_and_table(B, H, d, page_size, min_len, max_len, seed, seqlens=seqlens)
    P = meta["num_pages"]
    ks, vs = fp8_scales(Hkv)
    k8 = np.empty((P, Hkv, page_size, d), dtype=np.uint8)
    v8 = np.empty_like(k8)

    def fill(b):
        pb = int(meta["pages"][b])
        kx = _draw(np.random.default_rng([seed, 1, b]), (pb, Hkv, page_size, d), 1.0)
        vx = _draw(np.random.default_rng([seed, 2, b]), (pb, Hkv, page_size, d), 1.0)
        phys = meta["page_table"][b, :pb]
        k8[phys] = e4m3_encode(kx / ks[None, :, None, None])
        v8[phys] = e4m3_encode(vx / vs[None, :, None, None])

    with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(B)))
    meta.update(kcache8=k8, vcache8=v8, k_scale=ks, v_scale=vs)
    return meta



STRESS_KINDS = ("rising", "falling", "large", "flat")
_RAMP = np.float32(849.0)  # q[0] * ramp * scale ~ 300 at the end, for d = 128


def _shape_q(kind: str, q: np.ndarray) -> None:
    """Shape float32 query draws [..., d] in place."""
    if kind in ("rising", "falling"):
        q[..., 0] = np.float32(4.0)
    elif kind == "large":
        q *= np.float32(8.0)
    elif kind == "flat":
        q[...] = 0.0
    else:
        raise ValueError(f"unknown stress kind {kind!r}")


def _shape_k(kind: str, k: np.ndarray, span: int) -> None:
    """Shape float32 key draws [..., L, d] in place; key j sits at position j
    of its sequence and the ramp runs over ``span`` positions."""
    if kind in ("rising", "falling"):
        pos = np.arange(k.shape[-2], dtype=np.float32)
        ramp = (_RAMP * pos / np.float32(span)).astype(np.float32)
        k[..., 0] += ramp if kind == "rising" else -ramp
    elif kind == "large":
        k *= np.float32(8.0)


def stress_inputs(kind: str, B: int, H: int, Hkv: int, n: int, d: int, seed: int) -> dict:
    """Prefill inputs (layout and keys as ``prefill_inputs``, bf16) whose
    scores stress the running max and the rescaling of the online softmax:
    rising along the keys (the row max moves tile after tile), falling (the
    earliest visible key dominates, later ones underflow), large (scores
    spread over tens of units, rows near one-hot) or flat (all equal)."""
    rng = np.random.default_rng([seed, 9])
    x = {name: _draw(rng, (B, heads, n, d), 1.0)
         for name, heads in (("q", H), ("k", Hkv), ("v", Hkv))}
    _shape_q(kind, x["q"])
    _shape_k(kind, x["k"], n)
    out = {"dtype": "bf16", "seed": seed, "shape": (B, H, Hkv, n, d), "kind": kind}
    for name in ("q", "k", "v"):
        out[name], out[name + "_bits"] = bf16_round(x[name])
    return out


def decode_stress(meta: dict, kind: str, span: int) -> dict:
    """A decode workload (``decode_inputs`` with values) reshaped like
    ``stress_inputs``: token t of every sequence gets the ramp at position t
    (over ``span`` positions); q and the key cache are rounded to bf16 again.
    Returns a new dict; ``meta`` is left as it is."""
    out = dict(meta)
    q = np.array(meta["q"], dtype=np.float32)
    kc = np.array(meta["kcache"], dtype=np.float32)
    ps = kc.shape[2]
    _shape_q(kind, q)
    for b, L in enumerate(meta["seqlens"]):
        pages = meta["page_table"][b, :(int(L) + ps - 1) // ps]
        kb = kc[pages].transpose(1, 0, 2, 3)              # [Hkv, pages, ps, d]
        shp = kb.shape
        kb = np.ascontiguousarray(kb).reshape(shp[0], shp[1] * ps, shp[3])
        _shape_k(kind, kb, span)
        kc[pages] = kb.reshape(shp).transpose(1, 0, 2, 3)
    out["q"], out["q_bits"] = bf16_round(q)
    out["kcache"], out["kcache_bits"] = bf16_round(kc)
    return out

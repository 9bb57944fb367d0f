"""fp64 reference for ragged batches and for chunked prefill over a paged cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Product code never
imports this module.

Sources:
  * xxqk.cn sliding-window prefill article, §8.1: in batched prefill the
    requests have different lengths and share one window; the kernel clips
    each request's traversal to that request's own length instead of
    computing over padding.
  * charles2530 blog "算子与编译器：FlashAttention 与长上下文", §7: requests
    that share a long prefix should not redo its prefill, the cached history
    is reused; §5: the KV history is held in fixed-size pages.

Definitions (each reduces to ``attention_rows`` of attention.py, the plain
definition with an explicit mask):
  * ragged batch: the tokens of B sequences are packed per head as
    [heads, T, d], sequence b owning rows cu[b] .. cu[b+1]-1.  Every sequence
    is its own attention problem, positions counted from its first token.
  * chunked prefill over a paged cache: sequence b has L_b = seqlens_k[b]
    keys in pages (its cached prefix followed by the new chunk, already
    appended), and its q_b = cu_q[b+1] - cu_q[b] new queries are the last q_b
    positions: query i of the chunk sits at position L_b - q_b + i and sees
    the keys that the mask gives that position among the L_b keys.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_rows, gather_paged_kv

__all__ = ["attention_varlen", "attention_paged_prefill"]


def attention_varlen(q, k, v, cu_seqlens, causal: bool = False, window: int = -1,
                     scale: float | None = None):
    """Ragged batch: q [H, T, d], k/v [Hkv, T, d], cu_seqlens [B+1].

    Returns (o [H, T, dv], lse [H, T]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    H, T, d = q.shape
    Hkv = k.shape[0]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to T")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    o = np.zeros((H, T, v.shape[-1]), dtype=np.float64)
    lse = np.zeros((H, T), dtype=np.float64)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        rows = np.arange(s1 - s0)
        for h in range(H):
            g = h // group
            ob, lb = attention_rows(q[h, s0:s1], k[g, s0:s1], v[g, s0:s1], rows,
                                    causal, window, scale)
            o[h, s0:s1] = ob
            lse[h, s0:s1] = lb
    return o, lse


def attention_paged_prefill(q, kcache, vcache, page_table, cu_seqlens_q, seqlens_k,
                            causal: bool = True, window: int = -1,
                            scale: float | None = None):
    """New chunks over cached, paged histories.

    q: [H, Tq, d] packed chunks (sequence b owns rows cu_q[b] .. cu_q[b+1]-1);
    kcache, vcache: [num_pages, Hkv, page_size, d]; page_table [B, max_pages];
    seqlens_k [B]: keys of each sequence, the chunk's own keys included
    (each chunk is no longer than its sequence).
    Returns (o [H, Tq, d], lse [H, Tq]) in float64.
    """
    q = np.asarray(q)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    H, Tq, d = q.shape
    Hkv = np.asarray(kcache).shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    o = np.zeros((H, Tq, d), dtype=np.float64)
    lse = np.zeros((H, Tq), dtype=np.float64)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = int(seqlens_k[b])
        if s1 == s0:
            continue
        if s1 - s0 > L:
            raise ValueError("a chunk is longer than its sequence")
        kb, vb = gather_paged_kv(kcache, vcache, page_table, L, b)
        rows = np.arange(L - (s1 - s0), L)      # positions of the new queries
        for h in range(H):
            g = h // group
            ob, lb = attention_rows(q[h, s0:s1], kb[g], vb[g], rows, causal, window,
                                    scale)
            o[h, s0:s1] = ob
            lse[h, s0:s1] = lb
    return o, lse

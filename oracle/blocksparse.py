"""fp64 reference for block-sparse attention masks.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Product code never
imports this module.

Source: "FlashAttention 深度解析：大模型长序列的算力解放" (ruiowl.com), §四
names block-sparse FlashAttention, the version that accelerates sparse
attention; the xxqk.cn sliding-window prefill article §5 is the special case
where the kept blocks form a band.  The pages give no layout, so the plainest
one is taken: the score matrix of a head is cut into blocks of block_q query
rows by block_k key columns, and a 0/1 block layout says which blocks are
kept.  Key j is visible to query i when its block is kept AND the usual mask
(causal and/or window, attention.py) lets it through:

    V(i) = { j : layout[i // block_q, j // block_k] != 0 }  ∩  V_mask(i)

A row whose set is empty gets o = 0 and lse = -inf.  Everything else is the
plain definition with that explicit mask.
"""

from __future__ import annotations

import numpy as np

from .attention import visible_mask

__all__ = ["block_visible_mask", "attention_masked", "attention_block_sparse"]


def block_visible_mask(rows, n: int, layout, block_q: int, block_k: int, causal: bool,
                       window: int) -> np.ndarray:
    """Explicit boolean mask [len(rows), n] of the block-sparse visible sets."""
    rows = np.asarray(rows, dtype=np.int64)
    layout = np.asarray(layout) != 0
    keep = layout[rows // block_q][:, np.arange(n) // block_k]
    return keep & visible_mask(rows, n, causal, window)


def attention_masked(q_rows, k, v, mask, scale: float):
    """Attention of q_rows [R, d] over k, v [n, d] with an explicit mask [R, n].

    Full score rows, max-subtracted exponentials over the visible keys,
    lse = M + ln(sum), o = sum exp(s - lse) v; empty rows give o = 0 and
    lse = -inf.  Returns (o [R, dv], lse [R]) in float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    s = scale * (q_rows @ k.T)
    s_vis = np.where(mask, s, -np.inf)
    m = s_vis.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(mask, np.exp(s_vis - m_safe[:, None]), 0.0)
    z = e.sum(axis=1)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, z)))
    p = np.where(mask, np.exp(s_vis - np.where(empty, 0.0, lse)[:, None]), 0.0)
    o = p @ v
    return o, lse


def attention_block_sparse(q, k, v, layout, block_q: int, block_k: int,
                           causal: bool = False, window: int = -1,
                           scale: float | None = None, rows=None):
    """Block-sparse attention for a batch.

    q: [B, H, n, d]; k, v: [B, Hkv, n, d]; layout: [Lh, ceil(n/block_q),
    ceil(n/block_k)] with Lh = 1 (shared by all heads) or H (one per query
    head).  rows: optional query rows to evaluate.
    Returns (o [B, H, R, dv], lse [B, H, R]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    layout = np.asarray(layout)
    if layout.shape[0] not in (1, H):
        raise ValueError("layout must have 1 or H heads")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, H, rows.size, v.shape[-1]))
    lse = np.zeros((B, H, rows.size))
    for h in range(H):
        lay = layout[h if layout.shape[0] == H else 0]
        mask = block_visible_mask(rows, n, lay, block_q, block_k, causal, window)
        for b in range(B):
            o[b, h], lse[b, h] = attention_masked(q[b, h, rows], k[b, h // group],
                                                  v[b, h // group], mask, scale)
    return o, lse

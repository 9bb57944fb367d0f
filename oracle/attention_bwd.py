"""fp64 reference gradients of exact attention (the backward pass).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Product code never
imports this module.

The sources state only that the backward pass does not store the score or
probability matrices but recomputes them from the inputs (xxqk.cn
sliding-window prefill article §3.3; bomianfm.com Q&A "FlashAttention的原理是
什么？对Agent性能有何提升？" §一).  What is recomputed and differentiated is the
forward definition (see ``attention.py``): per (b, h), with the visible set
V(i) and P_ij = exp(s_ij - lse_i) for j in V(i) (0 elsewhere),

    O   = P V
    dV  = P^T dO                      (summed over the query heads of a group)
    dP  = dO V^T
    D_i = sum_j P_ij dP_ij = <dO_i, O_i>
    dS  = P o (dP - D 1^T)            (o: elementwise; zero off the mask)
    dQ  = scale * dS K
    dK  = scale * dS^T Q              (summed over the query heads of a group)

which is the chain rule through s_ij = scale <q_i, k_j> and the row softmax.
Everything is evaluated in float64 on full score rows with an explicit mask.
"""

from __future__ import annotations

import numpy as np

from .attention import visible_mask

__all__ = ["attention_bwd", "attention_bwd_rows", "attention_bwd_keys", "probabilities"]


def probabilities(q_rows, k, rows, causal: bool, window: int, scale: float):
    """Row-softmax probabilities [R, n] over the visible keys (fp64)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = k.shape[0]
    s = scale * (q_rows @ k.T)
    mask = visible_mask(rows, n, causal, window)
    s_vis = np.where(mask, s, -np.inf)
    m = s_vis.max(axis=1)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(s_vis - m[:, None]), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def attention_bwd(q, k, v, do, causal: bool = False, window: int = -1,
                  scale: float | None = None, chunk: int | None = None):
    """Gradients (dq [B,H,n,d], dk [B,Hkv,n,d], dv [B,Hkv,n,d]) in float64.

    q, do: [B, H, n, d]; k, v: [B, Hkv, n, d]; H % Hkv == 0, query head h
    uses key/value head h // (H // Hkv).  ``do`` is the gradient of the loss
    with respect to the forward output.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    group = H // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if chunk is None:
        chunk = max(1, min(n, (1 << 22) // max(n, 1)))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = h // group
            for r0 in range(0, n, chunk):
                rows = np.arange(r0, min(n, r0 + chunk))
                p = probabilities(q[b, h, rows], k[b, g], rows, causal, window, scale)
                o = p @ v[b, g]
                dp = do[b, h, rows] @ v[b, g].T
                dsum = np.sum(do[b, h, rows] * o, axis=1)
                ds = p * (dp - dsum[:, None])
                dq[b, h, rows] = scale * (ds @ k[b, g])
                dk[b, g] += scale * (ds.T @ q[b, h, rows])
                dv[b, g] += p.T @ do[b, h, rows]
    return dq, dk, dv


def _row_terms(q_rows, k, v, do_rows, rows, causal, window, scale):
    """P and dS of the given query rows of one head, over all n keys."""
    p = probabilities(q_rows, k, rows, causal, window, scale)
    o = p @ v
    dp = do_rows @ v.T
    dsum = np.sum(do_rows * o, axis=1)
    return p, p * (dp - dsum[:, None])


def attention_bwd_rows(q, k, v, do, rows, causal: bool = False, window: int = -1,
                       scale: float | None = None):
    """dq of the query rows ``rows`` of one batch element, in float64.

    q, do: [H, n, d]; k, v: [Hkv, n, d].  Returns dq [H, len(rows), d].
    Same definitions as ``attention_bwd``, evaluated only on those rows.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    H, n, d = q.shape
    group = H // k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((H, rows.size, d))
    for h in range(H):
        g = h // group
        _, ds = _row_terms(q[h, rows], k[g], v[g], do[h, rows], rows, causal, window, scale)
        out[h] = scale * (ds @ k[g])
    return out


def attention_bwd_keys(q, k, v, do, keys, rows, causal: bool = False, window: int = -1,
                       scale: float | None = None):
    """dk, dv of the keys ``keys`` of one batch element, in float64.

    q, do: [H, n, d]; k, v: [Hkv, n, d].  ``rows`` are the query rows summed
    over; they must include every row that sees one of ``keys`` (rows that see
    none add exactly zero).  Returns (dk, dv), each [Hkv, len(keys), d],
    summed over the query heads of each key/value head.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    H, n, d = q.shape
    Hkv = k.shape[0]
    group = H // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    keys = np.asarray(keys, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    dk = np.zeros((Hkv, keys.size, d))
    dv = np.zeros((Hkv, keys.size, d))
    for h in range(H):
        g = h // group
        p, ds = _row_terms(q[h, rows], k[g], v[g], do[h, rows], rows, causal, window, scale)
        dk[g] += scale * (ds[:, keys].T @ q[h, rows])
        dv[g] += p[:, keys].T @ do[h, rows]
    return dk, dv


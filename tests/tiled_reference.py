"""Second fp64 reference, tiled with an online softmax, used only to pin the oracle.

It follows the block algorithm the pages describe rather than the plain
definition, so agreement with the oracle checks both:
  * xxqk.cn sliding-window prefill article, §3.1-§3.2: Q, K, V split into
    blocks of B rows; per query block a running row max m, running sum l and
    an output accumulator; each new key block raises m, rescales l and the
    accumulator by exp(m_old - m_new) and adds its own exponentials.  With one
    block covering the whole sequence this is the ordinary softmax.
  * same article, §5.1 and §5.3: a key block entirely outside the window of the
    query block is skipped; the loop over ascending key blocks may stop at the
    first block that starts past the window; §5.2: partly covered blocks get a
    -inf mask added before the softmax update; §5.5: skipping an all -inf block
    is exact.
  * The page's sketch starts m at -inf; a row whose first visited block holds
    no visible key would then evaluate exp(-inf - (-inf)).  This version uses 0
    in place of a still -inf running max, which leaves every later update exact.
Also a split-then-merge reference for decode: partial (o_s, lse_s) over
disjoint key ranges merged by log-sum-exp weights.
"""

from __future__ import annotations

import numpy as np


def _visible_block(q0, q1, k0, k1, causal, window):
    """Index-range test: may any (i in [q0,q1], j in [k0,k1]) be visible?"""
    if causal:
        if k0 > q1:
            return False
        if window >= 0 and k1 < q0 - window:
            return False
        return True
    if window >= 0 and (k1 < q0 - window or k0 > q1 + window):
        return False
    return True


def tiled_attention(q, k, v, block: int, causal=False, window=-1, scale=None,
                    skip=True):
    """One head: q, k, v [n, d] -> (o [n, d], lse [n], visited_block_pairs)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros_like(q)
    lse = np.zeros(n)
    visited = 0
    for q0 in range(0, n, block):
        q1 = min(q0 + block, n) - 1
        rows = np.arange(q0, q1 + 1)
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, d))
        for k0 in range(0, n, block):
            k1 = min(k0 + block, n) - 1
            if skip:
                if not causal and window >= 0 and k0 > q1 + window:
                    break  # ascending key blocks: nothing further is visible
                if causal and k0 > q1:
                    break
                if not _visible_block(q0, q1, k0, k1, causal, window):
                    continue
            visited += 1
            cols = np.arange(k0, k1 + 1)
            s = scale * (q[q0:q1 + 1] @ k[k0:k1 + 1].T)
            ii = rows[:, None]
            jj = cols[None, :]
            ok = np.ones(s.shape, dtype=bool)
            if causal:
                ok &= jj <= ii
                if window >= 0:
                    ok &= jj >= ii - window
            elif window >= 0:
                ok &= np.abs(ii - jj) <= window
            s = np.where(ok, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            m_use = np.where(np.isfinite(m_new), m_new, 0.0)   # NaN guard
            p = np.exp(s - m_use[:, None])
            alpha = np.exp(m - m_use)
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[k0:k1 + 1]
            m = m_new
        m_fin = np.where(np.isfinite(m), m, 0.0)
        o[q0:q1 + 1] = acc / l[:, None]
        lse[q0:q1 + 1] = m_fin + np.log(l)
    return o, lse, visited


def split_merge_attention(qv, k, v, bounds, scale):
    """One query vector over keys split at ``bounds`` (sorted cut points).

    Each part yields a normalised partial output o_s and its log-sum-exp
    lse_s; the merge weights part s by exp(lse_s - lse) with
    lse = log sum_s exp(lse_s).  Returns (o [d], lse).
    """
    qv = np.asarray(qv, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cuts = [0] + list(bounds) + [k.shape[0]]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b <= a:
            continue
        s = scale * (k[a:b] @ qv)
        mx = s.max()
        e = np.exp(s - mx)
        z = e.sum()
        parts.append((e @ v[a:b] / z, mx + np.log(z)))
    lses = np.array([p[1] for p in parts])
    big = lses.max()
    w = np.exp(lses - big)
    lse = big + np.log(w.sum())
    o = sum(np.exp(ls - lse) * os_ for os_, ls in parts)
    return o, lse

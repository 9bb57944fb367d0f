"""Elementwise rounding bounds for the bf16 backward pass (test tolerance).

The HIP backward takes bf16 q, k, v, dO, the forward's bf16 O and fp32 lse,
and rounds two intermediates to bf16 before its matrix products: P (for dV)
and dS (for dQ and dK); everything else is fp32.  With u = 2^-8 (unit
roundoff of bf16, 8 significant bits, round to nearest) and, per query row
i,

    E_i = sum_c |dO_ic| |O_ic|      (bounds the error of D_i = <dO_i, O_i>
                                     caused by O being stored in bf16: u E_i)
    A_ij = |dS_ij| + P_ij E_i       (bounds |error of dS_ij| / u before and
                                     after its own rounding, to first order)

the first-order error of each gradient element is at most u times

    M_dq[i, c] = scale * sum_j A_ij |k_jc|
    M_dk[j, c] = scale * sum_i A_ij |q_ic|     (summed over the group's heads)
    M_dv[j, c] =         sum_i P_ij |dO_ic|    (summed over the group's heads)

fp32 accumulation, the fp32 lse and exp add far less (below 3e-4 M for the
sizes tested), so the tests accept |got - ref| <= 2u M = 2^-7 M elementwise.
A wrong term, sign, index, mask edge or scale moves elements by a large
fraction of M itself and fails.

P, O and dS are evaluated in float64 from the oracle's probabilities.
"""

from __future__ import annotations

import numpy as np

from oracle import probabilities

BOUND_FACTOR = 2.0 ** -7


def _row_bounds(q_rows, k, v, do_rows, rows, causal, window, scale):
    p = probabilities(q_rows, k, rows, causal, window, scale)
    o = p @ v
    dp = do_rows @ v.T
    dsum = np.sum(do_rows * o, axis=1)
    e = np.sum(np.abs(do_rows) * np.abs(o), axis=1)
    a = np.abs(p * (dp - dsum[:, None])) + p * e[:, None]
    return p, a


def bwd_bounds(q, k, v, do, causal, window, scale, rows=None, keys=None, key_rows=None):
    """Bounds M for one batch element: q, do [H, n, d]; k, v [Hkv, n, d].

    Returns (M_dq [H, len(rows), d], M_dk [Hkv, len(keys), d],
    M_dv [Hkv, len(keys), d]).  rows / keys default to all; key_rows (the
    query rows summed for the key bounds, a superset of the rows that see
    ``keys``) defaults to all rows.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    H, n, d = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    rows = np.arange(n) if rows is None else np.asarray(rows)
    keys = np.arange(n) if keys is None else np.asarray(keys)
    key_rows = np.arange(n) if key_rows is None else np.asarray(key_rows)
    m_dq = np.zeros((H, rows.size, d))
    m_dk = np.zeros((Hkv, keys.size, d))
    m_dv = np.zeros((Hkv, keys.size, d))
    for h in range(H):
        g = h // G
        _, a = _row_bounds(q[h, rows], k[g], v[g], do[h, rows], rows, causal, window, scale)
        m_dq[h] = scale * (a @ np.abs(k[g]))
        p, a = _row_bounds(q[h, key_rows], k[g], v[g], do[h, key_rows], key_rows, causal,
                           window, scale)
        m_dk[g] += scale * (a[:, keys].T @ np.abs(q[h, key_rows]))
        m_dv[g] += p[:, keys].T @ np.abs(do[h, key_rows])
    return m_dq, m_dk, m_dv

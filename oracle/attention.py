"""fp64 reference attention: the plain definition with an explicit mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Product code never
imports this module.

Definition evaluated, per batch b, query head h and query row i, with the
key/value head g = h // (H // Hkv) and the visible key set V(i):

    s_ij  = scale * <q[b,h,i,:], k[b,g,j,:]>             for j in V(i)
    M_i   = max_{j in V(i)} s_ij
    lse_i = M_i + ln( sum_{j in V(i)} exp(s_ij - M_i) )
    o_i   = sum_{j in V(i)} exp(s_ij - lse_i) * v[b,g,j,:]

Sources:
  * charles2530 blog "算子与编译器：FlashAttention 与长上下文", §1: the formula
    softmax(Q Kᵀ / √d) V (the caller passes scale = 1/√d by default).
  * xxqk.cn sliding-window prefill article, §4: a query sees the keys within
    distance w on both sides (bidirectional band); a causal model sees only
    the range from i-w up to i.  §5.2: keys outside the window receive a score
    of -inf before the softmax, so they carry zero probability.
  * The log-sum-exp row statistic is not printed on the pages; it is the
    natural-log normaliser of the same softmax, scale included.

Visible set V(i) for a sequence of n keys (window < 0 means "no window"):
  full            : 0 <= j < n
  causal          : 0 <= j <= i
  band  (w >= 0)  : |i - j| <= w        (inclusive, both sides)
  causal window   : i - w <= j <= i     (inclusive, w + 1 keys at most)

Numbers: inputs are upcast exactly to float64 and everything is evaluated in
float64; no tiling, reordering or online softmax is used.
"""

from __future__ import annotations

import multiprocessing as _mp
import os

import numpy as np

__all__ = [
    "visible_mask",
    "attention_rows",
    "attention_fwd",
    "gather_paged_kv",
    "decode_fwd",
]


def visible_mask(rows, n: int, causal: bool, window: int) -> np.ndarray:
    """Explicit boolean mask [len(rows), n]: True where key j is visible to row i.

    xxqk.cn sliding-window prefill article, §4 (band |i-j| <= w and the causal
    range [i-w, i]); §4.1 (everything outside the band is -inf).
    """
    i = np.asarray(rows, dtype=np.int64).reshape(-1, 1)
    j = np.arange(n, dtype=np.int64).reshape(1, -1)
    mask = np.ones((i.shape[0], n), dtype=bool)
    if causal:
        mask &= j <= i
        if window >= 0:
            mask &= j >= i - window
    elif window >= 0:
        mask &= np.abs(i - j) <= window
    return mask


def attention_rows(q_rows, k, v, rows, causal: bool, window: int, scale: float):
    """Attention for the query rows ``rows`` of one (batch, head).

    q_rows: [R, d]   the query vectors of those rows
    k, v  : [n, d]   all keys and values of the matching key/value head
    Returns (o [R, d], lse [R]) in float64.

    Steps follow the plain definition (charles2530 blog §1): full score rows,
    explicit mask, max-subtracted exponentials, normalise, multiply by V.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    s = scale * (q_rows @ k.T)                      # [R, n] all scores
    mask = visible_mask(rows, n, causal, window)    # [R, n]
    s_vis = np.where(mask, s, -np.inf)
    m = s_vis.max(axis=1)                           # row max over visible keys
    # A row with no visible key cannot occur for these masks (j = i is always
    # visible when i < n); guard anyway so such a row yields o = 0, lse = -inf.
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(s_vis - m_safe[:, None]), 0.0)
    z = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(z)
    p = np.where(mask, np.exp(s_vis - lse[:, None]), 0.0)
    o = p @ v
    return o, lse


# ---------------------------------------------------------------------------
# Batched driver (optionally over several processes).
# ---------------------------------------------------------------------------

_SHARED: dict = {}


def _task(args):
    b, h, row_chunk = args
    q, k, v, causal, window, scale, group = (
        _SHARED["q"], _SHARED["k"], _SHARED["v"], _SHARED["causal"],
        _SHARED["window"], _SHARED["scale"], _SHARED["group"])
    g = h // group
    o, lse = attention_rows(q[b, h, row_chunk], k[b, g], v[b, g], row_chunk,
                            causal, window, scale)
    return b, h, row_chunk, o, lse


def _worker_init():
    try:  # one BLAS thread per worker process: parallelism comes from the pool
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def attention_fwd(q, k, v, causal: bool = False, window: int = -1,
                  scale: float | None = None, rows=None, workers: int = 1,
                  chunk: int | None = None):
    """Reference attention for a batch.

    q: [B, H, n, d];  k, v: [B, Hkv, n, d] with H % Hkv == 0 (grouped-query
    attention: query head h reads key/value head h // (H // Hkv)).
    rows: optional 1-D array of query row indices to evaluate (all rows by
    default); the result then holds only those rows, in that order.
    workers: number of processes (fork) over (b, h, row-chunk) tasks.
    Returns (o [B, H, R, dv] float64, lse [B, H, R] float64), dv = v.shape[-1].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    if chunk is None:
        chunk = max(1, min(R, (1 << 22) // max(n, 1)))
    tasks = []
    offsets = []
    for b in range(B):
        for h in range(H):
            for c0 in range(0, R, chunk):
                tasks.append((b, h, rows[c0:c0 + chunk]))
                offsets.append(c0)
    o = np.zeros((B, H, R, v.shape[-1]), dtype=np.float64)
    lse = np.zeros((B, H, R), dtype=np.float64)
    _SHARED.update(q=q, k=k, v=v, causal=causal, window=window, scale=scale,
                   group=H // Hkv)
    try:
        if workers <= 1 or len(tasks) <= 1:
            results = map(_task, tasks)
            for (tb, th, _), off, res in zip(tasks, offsets, results):
                _, _, rc, ob, lb = res
                o[tb, th, off:off + len(rc)] = ob
                lse[tb, th, off:off + len(rc)] = lb
        else:
            # Workers are forked (they inherit the inputs without copying) and
            # end by returning from their task loop once the pool is closed;
            # they are never sent a signal (a profiler's handlers, inherited
            # through fork, must not run in them).
            ctx = _mp.get_context("fork")
            pool = ctx.Pool(workers, initializer=_worker_init)
            try:
                for (tb, th, _), off, res in zip(
                        tasks, offsets, pool.imap(_task, tasks, chunksize=1)):
                    _, _, rc, ob, lb = res
                    o[tb, th, off:off + len(rc)] = ob
                    lse[tb, th, off:off + len(rc)] = lb
            finally:
                pool.close()
                pool.join()
    finally:
        _SHARED.clear()
    return o, lse


# ---------------------------------------------------------------------------
# Decode over a paged KV cache.
# ---------------------------------------------------------------------------

def gather_paged_kv(kcache, vcache, page_table, seqlen: int, b: int):
    """Contiguous K, V [Hkv, L, d] of sequence b, read through its page table.

    Token t of sequence b lives in physical page page_table[b, t // ps] at
    slot t % ps, where ps is the page size (charles2530 blog §5 and the xxqk.cn
    article §8.2 describe KV held in fixed-size pages managed per block).
    """
    kcache = np.asarray(kcache)
    vcache = np.asarray(vcache)
    ps = kcache.shape[2]
    t = np.arange(seqlen)
    phys = np.asarray(page_table)[b, t // ps]
    slot = t % ps
    k = kcache[phys, :, slot, :]            # [L, Hkv, d]
    v = vcache[phys, :, slot, :]
    return np.transpose(k, (1, 0, 2)), np.transpose(v, (1, 0, 2))


def decode_fwd(q, kcache, vcache, page_table, seqlens, scale: float | None = None,
               batches=None):
    """Attention of one new query token per sequence over its whole KV cache.

    q: [B, H, d]; kcache, vcache: [num_pages, Hkv, page_size, d];
    page_table: [B, max_pages] physical page ids; seqlens: [B] (>= 1).
    The query attends to all seqlens[b] cached tokens (no mask): the decode
    step reads the whole history (charles2530 blog §3-§4, §6.2).
    batches: optional subset of batch indices to evaluate (others left zero).
    Returns (o [B, H, d] float64, lse [B, H] float64).
    """
    q = np.asarray(q)
    B, H, d = q.shape
    Hkv = np.asarray(kcache).shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = H // Hkv
    o = np.zeros((B, H, d), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for b in (range(B) if batches is None else batches):
        L = int(seqlens[b])
        kb, vb = gather_paged_kv(kcache, vcache, page_table, L, b)
        for h in range(H):
            g = h // group
            ob, lb = attention_rows(q[b, h][None, :], kb[g], vb[g], [L - 1],
                                    causal=False, window=-1, scale=scale)
            o[b, h] = ob[0]
            lse[b, h] = lb[0]
    return o, lse


def default_workers() -> int:
    """Host cores available to this process."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1

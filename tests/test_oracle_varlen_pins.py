"""Pins of the ragged-batch and paged-prefill oracle functions (CPU).

The ragged form against the pinned batched oracle and against brute force;
the paged prefill against decode (one-token chunks), against prefill over the
gathered cache (no prefix), and by the prefix-reuse identity: a chunk over a
cached prefix gives exactly the last rows of one causal prefill over the
whole sequence, whatever the split.
"""

import math

import numpy as np
import pytest

from oracle import attention_fwd, decode_fwd
from oracle.varlen import attention_paged_prefill, attention_varlen
from tests.test_oracle_pins import _brute

MODES = [(False, -1), (True, -1), (False, 3), (True, 2), (False, 0), (True, 0)]


def _packed(rng, H, Hkv, lens, d):
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((H, T, d))
    k = rng.standard_normal((Hkv, T, d))
    v = rng.standard_normal((Hkv, T, d))
    return q, k, v, cu


@pytest.mark.parametrize("causal,window", MODES)
def test_varlen_equal_lengths_is_the_batched_oracle(causal, window):
    rng = np.random.default_rng(70)
    B, H, Hkv, n, d = 3, 4, 2, 17, 8
    q, k, v, cu = _packed(rng, H, Hkv, [n] * B, d)
    o, lse = attention_varlen(q, k, v, cu, causal, window, 0.4)
    # [H, B*n, d] -> [B, H, n, d]
    qb = q.reshape(H, B, n, d).transpose(1, 0, 2, 3)
    kb = k.reshape(Hkv, B, n, d).transpose(1, 0, 2, 3)
    vb = v.reshape(Hkv, B, n, d).transpose(1, 0, 2, 3)
    o2, lse2 = attention_fwd(qb, kb, vb, causal, window, 0.4)
    np.testing.assert_allclose(o, o2.transpose(1, 0, 2, 3).reshape(H, B * n, d),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2.transpose(1, 0, 2).reshape(H, B * n),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", MODES)
def test_varlen_brute_force_and_independence(causal, window):
    rng = np.random.default_rng(71)
    H, Hkv, d = 2, 1, 3
    lens = [1, 4, 0, 3]
    q, k, v, cu = _packed(rng, H, Hkv, lens, d)
    o, lse = attention_varlen(q, k, v, cu, causal, window, 0.7)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        s0, s1 = cu[b], cu[b + 1]
        ob, lb = _brute(q[:, s0:s1].tolist(), k[:, s0:s1].tolist(), v[:, s0:s1].tolist(),
                        causal, window, 0.7)
        np.testing.assert_allclose(o[:, s0:s1], ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, s0:s1], lb, rtol=0, atol=1e-13)
    # changing another sequence's tokens leaves sequence 1 untouched
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 5:], k2[:, 5:], v2[:, 5:] = 0.0, 7.0, -3.0
    o2, lse2 = attention_varlen(q2, k2, v2, cu, causal, window, 0.7)
    assert np.array_equal(o2[:, 1:5], o[:, 1:5]) and np.array_equal(lse2[:, 1:5], lse[:, 1:5])


def _paged_cache(rng, Hkv, ps, d, lens):
    pages = [(L + ps - 1) // ps for L in lens]
    P = sum(pages)
    perm = rng.permutation(P)
    table = -np.ones((len(lens), max(pages)), dtype=np.int64)
    kc = rng.standard_normal((P, Hkv, ps, d))
    vc = rng.standard_normal((P, Hkv, ps, d))
    off = 0
    for b in range(len(lens)):
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    return kc, vc, table


def _contiguous(kc, vc, table, L, b):
    ps = kc.shape[2]
    t = np.arange(L)
    return (kc[table[b, t // ps], :, t % ps].transpose(1, 0, 2),
            vc[table[b, t // ps], :, t % ps].transpose(1, 0, 2))


def test_paged_one_token_chunks_are_decode():
    rng = np.random.default_rng(72)
    H, Hkv, d, ps = 4, 2, 8, 4
    lens = [1, 9, 16, 30]
    kc, vc, table = _paged_cache(rng, Hkv, ps, d, lens)
    q = rng.standard_normal((H, len(lens), d))
    cu = np.arange(len(lens) + 1)
    o, lse = attention_paged_prefill(q, kc, vc, table, cu, lens, True, -1, 0.3)
    od, lsed = decode_fwd(q.transpose(1, 0, 2), kc, vc, table, np.array(lens), 0.3)
    np.testing.assert_allclose(o.transpose(1, 0, 2), od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse.T, lsed, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", MODES)
def test_paged_without_prefix_is_prefill(causal, window):
    rng = np.random.default_rng(73)
    H, Hkv, d, ps = 2, 1, 6, 4
    lens = [7, 12, 1]
    kc, vc, table = _paged_cache(rng, Hkv, ps, d, lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((H, cu[-1], d))
    o, lse = attention_paged_prefill(q, kc, vc, table, cu, lens, causal, window, 0.5)
    for b, L in enumerate(lens):
        kb, vb = _contiguous(kc, vc, table, L, b)
        o2, l2 = attention_fwd(q[None, :, cu[b]:cu[b + 1]], kb[None], vb[None], causal,
                               window, 0.5)
        np.testing.assert_allclose(o[:, cu[b]:cu[b + 1]], o2[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, cu[b]:cu[b + 1]], l2[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", [(True, -1), (True, 5), (False, -1), (False, 4)])
@pytest.mark.parametrize("split", [0, 1, 13, 31, 32])
def test_prefix_reuse_identity(causal, window, split):
    """A chunk of queries over a cached prefix equals the chunk's rows of one
    prefill over the whole sequence (with its keys)."""
    rng = np.random.default_rng(74)
    H, Hkv, d, ps, L = 4, 2, 5, 8, 33
    kc, vc, table = _paged_cache(rng, Hkv, ps, d, [L])
    qfull = rng.standard_normal((H, L, d))
    kb, vb = _contiguous(kc, vc, table, L, 0)
    ofull, lfull = attention_fwd(qfull[None], kb[None], vb[None], causal, window, 0.6)
    chunk = qfull[:, split:]
    o, lse = attention_paged_prefill(chunk, kc, vc, table, [0, L - split], [L], causal,
                                     window, 0.6)
    np.testing.assert_allclose(o, ofull[0][:, split:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lfull[0][:, split:], rtol=0, atol=1e-13)


def test_chunk_by_chunk_rebuilds_causal_prefill():
    """Feeding a sequence as successive chunks, each over everything before
    it, yields every row of the causal prefill."""
    rng = np.random.default_rng(75)
    H, Hkv, d, ps, L = 2, 2, 4, 4, 23
    kc, vc, table = _paged_cache(rng, Hkv, ps, d, [L])
    qfull = rng.standard_normal((H, L, d))
    kb, vb = _contiguous(kc, vc, table, L, 0)
    ofull, lfull = attention_fwd(qfull[None], kb[None], vb[None], True, -1, 0.9)
    cuts = [0, 5, 6, 14, 23]
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, lse = attention_paged_prefill(qfull[:, a:b], kc, vc, table, [0, b - a], [b],
                                         True, -1, 0.9)
        np.testing.assert_allclose(o, ofull[0][:, a:b], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lfull[0][:, a:b], rtol=0, atol=1e-13)


def test_paged_prefill_brute_force():
    """Tiny case by pure-Python loops over explicit visible ranges."""
    rng = np.random.default_rng(76)
    H, Hkv, d, ps = 2, 1, 3, 2
    lens, qlens = [5, 3], [2, 3]
    kc, vc, table = _paged_cache(rng, Hkv, ps, d, lens)
    cu = np.concatenate([[0], np.cumsum(qlens)])
    q = rng.standard_normal((H, cu[-1], d))
    o, lse = attention_paged_prefill(q, kc, vc, table, cu, lens, True, 1, 0.8)
    for b, (L, ql) in enumerate(zip(lens, qlens)):
        for h in range(H):
            for i in range(ql):
                pos = L - ql + i
                js = range(max(0, pos - 1), pos + 1)
                s = {j: 0.8 * math.fsum(q[h, cu[b] + i, t] * kc[table[b, j // ps], 0, j % ps, t]
                                         for t in range(d)) for j in js}
                top = max(s.values())
                z = math.fsum(math.exp(x - top) for x in s.values())
                assert abs(lse[h, cu[b] + i] - (top + math.log(z))) < 1e-13
                for t in range(d):
                    ref = math.fsum(math.exp(s[j] - top) / z
                                    * vc[table[b, j // ps], 0, j % ps, t] for j in js)
                    assert abs(o[h, cu[b] + i, t] - ref) < 1e-13

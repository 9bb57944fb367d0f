"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test pins the oracle to brute force on tiny inputs, a library routine,
closed forms, invariants or numbers printed on the source pages, so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_fwd, attention_rows, decode_fwd, gather_paged_kv, visible_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MODES = [  # (causal, window)
    (False, -1), (True, -1), (False, 0), (False, 1), (False, 2), (False, 7),
    (True, 0), (True, 1), (True, 3),
]


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# Brute force on tiny inputs: explicit index ranges, math.fsum, scalar loops.
# --------------------------------------------------------------------------

def _visible_range(i, n, causal, window):
    """Visible keys of row i written as explicit ranges (not comparisons)."""
    if causal:
        lo = 0 if window < 0 else max(0, i - window)
        return range(lo, i + 1)
    if window < 0:
        return range(0, n)
    return range(max(0, i - window), min(n, i + window + 1))


def _brute(q, k, v, causal, window, scale):
    """q [H,n,d], k/v [Hkv,n,d] as nested lists; returns o, lse as lists."""
    H, n, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    o = [[[0.0] * d for _ in range(n)] for _ in range(H)]
    lse = [[0.0] * n for _ in range(H)]
    for h in range(H):
        g = h * Hkv // H
        for i in range(n):
            js = list(_visible_range(i, n, causal, window))
            s = {j: scale * math.fsum(q[h][i][t] * k[g][j][t] for t in range(d))
                 for j in js}
            top = max(s.values())
            z = math.fsum(math.exp(s[j] - top) for j in js)
            lse[h][i] = top + math.log(z)
            for t in range(d):
                o[h][i][t] = math.fsum(math.exp(s[j] - top) / z * v[g][j][t]
                                       for j in js)
    return o, lse


@pytest.mark.parametrize("n", [1, 2, 3, 5])
@pytest.mark.parametrize("causal,window", MODES)
def test_brute_force_tiny(n, causal, window):
    rng = np.random.default_rng(100 + n)
    H, Hkv, d = 2, 1, 3
    q, k, v = _rand(rng, 1, H, n, d), _rand(rng, 1, Hkv, n, d), _rand(rng, 1, Hkv, n, d)
    scale = 0.7
    o, lse = attention_fwd(q, k, v, causal, window, scale)
    ob, lb = _brute(q[0].tolist(), k[0].tolist(), v[0].tolist(), causal, window, scale)
    np.testing.assert_allclose(o[0], np.array(ob), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], np.array(lb), rtol=0, atol=1e-13)


def test_hand_cases():
    rng = np.random.default_rng(7)
    d = 4
    q, k, v = _rand(rng, 1, 1, 1, d), _rand(rng, 1, 1, 1, d), _rand(rng, 1, 1, 1, d)
    o, lse = attention_fwd(q, k, v, False, -1, 0.5)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 0.5 * q[0, 0, 0] @ k[0, 0, 0], rtol=0, atol=1e-15)
    # n = 2: a two-way softmax is a logistic sigmoid of the score difference.
    q, k, v = _rand(rng, 1, 1, 2, d), _rand(rng, 1, 1, 2, d), _rand(rng, 1, 1, 2, d)
    o, lse = attention_fwd(q, k, v, False, -1, 1.0)
    for i in range(2):
        s0 = q[0, 0, i] @ k[0, 0, 0]
        s1 = q[0, 0, i] @ k[0, 0, 1]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(o[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1],
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], np.logaddexp(s0, s1), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# Library routine: torch scaled_dot_product_attention in float64 on the CPU.
# --------------------------------------------------------------------------

def _torch_mask(n, causal, window):
    ones = torch.ones(n, n, dtype=torch.bool)
    if causal:
        m = torch.tril(ones)
        if window >= 0:
            m &= torch.triu(ones, diagonal=-window)
        return m
    if window >= 0:
        return torch.triu(ones, diagonal=-window) & torch.tril(ones, diagonal=window)
    return ones


@pytest.mark.parametrize("causal,window", MODES + [(False, 40), (True, 40)])
@pytest.mark.parametrize("n,d", [(67, 16), (130, 64)])
def test_sdpa_float64(n, d, causal, window):
    rng = np.random.default_rng(n * 31 + d)
    B, H, Hkv = 2, 4, 2
    q, k, v = _rand(rng, B, H, n, d), _rand(rng, B, Hkv, n, d), _rand(rng, B, Hkv, n, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_fwd(q, k, v, causal, window, scale)
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=1)
    mask = _torch_mask(n, causal, window)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    scores = torch.matmul(tq, tk.transpose(-1, -2)) * scale
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", MODES)
def test_probability_rows(causal, window):
    """With V = identity (d = n) the output rows are the probability rows:
    non-negative, zero outside the mask, summing to one."""
    n = 23
    rng = np.random.default_rng(5)
    q, k = _rand(rng, 1, 1, n, 8), _rand(rng, 1, 1, n, 8)
    v = np.eye(n)[None, None]
    p, _ = attention_fwd(q, k, v, causal, window, 0.9)
    p = p[0, 0]
    mask = visible_mask(np.arange(n), n, causal, window)
    assert np.all(p >= 0)
    assert np.all(p[~mask] == 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal,window", MODES)
def test_constant_and_linear_in_v(causal, window):
    n, d = 31, 6
    rng = np.random.default_rng(11)
    q, k = _rand(rng, 1, 2, n, d), _rand(rng, 1, 2, n, d)
    c = rng.standard_normal(d)
    v_const = np.broadcast_to(c, (1, 2, n, d)).copy()
    o, _ = attention_fwd(q, k, v_const, causal, window, 0.4)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)
    v1, v2 = _rand(rng, 1, 2, n, d), _rand(rng, 1, 2, n, d)
    o1, _ = attention_fwd(q, k, v1, causal, window, 0.4)
    o2, _ = attention_fwd(q, k, v2, causal, window, 0.4)
    o12, _ = attention_fwd(q, k, 2.5 * v1 - 0.75 * v2, causal, window, 0.4)
    np.testing.assert_allclose(o12, 2.5 * o1 - 0.75 * o2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", MODES)
def test_key_shift(causal, window):
    """Adding one vector c to every key shifts each score row by scale*q.c:
    the output is unchanged and the log-sum-exp moves by exactly that."""
    n, d, scale = 29, 5, 0.6
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    c = rng.standard_normal(d)
    o, lse = attention_fwd(q, k, v, causal, window, scale)
    o2, lse2 = attention_fwd(q, k + c, v, causal, window, scale)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2 - lse, scale * (q[0, 0] @ c)[None, None], rtol=0, atol=1e-13)


def test_full_mode_permutation_equivariance():
    n, d = 40, 8
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    perm = rng.permutation(n)
    o, lse = attention_fwd(q, k, v, False, -1, 0.3)
    o2, lse2 = attention_fwd(q, k[:, :, perm], v[:, :, perm], False, -1, 0.3)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# Reductions with closed forms.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 17, 64])
def test_window_covering_sequence(n):
    """A window of n-1 or more is no restriction: band == full, causal window
    == causal."""
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 1, 2, n, 8), _rand(rng, 1, 2, n, 8), _rand(rng, 1, 2, n, 8)
    for w in (n - 1, n, 5 * n):
        for causal in (False, True):
            a = attention_fwd(q, k, v, causal, w, 0.35)
            b = attention_fwd(q, k, v, causal, -1, 0.35)
            np.testing.assert_allclose(a[0], b[0], rtol=0, atol=0)
            np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_window_zero(causal):
    """Each row sees only itself: o_i = v_i and lse_i = scale * q_i.k_i."""
    n, d, scale = 33, 8, 0.45
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    o, lse = attention_fwd(q, k, v, causal, 0, scale)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], scale * np.einsum("id,id->i", q[0, 0], k[0, 0]),
                               rtol=0, atol=1e-14)


def _closed_form_count(i, n, causal, window):
    if causal:
        return i + 1 if window < 0 else min(i, window) + 1
    if window < 0:
        return n
    return min(i, window) + min(n - 1 - i, window) + 1


@pytest.mark.parametrize("causal,window", MODES + [(False, 10), (True, 10), (False, 100)])
def test_zero_query_gives_mean_and_log_count(causal, window):
    """Q = 0 makes every visible score 0: o_i is the mean of the visible values
    and lse_i = ln |V(i)|, whose size has a closed form per mask."""
    n, d = 37, 5
    rng = np.random.default_rng(16)
    q = np.zeros((1, 1, n, d))
    k, v = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    o, lse = attention_fwd(q, k, v, causal, window, 1.0)
    for i in range(n):
        cnt = _closed_form_count(i, n, causal, window)
        js = list(_visible_range(i, n, causal, window))
        assert len(js) == cnt
        np.testing.assert_allclose(lse[0, 0, i], math.log(cnt), rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, js].mean(axis=0), rtol=0, atol=1e-14)


def test_gqa_equals_repeated_kv():
    n, d = 45, 8
    rng = np.random.default_rng(17)
    B, H, Hkv = 2, 6, 2
    q, k, v = _rand(rng, B, H, n, d), _rand(rng, B, Hkv, n, d), _rand(rng, B, Hkv, n, d)
    a = attention_fwd(q, k, v, True, 9, 0.3)
    b = attention_fwd(q, np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1),
                      True, 9, 0.3)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=0)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)


def test_rows_subset_and_workers_match_full():
    n, d = 70, 8
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 2, 2, n, d), _rand(rng, 2, 1, n, d), _rand(rng, 2, 1, n, d)
    o, lse = attention_fwd(q, k, v, True, 20, 0.3)
    rows = np.array([0, 5, 69, 33, 34])
    o2, lse2 = attention_fwd(q, k, v, True, 20, 0.3, rows=rows, workers=2, chunk=2)
    np.testing.assert_allclose(o2, o[:, :, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, :, rows], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# Decode through a paged cache.
# --------------------------------------------------------------------------

def _paged(rng, B, Hkv, ps, d, lens):
    pages = [(L + ps - 1) // ps for L in lens]
    P = sum(pages)
    perm = rng.permutation(P)
    table = -np.ones((B, max(pages)), dtype=np.int64)
    kc = rng.standard_normal((P, Hkv, ps, d))
    vc = rng.standard_normal((P, Hkv, ps, d))
    off = 0
    for b in range(B):
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    return kc, vc, table


def test_gather_by_loops():
    rng = np.random.default_rng(19)
    lens = [5, 16, 33]
    kc, vc, table = _paged(rng, 3, 2, 4, 3, lens)
    for b, L in enumerate(lens):
        kb, vb = gather_paged_kv(kc, vc, table, L, b)
        for g in range(2):
            for t in range(L):
                page = table[b][t // 4]
                assert np.array_equal(kb[g, t], kc[page, g, t % 4])
                assert np.array_equal(vb[g, t], vc[page, g, t % 4])


def test_decode_matches_brute_and_last_causal_row():
    rng = np.random.default_rng(20)
    B, H, Hkv, d, ps = 3, 4, 2, 6, 4
    lens = [1, 7, 13]
    kc, vc, table = _paged(rng, B, Hkv, ps, d, lens)
    q = rng.standard_normal((B, H, d))
    o, lse = decode_fwd(q, kc, vc, table, np.array(lens), scale=0.5)
    for b, L in enumerate(lens):
        kb, vb = gather_paged_kv(kc, vc, table, L, b)
        # brute force with the query placed at the last position
        qq = np.zeros((H, L, d))
        qq[:, L - 1] = q[b]
        ob, lb = _brute(qq.tolist(), kb.tolist(), vb.tolist(), True, -1, 0.5)
        np.testing.assert_allclose(o[b], np.array(ob)[:, L - 1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], np.array(lb)[:, L - 1], rtol=0, atol=1e-13)
        # the last row of a causal prefill over the gathered cache
        qf = np.zeros((1, H, L, d))
        qf[0, :, L - 1] = q[b]
        of, lf = attention_fwd(qf, kb[None], vb[None], True, -1, 0.5, rows=[L - 1])
        np.testing.assert_allclose(o[b], of[0, :, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], lf[0, :, 0], rtol=0, atol=1e-14)


def test_decode_page_permutation_invariance():
    rng = np.random.default_rng(21)
    B, H, Hkv, d, ps = 2, 2, 1, 5, 4
    lens = [9, 14]
    kc, vc, table = _paged(rng, B, Hkv, ps, d, lens)
    q = rng.standard_normal((B, H, d))
    o, lse = decode_fwd(q, kc, vc, table, np.array(lens), 0.5)
    P = kc.shape[0]
    perm = rng.permutation(P)          # new physical position of each page
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2, lse2 = decode_fwd(q, kc2, vc2, table2, np.array(lens), 0.5)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(lse2, lse)


# --------------------------------------------------------------------------
# Numbers printed on the pages.
# --------------------------------------------------------------------------

def _count_visible(n, causal, window, chunk=1024):
    total = 0
    for r0 in range(0, n, chunk):
        total += int(visible_mask(np.arange(r0, min(n, r0 + chunk)), n, causal, window).sum())
    return total


def test_page_band_numbers():
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))["band_example"]
    n, w = g["n"], g["w"]
    full = _count_visible(n, False, -1)
    band = _count_visible(n, False, w)
    assert full == n * n
    assert abs(full - g["full_pairs_approx"]) <= g["rel_tol"] * g["full_pairs_approx"]
    assert abs(n * w - g["nw_approx"]) <= g["rel_tol"] * g["nw_approx"]
    # Exact band count n(2w+1) - w(w+1): the page's 1/16 is the one-sided
    # product n*w over n^2; the two-sided band is about twice that.
    assert band == n * (2 * w + 1) - w * (w + 1) == 130_054_144
    assert abs(band / full - 2 * g["claimed_fraction"]) < 0.01


def test_page_score_matrix_sizes():
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))
    for key in ("score_matrix_32k", "score_matrix_64k"):
        e = g[key]
        n = e["n"]
        # full-mode mask size of one row times n rows (counting one row only)
        elems = int(visible_mask([0], n, False, -1).sum()) * n
        assert abs(elems - e["elements_approx"]) <= e["rel_tol"] * e["elements_approx"]
        assert abs(2 * elems - e["fp16_bytes_approx"]) <= e["rel_tol"] * e["fp16_bytes_approx"]
    e = g["score_matrix_64k"]
    traffic = e["hbm_passes"] * 2 * 65536 ** 2
    assert abs(traffic - e["traffic_bytes_approx"]) <= e["rel_tol"] * e["traffic_bytes_approx"]
    t = e["traffic_bytes_approx"] / e["hbm_bandwidth_bytes_per_s"]
    assert abs(t - e["time_s_approx"]) < 1e-9


def test_attention_rows_direct():
    """attention_rows on an explicit small case equals the batch driver."""
    rng = np.random.default_rng(22)
    q, k, v = _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4)
    o, lse = attention_fwd(q, k, v, True, 2, 0.5)
    o2, lse2 = attention_rows(q[0, 0, [3, 8]], k[0, 0], v[0, 0], [3, 8], True, 2, 0.5)
    np.testing.assert_allclose(o2, o[0, 0, [3, 8]], rtol=0, atol=0)
    np.testing.assert_allclose(lse2, lse[0, 0, [3, 8]], rtol=0, atol=0)

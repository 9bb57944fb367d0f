"""The oracle against a tiled online-softmax reference and split-KV merging (CPU).

The tiled reference follows the pages' block algorithm (see
tests/tiled_reference.py); its agreement with the oracle's plain definition
pins the oracle and also shows that skipping out-of-band blocks is exact.
"""

import json
import os

import numpy as np
import pytest

from oracle import attention_fwd, decode_fwd
from tests.tiled_reference import split_merge_attention, tiled_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("block", [1, 7, 64, "n"])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (False, 16),
                                           (False, 37), (True, 16), (True, 37)])
def test_tiled_equals_oracle(block, causal, window):
    n, d = 150, 16
    rng = np.random.default_rng(30)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    b = n if block == "n" else block
    o_t, l_t, _ = tiled_attention(q, k, v, b, causal, window, 0.25)
    o, lse = attention_fwd(q[None, None], k[None, None], v[None, None], causal, window, 0.25)
    np.testing.assert_allclose(o_t, o[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_t, lse[0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,w,block", [(256, 100, 64), (300, 37, 64), (256, 64, 64),
                                       (257, 0, 32), (200, 199, 64)])
def test_skip_is_exact(n, w, block):
    """Skipping out-of-band blocks equals computing them (all -inf blocks)."""
    d = 8
    rng = np.random.default_rng(31)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for causal in (False, True):
        a = tiled_attention(q, k, v, block, causal, w, 0.3, skip=True)
        b = tiled_attention(q, k, v, block, causal, w, 0.3, skip=False)
        np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-13)
        assert not np.isnan(a[0]).any()
        o, lse = attention_fwd(q[None, None], k[None, None], v[None, None], causal, w, 0.3)
        np.testing.assert_allclose(a[0], o[0, 0], rtol=0, atol=1e-12)
        assert a[2] <= b[2]


def test_visited_block_pairs_page_example():
    """Block-pair accounting of the band example (n=32768, w=2048, B=128).

    The page estimates about 34 key blocks per query block and about 8704
    pairs in all; with aligned blocks an interior query block meets exactly
    33 key blocks (2w/B + 1), 8176 pairs in all, which is within the estimate.
    """
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))["block_pairs_example"]
    n, w, B = g["n"], g["w"], g["block"]
    nb = n // B
    assert nb * nb == g["full_block_pairs"]
    per_q = []
    for qb in range(nb):
        q0, q1 = qb * B, qb * B + B - 1
        cnt = sum(1 for kb in range(nb)
                  if not (kb * B + B - 1 < q0 - w or kb * B > q1 + w))
        per_q.append(cnt)
    total = sum(per_q)
    assert max(per_q) == 2 * w // B + 1 <= g["kv_blocks_per_q_block_approx"]
    assert total == 8176 <= g["band_block_pairs_approx"]
    assert abs(g["full_block_pairs"] / total - g["reduction_approx"]) < 0.6
    # The tiled reference visits exactly these blocks on a scaled-down copy.
    n2, w2, B2 = 1024, 64, 8
    rng = np.random.default_rng(32)
    q, k, v = (rng.standard_normal((n2, 4)) for _ in range(3))
    _, _, visited = tiled_attention(q, k, v, B2, False, w2, 0.5)
    nb2 = n2 // B2
    expect = sum(1 for qb in range(nb2) for kb in range(nb2)
                 if not (kb * B2 + B2 - 1 < qb * B2 - w2 or kb * B2 > qb * B2 + B2 - 1 + w2))
    assert visited == expect


@pytest.mark.parametrize("cuts", [[], [1], [5, 6], [16, 32, 48], [3, 50, 51, 60]])
def test_split_merge_equals_decode_oracle(cuts):
    """Any partition of the keys merged by log-sum-exp equals the unsplit result."""
    rng = np.random.default_rng(33)
    L, d, ps = 61, 8, 4
    pages = (L + ps - 1) // ps
    kc = rng.standard_normal((pages, 1, ps, d))
    vc = rng.standard_normal((pages, 1, ps, d))
    table = rng.permutation(pages)[None]
    kc_p = np.empty_like(kc)
    vc_p = np.empty_like(vc)
    kc_p[table[0]] = kc
    vc_p[table[0]] = vc
    q = rng.standard_normal((1, 1, d))
    o, lse = decode_fwd(q, kc_p, vc_p, table, np.array([L]), 0.4)
    kflat = kc[:, 0].reshape(-1, d)[:L]
    vflat = vc[:, 0].reshape(-1, d)[:L]
    o_m, lse_m = split_merge_attention(q[0, 0], kflat, vflat, cuts, 0.4)
    np.testing.assert_allclose(o_m, o[0, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_m, lse[0, 0], rtol=0, atol=1e-13)

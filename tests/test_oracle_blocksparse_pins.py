"""Pins of the block-sparse oracle (CPU): torch scaled_dot_product_attention in
float64 with the expanded element mask built independently (Kronecker product of
the layout with a ones block), reductions to dense and band attention, brute
force on tiny inputs, empty rows and head-specific layouts."""

import math

import numpy as np
import pytest
import torch

from oracle import attention_fwd
from oracle.blocksparse import attention_block_sparse, attention_masked, block_visible_mask
from tests.test_oracle_pins import _brute

MODES = [(False, -1), (True, -1), (False, 20), (True, 9)]


def _layout(rng, Lh, n, bq, bk, density=0.5):
    lay = (rng.random((Lh, -(-n // bq), -(-n // bk))) < density).astype(np.uint8)
    return lay


def _expanded(lay, n, bq, bk):
    """Element mask by Kronecker product with a ones block, cut to n x n."""
    return np.kron(lay != 0, np.ones((bq, bk), dtype=bool))[:n, :n]


def _torch_window(n, causal, window):
    ones = torch.ones(n, n, dtype=torch.bool)
    if causal:
        m = torch.tril(ones)
        return m & torch.triu(ones, diagonal=-window) if window >= 0 else m
    if window >= 0:
        return torch.triu(ones, diagonal=-window) & torch.tril(ones, diagonal=window)
    return ones


@pytest.mark.parametrize("causal,window", MODES)
@pytest.mark.parametrize("bq,bk", [(8, 4), (16, 16), (5, 7)])
def test_against_sdpa_with_expanded_mask(causal, window, bq, bk):
    rng = np.random.default_rng(80 + bq + bk)
    B, H, Hkv, n, d = 2, 4, 2, 45, 8
    q, k, v = (rng.standard_normal(s) for s in ((B, H, n, d), (B, Hkv, n, d), (B, Hkv, n, d)))
    lay = _layout(rng, H, n, bq, bk)
    for h in range(H):            # keep every row non-empty for the library comparison
        lay[h, :, 0] = 1
    o, lse = attention_block_sparse(q, k, v, lay, bq, bk, causal, window, 0.3)
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=1)
    mask = torch.stack([torch.from_numpy(_expanded(lay[h], n, bq, bk)) for h in range(H)])
    mask = mask & _torch_window(n, causal, window)
    ok = mask.any(dim=-1)          # rows with a visible key (causal row 0 may lose it)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=0.3)
    scores = torch.matmul(tq, tk.transpose(-1, -2)) * 0.3
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    okn = ok.numpy()
    for b in range(B):
        np.testing.assert_allclose(o[b][okn], ref.numpy()[b][okn], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b][okn], ref_lse.numpy()[b][okn], rtol=0, atol=1e-12)
        assert np.all(o[b][~okn] == 0) and np.all(lse[b][~okn] == -np.inf)


@pytest.mark.parametrize("causal,window", MODES)
def test_all_blocks_kept_is_dense(causal, window):
    rng = np.random.default_rng(81)
    q, k, v = (rng.standard_normal((1, 2, 50, 6)) for _ in range(3))
    lay = np.ones((1, 4, 7), dtype=np.uint8)
    o, lse = attention_block_sparse(q, k, v, lay, 16, 8, causal, window, 0.5)
    o2, l2 = attention_fwd(q, k, v, causal, window, 0.5)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-13)


def test_band_layout_with_window_is_band_attention():
    """Keeping exactly the blocks that meet the band (the sliding-window skip)
    and masking by the window equals band attention."""
    rng = np.random.default_rng(82)
    n, w, bq, bk = 97, 13, 16, 8
    q, k, v = (rng.standard_normal((1, 1, n, 4)) for _ in range(3))
    nq, nk = -(-n // bq), -(-n // bk)
    lay = np.zeros((1, nq, nk), dtype=np.uint8)
    for a in range(nq):
        for c in range(nk):
            q0, q1 = a * bq, min(n, a * bq + bq) - 1
            k0, k1 = c * bk, min(n, c * bk + bk) - 1
            lay[0, a, c] = not (k1 < q0 - w or k0 > q1 + w)
    o, lse = attention_block_sparse(q, k, v, lay, bq, bk, False, w, 0.7)
    o2, l2 = attention_fwd(q, k, v, False, w, 0.7)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-13)
    assert lay.sum() < nq * nk   # blocks really are skipped


def test_brute_force_tiny():
    rng = np.random.default_rng(83)
    n, d, bq, bk = 6, 3, 2, 3
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    lay = np.array([[[1, 0], [0, 1], [1, 1]]], dtype=np.uint8)
    o, lse = attention_block_sparse(q, k, v, lay, bq, bk, False, -1, 0.9)
    for i in range(n):
        js = [j for j in range(n) if lay[0, i // bq, j // bk]]
        s = {j: 0.9 * math.fsum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in js}
        top = max(s.values())
        z = math.fsum(math.exp(x - top) for x in s.values())
        assert abs(lse[0, 0, i] - (top + math.log(z))) < 1e-13
        for t in range(d):
            ref = math.fsum(math.exp(s[j] - top) / z * v[0, 0, j, t] for j in js)
            assert abs(o[0, 0, i, t] - ref) < 1e-13
    # a full layout matches the dense brute force
    ob, lb = _brute(q[0].tolist(), k[0].tolist(), v[0].tolist(), False, -1, 0.9)
    o1, l1 = attention_block_sparse(q, k, v, np.ones((1, 3, 2), np.uint8), bq, bk, False, -1,
                                    0.9)
    np.testing.assert_allclose(o1[0], ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1[0], lb, rtol=0, atol=1e-13)


def test_empty_rows_and_masked_helper():
    rng = np.random.default_rng(84)
    q, k, v = (rng.standard_normal((5, 4)) for _ in range(3))
    mask = np.zeros((5, 5), dtype=bool)
    mask[1, 2] = True
    o, lse = attention_masked(q, k, v, mask, 1.0)
    assert np.all(o[[0, 2, 3, 4]] == 0) and np.all(np.isneginf(lse[[0, 2, 3, 4]]))
    np.testing.assert_allclose(o[1], v[2], rtol=0, atol=1e-15)   # single key: o = v
    assert abs(lse[1] - q[1] @ k[2]) < 1e-13


def test_shared_layout_equals_repeated_and_mask_helper():
    rng = np.random.default_rng(85)
    q, k, v = (rng.standard_normal((1, 3, 40, 5)) for _ in range(3))
    lay = _layout(rng, 1, 40, 8, 8)
    a = attention_block_sparse(q, k, v, lay, 8, 8, True, -1, 0.4)
    b = attention_block_sparse(q, k, v, np.repeat(lay, 3, axis=0), 8, 8, True, -1, 0.4)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    m = block_visible_mask(np.arange(40), 40, lay[0], 8, 8, True, -1)
    assert np.array_equal(m, _expanded(lay[0], 40, 8, 8) & np.tril(np.ones((40, 40), bool)))

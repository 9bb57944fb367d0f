"""Pins of the fp64 backward oracle (CPU only).

Central finite differences of the forward oracle, torch autograd in float64,
closed forms (window 0, constant V) and invariants (key-shift invariance,
row sums), so that a dropped term, wrong sign, missing scale or transposed
operand in the gradient formulas fails at least one test.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_bwd, attention_bwd_keys, attention_bwd_rows, attention_fwd
from tests.gpu_util import rows_seeing

MODES = [(False, -1), (True, -1), (False, 0), (False, 1), (False, 3), (True, 0), (True, 2)]


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, w, causal, window, scale):
    o, _ = attention_fwd(q, k, v, causal, window, scale)
    return float(np.sum(o * w))


@pytest.mark.parametrize("causal,window", MODES)
def test_finite_differences(causal, window):
    """dL/dx for L = sum(O * W) by central differences, every input element."""
    rng = np.random.default_rng(40)
    B, H, Hkv, n, d = 1, 2, 1, 5, 3
    q, k, v = _rand(rng, B, H, n, d), _rand(rng, B, Hkv, n, d), _rand(rng, B, Hkv, n, d)
    w = _rand(rng, B, H, n, d)
    scale = 0.8
    dq, dk, dv = attention_bwd(q, k, v, w, causal, window, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], w, causal, window, scale)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], w, causal, window, scale)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


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


@pytest.mark.parametrize("causal,window", MODES + [(False, 20), (True, 20)])
def test_torch_autograd_float64(causal, window):
    rng = np.random.default_rng(41)
    B, H, Hkv, n, d = 2, 4, 2, 47, 16
    q, k, v = _rand(rng, B, H, n, d), _rand(rng, B, Hkv, n, d), _rand(rng, B, Hkv, n, d)
    do = _rand(rng, B, H, n, d)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = attention_bwd(q, k, v, do, causal, window, scale)
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    kk = tk.repeat_interleave(H // Hkv, dim=1)
    vv = tv.repeat_interleave(H // Hkv, dim=1)
    mask = _torch_mask(n, causal, window)
    o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=mask, scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-12, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_window_zero_closed_form(causal):
    """Each row sees only itself: O = V, so dQ = dK = 0 and dV = dO."""
    rng = np.random.default_rng(42)
    q, k, v, do = (_rand(rng, 1, 1, 19, 6) for _ in range(4))
    dq, dk, dv = attention_bwd(q, k, v, do, causal, 0, 0.5)
    np.testing.assert_allclose(dq, 0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal,window", MODES)
def test_invariants(causal, window):
    """Adding one vector to every key leaves O unchanged, so the key gradients
    sum to zero; rows of P sum to one, so the value gradients sum to the sum of
    dO; constant V gives O = V, so dQ and dK vanish."""
    rng = np.random.default_rng(43)
    B, H, n, d = 1, 2, 23, 5
    q, k, v, do = (_rand(rng, B, H, n, d) for _ in range(4))
    dq, dk, dv = attention_bwd(q, k, v, do, causal, window, 0.7)
    np.testing.assert_allclose(dk.sum(axis=2), 0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-12)
    c = rng.standard_normal(d)
    vc = np.broadcast_to(c, v.shape).copy()
    dq0, dk0, _ = attention_bwd(q, k, vc, do, causal, window, 0.7)
    np.testing.assert_allclose(dq0, 0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk0, 0, rtol=0, atol=1e-12)


def test_gqa_sums_over_group():
    rng = np.random.default_rng(44)
    B, H, Hkv, n, d = 1, 6, 2, 21, 4
    q, do = _rand(rng, B, H, n, d), _rand(rng, B, H, n, d)
    k, v = _rand(rng, B, Hkv, n, d), _rand(rng, B, Hkv, n, d)
    dq, dk, dv = attention_bwd(q, k, v, do, True, 5, 0.6)
    dq2, dk2, dv2 = attention_bwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), do,
                                  True, 5, 0.6)
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, 3, n, d).sum(axis=2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, 3, n, d).sum(axis=2), rtol=0, atol=1e-13)


def test_linear_in_do_and_chunking():
    rng = np.random.default_rng(45)
    q, k, v, d1, d2 = (_rand(rng, 1, 1, 30, 4) for _ in range(5))
    a = attention_bwd(q, k, v, d1, True, 7, 0.5)
    b = attention_bwd(q, k, v, d2, True, 7, 0.5)
    c = attention_bwd(q, k, v, 2 * d1 - 3 * d2, True, 7, 0.5, chunk=4)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2 * x - 3 * y, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window", MODES + [(False, 20), (True, 20)])
def test_subset_functions_equal_full(causal, window):
    """Row and key subsets give the full computation's values on those rows/keys,
    also when the summed rows are cut down to the ones that see the keys."""
    rng = np.random.default_rng(46)
    H, Hkv, n, d = 4, 2, 41, 8
    q, do = _rand(rng, 1, H, n, d), _rand(rng, 1, H, n, d)
    k, v = _rand(rng, 1, Hkv, n, d), _rand(rng, 1, Hkv, n, d)
    dq, dk, dv = attention_bwd(q, k, v, do, causal, window, 0.35)
    rows = np.array([0, 1, 5, 17, 39, 40])
    np.testing.assert_allclose(attention_bwd_rows(q[0], k[0], v[0], do[0], rows, causal,
                                                  window, 0.35), dq[0][:, rows],
                               rtol=0, atol=1e-13)
    keys = np.array([0, 3, 20, 38, 40])
    a_dk, a_dv = attention_bwd_keys(q[0], k[0], v[0], do[0], keys, np.arange(n), causal,
                                    window, 0.35)
    np.testing.assert_allclose(a_dk, dk[0][:, keys], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a_dv, dv[0][:, keys], rtol=0, atol=1e-13)
    seeing = rows_seeing(keys, n, causal, window)
    b_dk, b_dv = attention_bwd_keys(q[0], k[0], v[0], do[0], keys, seeing, causal, window, 0.35)
    np.testing.assert_allclose(b_dk, a_dk, rtol=0, atol=1e-13)
    np.testing.assert_allclose(b_dv, a_dv, rtol=0, atol=1e-13)


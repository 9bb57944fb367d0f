"""The backward tolerance (tests/bwd_bounds.py) on the CPU.

An fp64 model of the HIP backward's roundings (O stored in bf16, P and dS
rounded to bf16 before the products, lse in fp32) must stay within the
first-order bound u*M (u = 2^-8) of the oracle, hence within the 2u*M the GPU
tests accept; the same model with a planted mistake must break the bound.
"""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import bf16_round, grad_output, prefill_inputs
from oracle import attention_bwd, attention_fwd
from oracle.attention import visible_mask
from tests.bwd_bounds import BOUND_FACTOR, bwd_bounds


def _bf16(x):
    return bf16_round(np.asarray(x, dtype=np.float32))[0].astype(np.float64)


def _model(q, k, v, do, causal, window, scale, mistake=None):
    """Gradients with the HIP path's roundings; ``mistake`` plants one error."""
    H, n, d = q.shape
    G = H // k.shape[0]
    o, lse = attention_fwd(q[None], k[None], v[None], causal, window, scale)
    o = _bf16(o[0])
    lse = lse[0].astype(np.float32).astype(np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mask = visible_mask(np.arange(n), n, causal, window)
    if mistake == "mask_edge":
        mask = mask | np.eye(n, k=1, dtype=bool)  # lets each row see one key too many
    for h in range(H):
        g = h // G
        p = np.where(mask, np.exp(scale * (q[h] @ k[g].T) - lse[h][:, None]), 0.0)
        dp = do[h] @ v[g].T
        dsum = np.sum(o[h] * do[h], axis=1).astype(np.float32)
        if mistake == "no_D":
            dsum = 0.0 * dsum
        ds = _bf16(p * (dp - dsum[:, None]))
        dv[g] += _bf16(p).T @ do[h]
        dk[g] += (1.0 if mistake == "dk_unscaled" else scale) * (ds.T @ q[h])
        dq[h] = scale * (ds @ (k[g] if mistake != "dq_uses_v" else v[g]))
    return dq, dk, dv


CASES = [(2, 1, 7, 128, True, -1), (2, 2, 200, 64, False, -1), (4, 2, 300, 128, True, -1),
         (2, 1, 300, 128, False, 37), (2, 2, 257, 128, True, 20), (2, 1, 100, 128, False, 0)]


@pytest.mark.parametrize("H,Hkv,n,d,causal,window", CASES)
def test_rounding_model_within_bound(H, Hkv, n, d, causal, window):
    inp = prefill_inputs(1, H, Hkv, n, d, seed=50 + n)
    do, _ = grad_output(1, H, n, d, seed=50 + n)
    q, k, v, do = (x[0].astype(np.float64) for x in (inp["q"], inp["k"], inp["v"], do))
    scale = 1.0 / math.sqrt(d)
    ref = attention_bwd(q[None], k[None], v[None], do[None], causal, window, scale)
    got = _model(q, k, v, do, causal, window, scale)
    bounds = bwd_bounds(q, k, v, do, causal, window, scale)
    for r, g, m in zip(ref, got, bounds):
        err = np.abs(g - r[0])
        # first order: within u*M (1% slack for second-order and fp32 terms)
        assert (err <= 2.0 ** -8 * m * 1.01 + 1e-12).all()
        assert (err <= BOUND_FACTOR * m + 1e-6).all()


@pytest.mark.parametrize("mistake", ["no_D", "mask_edge", "dk_unscaled", "dq_uses_v"])
def test_planted_mistakes_break_bound(mistake):
    H, Hkv, n, d, causal, window = 2, 1, 150, 64, True, -1
    inp = prefill_inputs(1, H, Hkv, n, d, seed=60)
    do, _ = grad_output(1, H, n, d, seed=60)
    q, k, v, do = (x[0].astype(np.float64) for x in (inp["q"], inp["k"], inp["v"], do))
    scale = 1.0 / math.sqrt(d)
    ref = attention_bwd(q[None], k[None], v[None], do[None], causal, window, scale)
    got = _model(q, k, v, do, causal, window, scale, mistake=mistake)
    bounds = bwd_bounds(q, k, v, do, causal, window, scale)
    broken = [bool((np.abs(g - r[0]) > BOUND_FACTOR * m + 1e-6).any())
              for r, g, m in zip(ref, got, bounds)]
    assert any(broken), mistake


def test_subset_bounds_equal_full():
    inp = prefill_inputs(1, 4, 2, 90, 32, seed=61)
    do, _ = grad_output(1, 4, 90, 32, seed=61)
    q, k, v, do = (x[0] for x in (inp["q"], inp["k"], inp["v"], do))
    full = bwd_bounds(q, k, v, do, True, 20, 0.2)
    rows, keys = np.array([0, 5, 89]), np.array([3, 40, 88])
    part = bwd_bounds(q, k, v, do, True, 20, 0.2, rows=rows, keys=keys,
                      key_rows=np.arange(3, 90))
    np.testing.assert_allclose(part[0], full[0][:, rows], rtol=1e-12, atol=0)
    np.testing.assert_allclose(part[1], full[1][:, keys], rtol=1e-12, atol=0)
    np.testing.assert_allclose(part[2], full[2][:, keys], rtol=1e-12, atol=0)

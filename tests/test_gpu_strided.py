"""GPU parity of the strided forward (fa_fwd_strided): the (batch, seq, heads,
dim) layout and q/k/v views into one packed qkv tensor must give exactly the
bits of fa_fwd on contiguous copies (same tiles, same arithmetic), and match
the oracle."""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import prefill_inputs
from oracle import attention_fwd
from tests.gpu_util import TOL_BF16, compare, prefill_device, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,Hkv,n,d,causal,window", [
    (2, 4, 2, 300, 128, 1, -1),
    (1, 8, 2, 1000, 128, 0, 100),
    (2, 4, 4, 129, 64, 0, -1),
    (1, 2, 1, 2049, 128, 1, 300),
])
def test_bshd_equals_contiguous_bitwise_and_oracle(B, H, Hkv, n, d, causal, window):
    import torch
    import io_aware_exact_fa_amd as fa
    say(f"bshd B{B} H{H} Hkv{Hkv} n{n} d{d} c{causal} w{window}")
    inp = prefill_inputs(B, H, Hkv, n, d, seed=7000 + n)
    q, k, v = prefill_device(inp)
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = fa.flash_attn_fwd(q, k, v, causal=causal, window=window, scale=scale)
    qs, ks, vs = (t.transpose(1, 2).contiguous() for t in (q, k, v))  # [B, n, heads, d]
    o, lse = fa.flash_attn_strided(qs, ks, vs, causal=causal, window=window, scale=scale,
                                   layout="bshd")
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, n, H, d)
    assert torch.equal(o.transpose(1, 2), o_ref) and torch.equal(lse, l_ref)
    o_np = o.transpose(1, 2).float().cpu().numpy()
    oo, ll = attention_fwd(inp["q"], inp["k"], inp["v"], causal, window, scale)
    compare(o_np, lse.cpu().numpy(), oo, ll, TOL_BF16, "bshd vs oracle")


def test_packed_qkv_views_bitwise():
    """q, k, v as views into one [B, n, 3, H, d] tensor (row stride 3*H*d)."""
    import torch
    import io_aware_exact_fa_amd as fa
    B, H, n, d = 2, 8, 777, 128
    g = torch.Generator(device="cpu").manual_seed(71)
    qkv = torch.randn((B, n, 3, H, d), generator=g).to(torch.bfloat16).cuda()
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]     # [B, n, H, d] views
    o, lse = fa.flash_attn_strided(q, k, v, causal=True, layout="bshd")
    qc, kc, vc = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    o2, l2 = fa.flash_attn_fwd(qc, kc, vc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.transpose(1, 2), o2) and torch.equal(lse, l2)


def test_bhsd_views_with_padding_bitwise():
    """Rows padded to a larger stride (a [B, H, n, d + 64] buffer cut to d)."""
    import torch
    import io_aware_exact_fa_amd as fa
    B, H, n, d = 1, 4, 500, 128
    g = torch.Generator(device="cpu").manual_seed(72)
    big = torch.randn((3, B, H, n, d + 64), generator=g).to(torch.bfloat16).cuda()
    q, k, v = big[0, ..., :d], big[1, ..., :d], big[2, ..., :d]
    o, lse = fa.flash_attn_strided(q, k, v, causal=False, window=70)
    o2, l2 = fa.flash_attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=False,
                               window=70)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)

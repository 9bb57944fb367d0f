"""fa_decode_noalloc (the decode entry point that allocates nothing: its split
partials live in the library's static device array) against fa_decode with a
caller workspace and against the oracle, on two calls in a row -- the second
with a smaller batch, shorter sequences and the other head dim -- so the
second call runs over what the first left in the array."""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import decode_inputs
from oracle import decode_fwd
from tests.gpu_util import TOL_BF16, compare, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu


def _both(meta, max_len):
    import torch
    import io_aware_exact_fa_amd as fa
    q, kc, vc = dev_bf16(meta["q_bits"]), dev_bf16(meta["kcache_bits"]), dev_bf16(meta["vcache_bits"])
    pt, sl = dev_i32(meta["page_table"]), dev_i32(meta["seqlens"])
    B, H, d = q.shape
    Hkv = kc.shape[1]
    scale = 1.0 / math.sqrt(d)
    o_na = torch.empty_like(q)
    l_na = torch.empty((B, H), dtype=torch.float32, device=q.device)
    fa.fa_decode_noalloc(q, kc, vc, pt, sl, o_na, l_na, B, H, Hkv, d, kc.shape[0], 16,
                         pt.shape[1], max_len, scale)
    o_ws, l_ws = fa.flash_decode(q, kc, vc, pt, sl, max_seqlen=max_len, scale=scale)
    torch.cuda.synchronize()
    return (o_na.float().cpu().numpy(), l_na.cpu().numpy(),
            o_ws.float().cpu().numpy(), l_ws.cpu().numpy(), scale)


def test_noalloc_decode_two_calls_match_workspace_decode_and_oracle():
    # First call: 16 sequences of up to 9000 tokens (several splits each).
    say("noalloc decode call 1: B16 H32 Hkv8 d128 L~U[1000,9000]")
    m1 = decode_inputs(16, 32, 8, 128, 16, 1000, 9000, seed=7001)
    o1, l1, w1, wl1, sc1 = _both(m1, 9000)
    assert np.array_equal(o1, w1) and np.array_equal(l1, wl1)
    r1, rl1 = decode_fwd(m1["q"], m1["kcache"], m1["vcache"], m1["page_table"], m1["seqlens"],
                         sc1)
    compare(o1, l1, r1, rl1, TOL_BF16, "noalloc call 1")
    # Second call, smaller: 3 sequences, other heads and head dim, 1 to 700 tokens.
    say("noalloc decode call 2: B3 H8 Hkv2 d64 L in {1, 333, 700}")
    m2 = decode_inputs(3, 8, 2, 64, 16, 1, 700, seed=7002, seqlens=[1, 333, 700])
    o2, l2, w2, wl2, sc2 = _both(m2, 700)
    assert np.array_equal(o2, w2) and np.array_equal(l2, wl2)
    r2, rl2 = decode_fwd(m2["q"], m2["kcache"], m2["vcache"], m2["page_table"], m2["seqlens"],
                         sc2)
    compare(o2, l2, r2, rl2, TOL_BF16, "noalloc call 2")


def test_noalloc_decode_rejects_partials_beyond_the_array():
    import torch
    import io_aware_exact_fa_amd as fa
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_noalloc(x, x, x, x, x, x, x, 128, 32, 8, 128, 1, 16, 2048, 32768, 0.1)
    assert e.value.status == -4

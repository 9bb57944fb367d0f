"""Decode over degenerate metadata: the device-side guards of fa_decode and
fa_decode_fp8, each checked against what the header promises.

  * a sequence of length 0 gives o = 0 and lse = -inf exactly;
  * a length past min(max_seqlen, max_pages * 16) is clamped to it;
  * a page id outside [0, num_pages) leaves that page's 16 tokens out.

Decode has no position-dependent mask, so leaving a page out equals decoding
the same cache through a table without that page (later pages moved up one
slot): the expected values are the oracle's on such a table.
"""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import decode_fp8_inputs, decode_inputs
from oracle import decode_fwd
from oracle.fp8 import decode_fwd_fp8
from tests.gpu_util import TOL_BF16, compare, dev_bf16, dev_f32, dev_i32, say

pytestmark = pytest.mark.gpu

B, H, HKV, D, MAX_LEN = 4, 8, 2, 128, 100
LENS = [0, 64, 70, 100]          # lengths the cache and table are built for
DEV_LENS = [0, 64, 70, 10 ** 6]  # lengths passed to the kernel


def _tables(meta):
    """(table the kernel gets, table and lengths the oracle gets)."""
    t = meta["page_table"].copy()
    P = meta["num_pages"]
    kernel = t.copy()
    kernel[1, 1] = -1  # sequence 1: its second page is left out
    kernel[2, 2] = P   # sequence 2: its third page is left out
    expect = -np.ones_like(t)
    expect[1, :3] = t[1, [0, 2, 3]]
    expect[2, :4] = t[2, [0, 1, 3, 4]]
    expect[3] = t[3]
    # sequence 3 is clamped to min(MAX_LEN, max_pages * 16) = 100 tokens
    assert t.shape[1] * 16 >= MAX_LEN
    lens = np.array([0, 48, 54, MAX_LEN], dtype=np.int32)
    return kernel, expect, lens


def _check(o, lse, o_ref, lse_ref, label):
    """Sequence 0 exactly; sequences 1.. against the oracle (which has no
    meaning for an empty sequence and is given sequences 1.. only)."""
    assert np.all(o[0] == 0.0), f"{label}: length 0 must give o = 0"
    assert np.all(np.isneginf(lse[0])), f"{label}: length 0 must give lse = -inf"
    compare(o[1:], lse[1:], o_ref, lse_ref, TOL_BF16, label)


def test_decode_guards_bf16():
    import torch
    import io_aware_exact_fa_amd as fa
    say("decode guards bf16")
    meta = decode_inputs(B, H, HKV, D, 16, 0, MAX_LEN, seed=71, seqlens=LENS)
    kernel_t, expect_t, lens = _tables(meta)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.flash_decode(dev_bf16(meta["q_bits"]), dev_bf16(meta["kcache_bits"]),
                             dev_bf16(meta["vcache_bits"]), dev_i32(kernel_t),
                             dev_i32(np.array(DEV_LENS, dtype=np.int32)), max_seqlen=MAX_LEN,
                             scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = decode_fwd(meta["q"][1:], meta["kcache"], meta["vcache"], expect_t[1:],
                                lens[1:], scale)
    _check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "decode guards bf16")


def test_decode_guards_fp8():
    import torch
    import io_aware_exact_fa_amd as fa
    say("decode guards fp8")
    meta = decode_fp8_inputs(B, H, HKV, D, 16, 0, MAX_LEN, seed=72, seqlens=LENS)
    kernel_t, expect_t, lens = _tables(meta)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.flash_decode_fp8(dev_bf16(meta["q_bits"]),
                                 torch.from_numpy(meta["kcache8"]).to("cuda"),
                                 torch.from_numpy(meta["vcache8"]).to("cuda"),
                                 dev_f32(meta["k_scale"]), dev_f32(meta["v_scale"]),
                                 dev_i32(kernel_t), dev_i32(np.array(DEV_LENS, dtype=np.int32)),
                                 MAX_LEN, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = decode_fwd_fp8(meta["q"][1:], meta["kcache8"], meta["vcache8"],
                                    meta["k_scale"], meta["v_scale"], expect_t[1:], lens[1:],
                                    scale)
    _check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "decode guards fp8")

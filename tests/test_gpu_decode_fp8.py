"""GPU parity of decode over an FP8 (E4M3) cache (fa_decode_fp8) against the
oracle (bytes decoded from the format's fields, per-head scales applied in
fp64).  Small batches over every output, the 64-sequence workload on sampled
sequences, and the bf16 decode over the same dequantised values."""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import decode_fp8_inputs
from oracle.fp8 import decode_fwd_fp8, e4m3_to_float
from tests.gpu_util import TOL_BF16, compare, dev_bf16, dev_f32, dev_i32, say

pytestmark = pytest.mark.gpu


def run_fp8(meta, Hkv, scale):
    import torch
    import io_aware_exact_fa_amd as fa
    q = dev_bf16(meta["q_bits"])
    kc = torch.from_numpy(meta["kcache8"]).to("cuda")
    vc = torch.from_numpy(meta["vcache8"]).to("cuda")
    o, lse = fa.flash_decode_fp8(q, kc, vc, dev_f32(meta["k_scale"]), dev_f32(meta["v_scale"]),
                                 dev_i32(meta["page_table"]), dev_i32(meta["seqlens"]),
                                 int(meta["seqlens"].max()), scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


# (B, H, Hkv, min_len, max_len, seqlens)
SMALL = [
    (1, 1, 1, 1, 1, None),
    (3, 8, 2, 1, 100, [1, 17, 100]),
    (4, 16, 8, 500, 3000, None),
    (2, 16, 1, 1000, 2000, None),
    (3, 12, 4, 10, 700, None),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"fp8dec{i}" for i in range(len(SMALL))])
def test_decode_fp8_small(case):
    B, H, Hkv, lo, hi, lens = case
    say(f"decode fp8 {case}")
    meta = decode_fp8_inputs(B, H, Hkv, 128, 16, lo, hi, seed=6000 + B + H, seqlens=lens)
    scale = 1.0 / math.sqrt(128)
    o, lse = run_fp8(meta, Hkv, scale)
    o_ref, lse_ref = decode_fwd_fp8(meta["q"], meta["kcache8"], meta["vcache8"],
                                    meta["k_scale"], meta["v_scale"], meta["page_table"],
                                    meta["seqlens"], scale)
    compare(o, lse, o_ref, lse_ref, TOL_BF16, f"decode fp8 {case}")


def test_decode_fp8_matches_bf16_decode_of_same_values():
    """The E4M3 values times a power-of-two scale are exact in bf16: the bf16
    decode over those values must agree closely (same math, other loads)."""
    import torch
    import io_aware_exact_fa_amd as fa
    meta = decode_fp8_inputs(4, 16, 4, 128, 16, 200, 1500, seed=6100)
    meta["k_scale"] = np.full(4, 0.125, np.float32)
    meta["v_scale"] = np.full(4, 0.25, np.float32)
    o8, l8 = run_fp8(meta, 4, 0.1)
    kvals = (e4m3_to_float(meta["kcache8"]) * 0.125).astype(np.float32)
    vvals = (e4m3_to_float(meta["vcache8"]) * 0.25).astype(np.float32)
    kb = torch.from_numpy(kvals).to(torch.bfloat16).to("cuda")
    vb = torch.from_numpy(vvals).to(torch.bfloat16).to("cuda")
    o, lse = fa.flash_decode(dev_bf16(meta["q_bits"]), kb, vb, dev_i32(meta["page_table"]),
                             dev_i32(meta["seqlens"]), int(meta["seqlens"].max()), scale=0.1)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o8, o.float().cpu().numpy(), rtol=0, atol=1e-2)
    np.testing.assert_allclose(l8, lse.cpu().numpy(), rtol=0, atol=1e-4)


def test_decode_fp8_full_size_sampled():
    """The paged decode workload (64 sequences, lengths U[1024, 32768]) with
    E4M3 caches; eight sequences checked against the oracle."""
    B, H, Hkv = 64, 32, 8
    say("decode fp8 full B=64")
    meta = decode_fp8_inputs(B, H, Hkv, 128, 16, 1024, 32768, seed=5)
    scale = 1.0 / math.sqrt(128)
    o, lse = run_fp8(meta, Hkv, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    picks = [0, 1, 17, 31, 40, 52, 62, 63]
    o_ref, lse_ref = decode_fwd_fp8(meta["q"], meta["kcache8"], meta["vcache8"],
                                    meta["k_scale"], meta["v_scale"], meta["page_table"],
                                    meta["seqlens"], scale, batches=picks)
    compare(o[picks], lse[picks], o_ref[picks], lse_ref[picks], TOL_BF16, "decode fp8 full")

"""GPU parity of decode over an FP8 (E4M3) cache (fa_decode_fp8) against the
oracle (bytes decoded from the format's fields, per-head scales applied in
fp64).  Small batches over every output, the 64-sequence workload on sampled
sequences, and the bf16 decode over the same dequantised values."""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import decode_fp8_inputs
from oracle.fp8 import decode_fwd_fp8, e4m3_to_float
from tests.gpu_util import (TOL_BF16, compare, decode_oracle_all, dev_bf16, dev_f32,
                             dev_i32, say)

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


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", SMALL, ids=[f"fp8dec{i}" for i in range(len(SMALL))])
def test_decode_fp8_small(case, d):
    B, H, Hkv, lo, hi, lens = case
    say(f"decode fp8 {case} d{d}")
    meta = decode_fp8_inputs(B, H, Hkv, d, 16, lo, hi, seed=6000 + B + H + d, seqlens=lens)
    scale = 1.0 / math.sqrt(d)
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


@pytest.mark.parametrize("d", [128, 64])
def test_decode_fp8_full_size_all_outputs(d):
    """The paged decode workload (64 sequences, lengths U[1024, 32768]) with
    E4M3 caches; every output of every sequence against the oracle."""
    B, H, Hkv = 64, 32, 8
    say(f"decode fp8 full B=64 d{d}")
    meta = decode_fp8_inputs(B, H, Hkv, d, 16, 1024, 32768, seed=5)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fp8(meta, Hkv, scale)
    o_ref, lse_ref = decode_oracle_all(meta, scale, fp8=True)
    compare(o, lse, o_ref, lse_ref, TOL_BF16, f"decode fp8 full d{d} (all 64 sequences)")


@pytest.mark.parametrize("ks", [0.0, -0.25])
def test_decode_fp8_zero_and_negative_key_scale(ks):
    """A head whose key scale is zero (quantised from an all-zero cache) sees
    all scores 0 and a uniform softmax; a negative scale flips its keys.  The
    other heads keep their scales.  Short tail pages and several splits make
    the masked tokens meet the scale."""
    B, H, Hkv = 3, 8, 4
    lens = [17, 700, 3001]
    say(f"decode fp8 key scale {ks}")
    meta = decode_fp8_inputs(B, H, Hkv, 128, 16, 1, 3001, seed=6200, seqlens=lens)
    meta["k_scale"] = meta["k_scale"].copy()
    meta["k_scale"][1] = ks
    meta["v_scale"] = meta["v_scale"].copy()
    meta["v_scale"][2] = 0.0
    scale = 1.0 / math.sqrt(128)
    o, lse = run_fp8(meta, Hkv, scale)
    o_ref, lse_ref = decode_fwd_fp8(meta["q"], meta["kcache8"], meta["vcache8"],
                                    meta["k_scale"], meta["v_scale"], meta["page_table"],
                                    meta["seqlens"], scale)
    compare(o, lse, o_ref, lse_ref, TOL_BF16, f"decode fp8 k_scale[1]={ks}, v_scale[2]=0")
    if ks == 0.0:
        # uniform softmax over L keys: lse = ln L for the two query heads of KV head 1
        want = np.repeat(np.log(np.array(lens, dtype=np.float64))[:, None], 2, axis=1)
        np.testing.assert_allclose(lse[:, 2:4], want, rtol=0, atol=1e-5)


def test_decode_fp8_split_count_multiple_of_8():
    """The padded split grid with an E4M3 cache: 16 sequences up to 30000
    tokens, 32 splits of 60 pages per row (launched as 33), 15 pages per wave
    (every position of the six-page key/value rotation); every output."""
    lens = [30000, 1024, 29999, 960, 15000, 7681, 23040, 28801, 3000, 1, 12345, 29000,
            17, 26000, 4097, 19200]
    say("decode fp8 B16 H32 Hkv8 d128 max_len 30000 (32 splits, padded grid)")
    meta = decode_fp8_inputs(16, 32, 8, 128, 16, 1, 30000, seed=72, seqlens=lens)
    scale = 1.0 / math.sqrt(128)
    o, lse = run_fp8(meta, 8, scale)
    o_ref, lse_ref = decode_oracle_all(meta, scale, fp8=True)
    compare(o, lse, o_ref, lse_ref, TOL_BF16, "decode fp8 B16 padded split grid")

"""GPU parity of paged flash-decoding (fa_decode through the C ABI) against the oracle."""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import decode_inputs
from oracle import decode_fwd
from tests.gpu_util import TOL_BF16, compare, decode_oracle_all, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu


def _device(meta):
    return (dev_bf16(meta["q_bits"]), dev_bf16(meta["kcache_bits"]),
            dev_bf16(meta["vcache_bits"]), dev_i32(meta["page_table"]),
            dev_i32(meta["seqlens"]))


def _run(meta, max_len, dev=None):
    import torch
    import io_aware_exact_fa_amd as fa
    q, kc, vc, pt, sl = dev if dev is not None else _device(meta)
    o, lse = fa.flash_decode(q, kc, vc, pt, sl, max_seqlen=max_len,
                             scale=1.0 / math.sqrt(q.shape[-1]))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


SMALL = [  # (B, H, Hkv, lengths)
    (6, 8, 2, [1, 15, 16, 17, 511, 513]),
    (4, 4, 4, [512, 1, 1000, 33]),
    (3, 6, 2, [100, 2000, 31]),
    (2, 16, 1, [1500, 64]),
    (5, 32, 8, [1024, 1025, 4096, 3000, 700]),
]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}H{c[1]}kv{c[2]}" for c in SMALL])
def test_decode_small(case, d):
    B, H, Hkv, lens = case
    say(f"case decode B{B} H{H} Hkv{Hkv} d{d} lens {lens}")
    max_len = max(lens) + 40
    meta = decode_inputs(B, H, Hkv, d, 16, 1, max_len, seed=50 + H + d, seqlens=lens)
    o, lse = _run(meta, max_len)
    o_ref, lse_ref = decode_fwd(meta["q"], meta["kcache"], meta["vcache"],
                                meta["page_table"], meta["seqlens"], 1.0 / math.sqrt(d))
    compare(o, lse, o_ref, lse_ref, TOL_BF16, f"decode B{B}H{H}kv{Hkv} d{d}")


def test_decode_page_permutation_bitwise():
    """Moving pages in memory (and the table with them) changes no bit."""
    B, H, Hkv = 3, 8, 2
    lens = [300, 77, 1030]
    meta = decode_inputs(B, H, Hkv, 128, 16, 1, 1100, seed=61, seqlens=lens)
    o1, l1 = _run(meta, 1100)
    rng = np.random.default_rng(62)
    P = meta["num_pages"]
    perm = rng.permutation(P)
    kb = np.empty_like(meta["kcache_bits"])
    vb = np.empty_like(meta["vcache_bits"])
    kb[perm] = meta["kcache_bits"]
    vb[perm] = meta["vcache_bits"]
    t = meta["page_table"]
    t2 = np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32)
    meta2 = dict(meta, kcache_bits=kb, vcache_bits=vb, page_table=t2)
    o2, l2 = _run(meta2, 1100)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("d", [128, 64])
def test_decode_full_size_all_outputs(d):
    """The paged decode workload: 64 sequences, 32 query / 8 KV heads, lengths
    uniform in [1024, 32768], 16-token pages behind a permuted table; every
    output of every sequence against the oracle (d = 128 is the benchmarked
    configuration; d = 64 the same batch at the other supported head dim)."""
    say(f"case decode B64 H32 Hkv8 d{d} L~U[1024,32768]")
    meta = decode_inputs(64, 32, 8, d, 16, 1024, 32768, seed=5, with_values=False)
    o, lse = _run(meta, 32768)
    o_ref, lse_ref = decode_oracle_all(meta, 1.0 / math.sqrt(d))
    compare(o, lse, o_ref, lse_ref, TOL_BF16, f"decode full size d{d} (all 64 sequences)")


def test_decode_split_count_multiple_of_8():
    """16 sequences up to 30000 tokens: 60-page splits, 32 of them per
    (sequence, KV head) row, so the launch adds one empty split per row (a
    split count that is a multiple of 8 is padded).  The longest sequence
    fills the last real split; every output against the oracle."""
    import io_aware_exact_fa_amd as fa
    lens = [30000, 1024, 29999, 960, 15000, 7681, 23040, 28801, 3000, 1, 12345, 29000,
            17, 26000, 4097, 19200]
    max_len = 30000
    assert fa.fa_decode_workspace_bytes(16, 32, max_len, 128) == \
        16 * 32 * 32 * (128 + 1) * 4   # 32 splits of 60 pages per row
    say(f"case decode B16 H32 Hkv8 d128 max_len {max_len} (32 splits, padded grid)")
    meta = decode_inputs(16, 32, 8, 128, 16, 1, max_len, seed=71, seqlens=lens,
                         with_values=False)
    o, lse = _run(meta, max_len)
    o_ref, lse_ref = decode_oracle_all(meta, 1.0 / math.sqrt(128))
    compare(o, lse, o_ref, lse_ref, TOL_BF16, "decode B16 padded split grid")

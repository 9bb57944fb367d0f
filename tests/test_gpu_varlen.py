"""GPU parity of the ragged-batch forward (fa_fwd_varlen) and of chunked prefill
over paged histories (fa_fwd_paged) against the oracle, through the C ABI.

Small cases are compared over every output; the full workloads on sampled
rows of sampled sequences, which the oracle computes one by one.
"""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import paged_prefill_inputs, varlen_inputs
from oracle import attention_rows, gather_paged_kv
from oracle.varlen import attention_paged_prefill, attention_varlen
from tests.gpu_util import TOL_BF16, compare, dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu


def run_varlen(inp, max_seqlen, causal, window, scale):
    import torch
    import io_aware_exact_fa_amd as fa
    q, k, v = (dev_bf16(inp[x + "_bits"]) for x in ("q", "k", "v"))
    o, lse = fa.flash_attn_varlen(q, k, v, dev_i32(inp["cu_seqlens"]), max_seqlen,
                                  causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


# (lengths, H, Hkv, d, causal, window)
VARLEN = [
    ([1], 1, 1, 128, 0, -1),
    ([5, 0, 300, 1, 129], 4, 2, 128, 1, -1),
    ([128, 127, 256, 2], 2, 1, 128, 0, -1),
    ([700, 33, 64], 2, 2, 64, 0, 37),
    ([600, 512, 65], 4, 1, 128, 1, 100),
    ([1000, 200, 0, 450], 8, 2, 128, 1, -1),
    ([333, 999], 2, 1, 64, 1, 0),
]


@pytest.mark.parametrize("case", VARLEN, ids=[f"varlen{i}" for i in range(len(VARLEN))])
def test_varlen_small(case):
    lengths, H, Hkv, d, causal, window = case
    say(f"varlen lengths={lengths} H={H} Hkv={Hkv} d={d} causal={causal} w={window}")
    inp = varlen_inputs(H, Hkv, d, seed=3000 + sum(lengths), lengths=lengths)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_varlen(inp, max(lengths), causal, window, scale)
    o_ref, lse_ref = attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], causal,
                                      window, scale)
    compare(o, lse, o_ref, lse_ref, TOL_BF16, f"varlen {lengths}")


def run_paged(inp, causal, window, scale):
    import torch
    import io_aware_exact_fa_amd as fa
    q = dev_bf16(inp["q_bits"])
    kc, vc = dev_bf16(inp["kcache_bits"]), dev_bf16(inp["vcache_bits"])
    o, lse = fa.flash_attn_paged(q, kc, vc, dev_i32(inp["page_table"]),
                                 dev_i32(inp["cu_seqlens_q"]), dev_i32(inp["seqlens_k"]),
                                 int(inp["chunk"].max()), causal=causal, window=window,
                                 scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


# (B, H, Hkv, d, prefix range, chunk range, causal, window, seed)
PAGED = [
    (1, 1, 1, 128, (0, 0), (1, 1), 1, -1, 1),          # one token, no history
    (3, 4, 2, 128, (0, 40), (1, 20), 1, -1, 2),
    (4, 8, 2, 128, (100, 700), (1, 1), 1, -1, 3),      # decode steps
    (3, 4, 1, 128, (0, 0), (50, 300), 1, -1, 4),       # no prefix: plain prefill
    (5, 4, 4, 128, (200, 900), (64, 300), 1, -1, 5),
    (3, 2, 1, 64, (10, 500), (5, 130), 1, 50, 6),
    (2, 4, 2, 128, (300, 600), (100, 200), 0, -1, 7),   # chunk sees all keys
    (2, 4, 2, 128, (300, 600), (100, 200), 0, 33, 8),
    (2, 4, 2, 64, (100, 700), (50, 300), 1, -1, 9),    # d 64, 8-wave workgroups
]


@pytest.mark.parametrize("case", PAGED, ids=[f"paged{i}" for i in range(len(PAGED))])
def test_paged_small(case):
    B, H, Hkv, d, pr, cr, causal, window, seed = case
    say(f"paged B={B} H={H} Hkv={Hkv} d={d} prefix={pr} chunk={cr} causal={causal} w={window}")
    inp = paged_prefill_inputs(B, H, Hkv, d, 16, pr[0], pr[1], cr[0], cr[1], seed=4000 + seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_paged(inp, causal, window, scale)
    o_ref, lse_ref = attention_paged_prefill(inp["q"], inp["kcache"], inp["vcache"],
                                             inp["page_table"], inp["cu_seqlens_q"],
                                             inp["seqlens_k"], causal, window, scale)
    compare(o, lse, o_ref, lse_ref, TOL_BF16, f"paged {case}")


def test_paged_page_permutation_is_bitwise_invariant():
    """Moving pages to other physical slots (same table contents' meaning)
    leaves every output bit unchanged."""
    inp = paged_prefill_inputs(3, 4, 2, 128, 16, 50, 400, 30, 100, seed=4100)
    a = run_paged(inp, 1, -1, 0.09)
    P = inp["num_pages"]
    perm = np.random.default_rng(1).permutation(P)
    inv = np.empty(P, dtype=np.int64)
    inv[perm] = np.arange(P)
    moved = dict(inp)
    moved["kcache_bits"] = inp["kcache_bits"][perm]
    moved["vcache_bits"] = inp["vcache_bits"][perm]
    t = inp["page_table"].copy()
    t[t >= 0] = inv[t[t >= 0]]
    moved["page_table"] = t
    b = run_paged(moved, 1, -1, 0.09)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [0, 1], ids=["noncausal", "causal"])
def test_paged_eight_and_four_wave_workgroups_agree_bitwise(causal):
    """Chunks over pages run 8-wave workgroups (256 query rows, two waves per
    page) when rows see 16K keys or more (no window) and 4-wave ones (one
    wave per page) otherwise.  A window of 16000 over sequences shorter than
    that leaves the visible set unchanged but takes the 4-wave launch; each
    wave visits the same key tiles in the same order, so the outputs must
    agree bit for bit."""
    inp = paged_prefill_inputs(3, 4, 2, 128, 16, 200, 900, 300, 700, seed=4200 + causal)
    assert int(inp["seqlens_k"].max()) < 16000
    a = run_paged(inp, causal, -1, 0.09)
    b = run_paged(inp, causal, 16000, 0.09)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# Full-size workloads.
VARLEN_FULL = dict(B=16, H=32, Hkv=8, d=128, min_len=1024, max_len=16384, seed=11)
PAGED_FULL = dict(B=16, H=32, Hkv=8, d=128, prefix=(1024, 32768), chunk=(2048, 2048), seed=12)


def test_varlen_full_size_sampled():
    c = VARLEN_FULL
    say(f"varlen full {c}")
    inp = varlen_inputs(c["H"], c["Hkv"], c["d"], seed=c["seed"], B=c["B"],
                        min_len=c["min_len"], max_len=c["max_len"])
    scale = 1.0 / math.sqrt(c["d"])
    o, lse = run_varlen(inp, int(inp["lengths"].max()), 1, -1, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    cu = inp["cu_seqlens"]
    G = c["H"] // c["Hkv"]
    rng = np.random.default_rng(5)
    for b in (0, 7, c["B"] - 1):
        s0, L = int(cu[b]), int(inp["lengths"][b])
        rows = np.unique(np.concatenate([[0, 1, 127, 128, L - 1], rng.integers(0, L, 6)]))
        for h in (0, c["H"] - 1):
            g = h // G
            o_ref, l_ref = attention_rows(inp["q"][h, s0 + rows], inp["k"][g, s0:s0 + L],
                                          inp["v"][g, s0:s0 + L], rows, True, -1, scale)
            compare(o[h, s0 + rows], lse[h, s0 + rows], o_ref, l_ref, TOL_BF16,
                    f"varlen full b{b} h{h}")


def test_paged_full_size_sampled():
    c = PAGED_FULL
    say(f"paged full {c}")
    inp = paged_prefill_inputs(c["B"], c["H"], c["Hkv"], c["d"], 16, c["prefix"][0],
                               c["prefix"][1], c["chunk"][0], c["chunk"][1], seed=c["seed"])
    scale = 1.0 / math.sqrt(c["d"])
    o, lse = run_paged(inp, 1, -1, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    cu = inp["cu_seqlens_q"]
    G = c["H"] // c["Hkv"]
    rng = np.random.default_rng(6)
    for b in (0, 9, c["B"] - 1):
        L, C = int(inp["seqlens_k"][b]), int(inp["chunk"][b])
        kb, vb = gather_paged_kv(inp["kcache"], inp["vcache"], inp["page_table"], L, b)
        rows = np.unique(np.concatenate([[0, 1, 127, 128, C - 1], rng.integers(0, C, 6)]))
        for h in (0, c["H"] - 1):
            g = h // G
            o_ref, l_ref = attention_rows(inp["q"][h, cu[b] + rows], kb[g], vb[g],
                                          L - C + rows, True, -1, scale)
            compare(o[h, cu[b] + rows], lse[h, cu[b] + rows], o_ref, l_ref, TOL_BF16,
                    f"paged full b{b} h{h}")

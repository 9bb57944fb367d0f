"""GPU parity of the block-sparse forward (fa_fwd_blocksparse) against the oracle.

Small shapes over every output (rows whose kept blocks hold no visible key
must come back as o = 0, lse = -inf exactly); the band layout with the window
must reproduce fa_fwd with that window bit for bit (same tiles, same
arithmetic); a 32768-token layout with local, global and random blocks over
two whole heads and one row of every block of every head.
"""

import math

import numpy as np
import pytest

from io_aware_exact_fa_amd.inputs import block_layout, prefill_inputs
from oracle.blocksparse import attention_block_sparse
from tests.gpu_util import (TOL_BF16, compare, dev_bf16, oracle_rows_parallel,
                             prefill_device, say, stratified_rows)

pytestmark = pytest.mark.gpu


def run_bs(inp, layout, block_k, causal, window, scale, dev=None):
    import torch
    import io_aware_exact_fa_amd as fa
    q, k, v = dev if dev is not None else prefill_device(inp)
    lay = torch.from_numpy(np.ascontiguousarray(layout, dtype=np.uint8)).to("cuda")
    o, lse = fa.flash_attn_blocksparse(q, k, v, lay, 128, block_k, causal=causal, window=window,
                                       scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check(o, lse, o_ref, lse_ref, label):
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{label}: empty rows differ"
    assert np.all(o[empty] == 0.0), f"{label}: empty rows not zero"
    compare(o[~empty], lse[~empty], o_ref[~empty], lse_ref[~empty], TOL_BF16, label)


# (B, H, Hkv, n, d, block_k, layout_heads, density, causal, window)
SMALL = [
    (1, 1, 1, 1, 128, 64, 1, 1.0, 0, -1),
    (1, 2, 1, 300, 128, 64, 1, 0.5, 0, -1),
    (2, 4, 2, 700, 128, 64, 4, 0.4, 1, -1),
    (1, 4, 4, 1000, 128, 128, 4, 0.3, 0, -1),
    (1, 2, 2, 513, 64, 64, 2, 0.6, 1, 100),
    (1, 2, 1, 1024, 128, 128, 1, 0.2, 0, 300),
    (2, 2, 1, 129, 64, 64, 1, 0.5, 1, -1),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"bs{i}" for i in range(len(SMALL))])
def test_blocksparse_small(case):
    B, H, Hkv, n, d, bk, lh, dens, causal, window = case
    say(f"blocksparse {case}")
    inp = prefill_inputs(B, H, Hkv, n, d, seed=5000 + n + d)
    lay = block_layout(lh, n, 128, bk, seed=n + lh, density=dens)
    if n > 256:
        lay[:, 1, :] = 0   # a query block with nothing kept: o = 0, lse = -inf
    scale = 1.0 / math.sqrt(d)
    o, lse = run_bs(inp, lay, bk, causal, window, scale)
    o_ref, lse_ref = attention_block_sparse(inp["q"], inp["k"], inp["v"], lay, 128, bk, causal,
                                            window, scale)
    check(o, lse, o_ref, lse_ref, f"bs {case}")


@pytest.mark.parametrize("causal,window", [(False, 200), (True, 200), (False, 1000)])
def test_band_layout_equals_windowed_forward_bitwise(causal, window):
    """Keeping exactly the tiles the band meets reproduces fa_fwd's skip."""
    import io_aware_exact_fa_amd as fa
    n, bk = 2100, 64
    inp = prefill_inputs(1, 4, 2, n, 128, seed=5100)
    dev = prefill_device(inp)
    nq, nk = -(-n // 128), -(-n // bk)
    lay = np.zeros((1, nq, nk), dtype=np.uint8)
    for a in range(nq):
        q0, q1 = a * 128, min(n, a * 128 + 128) - 1
        lo = q0 - window
        hi = q1 if causal else q1 + window
        for c in range(nk):
            k0, k1 = c * bk, min(n, c * bk + bk) - 1
            lay[0, a, c] = not (k1 < lo or k0 > hi)
    o, lse = run_bs(inp, lay, bk, causal, window, 0.08, dev=dev)
    import torch
    o2, l2 = fa.flash_attn_fwd(*dev, causal=causal, window=window, scale=0.08)
    torch.cuda.synchronize()
    assert np.array_equal(o, o2.float().cpu().numpy())
    assert np.array_equal(lse, l2.cpu().numpy())


def test_blocksparse_paired_grid_empty_first_block():
    """Short causal grids pair query blocks (a workgroup runs block NQ-1-t,
    then t).  With the first block of every pair empty (no kept tile, so no
    barrier in its tile loop), the workgroup's second block list must still
    be built only after every wave has read the first block's count."""
    B, H, Hkv, n, d = 2, 4, 2, 1024, 128
    inp = prefill_inputs(B, H, Hkv, n, d, seed=5200)
    lay = block_layout(H, n, 128, 64, seed=5201, density=0.5)
    lay[:, 4:, :] = 0  # blocks 4..7, the first of each pair (7-t, t), keep nothing
    scale = 1.0 / math.sqrt(d)
    o, lse = run_bs(inp, lay, 64, 1, -1, scale)
    o_ref, lse_ref = attention_block_sparse(inp["q"], inp["k"], inp["v"], lay, 128, 64, True, -1,
                                            scale)
    check(o, lse, o_ref, lse_ref, "bs paired, first blocks empty")


def test_blocksparse_full_size():
    """n = 32768, 32 heads sharing 8 KV heads: one local block either side of the
    diagonal, the first key block column, 10 % random blocks, causal.  Two
    whole heads, and in every head one row of every 128-row block plus edges."""
    B, H, Hkv, n, d = 1, 32, 8, 32768, 128
    say("blocksparse full n=32768")
    inp = prefill_inputs(B, H, Hkv, n, d, seed=13)
    lay = block_layout(H, n, 128, 64, seed=13, density=0.1, local=2, global_cols=1)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_bs(inp, lay, 64, 1, -1, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for h in (0, H - 1):
        g = h // (H // Hkv)

        def head_rows(rows, h=h, g=g):
            return attention_block_sparse(inp["q"][:, h:h + 1], inp["k"][:, g:g + 1],
                                          inp["v"][:, g:g + 1], lay[h:h + 1], 128, 64, True, -1,
                                          scale, rows=rows)

        o_ref, l_ref = oracle_rows_parallel(head_rows, np.arange(n), chunk=512)
        check(o[:, h:h + 1], lse[:, h:h + 1], o_ref, l_ref, f"bs full h{h} (every row)")
    rows = stratified_rows(n, 128, seed=7, extra=[0, 1, 127, 128, 16383, n - 1])
    o_ref, l_ref = oracle_rows_parallel(
        lambda r: attention_block_sparse(inp["q"], inp["k"], inp["v"], lay, 128, 64, True, -1,
                                         scale, rows=r), rows, chunk=16)
    check(o[:, :, rows], lse[:, :, rows], o_ref, l_ref, f"bs full all heads, {rows.size} rows")

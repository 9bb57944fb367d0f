"""C-ABI library: loads, exports every declared symbol, rejects bad arguments
on the host before any launch (CPU only: no kernel is ever enqueued here)."""

import ctypes
import os
import re

import pytest

import io_aware_exact_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = 256  # a non-NULL address that validation rejects before any use


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"fa_fwd", "fa_decode", "fa_decode_workspace_bytes",
                          "fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd_varlen", "fa_fwd_paged",
                          "fa_fwd_blocksparse", "fa_decode_fp8", "fa_fwd_strided",
                          "fa_fwd_tile_count", "fa_decode_noalloc", "fa_strerror",
                          "fa_version"}
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strerror(lib):
    assert fa.fa_version() >> 16 == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert fa.fa_strerror(st) and fa.fa_strerror(st) != "unknown status"
    assert fa.fa_strerror(-99) == "unknown status"


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Hkv=1, n=16, d=128,
                causal=0, window=-1, scale=0.1, dtype=0)
    args.update(kw)
    return fa.lib().fa_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"],
                           args["B"], args["H"], args["Hkv"], args["n"], args["d"],
                           args["causal"], args["window"], ctypes.c_float(args["scale"]),
                           args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(Hkv=0), -2), (dict(n=0), -2), (dict(d=0), -2),
    (dict(H=3, Hkv=2), -2), (dict(causal=2), -2), (dict(scale=0.0), -2),
    (dict(scale=-1.0), -2), (dict(scale=float("inf")), -2), (dict(scale=float("nan")), -2),
    (dict(n=1 << 25, d=128), -2),
    (dict(H=1 << 28, Hkv=1 << 28, n=1024), -2),  # 2^31 workgroups
    (dict(d=96), -3), (dict(d=256), -3), (dict(dtype=7), -3),
])
def test_fwd_rejects(lib, kw, status):
    assert _fwd(**kw) == status


def _dec_na(**kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, pt=FAKE, sl=FAKE, o=FAKE, lse=FAKE, B=2, H=8,
                Hkv=2, d=128, P=10, ps=16, maxp=4, maxs=64, scale=0.1)
    args.update(kw)
    return fa.lib().fa_decode_noalloc(args["q"], args["kc"], args["vc"], args["pt"], args["sl"],
                                      args["o"], args["lse"], args["B"], args["H"], args["Hkv"],
                                      args["d"], args["P"], args["ps"], args["maxp"],
                                      args["maxs"], ctypes.c_float(args["scale"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(pt=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(maxs=0), -2), (dict(H=6, Hkv=4), -2), (dict(scale=0.0), -2),
    (dict(maxp=1 << 28), -2),
    (dict(d=96), -3), (dict(ps=32), -3), (dict(H=34, Hkv=2), -3),
    # partials beyond the 32 MiB array: 128 sequences x 32 heads at 32K tokens
    (dict(B=128, H=32, Hkv=8, maxp=2048, maxs=32768), -4),
])
def test_decode_noalloc_rejects(lib, kw, status):
    assert _dec_na(**kw) == status


def test_decode_noalloc_limit_matches_workspace_size(lib):
    limit = 32 << 20
    assert fa.fa_decode_workspace_bytes(64, 32, 32768, 128) <= limit   # the decode workload
    assert fa.fa_decode_workspace_bytes(128, 32, 32768, 128) > limit


def _count(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, H=8, Hkv=2, n=1000, d=128,
                causal=1, window=-1, scale=0.1, counters=FAKE)
    args.update(kw)
    return fa.lib().fa_fwd_tile_count(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                      args["B"], args["H"], args["Hkv"], args["n"], args["d"],
                                      args["causal"], args["window"],
                                      ctypes.c_float(args["scale"]), args["counters"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(counters=None), -1), (dict(q=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(n=0), -2), (dict(H=3, Hkv=2), -2), (dict(causal=2), -2),
    (dict(scale=0.0), -2), (dict(n=1 << 25, d=128), -2),
    (dict(d=96), -3),
])
def test_tile_count_rejects(lib, kw, status):
    assert _count(**kw) == status


def _dec(**kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, pt=FAKE, sl=FAKE, o=FAKE, lse=FAKE, B=2, H=8,
                Hkv=2, d=128, P=10, ps=16, maxp=4, maxs=64, scale=0.1, ws=FAKE,
                wsb=1 << 30)
    args.update(kw)
    return fa.lib().fa_decode(args["q"], args["kc"], args["vc"], args["pt"], args["sl"],
                              args["o"], args["lse"], args["B"], args["H"], args["Hkv"],
                              args["d"], args["P"], args["ps"], args["maxp"], args["maxs"],
                              ctypes.c_float(args["scale"]), args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(kc=None), -1), (dict(vc=None), -1), (dict(pt=None), -1),
    (dict(sl=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(Hkv=0), -2), (dict(P=0), -2), (dict(ps=0), -2),
    (dict(maxp=0), -2), (dict(maxs=0), -2), (dict(H=6, Hkv=4), -2), (dict(scale=0.0), -2),
    (dict(maxp=1 << 28), -2),  # max_pages * 16 overflows 32 bits
    (dict(d=96), -3), (dict(d=256), -3), (dict(ps=32), -3), (dict(H=34, Hkv=2), -3),
    (dict(ws=None), -4), (dict(wsb=16), -4),
])
def test_decode_rejects(lib, kw, status):
    assert _dec(**kw) == status


def test_workspace_size(lib):
    assert fa.fa_decode_workspace_bytes(0, 8, 64, 128) == 0
    small = fa.fa_decode_workspace_bytes(2, 8, 64, 128)
    big = fa.fa_decode_workspace_bytes(64, 32, 32768, 128)
    assert 0 < small < big
    # partial output (d floats) + log-sum-exp per (b, h, split), at least one split
    assert big >= 64 * 32 * (128 + 1) * 4
    assert fa.fa_decode_workspace_bytes(64, 32, 65536, 128) >= big
    ws = fa.fa_decode_workspace_bytes(2, 8, 64, 128)
    assert _dec(wsb=ws - 1) == -4


def _decode_plan_bytes(B, H, max_seqlen, d):
    """The documented split plan: 120 pages (1920 tokens) per split, halved
    (down to 8) while fewer than 2048 (sequence, H/4 head group) splits of an
    average sequence (half of max_seqlen) would exist; one partial (d floats)
    and one log-sum-exp per (sequence, query head, split), each array padded
    to 256 bytes.  Padding the launch grid by an empty split adds no partial."""
    pages = -(-max_seqlen // 16)
    groups = B * (H // 4 if H >= 4 else 1)
    avg = (pages + 1) // 2
    sp = 120
    while sp > 8 and groups * (-(-avg // sp)) < 2048:
        sp = sp // 2 if sp > 16 else 8
    rows = B * H * (-(-pages // sp))
    up = lambda x: -(-x // 256) * 256
    return up(rows * d * 4) + up(rows * 4)


@pytest.mark.parametrize("B,H,max_seqlen,d", [
    (64, 32, 32768, 128), (64, 32, 32768, 64), (16, 32, 30000, 128), (5, 32, 4136, 128),
    (1, 8, 1, 128), (2, 16, 1500, 64), (128, 32, 65536, 128), (3, 2, 777, 128),
    (64, 32, 30000, 128), (8, 64, 131072, 128),
])
def test_decode_workspace_follows_split_plan(lib, B, H, max_seqlen, d):
    assert fa.fa_decode_workspace_bytes(B, H, max_seqlen, d) == _decode_plan_bytes(B, H, max_seqlen, d)


def test_decode_split_plan_of_the_workload(lib):
    """The 64-sequence workload (up to 32768 tokens): 18 splits of 120 pages."""
    rows = 64 * 32 * 18
    assert fa.fa_decode_workspace_bytes(64, 32, 32768, 128) == rows * 128 * 4 + rows * 4


def _bwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                B=1, H=2, Hkv=1, n=16, d=128, causal=0, window=-1, scale=0.1, dtype=0,
                ws=FAKE, wsb=1 << 20)
    args.update(kw)
    return fa.lib().fa_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"],
                           args["dq"], args["dk"], args["dv"], args["B"], args["H"],
                           args["Hkv"], args["n"], args["d"], args["causal"], args["window"],
                           ctypes.c_float(args["scale"]), args["dtype"], args["ws"],
                           args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1), (dict(do=None), -1), (dict(dq=None), -1), (dict(dk=None), -1),
    (dict(dv=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(Hkv=0), -2), (dict(n=0), -2), (dict(d=0), -2),
    (dict(H=3, Hkv=2), -2), (dict(causal=2), -2), (dict(scale=0.0), -2),
    (dict(scale=float("nan")), -2), (dict(n=1 << 25, d=128), -2),
    (dict(B=1 << 10, H=1 << 18, Hkv=1 << 18, n=1024), -2),  # 2^31 workgroups
    (dict(d=96), -3), (dict(dtype=1), -3), (dict(dtype=7), -3),
    (dict(ws=None), -4), (dict(wsb=1 * 2 * 16 * 4 - 1), -4),
])
def test_bwd_rejects(lib, kw, status):
    assert _bwd(**kw) == status


def test_bwd_workspace_size(lib):
    # one float (D_i = <dO_i, O_i>) per query row
    assert fa.fa_bwd_workspace_bytes(2, 8, 100, 128) == 2 * 8 * 100 * 4
    assert fa.fa_bwd_workspace_bytes(0, 8, 100, 128) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 1 << 25, 128) == 0


def _varlen(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, B=2, H=4, Hkv=2, total=100,
                maxs=60, d=128, causal=1, window=-1, scale=0.1, dtype=0)
    args.update(kw)
    return fa.lib().fa_fwd_varlen(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                  args["cu"], args["B"], args["H"], args["Hkv"], args["total"],
                                  args["maxs"], args["d"], args["causal"], args["window"],
                                  ctypes.c_float(args["scale"]), args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1), (dict(cu=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(Hkv=0), -2), (dict(total=0), -2),
    (dict(maxs=0), -2), (dict(d=0), -2), (dict(H=3, Hkv=2), -2), (dict(causal=3), -2),
    (dict(scale=0.0), -2), (dict(total=1 << 24, H=8), -2),
    (dict(B=1 << 20, H=1 << 10, Hkv=1 << 10, total=256, maxs=256), -2),  # 2^31 workgroups
    (dict(d=96), -3), (dict(dtype=1), -3),
])
def test_varlen_rejects(lib, kw, status):
    assert _varlen(**kw) == status


def _paged_fwd(**kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, pt=FAKE, cu=FAKE, sk=FAKE, o=FAKE, lse=FAKE, B=2,
                H=8, Hkv=2, d=128, total=64, maxs=32, P=10, ps=16, maxp=4, causal=1,
                window=-1, scale=0.1, dtype=0)
    args.update(kw)
    return fa.lib().fa_fwd_paged(args["q"], args["kc"], args["vc"], args["pt"], args["cu"],
                                 args["sk"], args["o"], args["lse"], args["B"], args["H"],
                                 args["Hkv"], args["d"], args["total"], args["maxs"], args["P"],
                                 args["ps"], args["maxp"], args["causal"], args["window"],
                                 ctypes.c_float(args["scale"]), args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(kc=None), -1), (dict(vc=None), -1), (dict(pt=None), -1),
    (dict(cu=None), -1), (dict(sk=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(Hkv=0), -2), (dict(total=0), -2),
    (dict(maxs=0), -2), (dict(P=0), -2), (dict(ps=0), -2), (dict(maxp=0), -2),
    (dict(H=6, Hkv=4), -2), (dict(causal=-1), -2), (dict(scale=float("inf")), -2),
    (dict(d=96), -3), (dict(ps=32), -3), (dict(dtype=1), -3),
])
def test_paged_fwd_rejects(lib, kw, status):
    assert _paged_fwd(**kw) == status


def _bsparse(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, lay=FAKE, lh=1, B=1, H=4, Hkv=2,
                n=1000, d=128, bq=128, bk=64, causal=1, window=-1, scale=0.1, dtype=0)
    args.update(kw)
    return fa.lib().fa_fwd_blocksparse(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                       args["lay"], args["lh"], args["B"], args["H"],
                                       args["Hkv"], args["n"], args["d"], args["bq"],
                                       args["bk"], args["causal"], args["window"],
                                       ctypes.c_float(args["scale"]), args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1), (dict(lay=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(n=0), -2), (dict(H=3, Hkv=2), -2),
    (dict(lh=2), -2), (dict(lh=0), -2), (dict(causal=2), -2), (dict(scale=0.0), -2),
    (dict(n=131073), -3), (dict(d=96), -3), (dict(bq=64), -3), (dict(bk=32), -3),
    (dict(bk=256), -3), (dict(dtype=1), -3),
])
def test_blocksparse_rejects(lib, kw, status):
    assert _bsparse(**kw) == status


def _dec8(**kw):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, pt=FAKE, sl=FAKE, o=FAKE, lse=FAKE,
                B=2, H=8, Hkv=2, d=128, P=10, ps=16, maxp=4, maxs=64, scale=0.1, ws=FAKE,
                wsb=1 << 30)
    args.update(kw)
    return fa.lib().fa_decode_fp8(args["q"], args["kc"], args["vc"], args["ks"], args["vs"],
                                  args["pt"], args["sl"], args["o"], args["lse"], args["B"],
                                  args["H"], args["Hkv"], args["d"], args["P"], args["ps"],
                                  args["maxp"], args["maxs"], ctypes.c_float(args["scale"]),
                                  args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(kc=None), -1), (dict(vc=None), -1), (dict(ks=None), -1),
    (dict(vs=None), -1), (dict(pt=None), -1), (dict(sl=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(Hkv=0), -2), (dict(P=0), -2), (dict(maxs=0), -2),
    (dict(H=6, Hkv=4), -2), (dict(scale=-1.0), -2),
    (dict(maxp=1 << 28), -2),  # max_pages * 16 overflows 32 bits
    (dict(d=96), -3), (dict(ps=8), -3), (dict(H=34, Hkv=2), -3),
    (dict(ws=None), -4), (dict(wsb=16), -4),
])
def test_decode_fp8_rejects(lib, kw, status):
    assert _dec8(**kw) == status


def _strided(strides=None, **kw):
    B, H, n, d = 2, 4, 100, 128
    if strides is None:  # BSHD
        strides = [n * H * d, d, H * d, n * 2 * d, d, 2 * d, n * 2 * d, d, 2 * d,
                   n * H * d, d, H * d]
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=B, H=H, Hkv=2, n=n, d=d, causal=1,
                window=-1, scale=0.1, dtype=0)
    args.update(kw)
    arr = (ctypes.c_int64 * 12)(*strides)
    ptr = None if kw.get("null_strides") else ctypes.cast(arr, ctypes.c_void_p)
    return fa.lib().fa_fwd_strided(args["q"], args["k"], args["v"], args["o"], args["lse"], ptr,
                                   args["B"], args["H"], args["Hkv"], args["n"], args["d"],
                                   args["causal"], args["window"],
                                   ctypes.c_float(args["scale"]), args["dtype"], None)


def _bad(i, val):
    B, H, n, d = 2, 4, 100, 128
    s = [n * H * d, d, H * d, n * 2 * d, d, 2 * d, n * 2 * d, d, 2 * d, n * H * d, d, H * d]
    s[i] = val
    return s


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(null_strides=True), -1),
    (dict(B=0), -2), (dict(H=3, Hkv=2), -2), (dict(causal=5), -2), (dict(scale=0.0), -2),
    (dict(strides=_bad(2, 64)), -2),         # q row stride < d
    (dict(strides=_bad(5, 4 * 128)), -2),    # k and v row strides differ
    (dict(strides=_bad(0, -8)), -2),         # negative
    (dict(strides=_bad(1, 129)), -2),        # not a multiple of 8
    (dict(d=96), -3), (dict(dtype=1), -3),
])
def test_strided_rejects(lib, kw, status):
    kw = dict(kw)
    strides = kw.pop("strides", None)
    assert _strided(strides, **kw) == status


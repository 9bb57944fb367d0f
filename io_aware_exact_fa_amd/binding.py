"""ctypes binding over libfa.so (declared in include/fa.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a negative status becomes ``FaError``.
Every step of the computation runs in the library's HIP kernels.  Loading
fails loudly when the library has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

FA_BF16 = 0
FA_F32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FaError(RuntimeError):
    """A libfa call returned a negative status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {fa_strerror(status)} (status {status})")


def lib_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def lib() -> ctypes.CDLL:
    """Load libfa.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                         f32, i32, vp]
    L.fa_fwd.restype = i32
    L.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.fa_decode_workspace_bytes.restype = sz
    L.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                            i32, i32, i32, f32, vp, sz, vp]
    L.fa_decode.restype = i32
    L.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.fa_bwd_workspace_bytes.restype = sz
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                         i32, i32, i32, f32, i32, vp, sz, vp]
    L.fa_bwd.restype = i32
    L.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                i32, i32, f32, i32, vp]
    L.fa_fwd_varlen.restype = i32
    L.fa_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                               i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.fa_fwd_paged.restype = i32
    L.fa_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i32, i32, i32, f32, i32, vp]
    L.fa_fwd_blocksparse.restype = i32
    L.fa_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                i32, i32, i32, f32, vp, sz, vp]
    L.fa_decode_fp8.restype = i32
    L.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                 f32, i32, vp]
    L.fa_fwd_strided.restype = i32
    L.fa_fwd_tile_count.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, vp, vp]
    L.fa_fwd_tile_count.restype = i32
    L.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                    i32, i32, i32, f32, vp]
    L.fa_decode_noalloc.restype = i32
    L.fa_strerror.argtypes = [i32]
    L.fa_strerror.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = i32
    _LIB = L
    return L


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def fa_strerror(status: int) -> str:
    return lib().fa_strerror(int(status)).decode()


def fa_version() -> int:
    return int(lib().fa_version())


def fa_fwd(q, k, v, o, lse, B, H, Hkv, n, d, causal, window, scale, dtype,
           stream=None) -> None:
    """Raw C-ABI call; tensors or integer device addresses."""
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B),
                      int(H), int(Hkv), int(n), int(d), int(causal), int(window),
                      float(scale), int(dtype), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd")


def fa_decode_noalloc(q, kcache, vcache, page_table, seqlens, o, lse, B, H, Hkv, d, num_pages,
                      page_size, max_pages, max_seqlen, scale, stream=None) -> None:
    """Raw C-ABI call: fa_decode with the split partials in the library's own
    static device array (no workspace, no allocation)."""
    st = lib().fa_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(page_table),
                                 _ptr(seqlens), _ptr(o), _ptr(lse), int(B), int(H), int(Hkv),
                                 int(d), int(num_pages), int(page_size), int(max_pages),
                                 int(max_seqlen), float(scale), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_decode_noalloc")


def fa_fwd_tile_count(q, k, v, o, lse, B, H, Hkv, n, d, causal, window, scale, counters,
                      stream=None) -> None:
    """Raw C-ABI call (bf16 forward that adds its visited / staged key-tile
    counts to the two uint64 ``counters``); tensors or device addresses."""
    st = lib().fa_fwd_tile_count(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                 int(Hkv), int(n), int(d), int(causal), int(window),
                                 float(scale), _ptr(counters), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_tile_count")


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d, causal,
                  window, scale, dtype, stream=None) -> None:
    """Raw C-ABI call; tensors or integer device addresses."""
    st = lib().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                             int(B), int(H), int(Hkv), int(total), int(max_seqlen), int(d),
                             int(causal), int(window), float(scale), int(dtype),
                             _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_varlen")


def fa_fwd_paged(q, kcache, vcache, page_table, cu_seqlens_q, seqlens_k, o, lse, B, H, Hkv,
                 d, total_q, max_seqlen_q, num_pages, page_size, max_pages, causal, window,
                 scale, dtype, stream=None) -> None:
    """Raw C-ABI call; tensors or integer device addresses."""
    st = lib().fa_fwd_paged(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(page_table),
                            _ptr(cu_seqlens_q), _ptr(seqlens_k), _ptr(o), _ptr(lse), int(B),
                            int(H), int(Hkv), int(d), int(total_q), int(max_seqlen_q),
                            int(num_pages), int(page_size), int(max_pages), int(causal),
                            int(window), float(scale), int(dtype), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_paged")


def fa_fwd_blocksparse(q, k, v, o, lse, layout, layout_heads, B, H, Hkv, n, d, block_q,
                       block_k, causal, window, scale, dtype, stream=None) -> None:
    """Raw C-ABI call; tensors or integer device addresses."""
    st = lib().fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(layout),
                                  int(layout_heads), int(B), int(H), int(Hkv), int(n), int(d),
                                  int(block_q), int(block_k), int(causal), int(window),
                                  float(scale), int(dtype), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_blocksparse")


def fa_decode_fp8(q, kcache, vcache, k_scale, v_scale, page_table, seqlens, o, lse, B, H,
                  Hkv, d, num_pages, page_size, max_pages, max_seqlen, scale, workspace,
                  workspace_bytes, stream=None) -> None:
    """Raw C-ABI call; tensors or integer device addresses."""
    st = lib().fa_decode_fp8(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(k_scale), _ptr(v_scale),
                             _ptr(page_table), _ptr(seqlens), _ptr(o), _ptr(lse), int(B),
                             int(H), int(Hkv), int(d), int(num_pages), int(page_size),
                             int(max_pages), int(max_seqlen), float(scale), _ptr(workspace),
                             int(workspace_bytes), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_decode_fp8")


def fa_fwd_strided(q, k, v, o, lse, strides, B, H, Hkv, n, d, causal, window, scale, dtype,
                   stream=None) -> None:
    """Raw C-ABI call; ``strides`` is a sequence of 12 element strides."""
    arr = (ctypes.c_int64 * 12)(*[int(x) for x in strides])
    st = lib().fa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              ctypes.cast(arr, ctypes.c_void_p), int(B), int(H), int(Hkv),
                              int(n), int(d), int(causal), int(window), float(scale), int(dtype),
                              _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_strided")


def fa_decode_workspace_bytes(B, H, max_seqlen, d) -> int:
    return int(lib().fa_decode_workspace_bytes(int(B), int(H), int(max_seqlen), int(d)))


def fa_decode(q, kcache, vcache, page_table, seqlens, o, lse, B, H, Hkv, d,
              num_pages, page_size, max_pages, max_seqlen, scale, workspace,
              workspace_bytes, stream=None) -> None:
    """Raw C-ABI call; tensors or integer device addresses."""
    st = lib().fa_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(page_table),
                         _ptr(seqlens), _ptr(o), _ptr(lse), int(B), int(H),
                         int(Hkv), int(d), int(num_pages), int(page_size),
                         int(max_pages), int(max_seqlen), float(scale),
                         _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_decode")


def fa_bwd_workspace_bytes(B, H, n, d) -> int:
    return int(lib().fa_bwd_workspace_bytes(int(B), int(H), int(n), int(d)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, n, d, causal, window,
           scale, dtype, workspace, workspace_bytes, stream=None) -> None:
    """Raw C-ABI call; tensors or integer device addresses."""
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                      _ptr(dq), _ptr(dk), _ptr(dv), int(B), int(H), int(Hkv),
                      int(n), int(d), int(causal), int(window), float(scale),
                      int(dtype), _ptr(workspace), int(workspace_bytes),
                      _stream(stream))
    if st != 0:
        raise FaError(st, "fa_bwd")


# ---------------------------------------------------------------------------
# Convenience wrappers: allocate outputs with torch, then call the ABI.
# ---------------------------------------------------------------------------

def _check_contig(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (row-major)")


def flash_attn_fwd(q, k, v, causal: bool = False, window: int = -1,
                   scale: float | None = None, out=None, lse=None, stream=None):
    """q [B,H,n,d], k/v [B,Hkv,n,d] (bf16 or fp32 CUDA tensors) -> (o, lse)."""
    import torch
    _check_contig(q, k, v)
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if q.dtype == torch.bfloat16:
        dt = FA_BF16
    elif q.dtype == torch.float32:
        dt = FA_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if not (k.dtype == v.dtype == q.dtype):
        raise ValueError("q, k, v must share a dtype")
    if tuple(k.shape) != (B, Hkv, n, d) or tuple(v.shape) != (B, Hkv, n, d):
        raise ValueError("k and v must be [B, Hkv, n, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, out, lse, B, H, Hkv, n, d, int(bool(causal)), int(window),
           scale, dt, stream)
    return out, lse


def flash_decode(q, kcache, vcache, page_table, seqlens, max_seqlen: int,
                 scale: float | None = None, workspace=None, out=None, lse=None,
                 stream=None):
    """q [B,H,d] bf16; caches [P,Hkv,ps,d] bf16; table [B,maxp] / seqlens [B] int32."""
    import torch
    _check_contig(q, kcache, vcache, page_table, seqlens)
    B, H, d = q.shape
    P, Hkv, ps, d2 = kcache.shape
    if d2 != d or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError("cache shapes disagree with q")
    if page_table.dtype != torch.int32 or seqlens.dtype != torch.int32:
        raise ValueError("page_table and seqlens must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = fa_decode_workspace_bytes(B, H, max_seqlen, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    fa_decode(q, kcache, vcache, page_table, seqlens, out, lse, B, H, Hkv, d, P,
              ps, page_table.shape[1], max_seqlen, scale, workspace,
              workspace.numel() * workspace.element_size(), stream)
    return out, lse


def flash_attn_bwd(q, k, v, o, lse, dout, causal: bool = False, window: int = -1,
                   scale: float | None = None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) as float32 tensors for bf16 q/k/v/o/dout.

    o and lse must be what flash_attn_fwd returned for the same q, k, v,
    causal, window and scale.
    """
    import torch
    _check_contig(q, k, v, o, lse, dout)
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    for t in (q, k, v, o, dout):
        if t.dtype != torch.bfloat16:
            raise ValueError("fa_bwd takes bf16 q, k, v, o and dout")
    if tuple(k.shape) != (B, Hkv, n, d) or tuple(v.shape) != (B, Hkv, n, d):
        raise ValueError("k and v must be [B, Hkv, n, d]")
    if tuple(o.shape) != (B, H, n, d) or tuple(dout.shape) != (B, H, n, d):
        raise ValueError("o and dout must be [B, H, n, d]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n):
        raise ValueError("lse must be float32 [B, H, n]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = fa_bwd_workspace_bytes(B, H, n, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, H, n, d), **f32)
    dk = torch.empty((B, Hkv, n, d), **f32)
    dv = torch.empty((B, Hkv, n, d), **f32)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, n, d, int(bool(causal)),
           int(window), scale, FA_BF16, workspace,
           workspace.numel() * workspace.element_size(), stream)
    return dq, dk, dv


def flash_attn_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False,
                      window: int = -1, scale: float | None = None, stream=None):
    """Ragged batch: q [H,total,d], k/v [Hkv,total,d] bf16; cu_seqlens [B+1] int32
    (device) -> (o [H,total,d] bf16, lse [H,total] fp32)."""
    import torch
    _check_contig(q, k, v, cu_seqlens)
    H, total, d = q.shape
    Hkv = k.shape[0]
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("fa_fwd_varlen takes bf16 q, k, v")
    if tuple(k.shape) != (Hkv, total, d) or tuple(v.shape) != (Hkv, total, d):
        raise ValueError("k and v must be [Hkv, total, d]")
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, cu_seqlens.numel() - 1, H, Hkv, total,
                  max_seqlen, d, int(bool(causal)), int(window), scale, FA_BF16, stream)
    return o, lse


def flash_attn_paged(q, kcache, vcache, page_table, cu_seqlens_q, seqlens_k,
                     max_seqlen_q: int, causal: bool = True, window: int = -1,
                     scale: float | None = None, stream=None):
    """Chunks over paged histories: q [H,total_q,d] bf16; caches [P,Hkv,16,d] bf16;
    page_table [B,max_pages], cu_seqlens_q [B+1], seqlens_k [B] int32 (device)
    -> (o [H,total_q,d] bf16, lse [H,total_q] fp32)."""
    import torch
    _check_contig(q, kcache, vcache, page_table, cu_seqlens_q, seqlens_k)
    H, total_q, d = q.shape
    P, Hkv, ps, d2 = kcache.shape
    if d2 != d or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError("cache shapes disagree with q")
    for t in (page_table, cu_seqlens_q, seqlens_k):
        if t.dtype != torch.int32:
            raise ValueError("page_table, cu_seqlens_q and seqlens_k must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    fa_fwd_paged(q, kcache, vcache, page_table, cu_seqlens_q, seqlens_k, o, lse,
                 seqlens_k.numel(), H, Hkv, d, total_q, max_seqlen_q, P, ps,
                 page_table.shape[1], int(bool(causal)), int(window), scale, FA_BF16, stream)
    return o, lse


def flash_attn_blocksparse(q, k, v, layout, block_q: int = 128, block_k: int = 64,
                           causal: bool = False, window: int = -1,
                           scale: float | None = None, stream=None):
    """q [B,H,n,d], k/v [B,Hkv,n,d] bf16; layout uint8 [1 or H, ceil(n/block_q),
    ceil(n/block_k)] (device) -> (o, lse) as flash_attn_fwd."""
    import torch
    _check_contig(q, k, v, layout)
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("fa_fwd_blocksparse takes bf16 q, k, v")
    if tuple(k.shape) != (B, Hkv, n, d) or tuple(v.shape) != (B, Hkv, n, d):
        raise ValueError("k and v must be [B, Hkv, n, d]")
    lh = layout.shape[0]
    if layout.dtype != torch.uint8 or tuple(layout.shape[1:]) != (-(-n // block_q),
                                                                    -(-n // block_k)):
        raise ValueError("layout must be uint8 [1 or H, ceil(n/block_q), ceil(n/block_k)]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    fa_fwd_blocksparse(q, k, v, o, lse, layout, lh, B, H, Hkv, n, d, block_q, block_k,
                       int(bool(causal)), int(window), scale, FA_BF16, stream)
    return o, lse


def flash_decode_fp8(q, kcache, vcache, k_scale, v_scale, page_table, seqlens,
                     max_seqlen: int, scale: float | None = None, workspace=None,
                     stream=None):
    """q [B,H,d] bf16; caches [P,Hkv,ps,d] uint8 (E4M3 bytes); k_scale/v_scale
    [Hkv] float32; table [B,maxp] / seqlens [B] int32 -> (o, lse)."""
    import torch
    _check_contig(q, kcache, vcache, k_scale, v_scale, page_table, seqlens)
    B, H, d = q.shape
    P, Hkv, ps, d2 = kcache.shape
    if d2 != d or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError("cache shapes disagree with q")
    if kcache.dtype != torch.uint8 or vcache.dtype != torch.uint8:
        raise ValueError("FP8 caches are uint8 tensors of E4M3 bytes")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32 or \
            k_scale.numel() != Hkv or v_scale.numel() != Hkv:
        raise ValueError("k_scale and v_scale must be float32 [Hkv]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = fa_decode_workspace_bytes(B, H, max_seqlen, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    fa_decode_fp8(q, kcache, vcache, k_scale, v_scale, page_table, seqlens, o, lse, B, H, Hkv,
                  d, P, ps, page_table.shape[1], max_seqlen, scale, workspace,
                  workspace.numel() * workspace.element_size(), stream)
    return o, lse


def flash_attn_strided(q, k, v, causal: bool = False, window: int = -1,
                       scale: float | None = None, out=None, stream=None, layout: str = "bhsd"):
    """Attention over strided bf16 views.

    ``layout`` names how the four dims of q, k, v (and ``out``) are ordered:
    "bhsd" (batch, heads, seq, dim) or "bshd" (batch, seq, heads, dim, the
    layout of the library call in the sources).  Any strides are accepted as
    long as the head dim is contiguous (e.g. views into a packed qkv tensor).
    Returns (o in the same layout as q, lse [B, H, n] float32).
    """
    import torch
    if layout not in ("bhsd", "bshd"):
        raise ValueError("layout must be 'bhsd' or 'bshd'")
    perm = (0, 1, 2, 3) if layout == "bhsd" else (0, 2, 1, 3)
    qv, kv_, vv = (t.permute(*perm) for t in (q, k, v))  # -> [B, heads, n, d] views
    B, H, n, d = qv.shape
    Hkv = kv_.shape[1]
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1:
            raise ValueError("bf16 tensors with a contiguous head dim are required")
    if out is None:
        out = torch.empty_like(q)
    ov = out.permute(*perm)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    strides = [*qv.stride()[:3], *kv_.stride()[:3], *vv.stride()[:3], *ov.stride()[:3]]
    fa_fwd_strided(q, k, v, out, lse, strides, B, H, Hkv, n, d, int(bool(causal)), int(window),
                   scale, FA_BF16, stream)
    return out, lse


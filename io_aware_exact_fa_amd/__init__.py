"""Exact FlashAttention for MI355X / gfx950: prefill forward, paged
flash-decoding and the backward pass.

The compute path is the HIP library ``libfa.so`` built from ``csrc/``; this
package is a thin ctypes binding over its C ABI (see ``include/fa.h``).
The library is loaded lazily on first use and loading fails loudly if it has
not been built.
"""

from .binding import (  # noqa: F401
    FA_BF16, FA_F32, FaError, lib, lib_path,
    fa_fwd, fa_decode, fa_decode_workspace_bytes, fa_bwd, fa_bwd_workspace_bytes,
    fa_fwd_varlen, fa_fwd_paged, fa_strerror, fa_version, flash_attn_fwd, flash_decode,
    flash_attn_bwd, flash_attn_varlen, flash_attn_paged, fa_fwd_blocksparse,
    flash_attn_blocksparse, fa_decode_fp8, flash_decode_fp8, fa_fwd_strided,
    flash_attn_strided, fa_fwd_tile_count, fa_decode_noalloc,
)

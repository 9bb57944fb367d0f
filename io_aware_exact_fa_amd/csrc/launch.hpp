// Internal launch entry points behind the C ABI (include/fa.h).
// Arguments have been validated by the caller; these only build grids and
// enqueue kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Prefill: q [B,H,n,d], k/v [B,Hkv,n,d], o like q, lse [B,H,n].  window has
// been clamped to [-1, n].  scale > 0.
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o,
                               float* lse, int B, int H, int Hkv, int n, int d,
                               int causal, int window, float scale, hipStream_t stream);
// As launch_prefill_bf16, and counters[0] += (wave, key tile) pairs whose
// products are computed, counters[1] += key/value tiles staged (device).
hipError_t launch_prefill_bf16_counted(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int H, int Hkv, int n, int d,
                                       int causal, int window, float scale,
                                       unsigned long long* counters, hipStream_t stream);
// Ragged batch: q, o [H, total, d]; k, v [Hkv, total, d]; lse [H, total];
// cu_seqlens [B+1] device offsets.
hipError_t launch_prefill_bf16_varlen(const void* q, const void* k, const void* v, void* o,
                                      float* lse, const int* cu_seqlens, int B, int H, int Hkv,
                                      int total, int max_seqlen, int d, int causal, int window,
                                      float scale, hipStream_t stream);
// Chunks over paged histories: q, o [H, total_q, d]; lse [H, total_q];
// caches [num_pages, Hkv, 16, d]; page_table [B, max_pages].
hipError_t launch_prefill_bf16_paged(const void* q, const void* kcache, const void* vcache,
                                     const int* page_table, const int* cu_seqlens_q,
                                     const int* seqlens_k, void* o, float* lse, int B, int H,
                                     int Hkv, int d, int total_q, int max_seqlen_q, int num_pages,
                                     int max_pages, int causal, int window, float scale,
                                     hipStream_t stream);
// Block-sparse: dense layout plus layout [layout_heads, ceil(n/128), ceil(n/block_k)].
hipError_t launch_prefill_bf16_blocksparse(const void* q, const void* k, const void* v, void* o,
                                           float* lse, const unsigned char* layout,
                                           int layout_heads, int B, int H, int Hkv, int n, int d,
                                           int block_k, int causal, int window, float scale,
                                           hipStream_t stream);
// Strided dense problem: strides[12] (elements) = q (batch, head, row), k (...),
// v (...), o (...); k and v share the row stride.
hipError_t launch_prefill_bf16_strided(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const long long* strides, int B, int H,
                                       int Hkv, int n, int d, int causal, int window, float scale,
                                       hipStream_t stream);
hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* o,
                              float* lse, int B, int H, int Hkv, int n, int d,
                              int causal, int window, float scale, hipStream_t stream);

// Decode: tokens per split and the workspace the split partials need.
int decode_split_pages(int B, int H, int max_seqlen);
int decode_max_splits(int B, int H, int max_seqlen);
size_t decode_workspace_bytes(int B, int H, int max_seqlen, int d);
// FP8 decode: caches of E4M3 bytes, scales [Hkv] (device).
hipError_t launch_decode_fp8(const void* q, const void* kcache, const void* vcache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* page_table, const int32_t* seqlens, void* o,
                             float* lse, int B, int H, int Hkv, int d, int num_pages,
                             int max_pages, int max_seqlen, float scale, void* workspace,
                             hipStream_t stream);
hipError_t launch_decode(const void* q, const void* kcache, const void* vcache,
                         const int32_t* page_table, const int32_t* seqlens, void* o,
                         float* lse, int B, int H, int Hkv, int d, int num_pages,
                         int max_pages, int max_seqlen, float scale, void* workspace,
                         hipStream_t stream);
// Decode with the split partials in the library's static device array
// (kDecodeScratchBytes per device) instead of a caller workspace; fails with
// hipErrorInvalidValue when the partials would not fit.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t launch_decode_static(const void* q, const void* kcache, const void* vcache,
                                const int32_t* page_table, const int32_t* seqlens, void* o,
                                float* lse, int B, int H, int Hkv, int d, int num_pages,
                                int max_pages, int max_seqlen, float scale,
                                hipStream_t stream);

// Backward: delta workspace [B,H,n] floats; window clamped as for prefill.
size_t bwd_workspace_bytes(int B, int H, int n);
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* delta, int B, int H, int Hkv, int n, int d, int causal,
                           int window, float scale, hipStream_t stream);

}  // namespace fa

// C ABI of libfa.so (declared in include/fa.h): argument checks on the host,
// then dispatch to the gfx950 kernels.  Nothing here allocates, frees or
// synchronises; every kernel is enqueued on the caller's stream.

#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>

#include "launch.hpp"

static_assert(FA_DECODE_NOALLOC_MAX_BYTES == fa::kDecodeScratchBytes,
              "the header states the library's static decode array size");

namespace {

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

bool fits_i32(long long x) { return x >= 0 && x < (long long)INT_MAX; }

// Workgroups of a prefill or backward grid: one per 128 query rows of every
// (batch, head).  The 1-D grid and the kernels' block indices are 32-bit.
bool grid_ok(long long rows, long long B, long long H) {
  return fits_i32((rows + 127) / 128 * B * H);
}

}  // namespace

extern "C" {

int fa_version(void) { return (1 << 16) | 5; }

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "sizes out of range or inconsistent";
    case FA_ERR_UNSUPPORTED: return "request not supported by this build";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_LAUNCH: return "kernel launch rejected by the HIP runtime";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int Hkv, int n, int d, int causal, int window, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || n < 1 || d < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)n * d)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)B * H) || !grid_ok(n, B, H)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // A window of n or more restricts nothing; clamp so index sums cannot overflow.
  if (window < 0) window = -1;
  if (window > n) window = n;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == FA_BF16)
    e = fa::launch_prefill_bf16(q, k, v, o, lse, B, H, Hkv, n, d, causal, window, scale, st);
  else if (dtype == FA_F32)
    e = fa::launch_prefill_f32(q, k, v, o, lse, B, H, Hkv, n, d, causal, window, scale, st);
  else
    return FA_ERR_UNSUPPORTED;
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_tile_count(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Hkv, int n, int d, int causal, int window, float scale,
                      unsigned long long* counters, void* stream) {
  if (!counters) return FA_ERR_NULL;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || n < 1 || d < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)n * d)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)B * H) || !grid_ok(n, B, H)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (window < 0) window = -1;
  if (window > n) window = n;
  hipError_t e = fa::launch_prefill_bf16_counted(q, k, v, o, lse, B, H, Hkv, n, d, causal, window,
                                                 scale, counters,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen,
                  int d, int causal, int window, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || total < 1 || max_seqlen < 1 || d < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)total * d) || !fits_i32((long long)B * H) ||
      !fits_i32((long long)B + 1) || !grid_ok(std::min(max_seqlen, total), B, H))
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (max_seqlen > total) max_seqlen = total;
  if (window < 0) window = -1;
  if (window > max_seqlen) window = max_seqlen;
  hipError_t e = fa::launch_prefill_bf16_varlen(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total,
                                                max_seqlen, d, causal, window, scale,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int64_t* strides, int B, int H, int Hkv, int n, int d, int causal,
                   int window, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !strides) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || n < 1 || d < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)n * d) || !fits_i32((long long)B * H) || !grid_ok(n, B, H))
    return FA_ERR_SHAPE;
  for (int i = 0; i < 12; ++i)
    if (strides[i] < 0 || strides[i] % 8 != 0) return FA_ERR_SHAPE;
  const long long rs[4] = {strides[2], strides[5], strides[8], strides[11]};
  for (long long r : rs)
    if (r < d || r > (1LL << 24)) return FA_ERR_SHAPE;
  if (strides[5] != strides[8]) return FA_ERR_SHAPE;  // k and v row strides
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (window < 0) window = -1;
  if (window > n) window = n;
  long long st[12];
  for (int i = 0; i < 12; ++i) st[i] = strides[i];
  hipError_t e = fa::launch_prefill_bf16_strided(q, k, v, o, lse, st, B, H, Hkv, n, d, causal,
                                                 window, scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       const uint8_t* layout, int layout_heads, int B, int H, int Hkv, int n,
                       int d, int block_q, int block_k, int causal, int window, float scale,
                       int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !layout) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || n < 1 || d < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (layout_heads != 1 && layout_heads != H) return FA_ERR_SHAPE;
  if (!fits_i32((long long)n * d) || !fits_i32((long long)B * H) || !grid_ok(n, B, H))
    return FA_ERR_SHAPE;
  if (n > 131072) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (block_q != 128 || (block_k != 64 && block_k != 128)) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (window < 0) window = -1;
  if (window > n) window = n;
  hipError_t e = fa::launch_prefill_bf16_blocksparse(q, k, v, o, lse, layout, layout_heads, B,
                                                     H, Hkv, n, d, block_k, causal, window,
                                                     scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_paged(const void* q, const void* kcache, const void* vcache, const int32_t* page_table,
                 const int32_t* cu_seqlens_q, const int32_t* seqlens_k, void* o, float* lse,
                 int B, int H, int Hkv, int d, int total_q, int max_seqlen_q, int num_pages,
                 int page_size, int max_pages, int causal, int window, float scale, int dtype,
                 void* stream) {
  if (!q || !kcache || !vcache || !page_table || !cu_seqlens_q || !seqlens_k || !o || !lse)
    return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || d < 1 || total_q < 1 || max_seqlen_q < 1 || num_pages < 1 ||
      page_size < 1 || max_pages < 1)
    return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)total_q * d) || !fits_i32((long long)B * H) ||
      !fits_i32((long long)B * max_pages) || !fits_i32((long long)max_pages * 16) ||
      !fits_i32((long long)B + 1) || !grid_ok(std::min(max_seqlen_q, total_q), B, H))
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 16 || dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (max_seqlen_q > total_q) max_seqlen_q = total_q;
  if (window < 0) window = -1;
  if (window > max_pages * 16) window = max_pages * 16;
  hipError_t e = fa::launch_prefill_bf16_paged(q, kcache, vcache, page_table, cu_seqlens_q,
                                               seqlens_k, o, lse, B, H, Hkv, d, total_q,
                                               max_seqlen_q, num_pages, max_pages, causal,
                                               window, scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_decode_workspace_bytes(int B, int H, int max_seqlen, int d) {
  if (B < 1 || H < 1 || max_seqlen < 1 || d < 1) return 0;
  return fa::decode_workspace_bytes(B, H, max_seqlen, d);
}

int fa_decode(const void* q, const void* kcache, const void* vcache, const int32_t* page_table,
              const int32_t* seqlens, void* o, float* lse, int B, int H, int Hkv, int d,
              int num_pages, int page_size, int max_pages, int max_seqlen, float scale,
              void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !kcache || !vcache || !page_table || !seqlens || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || d < 1 || num_pages < 1 || page_size < 1 || max_pages < 1 ||
      max_seqlen < 1)
    return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)B * H) || !fits_i32((long long)B * max_pages) ||
      !fits_i32((long long)max_pages * 16))
    return FA_ERR_SHAPE;
  if ((d != 64 && d != 128) || page_size != 16 || H / Hkv > 16) return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < fa::decode_workspace_bytes(B, H, max_seqlen, d))
    return FA_ERR_WORKSPACE;
  hipError_t e = fa::launch_decode(q, kcache, vcache, page_table, seqlens, o, lse, B, H, Hkv, d,
                                   num_pages, max_pages, max_seqlen, scale, workspace,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                      const int32_t* page_table, const int32_t* seqlens, void* o, float* lse,
                      int B, int H, int Hkv, int d, int num_pages, int page_size, int max_pages,
                      int max_seqlen, float scale, void* stream) {
  if (!q || !kcache || !vcache || !page_table || !seqlens || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || d < 1 || num_pages < 1 || page_size < 1 || max_pages < 1 ||
      max_seqlen < 1)
    return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)B * H) || !fits_i32((long long)B * max_pages) ||
      !fits_i32((long long)max_pages * 16))
    return FA_ERR_SHAPE;
  if ((d != 64 && d != 128) || page_size != 16 || H / Hkv > 16) return FA_ERR_UNSUPPORTED;
  if (fa::decode_workspace_bytes(B, H, max_seqlen, d) > fa::kDecodeScratchBytes)
    return FA_ERR_WORKSPACE;
  hipError_t e = fa::launch_decode_static(q, kcache, vcache, page_table, seqlens, o, lse, B, H,
                                          Hkv, d, num_pages, max_pages, max_seqlen, scale,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_decode_fp8(const void* q, const void* kcache, const void* vcache, const float* k_scale,
                  const float* v_scale, const int32_t* page_table, const int32_t* seqlens,
                  void* o, float* lse, int B, int H, int Hkv, int d, int num_pages,
                  int page_size, int max_pages, int max_seqlen, float scale, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!q || !kcache || !vcache || !k_scale || !v_scale || !page_table || !seqlens || !o || !lse)
    return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || d < 1 || num_pages < 1 || page_size < 1 || max_pages < 1 ||
      max_seqlen < 1)
    return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)B * H) || !fits_i32((long long)B * max_pages) ||
      !fits_i32((long long)max_pages * 16))
    return FA_ERR_SHAPE;
  if ((d != 64 && d != 128) || page_size != 16 || H / Hkv > 16) return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < fa::decode_workspace_bytes(B, H, max_seqlen, d))
    return FA_ERR_WORKSPACE;
  hipError_t e = fa::launch_decode_fp8(q, kcache, vcache, k_scale, v_scale, page_table, seqlens,
                                       o, lse, B, H, Hkv, d, num_pages, max_pages, max_seqlen,
                                       scale, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_workspace_bytes(int B, int H, int n, int d) {
  if (B < 1 || H < 1 || n < 1 || d < 1) return 0;
  if (!fits_i32((long long)B * H) || !fits_i32((long long)n * d)) return 0;
  return fa::bwd_workspace_bytes(B, H, n);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, float* dq, float* dk, float* dv, int B, int H, int Hkv, int n, int d,
           int causal, int window, float scale, int dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Hkv < 1 || n < 1 || d < 1) return FA_ERR_SHAPE;
  if (H % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)n * d)) return FA_ERR_SHAPE;
  if (!fits_i32((long long)B * H) || !grid_ok(n, B, H)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < fa::bwd_workspace_bytes(B, H, n)) return FA_ERR_WORKSPACE;
  if (window < 0) window = -1;
  if (window > n) window = n;
  hipError_t e = fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv,
                                     static_cast<float*>(workspace), B, H, Hkv, n, d, causal,
                                     window, scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

// float32 attention prefill (vector ALU, fp32 storage and arithmetic).
//
// Same tiled method as the bf16 kernel (xxqk.cn sliding-window prefill
// article §3.1-§3.2 for tiles and the online softmax, §5.1-§5.3 for visiting
// only key tiles inside the band and masking the straddling ones), kept in
// float32 end to end: no bf16 rounding anywhere.  Intended for small
// latency-bound problems; one lane owns one query row.
//
// Layout: workgroup = one wave of 64 lanes = 64 query rows of one (b, h);
// key/value tiles of 32 rows staged in LDS and read back as broadcasts.

#include "common.hpp"
#include "launch.hpp"

namespace fa {

struct PrefillF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, H, Hkv, n, causal, window, nqb;
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillF32Args a) {
  constexpr int BQ = 64, BC = 32;
  __shared__ __attribute__((aligned(16))) float Ks[BC * D];
  __shared__ __attribute__((aligned(16))) float Vs[BC * D];

  const int lane = threadIdx.x;
  const int n = a.n;
  const int qb = blockIdx.x % a.nqb;
  const int bh = blockIdx.x / a.nqb;
  const int b = bh / a.H, h = bh - b * a.H;
  const int g = h / (a.H / a.Hkv);
  const float* Qh = a.q + (size_t)(b * a.H + h) * n * D;
  const float* Kh = a.k + (size_t)(b * a.Hkv + g) * n * D;
  const float* Vh = a.v + (size_t)(b * a.Hkv + g) * n * D;
  const int causal = a.causal, window = a.window;
  auto lo_of = [&](int i) { return window >= 0 ? i - window : 0; };
  auto hi_of = [&](int i) {
    int v = causal ? i : (window >= 0 ? i + window : n - 1);
    return v < n - 1 ? v : n - 1;
  };

  const int q0 = qb * BQ;
  const int qlast = min(q0 + BQ, n) - 1;
  const int kt_lo = max(lo_of(q0), 0) / BC;
  const int kt_hi = hi_of(qlast) / BC;
  const int row = q0 + lane;
  const bool valid = row < n;
  const int rlo = lo_of(row), rhi = hi_of(row);

  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    f32x4 x = valid ? *reinterpret_cast<const f32x4*>(Qh + (size_t)row * D + d) : f32x4{};
    q[d] = x[0]; q[d + 1] = x[1]; q[d + 2] = x[2]; q[d + 3] = x[3];
    acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.f;
  }
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.scale_log2;

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int k0 = kt * BC;
    __syncthreads();
#pragma unroll
    for (int i = lane; i < BC * D / 4; i += 64) {
      const int r = i / (D / 4), c = (i - r * (D / 4)) * 4;
      const int key = k0 + r;
      f32x4 kx{}, vx{};
      if (key < n) {
        kx = *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + c);
        vx = *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + c);
      }
      *reinterpret_cast<f32x4*>(Ks + r * D + c) = kx;
      *reinterpret_cast<f32x4*>(Vs + r * D + c) = vx;
    }
    __syncthreads();

    float s[BC];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const f32x4 kx = *reinterpret_cast<const f32x4*>(Ks + j * D + d);
        dot = __builtin_fmaf(q[d], kx[0], dot);
        dot = __builtin_fmaf(q[d + 1], kx[1], dot);
        dot = __builtin_fmaf(q[d + 2], kx[2], dot);
        dot = __builtin_fmaf(q[d + 3], kx[3], dot);
      }
      const int key = k0 + j;
      s[j] = (key < rlo || key > rhi) ? kNegInf : dot;
      mx = fmax2(mx, s[j]);
    }
    const float m_new = fmax2(m_run, mx * c2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      s[j] = exp2_fast(__builtin_fmaf(s[j], c2, -m_use));
      rs += s[j];
    }
    l_run = alpha * l_run + rs;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const f32x4 vx = *reinterpret_cast<const f32x4*>(Vs + j * D + d);
        acc[d] = __builtin_fmaf(s[j], vx[0], acc[d]);
        acc[d + 1] = __builtin_fmaf(s[j], vx[1], acc[d + 1]);
        acc[d + 2] = __builtin_fmaf(s[j], vx[2], acc[d + 2]);
        acc[d + 3] = __builtin_fmaf(s[j], vx[3], acc[d + 3]);
      }
    }
  }

  if (!valid) return;
  const float inv = 1.f / l_run;
  float* orow = a.o + ((size_t)(b * a.H + h) * n + row) * D;
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    f32x4 x;
    x[0] = acc[d] * inv; x[1] = acc[d + 1] * inv; x[2] = acc[d + 2] * inv; x[3] = acc[d + 3] * inv;
    *reinterpret_cast<f32x4*>(orow + d) = x;
  }
  const float m_use = (m_run == kNegInf) ? 0.f : m_run;
  a.lse[(size_t)(b * a.H + h) * n + row] = (m_use + log2_fast(l_run)) * kLn2;
}

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Hkv, int n, int d, int causal, int window,
                              float scale, hipStream_t stream) {
  PrefillF32Args a;
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.o = static_cast<float*>(o);
  a.lse = lse;
  a.B = B; a.H = H; a.Hkv = Hkv; a.n = n; a.causal = causal; a.window = window;
  a.nqb = (n + 63) / 64;
  a.scale_log2 = scale * kLog2e;
  const long long grid = (long long)a.nqb * B * H;
  if (d == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)grid), dim3(64), 0, stream, a);
  else if (d == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)grid), dim3(64), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa

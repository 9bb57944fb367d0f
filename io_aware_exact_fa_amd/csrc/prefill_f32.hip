// float32 attention prefill (vector ALU, fp32 storage and arithmetic).
//
// Same tiled method as the bf16 kernel (xxqk.cn sliding-window prefill
// article §3.1-§3.2 for tiles and the online softmax, §5.1-§5.3 for visiting
// only key tiles inside the band and masking the straddling ones), kept in
// float32 end to end: no bf16 rounding anywhere.  Intended for small
// latency-bound problems.
//
// Layout: a workgroup owns 64 query rows of one (b, h); each of its NW waves
// holds all 64 rows (one lane per row) and takes every NW-th key tile of the
// band, staged in its own LDS buffer and read back as broadcasts, so the loop
// needs no workgroup barrier.  Each wave keeps its own running max, sum and
// accumulator; at the end the NW partial softmaxes are merged through LDS with
// the rescaling of the online update: weights exp(m_w - M), M the largest
// partial max (the split-and-merge of the same article's §3.2 algebra that
// the decode kernel applies across splits).  Splitting the keys over waves
// cuts the serial chain of a lane NW-fold, which is what bounds these sizes.

#include "common.hpp"
#include "launch.hpp"

namespace fa {

template <int D>
struct F32Shape {
  static constexpr int NW = D == 64 ? 8 : 4;  // waves per workgroup
  static constexpr int BC = 2048 / D;         // keys per tile: 16 KB of K+V per wave
  static constexpr int BQ = 64;               // query rows per workgroup
  static constexpr int STAGE = NW * 2 * BC * D * 4;
  static constexpr int MERGE = NW * BQ * D * 4;
  static constexpr int LDS = STAGE > MERGE ? STAGE : MERGE;
};

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
__global__ __launch_bounds__(F32Shape<D>::NW * 64) void prefill_f32_kernel(PrefillF32Args a) {
  using S = F32Shape<D>;
  constexpr int BQ = S::BQ, BC = S::BC, NW = S::NW;
  static_assert(S::LDS + 2 * NW * BQ * 4 <= 160 * 1024, "LDS budget");
  // Staging tiles during the loop, the waves' partial accumulators after it.
  __shared__ __attribute__((aligned(16))) char smem[S::LDS];
  __shared__ float sm[NW][BQ], sl[NW][BQ];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
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
  float* Ks = reinterpret_cast<float*>(smem) + wave * 2 * BC * D;
  float* Vs = Ks + BC * D;

  for (int kt = kt_lo + wave; kt <= kt_hi; kt += NW) {
    const int k0 = kt * BC;
    // The wave's own buffer: its previous reads precede these writes in the
    // wave's in-order LDS stream; the fence orders the writes before the reads
    // of other lanes below.
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
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();

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

  // ---- merge the waves' partial softmaxes ----
  sm[wave][lane] = m_run;
  sl[wave][lane] = l_run;
  __syncthreads();  // every wave is past its loop: the staging buffers are free
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmax2(M, sm[w][lane]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L = __builtin_fmaf(exp2_fast(sm[w][lane] - Mu), sl[w][lane], L);
  // Partial accumulators, weighted, as [wave][dim][row]: a lane's stores and
  // the reads below touch consecutive words across the wave.
  float* part = reinterpret_cast<float*>(smem);
  const float wgt = exp2_fast(m_run - Mu);
#pragma unroll
  for (int d = 0; d < D; ++d) part[(wave * D + d) * BQ + lane] = acc[d] * wgt;
  __syncthreads();
  if (!valid) return;
  // Wave w finishes dims [w*D/NW, (w+1)*D/NW) of every row.
  constexpr int DW = D / NW;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* orow = a.o + ((size_t)(b * a.H + h) * n + row) * D + wave * DW;
#pragma unroll
  for (int d = 0; d < DW; d += 4) {
    f32x4 x = f32x4{};
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += part[(w * D + wave * DW + d + e) * BQ + lane];
    *reinterpret_cast<f32x4*>(orow + d) = x * inv;
  }
  if (wave == 0)
    a.lse[(size_t)(b * a.H + h) * n + row] = L > 0.f ? (Mu + log2_fast(L)) * kLn2 : kNegInf;
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
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)grid),
                       dim3(F32Shape<128>::NW * 64), 0, stream, a);
  else if (d == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)grid),
                       dim3(F32Shape<64>::NW * 64), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa

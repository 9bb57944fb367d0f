// bf16 attention prefill on gfx950 matrix cores (MFMA), fp32 accumulation.
//
// Method (web pages on IO-aware exact attention):
//   * xxqk.cn sliding-window prefill article §3.1-§3.2: one workgroup per query
//     tile; the key/value tiles stream through on-chip memory; per query row a
//     running max m, running sum l and an accumulator rescaled by
//     exp(m_old - m_new) when m grows; the output is acc / l.
//   * same article §5.1/§5.3/§7.3: the workgroup visits only the key tiles whose
//     index range meets the band of its query rows; §5.2: tiles that straddle
//     the band edge get a -inf mask before the max/sum update; §5.5: skipping a
//     tile that would be all -inf is exact.
//   * ruiowl.com deep-dive page §二: tiles of 64-128 tokens, one query tile and
//     the matching key/value tile on chip at a time.
//
// gfx950 design (prior art above is NVIDIA-shaped; this is not a translation):
//   * Workgroup = NW waves of 64 lanes; wave w owns 32*NQB query rows.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims (one ds_read_b128 per
//     lane from LDS), B = Q^T fragment held in VGPRs for the whole loop.  In the
//     32x32 accumulator layout lane l owns query column l%32 and 16 key rows,
//     so the row max / row sum of a query is a 16-value in-lane reduction plus
//     one cross-half swap (v_permlane32_swap) -- no LDS round trip.
//   * The same registers, rounded to bf16, are directly the B operand P^T of
//     the O^T += V^T P^T MFMA: the MFMA's k index is mapped onto the key order
//     the accumulator layout produced, and V^T is gathered from LDS to match.
//   * Softmax runs in the base-2 domain: scale*log2(e) is folded into one FMA
//     before v_exp_f32.
//   * K/V tiles are double-buffered in LDS; the next tile's global loads are
//     in flight while the current tile is computed; one barrier per tile.
//   * Grid order: heaviest causal query tiles first; inside each round of B*H
//     tiles, workgroups that share a key/value head are placed on the same XCD
//     (dispatch is round-robin over the 8 XCDs), so their K/V reads share L2.

#include "common.hpp"
#include "launch.hpp"

namespace fa {

struct PrefillArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int B, H, Hkv, n, causal, window, nqb;
  float scale_log2;  // scale * log2(e)
};

template <int D, int NW, int NQB, int BC>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int BR = NW * 32 * NQB;   // query rows per workgroup
  constexpr int LS = D + 8;           // LDS row stride in elements (16 B pad)
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CPT = BC * CPR / NT;  // chunks per thread per tensor per tile
  constexpr int NKB = BC / 32;        // 32-key MFMA blocks per tile
  constexpr int NDC = D / 16;         // 16-wide head-dim chunks (QK^T contraction)
  constexpr int NDB = D / 32;         // 32-wide head-dim blocks (PV output)
  constexpr int NKC = BC / 16;        // 16-key chunks (PV contraction)
  static_assert(BC * CPR % NT == 0, "tile must split evenly over threads");

  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BC * LS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int n = a.n;
  const int BH = a.B * a.H;

  // ---- workgroup -> (b, h, query tile) ----
  const int idx = blockIdx.x;
  const int round = idx / BH;
  const int p = idx - round * BH;
  const int qb = a.causal ? (a.nqb - 1 - round) : round;
  int bh = p;
  if ((BH & 7) == 0) bh = (p & 7) * (BH >> 3) + (p >> 3);
  const int b = bh / a.H, h = bh - b * a.H;
  const int g = h / (a.H / a.Hkv);
  const __bf16* Qh = a.q + (size_t)(b * a.H + h) * n * D;
  const __bf16* Kh = a.k + (size_t)(b * a.Hkv + g) * n * D;
  const __bf16* Vh = a.v + (size_t)(b * a.Hkv + g) * n * D;
  __bf16* Oh = a.o + (size_t)(b * a.H + h) * n * D;
  float* Lh = a.lse + (size_t)(b * a.H + h) * n;

  const int causal = a.causal, window = a.window;
  // Visible keys of row i form the interval [lo(i), hi(i)], both monotone in i.
  auto lo_of = [&](int i) { return window >= 0 ? i - window : 0; };
  auto hi_of = [&](int i) {
    int v = causal ? i : (window >= 0 ? i + window : n - 1);
    return v < n - 1 ? v : n - 1;
  };

  const int q0 = qb * BR;
  const int qlast = min(q0 + BR, n) - 1;
  const int kt_lo = max(lo_of(q0), 0) / BC;
  const int kt_hi = hi_of(qlast) / BC;

  // ---- this wave's query rows ----
  const int wq0 = q0 + wave * 32 * NQB;
  const bool wave_rows = wq0 < n;
  const int wr1 = min(wq0 + 32 * NQB, n) - 1;
  const int wlo0 = lo_of(wq0), whi0 = hi_of(wq0);
  const int wlo1 = lo_of(wr1), whi1 = hi_of(wr1);

  bf16x8 qf[NQB][NDC];
#pragma unroll
  for (int nq = 0; nq < NQB; ++nq) {
    const int row = wq0 + nq * 32 + l32;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      if (row < n)
        qf[nq][dc] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)row * D + dc * 16 + hi * 8);
      else
        qf[nq][dc] = bf16x8{};
    }
  }

  f32x16 acc[NQB][NDB];
  float m_run[NQB], l_run[NQB];
#pragma unroll
  for (int nq = 0; nq < NQB; ++nq) {
    m_run[nq] = kNegInf;
    l_run[nq] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[nq][db] = f32x16{};
  }

  // ---- K/V staging: global -> registers -> LDS ----
  u32x4 stK[CPT], stV[CPT];
  auto gload = [&](int kt) {
    const int k0 = kt * BC;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      const int r = ch / CPR, cc = ch - (ch / CPR) * CPR;
      const int key = k0 + r;
      if (key < n) {
        stK[c] = *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + cc * 8);
        stV[c] = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + cc * 8);
      } else {
        stK[c] = u32x4{};
        stV[c] = u32x4{};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      const int r = ch / CPR, cc = ch - (ch / CPR) * CPR;
      *reinterpret_cast<u32x4*>(&smem[buf][0][r * LS + cc * 8]) = stK[c];
      *reinterpret_cast<u32x4*>(&smem[buf][1][r * LS + cc * 8]) = stV[c];
    }
  };

  const float c2 = a.scale_log2;

  gload(kt_lo);
  sstore(0);
  __syncthreads();

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int buf = (kt - kt_lo) & 1;
    if (kt < kt_hi) gload(kt + 1);
    const int k0 = kt * BC, k1 = k0 + BC - 1;
    // Wave-level classification of this tile against the wave's rows.
    const bool active = wave_rows && !(k1 < wlo0 || k0 > whi1);
    const bool full = (k0 >= wlo1) && (k1 <= whi0);
    if (active) {
      const __bf16* Ks = smem[buf][0];
      const __bf16* Vs = smem[buf][1];
      // S^T = K Q^T for NKB key blocks x NQB query blocks.
      f32x16 s[NQB][NKB];
#pragma unroll
      for (int nq = 0; nq < NQB; ++nq)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[nq][kb] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + l32) * LS + dc * 16 + hi * 8);
#pragma unroll
          for (int nq = 0; nq < NQB; ++nq)
            s[nq][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nq][dc], s[nq][kb], 0, 0, 0);
        }
      }
      // Online softmax, one query row per lane (pair of lanes l, l^32).
      bf16x8 pf[NQB][NKC];
#pragma unroll
      for (int nq = 0; nq < NQB; ++nq) {
        if (!full) {
          const int row = wq0 + nq * 32 + l32;
          const int rlo = lo_of(row), rhi = hi_of(row);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (key < rlo || key > rhi) s[nq][kb][r] = kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmax2(mx, s[nq][kb][r]);
        mx = max_xor32(mx);
        const float m_new = fmax2(m_run[nq], mx * c2);
        // A row with no visible key so far keeps m = -inf; use 0 so that
        // exp2(-inf - m) stays 0 instead of NaN.
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run[nq] - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = exp2_fast(__builtin_fmaf(s[nq][kb][r], c2, -m_use));
            rs += pv;
            pf[nq][kb * 2 + (r >> 3)][r & 7] = (__bf16)pv;
          }
        l_run[nq] = alpha * l_run[nq] + rs;
        m_run[nq] = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[nq][db] *= alpha;
      }
      // O^T += V^T P^T.  MFMA k index kk = 8*hi + t stands for key
      // 16*kc + 8*(t/4) + 4*hi + t%4, the order the S^T accumulator holds.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          bf16x8 vf;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int key = kc * 16 + 8 * (t >> 2) + 4 * hi + (t & 3);
            vf[t] = Vs[key * LS + db * 32 + l32];
          }
#pragma unroll
          for (int nq = 0; nq < NQB; ++nq)
            acc[nq][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nq][kc], acc[nq][db], 0, 0, 0);
        }
      }
    }
    if (kt < kt_hi) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, lse = ln(2) * (m + log2 l) ----
  if (!wave_rows) return;
#pragma unroll
  for (int nq = 0; nq < NQB; ++nq) {
    const int row = wq0 + nq * 32 + l32;
    const float lt = sum_xor32(l_run[nq]);
    if (row >= n) continue;
    const float inv = 1.f / lt;
    __bf16* orow = Oh + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(acc[nq][db][4 * g4 + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g4 + 4 * hi) = ov;
      }
    if (hi == 0) {
      const float m_use = (m_run[nq] == kNegInf) ? 0.f : m_run[nq];
      Lh[row] = (m_use + log2_fast(lt)) * kLn2;
    }
  }
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a0, int B, int H, int n, hipStream_t stream) {
  constexpr int NW = 4, NQB = 1, BC = 64;
  constexpr int BR = NW * 32 * NQB;
  PrefillArgs a = a0;
  a.nqb = (n + BR - 1) / BR;
  const long long grid = (long long)a.nqb * B * H;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, NQB, BC>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Hkv, int n, int d, int causal, int window,
                               float scale, hipStream_t stream) {
  PrefillArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.n = n;
  a.causal = causal;
  a.window = window;
  a.nqb = 0;
  a.scale_log2 = scale * kLog2e;
  if (d == 128) return launch_d<128>(a, B, H, n, stream);
  if (d == 64) return launch_d<64>(a, B, H, n, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

// Paged flash-decoding on gfx950: split-KV partial softmax + log-sum-exp merge.
//
// Method: one new query token per sequence reads its whole key/value history,
// so the work is parallelised along that history rather than along queries
// (charles2530 blog "算子与编译器：FlashAttention 与长上下文" §4 and §6.2); the
// history lives in fixed-size pages reached through a per-sequence page table
// (same page §5; xxqk.cn sliding-window prefill article §8.2).  Each split
// computes an exact softmax over its pages with the running max / running sum
// of the tiled method (xxqk.cn article §3.2); the merge applies the same
// rescaling algebra across splits: partial outputs are weighted by
// exp(lse_s - lse), lse = log sum_s exp(lse_s).
//
// gfx950 design (HBM bound: every K/V byte is read exactly once):
//   * One workgroup per (sequence b, key/value head g, split of SPLIT pages);
//     its 4 waves take the split's pages round-robin.  All G = H/Hkv query
//     heads of the group are served from the same K/V bytes.
//   * Scores: v_mfma_f32_16x16x32_bf16 with A = the page's 16 tokens x 32 dims
//     loaded straight from HBM into the A-operand layout (16 B per lane), B =
//     the G query vectors (columns >= G are zero).  In the 16x16 accumulator
//     lane l owns query column l%16 and 4 tokens; max/sum over the page's 16
//     tokens are 4 in-lane values plus two lane swaps (permlane16/32).
//   * Probabilities go through a 1 KB LDS slab per wave; P.V runs on the vector
//     ALU with each lane owning 8 head dims of one token row, so V rows are
//     read with coalesced 16 B loads and no transpose is needed.
//   * Waves merge in LDS at the end; the split writes a normalised fp32
//     partial output and its base-2 log-sum-exp to the workspace.
//   * The merge kernel reads the valid splits of each (b, h) and writes bf16
//     output and the natural-log lse.

#include "common.hpp"
#include "launch.hpp"

namespace fa {

constexpr int kPage = 16;
constexpr int kDecodeWaves = 4;

struct DecodeArgs {
  const __bf16* q;
  const __bf16* kc;
  const __bf16* vc;
  const int32_t* page_table;
  const int32_t* seqlens;
  float* ws_o;    // [B, H, max_splits, D]
  float* ws_lse;  // [B, H, max_splits]   base-2 log-sum-exp, scale included
  __bf16* o;
  float* lse;
  int B, H, Hkv, G, num_pages, max_pages, max_seqlen, split_pages, max_splits;
  float scale_log2;
};

__device__ __forceinline__ int decode_len(const DecodeArgs& a, int b) {
  int L = a.seqlens[b];
  const int cap = min(a.max_seqlen, a.max_pages * kPage);
  L = L < 0 ? 0 : L;
  return L > cap ? cap : L;
}

// Threshold (base-2 exponent units) for moving a query's reference max; see
// the prefill kernel: the result is unchanged, most pages skip the rescale.
constexpr float kDecodeRescaleThreshold = 8.0f;

template <int D, int GP>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_split_kernel(DecodeArgs a) {
  static_assert(D == 128, "decode kernel is written for head dim 128");
  constexpr int NC = D / 32;  // 32-dim chunks of the QK contraction
  __shared__ float Pl[kDecodeWaves][kPage * GP];
  __shared__ float Wm[kDecodeWaves][GP];
  __shared__ float Wl[kDecodeWaves][GP];
  __shared__ float Wacc[kDecodeWaves][GP][D];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = decode_len(a, b);
  const int npg = (L + kPage - 1) / kPage;
  const int p0 = s * a.split_pages;
  if (p0 >= npg) return;  // whole workgroup exits together
  const int p1 = min(p0 + a.split_pages, npg);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int G = a.G;

  // This wave's pages are p0 + wave + 4*i, i < cnt; their physical ids are
  // read once, one per lane, and broadcast with readlane in the loop.
  const int cnt = p1 - p0 > wave ? (p1 - p0 - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
  const int32_t* table = a.page_table + (size_t)b * a.max_pages;
  int my_phys = -1;
  if (lane < cnt) my_phys = table[p0 + wave + kDecodeWaves * lane];

  // Query fragments: B operand (32 dims x 16 query columns) per chunk.
  bf16x8 qf[NC];
  {
    const __bf16* qrow = a.q + ((size_t)b * a.H + (size_t)g * G + col) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = (col < G) ? *reinterpret_cast<const bf16x8*>(qrow + 32 * c + 8 * grp) : bf16x8{};
  }

  float m_ref = kNegInf, l_part = 0.f;
  float acc[GP][8];
#pragma unroll
  for (int qq = 0; qq < GP; ++qq)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qq][e] = 0.f;

  const float c2 = a.scale_log2;

  // Registers of one page: K in the MFMA A-operand layout (token = lane%16,
  // dims 32c + 8*(lane/16) .. +8) and four V rows (token lane/16 + 4i, dims
  // 8*(lane%16) .. +8).  A page id outside [0, num_pages) is replaced by page
  // 0 for the load and all its tokens are masked.
  struct PageRegs {
    bf16x8 k[NC];
    u32x4 v[4];
  };
  auto load_page = [&](int i, PageRegs& r) {
    int phys = __builtin_amdgcn_readlane(my_phys, i);
    if (phys < 0 || phys >= a.num_pages) phys = 0;
    const size_t base = ((size_t)phys * a.Hkv + g) * kPage * D;
    const __bf16* kp = a.kc + base;
    const __bf16* vp = a.vc + base;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      r.k[c] = *reinterpret_cast<const bf16x8*>(kp + col * D + 32 * c + 8 * grp);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      r.v[i4] = *reinterpret_cast<const u32x4*>(vp + (grp + 4 * i4) * D + 8 * col);
  };

  auto process_page = [&](int i, const PageRegs& r) {
    const int phys = __builtin_amdgcn_readlane(my_phys, i);
    const bool valid = phys >= 0 && phys < a.num_pages;
    const int tok0 = (p0 + wave + kDecodeWaves * i) * kPage;
    // Tokens at or past `lim` are masked (the sequence end, or the whole page
    // when its id is invalid).
    const int lim = valid ? L : tok0;
    const bool tail = tok0 + kPage > lim;

    f32x4 sc = f32x4{};
#pragma unroll
    for (int c = 0; c < NC; ++c) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[c], qf[c], sc, 0, 0, 0);
    if (tail) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (tok0 + 4 * grp + rr >= lim) sc[rr] = kNegInf;
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3]));
    mx = max_xor32(max_xor16(mx)) * c2;
    const bool need = mx > m_ref + kDecodeRescaleThreshold;
    const float alpha = need ? exp2_fast(m_ref - mx) : 1.f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      m_ref = need ? mx : m_ref;
      l_part *= alpha;
      float al[GP];
#pragma unroll
      for (int qq = 0; qq < GP; ++qq)
        al[qq] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), qq));
#pragma unroll
      for (int qq = 0; qq < GP; ++qq)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qq][e] *= al[qq];
    }
    const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
    float pr[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      pr[rr] = exp2_fast(__builtin_fmaf(sc[rr], c2, -m_use));
      l_part += pr[rr];
    }

    // Hand the probabilities to the lanes that hold the matching V rows.
    if (col < GP) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) Pl[wave][(4 * grp + rr) * GP + col] = pr[rr];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int t = grp + 4 * i4;
      float vv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = bf16lo_to_f32(r.v[i4][e]);
        vv[2 * e + 1] = bf16hi_to_f32(r.v[i4][e]);
      }
      if (tail && tok0 + t >= lim) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = 0.f;  // slots past the end may hold anything
      }
      float pq[GP];
#pragma unroll
      for (int qq = 0; qq < GP; ++qq) pq[qq] = Pl[wave][t * GP + qq];
#pragma unroll
      for (int qq = 0; qq < GP; ++qq)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qq][e] = __builtin_fmaf(pq[qq], vv[e], acc[qq][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Two register sets: page i+1 is in flight while page i is processed.
  PageRegs ra, rb;
  if (cnt > 0) load_page(0, ra);
  for (int i = 0; i < cnt; i += 2) {
    if (i + 1 < cnt) load_page(i + 1, rb);
    process_page(i, ra);
    if (i + 1 >= cnt) break;
    if (i + 2 < cnt) load_page(i + 2, ra);
    process_page(i + 1, rb);
  }

  // Sum the four token groups of each column, then merge the waves.
  float l_tot = sum_xor32(sum_xor16(l_part));
#pragma unroll
  for (int qq = 0; qq < GP; ++qq)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qq][e] = sum_xor32(sum_xor16(acc[qq][e]));
  if (grp == 0) {
    if (col < GP) {
      Wm[wave][col] = m_ref;
      Wl[wave][col] = l_tot;
    }
#pragma unroll
    for (int qq = 0; qq < GP; ++qq)
#pragma unroll
      for (int e = 0; e < 8; ++e) Wacc[wave][qq][8 * col + e] = acc[qq][e];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += kDecodeWaves * 64) {
    const int qq = i / D, d = i - (i / D) * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmax2(M, Wm[w][qq]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float wsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float wt = exp2_fast(Wm[w][qq] - Mu);
      wsum = __builtin_fmaf(wt, Wl[w][qq], wsum);
      osum = __builtin_fmaf(wt, Wacc[w][qq][d], osum);
    }
    const size_t row = ((size_t)b * a.H + (size_t)g * G + qq) * a.max_splits + s;
    a.ws_o[row * D + d] = wsum > 0.f ? osum / wsum : 0.f;
    if (d == 0) a.ws_lse[row] = wsum > 0.f ? Mu + log2_fast(wsum) : kNegInf;
  }
}

// Merge of the splits of one (b, h): one wave; lanes take splits for the
// max / weight sums and two head dims each for the weighted output sum.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  static_assert(D == 128, "two head dims per lane");
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int lane = threadIdx.x;
  const int L = decode_len(a, b);
  const int npg = (L + kPage - 1) / kPage;
  const int ns = (npg + a.split_pages - 1) / a.split_pages;
  const float* lse_s = a.ws_lse + (size_t)bh * a.max_splits;
  const float* o_s = a.ws_o + (size_t)bh * a.max_splits * D;
  float M = kNegInf;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) M = fmax2(M, lse_s[s0 + lane]);
  for (int off = 32; off >= 1; off >>= 1) M = fmax2(M, __shfl_xor(M, off));
  const float Mu = (M == kNegInf) ? 0.f : M;
  float W = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) W += exp2_fast(lse_s[s0 + lane] - Mu);
  for (int off = 32; off >= 1; off >>= 1) W += __shfl_xor(W, off);
  float o0 = 0.f, o1 = 0.f;
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    float w[4];
    f32x2 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = exp2_fast(lse_s[s + u] - Mu);
      x[u] = *reinterpret_cast<const f32x2*>(o_s + (size_t)(s + u) * D + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      o0 = __builtin_fmaf(w[u], x[u][0], o0);
      o1 = __builtin_fmaf(w[u], x[u][1], o1);
    }
  }
  for (; s < ns; ++s) {
    const float w = exp2_fast(lse_s[s] - Mu);
    const f32x2 x = *reinterpret_cast<const f32x2*>(o_s + (size_t)s * D + 2 * lane);
    o0 = __builtin_fmaf(w, x[0], o0);
    o1 = __builtin_fmaf(w, x[1], o1);
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  bf16x2 ov;
  ov[0] = (__bf16)(o0 * inv);
  ov[1] = (__bf16)(o1 * inv);
  *reinterpret_cast<bf16x2*>(a.o + (size_t)bh * D + 2 * lane) = ov;
  if (lane == 0) a.lse[bh] = W > 0.f ? (Mu + log2_fast(W)) * kLn2 : kNegInf;
}

int decode_split_pages(int B, int H, int max_seqlen) {
  (void)B;
  (void)H;
  (void)max_seqlen;
  return 32;  // 512 tokens per split
}
// A wave holds the page ids of its share of a split one per lane.
static_assert(kDecodeWaves * 64 >= 32, "split pages per wave must fit in 64 lanes");

int decode_max_splits(int B, int H, int max_seqlen) {
  const int sp = decode_split_pages(B, H, max_seqlen);
  const long long pages = ((long long)max_seqlen + kPage - 1) / kPage;
  return (int)((pages + sp - 1) / sp);
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t decode_workspace_bytes(int B, int H, int max_seqlen, int d) {
  const size_t ms = (size_t)decode_max_splits(B, H, max_seqlen);
  const size_t rows = (size_t)B * H * ms;
  return align_up(rows * d * sizeof(float), 256) + align_up(rows * sizeof(float), 256);
}

template <int GP>
static void launch_split(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<128, GP>), grid, dim3(kDecodeWaves * 64), 0, stream, a);
}

hipError_t launch_decode(const void* q, const void* kcache, const void* vcache,
                         const int32_t* page_table, const int32_t* seqlens, void* o, float* lse,
                         int B, int H, int Hkv, int d, int num_pages, int max_pages,
                         int max_seqlen, float scale, void* workspace, hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  DecodeArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.kc = static_cast<const __bf16*>(kcache);
  a.vc = static_cast<const __bf16*>(vcache);
  a.page_table = page_table;
  a.seqlens = seqlens;
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.B = B; a.H = H; a.Hkv = Hkv; a.G = H / Hkv;
  a.num_pages = num_pages; a.max_pages = max_pages; a.max_seqlen = max_seqlen;
  a.split_pages = decode_split_pages(B, H, max_seqlen);
  a.max_splits = decode_max_splits(B, H, max_seqlen);
  a.scale_log2 = scale * kLog2e;
  const size_t rows = (size_t)B * H * a.max_splits;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      align_up(rows * d * sizeof(float), 256));
  dim3 grid(a.max_splits, Hkv, B);
  const int G = a.G;
  if (G <= 1) launch_split<1>(a, grid, stream);
  else if (G <= 2) launch_split<2>(a, grid, stream);
  else if (G <= 4) launch_split<4>(a, grid, stream);
  else if (G <= 8) launch_split<8>(a, grid, stream);
  else if (G <= 16) launch_split<16>(a, grid, stream);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(B * H), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa

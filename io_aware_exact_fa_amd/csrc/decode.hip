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
//   * One workgroup per (sequence b, key/value head g, split of up to 96
//     pages); its 4 waves take the split's pages round-robin, one page (16
//     tokens) at a time, with the next page's loads in flight.  The loads go
//     through range-checked buffer descriptors, so the prefetch is issued
//     unconditionally (empty range past the wave's last page) and the
//     compiler waits only for the current page's loads.  All G = H/Hkv query
//     heads of the group are served from the same K/V bytes.
//   * Scores: v_mfma_f32_16x16x32_bf16, A = the page's 16 tokens x 32 dims,
//     B = the G query vectors (columns >= G are zero).  The bf16 keys are
//     loaded lane-linearly (whole 128-byte lines per instruction) one page
//     ahead into registers and pass through a per-wave LDS buffer into the
//     A-operand layout just before use.  Lane l owns query column l%16
//     and tokens 4*(l/16) .. +3, so the max / sum over the page's 16 tokens is
//     4 in-lane values plus two lane swaps (permlane16/32).
//   * P.V: v_mfma_f32_16x16x16_bf16 over the page's 16 tokens.  Its B operand
//     (tokens x query columns) has exactly the score accumulator's layout, so
//     the bf16-rounded probabilities never leave registers; its A operand
//     (dims x tokens) comes from the V page, DMA'd HBM -> LDS into a per-wave
//     buffer and read back transposed with ds_read_b64_tr_b16.  V needs no
//     registers and the accumulator is 32 registers for any G <= 16.
//   * The 4 waves merge through LDS at the end (their idle V buffers hold the
//     partial outputs); the split writes a normalised fp32 partial output and
//     its base-2 log-sum-exp to the workspace.
//   * The merge kernel (4 waves per (b, h)) reads the valid splits of each
//     (b, h) and writes bf16 output and the natural-log lse.
//   * FP8 caches (quantised KV, charles2530 blog §9): keys and values are
//     bytes in the OCP E4M3 format with one scale per KV head.  Every E4M3
//     value is exact in bf16, so a page's bytes are loaded into registers
//     one page ahead, widened with v_cvt_scalef32_pk_bf16_fp8 (two bytes
//     per instruction, unit scale) and fed to the same
//     bf16 MFMAs (V goes through the same LDS buffers, written from
//     registers); the key scale joins the score scale and the value scale
//     multiplies the split's output.  Half the bytes of the bf16 cache move.

#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace fa {

constexpr int kPage = 16;
constexpr int kDecodeWaves = 4;

struct DecodeArgs {
  const __bf16* q;
  const __bf16* kc;
  const __bf16* vc;
  const unsigned char* kc8;  // FP8 caches (E4M3 bytes)
  const unsigned char* vc8;
  const float* k_scale;      // [Hkv] FP8 dequantisation scales
  const float* v_scale;
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

// Swizzle of the 16-byte chunks of a V page row in LDS (16 rows x 2*D bytes):
// chunk c of row r sits at c ^ vswz<D>(r), so the transposed reads of one
// instruction (16 rows x 32 B) spread over the banks.  The XOR value is even,
// so chunks 2k and 2k+1 stay side by side (the FP8 path writes them as one
// widened 16-byte piece).
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 2 * (r & 7) : 2 * (r & 3);
}

// Range-checked view of one (page, KV head) slab: loads at offsets past
// nbytes return zeros without touching memory, so a prefetch past the last
// page can be issued unconditionally with nbytes = 0.  (Unconditional loads
// let the compiler count the loads in flight; a load under a branch makes it
// wait for all of them before the current page's work.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
}

// Every K/V byte of the cache is read once per launch: the page loads carry
// the non-temporal hint (cache-policy bit nt), which let a plain 16-byte-per-
// lane stream over 4 GiB read at 6.94 TB/s instead of 6.25.
constexpr int kStream = 2;

// 16 bytes per lane from HBM straight into LDS (lane i -> lds + 16*i).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, 0, 0, kStream);
}

// Eight E4M3 bytes (little-endian in two words) widened to bf16; exact, as
// every E4M3 value has at most 4 significant bits and a bf16-range exponent.
// One v_cvt_scalef32_pk_bf16_fp8 per byte pair, with a unit scale (the
// per-head scales are applied in fp32 elsewhere), so no rounding occurs.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x8 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, true);
    r[4 * h + 0] = lo[0];
    r[4 * h + 1] = lo[1];
    r[4 * h + 2] = hi[0];
    r[4 * h + 3] = hi[1];
  }
  return r;
}

template <int D, int GP, bool FP8>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_split_kernel(DecodeArgs a) {
  static_assert(D == 128 || D == 64, "head dim 64 or 128");
  constexpr int NC = D / 32;   // 32-dim chunks of the QK contraction
  constexpr int NDB = D / 16;  // 16-dim blocks of the PV output
  constexpr int PAGE_BYTES = kPage * D * 2;
  constexpr int CPR = D / 8;   // 16-byte bf16 chunks per page row
  constexpr int NVJ = PAGE_BYTES / 1024;  // 1 KB V DMA instructions per page
  // Per wave: two V page buffers (double-buffered), filled by LDS DMA.
  __shared__ __attribute__((aligned(1024))) char sV0[kDecodeWaves][PAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[kDecodeWaves][PAGE_BYTES];
  // bf16 keys: the page's keys, loaded lane-linearly, pass through this
  // per-wave buffer on their way into the MFMA operand layout.
  __shared__ __attribute__((aligned(1024))) char sK[FP8 ? 1 : kDecodeWaves][FP8 ? 16 : PAGE_BYTES];
  __shared__ float Wm[kDecodeWaves][16];
  __shared__ float Wl[kDecodeWaves][16];
  static_assert(GP * D * 4 <= 2 * PAGE_BYTES, "wave partials must fit in its two V buffers");

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

  // Query fragments: B operand (32 dims x 16 query columns) per chunk.  The
  // contraction's k index may follow any order of the head dims as long as
  // K and Q agree.  bf16 cache: chunk c, lane group grp holds dims
  // 32c + 8*grp .. +7.  FP8 cache: chunks 2m and 2m+1 hold dims
  // 64m + 16*grp .. +7 and .. +15, so a lane's key bytes for both chunks are
  // one 16-byte load.
  bf16x8 qf[NC];
  {
    const __bf16* qrow = a.q + ((size_t)b * a.H + (size_t)g * G + col) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int dim0 = FP8 ? 64 * (c >> 1) + 16 * grp + 8 * (c & 1) : 32 * c + 8 * grp;
      qf[c] = (col < G) ? *reinterpret_cast<const bf16x8*>(qrow + dim0) : bf16x8{};
    }
  }

  // O^T accumulator: 8 blocks of 16 dims x 16 query columns; lane (col q,
  // grp) holds dims 16*db + 4*grp + r of query q.
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
  float m_ref = kNegInf, l_part = 0.f;
  float c2 = a.scale_log2, vmul = 1.f;
  if constexpr (FP8) {
    c2 *= a.k_scale[g];  // scores scale by the key scale
    vmul = a.v_scale[g];  // the output by the value scale
  }

  // V DMA: lane i of instruction j writes LDS slot 64*j + i (16 B), which holds
  // physical chunk slot%CPR of page row slot/CPR.
  unsigned v_off[NVJ];
#pragma unroll
  for (int j = 0; j < NVJ; ++j) {
    const int slot = 64 * j + lane;
    const int r = slot / CPR;
    const int c = (slot % CPR) ^ vswz<D>(r);
    v_off[j] = (unsigned)(r * D * 2 + c * 16);
  }
  // Transposed V read (block db): lane supplies row 4*grp + (lane%16)/4,
  // dims 16*db + 4*(lane%4) .. +4 (8 bytes).
  const int vr_row = 4 * grp + ((lane & 15) >> 2);
  const int vr_sw = vswz<D>(vr_row);

  struct PageK {
    bf16x8 k[NC];
  };
  struct PageK8 {  // FP8: a page's key bytes (k) or value bytes (v) held by this lane
    u32x4 k[NC / 2];   // token col, dims 64m + 16*grp .. +15
    u32x4 v[D / 64];   // 16-byte piece 64j + lane of the page (row-major)
  };
  using PageRegs = typename std::conditional<FP8, PageK8, PageK>::type;
  auto phys_of = [&](int i) {
    int phys = __builtin_amdgcn_readlane(my_phys, i);
    return (phys < 0 || phys >= a.num_pages) ? -1 : phys;
  };
  // bf16 page i: K into registers (lane-linear 16-byte pieces, rearranged
  // through LDS before use) and V into the LDS buffer vdst by DMA.  An invalid
  // page id loads page 0 (in bounds) and its tokens are masked; a page past the
  // wave's last one (i >= cnt) loads nothing (zero-sized range).
  auto load_page = [&](int i, PageRegs& r, char* vdst) {
    int phys = phys_of(i);
    if (phys < 0) phys = 0;
    const size_t base = ((size_t)phys * a.Hkv + g) * kPage * D;
    if constexpr (!FP8) {
      const int nb = i < cnt ? PAGE_BYTES : 0;
      const __amdgpu_buffer_rsrc_t rk = page_rsrc(a.kc + base, nb);
      const __amdgpu_buffer_rsrc_t rv = page_rsrc(a.vc + base, nb);
      static_assert(PAGE_BYTES == NC * 1024, "one 1 KB key piece per register slot");
#pragma unroll
      for (int j = 0; j < NC; ++j)
        r.k[j] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, 1024 * j + 16 * lane, 0, kStream));
#pragma unroll
      for (int j = 0; j < NVJ; ++j) dma16(rv, v_off[j], vdst + 1024 * j);
    }
  };
  // FP8 page i, into registers: its key bytes (keys = true; token col, dims
  // 64m + 16*grp .. +15) or its value bytes (16-byte piece 64j + lane of the
  // row-major slab).  Same page-id and range rules as above.
  auto load_page8 = [&](int i, PageRegs& r, bool keys) {
    int phys = phys_of(i);
    if (phys < 0) phys = 0;
    const size_t base = ((size_t)phys * a.Hkv + g) * kPage * D;
    const int nb = i < cnt ? kPage * D : 0;
    if constexpr (FP8) {
      if (keys) {
        const __amdgpu_buffer_rsrc_t rk = page_rsrc(a.kc8 + base, nb);
#pragma unroll
        for (int m = 0; m < NC / 2; ++m)
          r.k[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rk, col * D + 64 * m + 16 * grp, 0, kStream));
      } else {
        const __amdgpu_buffer_rsrc_t rv = page_rsrc(a.vc8 + base, nb);
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
          r.v[j] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 1024 * j + 16 * lane, 0, kStream));
      }
    }
  };

  // Page i with its keys in rk (both paths) and, FP8, its values in rv.
  auto process_page = [&](int i, const PageRegs& r, const PageRegs& rvv, const char* vsrc) {
    const bool valid = phys_of(i) >= 0;
    const int tok0 = (p0 + wave + kDecodeWaves * i) * kPage;
    const int lim = valid ? L : tok0;  // tokens at or past lim are masked
    const bool tail = tok0 + kPage > lim;

    bf16x8 kf[NC];
    if constexpr (FP8) {
      // V: widen and write the page into this wave's buffer in the swizzled
      // layout the DMA gives the bf16 cache (the reads below follow in
      // program order).  Piece 64j + lane is row r, dims 16k .. +15, i.e.
      // bf16 chunks 2k and 2k+1, which the swizzle (an XOR with an even
      // value) keeps side by side.
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        const int piece = 64 * j + lane, r8 = piece / (D / 16), k8 = piece % (D / 16);
        char* dst = const_cast<char*>(vsrc) + r8 * D * 2 + 16 * ((2 * k8) ^ vswz<D>(r8));
        *reinterpret_cast<bf16x8*>(dst) = e4m3x8_to_bf16(u32x2{rvv.v[j][0], rvv.v[j][1]});
        *reinterpret_cast<bf16x8*>(dst + 16) = e4m3x8_to_bf16(u32x2{rvv.v[j][2], rvv.v[j][3]});
      }
#pragma unroll
      for (int m = 0; m < NC / 2; ++m) {
        kf[2 * m] = e4m3x8_to_bf16(u32x2{r.k[m][0], r.k[m][1]});
        kf[2 * m + 1] = e4m3x8_to_bf16(u32x2{r.k[m][2], r.k[m][3]});
      }
    } else {
      // Piece j of lane l is row (64j + l)/CPR, 16-byte chunk l%CPR; it is
      // stored at chunk (l%CPR) ^ (row%CPR) of its row, so that the fragment
      // reads (16 rows, one chunk each) spread over the banks.
      char* ks = sK[FP8 ? 0 : wave];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int kr = (64 * j + lane) / CPR;
        *reinterpret_cast<bf16x8*>(ks + kr * D * 2 + 16 * ((lane % CPR) ^ (kr % CPR))) = r.k[j];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kf[c] = *reinterpret_cast<const bf16x8*>(ks + col * D * 2 +
                                                 16 * ((4 * c + grp) ^ (col % CPR)));
    }

    // S^T = K Q^T: lane (col q, grp) holds tokens 4*grp + rr of query q.
    f32x4 sc = f32x4{};
#pragma unroll
    for (int c = 0; c < NC; ++c) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[c], sc, 0, 0, 0);
    // Scores in base-2 units, scaled before the mask: the FP8 key scale may
    // be zero (a head quantised from zeros) or negative, and -inf * 0 or a
    // max taken before a negative scale would be wrong.
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sc[rr] *= c2;
    if (tail) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (tok0 + 4 * grp + rr >= lim) sc[rr] = kNegInf;
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3]));
    mx = max_xor32(max_xor16(mx));
    const bool need = mx > m_ref + kDecodeRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? exp2_fast(m_ref - mx) : 1.f;
      m_ref = need ? mx : m_ref;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
    bf16x4 pb;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float pv = exp2_fast(sc[rr] - m_use);
      l_part += pv;
      pb[rr] = (__bf16)pv;
    }
    // Slots past the end of the sequence may hold anything: zero P is not
    // enough (0 * NaN), so masked tokens' V rows must not enter the product.
    // Their P is exactly 0 and finite V is guaranteed by zeroing the A operand
    // below only on the (rare) tail page.
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const i16x4 pbi = __builtin_bit_cast(i16x4, pb);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int cbyte = (16 * db + 4 * (lane & 3)) * 2;
      const int off = vr_row * D * 2 + ((((cbyte >> 4) ^ vr_sw) << 4) | (cbyte & 15));
      i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(
              (__attribute__((address_space(3))) char*)(vsrc) + off));
      if (tail) {
        // element t of vt is token 4*grp + t of this page
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (tok0 + 4 * grp + t >= lim) vt[t] = 0;
      }
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pbi, acc[db], 0, 0, 0);
    }
  };

  // bf16: two page register sets and two V buffers, page i+1 in flight while
  // page i is processed.  FP8: keys two pages ahead (three register sets),
  // values one (two sets), which still fits three waves per SIMD (whole FP8
  // pages two ahead would not); the loop is unrolled by six so that every
  // set is a fixed register range.
  if constexpr (FP8) {
    PageRegs k0, k1, k2, v0, v1;
    load_page8(0, k0, true);
    load_page8(0, v0, false);
    load_page8(1, k1, true);
    auto step = [&](int i, const PageRegs& kc, const PageRegs& vc, PageRegs& kn, PageRegs& vn,
                    const char* vsrc) __attribute__((always_inline)) {
      load_page8(i + 2, kn, true);
      load_page8(i + 1, vn, false);
      process_page(i, kc, vc, vsrc);
    };
    for (int i = 0; i < cnt; i += 6) {
      step(i, k0, v0, k2, v1, sV0[wave]);
      if (i + 1 >= cnt) break;
      step(i + 1, k1, v1, k0, v0, sV1[wave]);
      if (i + 2 >= cnt) break;
      step(i + 2, k2, v0, k1, v1, sV0[wave]);
      if (i + 3 >= cnt) break;
      step(i + 3, k0, v1, k2, v0, sV1[wave]);
      if (i + 4 >= cnt) break;
      step(i + 4, k1, v0, k0, v1, sV0[wave]);
      if (i + 5 >= cnt) break;
      step(i + 5, k2, v1, k1, v0, sV1[wave]);
    }
  } else {
    PageRegs ka, kb;
    load_page(0, ka, sV0[wave]);
    for (int i = 0; i < cnt; i += 2) {
      load_page(i + 1, kb, sV1[wave]);
      process_page(i, ka, ka, sV0[wave]);
      if (i + 1 >= cnt) break;
      load_page(i + 2, ka, sV0[wave]);
      process_page(i + 1, kb, kb, sV1[wave]);
    }
  }

  // The last prefetch (past the wave's pages, zero-sized) may still be in
  // flight into a V buffer that holds the partial outputs below.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Row sums: sum the four token groups of each column.  The accumulator
  // needs no cross-lane sum (lanes hold distinct dims).
  const float l_tot = sum_xor32(sum_xor16(l_part));
  if (grp == 0 && col < GP) {
    Wm[wave][col] = m_ref;
    Wl[wave][col] = l_tot;
  }
  // The wave's partial outputs go to its own V buffers, idle from here on
  // (every DMA into them was waited for before its page was read).
  float* wacc_own = reinterpret_cast<float*>(col * D * 4 < PAGE_BYTES ? sV0[wave] : sV1[wave]);
  if (col < GP) {
    const int base = (col * D) % (PAGE_BYTES / 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(wacc_own + base + 16 * db + 4 * grp) = acc[db];
  }
  __syncthreads();
  auto wacc = [&](int w, int qq, int d) {
    const float* buf = reinterpret_cast<const float*>(qq * D * 4 < PAGE_BYTES ? sV0[w] : sV1[w]);
    return buf[(qq * D) % (PAGE_BYTES / 4) + d];
  };

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
      osum = __builtin_fmaf(wt, wacc(w, qq, d), osum);
    }
    const size_t row = ((size_t)b * a.H + (size_t)g * G + qq) * a.max_splits + s;
    a.ws_o[row * D + d] = wsum > 0.f ? vmul * osum / wsum : 0.f;
    if (d == 0) a.ws_lse[row] = wsum > 0.f ? Mu + log2_fast(wsum) : kNegInf;
  }
}

// Merge of the split partials of one (b, h): 4 waves.  The workgroup first
// finds the largest partial lse; wave w then sums splits w, w+4, ... with weights
// exp2(lse_e - max), each lane owning D/64 head dims; the waves' sums are
// added through LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  static_assert(D == 128 || D == 64, "one or two head dims per lane");
  constexpr int DPL = D / 64;
  typedef float fdpl __attribute__((ext_vector_type(DPL)));
  __shared__ float red[4];
  __shared__ float part_o[4][D];
  __shared__ float part_w[4];
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = decode_len(a, b);
  const int npg = (L + kPage - 1) / kPage;
  const int ne = (npg + a.split_pages - 1) / a.split_pages;
  const size_t row0 = (size_t)bh * a.max_splits;
  const float* lse_e = a.ws_lse + row0;
  const float* o_e = a.ws_o + row0 * D;
  float M = kNegInf;
  for (int e = tid; e < ne; e += 256) M = fmax2(M, lse_e[e]);
  for (int off = 32; off >= 1; off >>= 1) M = fmax2(M, __shfl_xor(M, off));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmax2(fmax2(red[0], red[1]), fmax2(red[2], red[3]));
  const float Mu = (M == kNegInf) ? 0.f : M;
  float W = 0.f;
  float ov_acc[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) ov_acc[u] = 0.f;
  auto part = [&](int e) {
    return *reinterpret_cast<const fdpl*>(o_e + (size_t)e * D + DPL * lane);
  };
  int e = wave;
  for (; e + 12 < ne; e += 16) {
    float w[4];
    fdpl x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = exp2_fast(lse_e[e + 4 * u] - Mu);
      x[u] = part(e + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      W += w[u];
#pragma unroll
      for (int c = 0; c < DPL; ++c) ov_acc[c] = __builtin_fmaf(w[u], x[u][c], ov_acc[c]);
    }
  }
  for (; e < ne; e += 4) {
    const float w = exp2_fast(lse_e[e] - Mu);
    const fdpl x = part(e);
    W += w;
#pragma unroll
    for (int c = 0; c < DPL; ++c) ov_acc[c] = __builtin_fmaf(w, x[c], ov_acc[c]);
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) part_o[wave][DPL * lane + c] = ov_acc[c];
  if (lane == 0) part_w[wave] = W;
  __syncthreads();
  if (wave != 0) return;
  const float Wt = part_w[0] + part_w[1] + part_w[2] + part_w[3];
  const float inv = Wt > 0.f ? 1.f / Wt : 0.f;
  __bf16 ov[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) {
    const int d = DPL * lane + u;
    ov[u] = (__bf16)((part_o[0][d] + part_o[1][d] + part_o[2][d] + part_o[3][d]) * inv);
  }
  if constexpr (DPL == 2)
    *reinterpret_cast<bf16x2*>(a.o + (size_t)bh * D + 2 * lane) = bf16x2{ov[0], ov[1]};
  else
    a.o[(size_t)bh * D + lane] = ov[0];
  if (lane == 0) a.lse[bh] = Wt > 0.f ? (Mu + log2_fast(Wt)) * kLn2 : kNegInf;
}

// Pages per split.  Long splits amortise each workgroup's start-up (lengths,
// page ids, first page) and its end (merge of the 4 waves); on the
// 64-sequence workload (up to 2048 pages) 120 pages measured best among 72
// to 240 (0.675 ms against 0.682 at 96 and 0.709 at 72).  With few
// sequences x heads the split shrinks so that enough workgroups exist: the
// estimate uses H/4 KV heads and half of max_seqlen as the typical length.
int decode_split_pages(int B, int H, int max_seqlen) {
  const long long max_pages = ((long long)max_seqlen + kPage - 1) / kPage;
  const long long groups = (long long)B * (H >= 4 ? H / 4 : 1);
  const long long avg_pages = (max_pages + 1) / 2;
  int sp = 120;
  while (sp > 8 && groups * ((avg_pages + sp - 1) / sp) < 2048) sp = sp > 16 ? sp / 2 : 8;
  return sp;
}
// A wave holds the page ids of its share of a split one per lane and reads
// up to lane cnt + 1 (the FP8 keys are prefetched two pages ahead).
static_assert((120 + kDecodeWaves - 1) / kDecodeWaves + 2 <= 64,
              "a wave's pages plus two must fit in 64 lanes");

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

// The split index is fastest in the grid and workgroups go round-robin over
// the 8 XCDs in dispatch order, so with a split count that is a multiple of 8
// split s of every (KV head, sequence) row lands on XCD s mod 8: the low
// splits, live in every sequence, crowd a few XCDs while the high ones sit
// idle (16 splits of 136 pages: 0.84 ms, against 0.69 with 17).  One more
// split per row, empty (it starts past every sequence's last page and exits
// at once), rotates the rows over the XCDs.
static int decode_grid_splits(int max_splits) {
  return max_splits % 8 == 0 ? max_splits + 1 : max_splits;
}

template <int D, int GP, bool FP8>
static void launch_split(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, GP, FP8>),
                     dim3(decode_grid_splits(a.max_splits), a.Hkv, a.B),
                     dim3(kDecodeWaves * 64), 0, stream, a);
}

template <int D, bool FP8>
static hipError_t launch_decode_d(DecodeArgs& a, int B, int H, void* workspace,
                                  hipStream_t stream) {
  const size_t rows = (size_t)B * H * a.max_splits;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      align_up(rows * D * sizeof(float), 256));
  const int G = a.G;
  if (G <= 1) launch_split<D, 1, FP8>(a, stream);
  else if (G <= 2) launch_split<D, 2, FP8>(a, stream);
  else if (G <= 4) launch_split<D, 4, FP8>(a, stream);
  else if (G <= 8) launch_split<D, 8, FP8>(a, stream);
  else if (G <= 16) launch_split<D, 16, FP8>(a, stream);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(B * H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool FP8>
static hipError_t launch_decode_t(DecodeArgs& a, int B, int H, int d, void* workspace,
                                  hipStream_t stream) {
  if (d == 128) return launch_decode_d<128, FP8>(a, B, H, workspace, stream);
  if (d == 64) return launch_decode_d<64, FP8>(a, B, H, workspace, stream);
  return hipErrorInvalidValue;
}

static DecodeArgs decode_args(const void* q, const int32_t* page_table, const int32_t* seqlens,
                              void* o, float* lse, int B, int H, int Hkv, int num_pages,
                              int max_pages, int max_seqlen, float scale) {
  DecodeArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.page_table = page_table;
  a.seqlens = seqlens;
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.B = B; a.H = H; a.Hkv = Hkv; a.G = H / Hkv;
  a.num_pages = num_pages; a.max_pages = max_pages; a.max_seqlen = max_seqlen;
  a.split_pages = decode_split_pages(B, H, max_seqlen);
  a.max_splits = decode_max_splits(B, H, max_seqlen);
  a.scale_log2 = scale * kLog2e;
  return a;
}

hipError_t launch_decode_fp8(const void* q, const void* kcache, const void* vcache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* page_table, const int32_t* seqlens, void* o,
                             float* lse, int B, int H, int Hkv, int d, int num_pages,
                             int max_pages, int max_seqlen, float scale, void* workspace,
                             hipStream_t stream) {
  DecodeArgs a = decode_args(q, page_table, seqlens, o, lse, B, H, Hkv, num_pages, max_pages,
                             max_seqlen, scale);
  a.kc8 = static_cast<const unsigned char*>(kcache);
  a.vc8 = static_cast<const unsigned char*>(vcache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return launch_decode_t<true>(a, B, H, d, workspace, stream);
}

// ---- allocation-free decode: split partials in a static device array ----
//
// For callers that cannot allocate device memory.  Each GPU the library runs
// on holds one copy of this array until the process ends; the kernels get it
// as their workspace pointer like any caller-owned buffer.  Every call on a
// device shares that device's copy, so calls that overlap on one GPU race.
// Every partial the merge reads is written by the split kernel of the same
// call, so nothing needs clearing between calls.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

// The array's device address on the current device, looked up once per
// device (the host-side name is only a stand-in for the symbol).
static hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode_static(const void* q, const void* kcache, const void* vcache,
                                const int32_t* page_table, const int32_t* seqlens, void* o,
                                float* lse, int B, int H, int Hkv, int d, int num_pages,
                                int max_pages, int max_seqlen, float scale,
                                hipStream_t stream) {
  if (decode_workspace_bytes(B, H, max_seqlen, d) > kDecodeScratchBytes)
    return hipErrorInvalidValue;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_decode(q, kcache, vcache, page_table, seqlens, o, lse, B, H, Hkv, d, num_pages,
                       max_pages, max_seqlen, scale, ws, stream);
}

hipError_t launch_decode(const void* q, const void* kcache, const void* vcache,
                         const int32_t* page_table, const int32_t* seqlens, void* o, float* lse,
                         int B, int H, int Hkv, int d, int num_pages, int max_pages,
                         int max_seqlen, float scale, void* workspace, hipStream_t stream) {
  DecodeArgs a = decode_args(q, page_table, seqlens, o, lse, B, H, Hkv, num_pages, max_pages,
                             max_seqlen, scale);
  a.kc = static_cast<const __bf16*>(kcache);
  a.vc = static_cast<const __bf16*>(vcache);
  return launch_decode_t<false>(a, B, H, d, workspace, stream);
}

}  // namespace fa

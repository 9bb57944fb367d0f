// Attention backward pass on gfx950 (bf16 inputs, fp32 gradients).
//
// Method: the backward pass keeps no score or probability matrix from the
// forward pass; it recomputes them tile by tile from Q, K and the saved
// row log-sum-exp (xxqk.cn sliding-window prefill article §3.3; bomianfm.com
// Q&A "FlashAttention的原理是什么？对Agent性能有何提升？" §一).  With
// P = exp(scale*Q K^T - lse) on the visible pairs and D_i = <dO_i, O_i>:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q   (dK, dV summed over the query heads of a KV group).
// Key tiles outside a query tile's band are skipped exactly as in the forward
// pass (xxqk.cn article §5.1-§5.5).
//
// Three kernels, no atomics (deterministic):
//   * bwd_delta_kernel: D_i = <dO_i, O_i> in fp32.
//   * bwd_dkdv_kernel: a workgroup owns 128 keys of one (b, KV head); wave w
//     owns 32 of them with K and V held in registers as MFMA B operands.  It
//     streams (32-query tile, query head) pairs, top tile first, through
//     three LDS stage buffers (each tile's loads issued two tiles ahead):
//     S = Q K^T and dP = dO V^T (v_mfma_f32_32x32x16_bf16; in the accumulator
//     lane l owns key l%32 and 16 query rows), P and dS elementwise, then
//     dV += P^T dO and dK += dS^T Q with P^T / dS^T taken straight from those
//     registers (the MFMA k index follows the accumulator's query order) and
//     dO / Q read transposed from LDS with ds_read_b64_tr_b16.
//   * bwd_dq_kernel: a workgroup owns 256 query rows (8 waves; 128 and 4
//     waves with a window) of one (b, h); wave w owns 32 with Q and dO in
//     registers (lane = query, as in the forward kernel), streams K/V tiles,
//     recomputes S^T and dP^T = V dO^T, forms dS^T and accumulates
//     dQ^T += K^T dS^T with K^T read transposed from LDS.

#include "common.hpp"
#include "launch.hpp"

namespace fa {

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const float* lse;  // natural log
  const __bf16* dout;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // [B, H, n]
  int B, H, Hkv, n, causal, window;
  float scale;
  float scale_log2;  // scale * log2(e)
};

// Same LDS chunk swizzle as the forward kernel (256-byte rows).
template <int D>
__device__ __forceinline__ int bswz(int row) {
  if constexpr (D == 128)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return row & 7;
}

__device__ __forceinline__ void bwd_load_lds16(const void* base, int nbytes, unsigned off,
                                               void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, 0, 0, 0);
}

__device__ __forceinline__ void bwd_load_lds4(const void* base, int nbytes, unsigned off,
                                              void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           off, 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed 32x16 fragment from a row-major LDS tile (rows of D bf16, chunk
// swizzle bswz): lane (l32, hi) receives, for t = 0..7, element
// [row0 + 8*(t/4) + 4*hi + t%4][col0 + l32].
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int row0, int col0, int lane) {
  const int hi = lane >> 5;
  const int vrow = 4 * hi + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  bf16x8 f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = row0 + 8 * half + vrow;
    const int cbyte = (col0 + vcol) * 2;
    const int off = r * D * 2 + ((((cbyte >> 4) ^ bswz<D>(r)) << 4) | (cbyte & 15));
    const i16x4 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)(tile) +
                                                     off));
    const bf16x4 b4 = __builtin_bit_cast(bf16x4, t4);
    f[4 * half + 0] = b4[0];
    f[4 * half + 1] = b4[1];
    f[4 * half + 2] = b4[2];
    f[4 * half + 3] = b4[3];
  }
  return f;
}

// Row fragment (A operand, 32 rows x 16 dims): lane (l32, hi) gets
// [row0 + l32][16*dc + 8*hi .. +8].
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int row0, int dc, int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  const int r = row0 + l32;
  const int off = r * D * 2 + (((2 * dc + hi) ^ bswz<D>(r)) << 4);
  return *reinterpret_cast<const bf16x8*>(tile + off);
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const long long rows = (long long)a.B * a.H * a.n;
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const __bf16* orow = a.o + r * D;
  const __bf16* drow = a.dout + r * D;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(orow + c);
    const u32x4 y = *reinterpret_cast<const u32x4*>(drow + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(bf16lo_to_f32(x[e]), bf16lo_to_f32(y[e]), acc);
      acc = __builtin_fmaf(bf16hi_to_f32(x[e]), bf16hi_to_f32(y[e]), acc);
    }
  }
  a.delta[r] = acc;
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 4, BK = NW * 32, BQ = 32;
  constexpr int RB = D * 2, CPR = D / 8, TILE = BQ * RB;
  constexpr int IPW = BQ * CPR / (64 * NW);
  constexpr int NDC = D / 16, NDB = D / 32;
  static_assert(BQ * CPR % (64 * NW) == 0, "tile must split evenly over waves");
  // Three stage buffers, each one LDS object holding a Q tile, a dO tile,
  // then lse and D of the staged query rows (64 slots each, the first BQ
  // used).  One object per stage lets the compiler tell the buffer being read
  // from those that in-flight loads fill.
  constexpr int STAGE = 2 * TILE + 2 * 64 * 4;
  __shared__ __attribute__((aligned(1024))) char sB0[STAGE];
  __shared__ __attribute__((aligned(1024))) char sB1[STAGE];
  __shared__ __attribute__((aligned(1024))) char sB2[STAGE];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.n, G = a.H / a.Hkv;
  const int nkb = (n + BK - 1) / BK;
  // Rounds of B*Hkv workgroups, one key block each (heaviest causal blocks,
  // the first ones, first); inside a round, groups are spread so that each
  // XCD keeps the same (b, g) from round to round.
  const int BG = a.B * a.Hkv;
  const int kblk = blockIdx.x / BG;
  const int p = blockIdx.x - kblk * BG;
  const int bg = (BG & 7) == 0 ? (p & 7) * (BG >> 3) + (p >> 3) : p;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int causal = a.causal, window = a.window;
  auto lo_of = [&](int i) { return window >= 0 ? i - window : 0; };
  auto hi_of = [&](int i) {
    int v = causal ? i : (window >= 0 ? i + window : n - 1);
    return v < n - 1 ? v : n - 1;
  };

  const int k0 = kblk * BK;
  const int k1 = min(k0 + BK, n) - 1;
  // Query rows whose band meets this key block.
  const int i_min = causal ? k0 : (window >= 0 ? max(0, k0 - window) : 0);
  const int i_max = window >= 0 ? min(n - 1, k1 + window) : n - 1;
  const int qt_lo = i_min / BQ, qt_hi = i_max / BQ;
  const int nqt = qt_hi - qt_lo + 1;
  const int T = G * nqt;  // (query head, query tile) pairs

  const int kw0 = k0 + 32 * wave;  // this wave's keys kw0 .. kw0+31
  const int kw1 = min(kw0 + 31, n - 1);
  const bool wave_keys = kw0 < n;
  const int key = kw0 + l32;  // the key this lane owns in the accumulators
  const size_t kvbase = (size_t)(b * a.Hkv + g) * n;
  bf16x8 kb[NDC], vb[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    if (key < n) {
      kb[dc] = *reinterpret_cast<const bf16x8*>(a.k + (kvbase + key) * D + 16 * dc + 8 * hi);
      vb[dc] = *reinterpret_cast<const bf16x8*>(a.v + (kvbase + key) * D + 16 * dc + 8 * hi);
    } else {
      kb[dc] = bf16x8{};
      vb[dc] = bf16x8{};
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  unsigned st_off[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int s = (wave * IPW + j) * 64 + lane;
    const int r = s / CPR;
    const int c = (s % CPR) ^ bswz<D>(r);
    st_off[j] = (unsigned)(r * RB + c * 16);
  }
  // Query tiles are walked from the last one down, the group's heads
  // innermost: the workgroups of one (b, g) that an XCD runs together start
  // on the same tiles, and a replacement workgroup starts where the others
  // started shortly before, so Q and dO tiles are mostly read from L2 (a key
  // block further down simply stops earlier).  Step t is (query head
  // g*G + t%G, query tile qt_hi - t/G); a cursor holds both and moves one step.
  struct Cursor {
    int hq, qt;
  };
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.hq == G) {
      c.hq = 0;
      --c.qt;
    }
  };
  // Every step stages one (Q, dO, lse, D) tile; a step past the last one
  // issues the same loads with an empty descriptor (no memory access), so
  // that each wave has the same number of loads in flight on every path.
  // Even waves load lse, odd waves D (waves 2 and 3 repeat the values 0 and 1
  // write).  Rows past n read as zero.
  auto stage = [&](int t, const Cursor& c, char* buf) __attribute__((always_inline)) {
    const bool live = t < T;
    const int h = g * G + c.hq, q0 = max(c.qt, 0) * BQ;
    const size_t row0 = (size_t)(b * a.H + h) * n + q0;
    const int bytes = live ? (n - q0) * RB : 0;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      bwd_load_lds16(a.q + row0 * D, bytes, st_off[j], buf + (wave * IPW + j) * 1024);
      bwd_load_lds16(a.dout + row0 * D, bytes, st_off[j], buf + TILE + (wave * IPW + j) * 1024);
    }
    const float* src = (wave & 1) ? a.delta : a.lse;
    bwd_load_lds4(src + row0, live ? (n - q0) * 4 : 0, 4u * lane,
                  buf + 2 * TILE + 256 * (wave & 1));
  };

  const float c2 = a.scale_log2;
  const float log2e = kLog2e;

  auto tile = [&](int qt, const char* buf) __attribute__((always_inline)) {
    if (!wave_keys) return;
    const char* Qs = buf;
    const char* Os = buf + TILE;
    const float* Ls = reinterpret_cast<const float*>(buf + 2 * TILE);
    const float* Ds = Ls + 64;
    const int q0 = qt * BQ;
    const int q1 = min(q0 + BQ, n) - 1;
    // band test over this wave's keys [kw0, kw1] and the tile's queries [q0, q1]
    if (hi_of(q1) < kw0 || lo_of(q0) > kw1) return;
    const bool full = (q0 + BQ <= n) && (kw0 + 31 < n) && (lo_of(q1) <= kw0) && (hi_of(q0) >= kw0 + 31);
    // lse (base 2) and D of the 16 query rows this lane holds.
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      l4[j] = *reinterpret_cast<const f32x4*>(Ls + 8 * j + 4 * hi);
      d4[j] = *reinterpret_cast<const f32x4*>(Ds + 8 * j + 4 * hi);
    }
    // The tile is one stream of 4*NDC products, each with one operand
    // fragment read from LDS two products ahead: S = Q K^T (Q rows; lane: key
    // l32, 16 query rows), dP = dO V^T (dO rows), dV += P^T dO (dO
    // transposed), dK += dS^T Q (Q transposed).  The vector work rides
    // between the products that do not depend on it: the base-2 -lse terms
    // beside S, P beside dP, dS beside dV.  A scheduling fence after each
    // product keeps this order.  In dV and dK the MFMA k index 8*hi + t of
    // chunk c stands for query 16*c + 8*(t/4) + 4*hi + t%4, the order the
    // accumulator holds.
    f32x16 s = f32x16{}, dp = f32x16{};
    float nl[16], p[16];
    bf16x8 pbf[2], dsbf[2];
    bf16x8 f0 = row_frag<D>(Qs, 0, 0, lane);
    bf16x8 f1 = row_frag<D>(Qs, 0, 1, lane);
    constexpr int RPK = 16 / NDC;  // rows of vector work per product
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const bf16x8 f2 = dc + 2 < NDC ? row_frag<D>(Qs, 0, dc + 2, lane)
                                     : row_frag<D>(Os, 0, dc + 2 - NDC, lane);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, kb[dc], s, 0, 0, 0);
#pragma unroll
      for (int r = RPK * dc; r < RPK * (dc + 1); ++r) nl[r] = -l4[r >> 2][r & 3] * log2e;
      f0 = f1;
      f1 = f2;
      __builtin_amdgcn_sched_barrier(0);
    }
    // -inf for pairs outside the band (or past n): P = 0 there.  A
    // wave-uniform branch of selects on the -lse terms, not on the MFMA
    // results.
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool vis = qi < n && key < n && key >= lo_of(qi) && key <= hi_of(qi);
        nl[r] = vis ? nl[r] : kNegInf;
      }
    }
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const bf16x8 f2 = dc + 2 < NDC ? row_frag<D>(Os, 0, dc + 2, lane)
                                     : tr_frag<D>(Os, 0, 32 * (dc + 2 - NDC), lane);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, vb[dc], dp, 0, 0, 0);
#pragma unroll
      for (int r = RPK * dc; r < RPK * (dc + 1); ++r) {
        p[r] = exp2_fast(__builtin_fmaf(s[r], c2, nl[r]));
        pbf[r >> 3][r & 7] = (__bf16)p[r];
      }
      f0 = f1;
      f1 = f2;
      __builtin_amdgcn_sched_barrier(0);
    }
    // dS rows formed beside dV product u: none beside the first (it would
    // wait for dP to finish), the 16 spread over the rest.
    constexpr int NU = 2 * NDB;  // products in dV (and in dK)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = u / NDB, db = u % NDB;
      const int un = u + 2;
      const bf16x8 f2 = un < NU ? tr_frag<D>(Os, 16 * (un / NDB), 32 * (un % NDB), lane)
                                : tr_frag<D>(Qs, 16 * ((un - NU) / NDB), 32 * ((un - NU) % NDB), lane);
      dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pbf[c], f0, dv[db], 0, 0, 0);
      const int r0 = u == 0 ? 0 : ((u - 1) * 16 + NU - 2) / (NU - 1);
      const int r1 = ((u) * 16 + NU - 2) / (NU - 1);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (u > 0 && r >= r0 && r < r1)
          dsbf[r >> 3][r & 7] = (__bf16)(p[r] * (dp[r] - d4[r >> 2][r & 3]));
      f0 = f1;
      f1 = f2;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = u / NDB, db = u % NDB;
      const int un = u + 2;
      bf16x8 f2 = f1;
      if (un < NU) f2 = tr_frag<D>(Qs, 16 * (un / NDB), 32 * (un % NDB), lane);
      dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsbf[c], f0, dk[db], 0, 0, 0);
      f0 = f1;
      f1 = f2;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Three buffers: the tiles two steps ahead are in flight while a tile is
  // used.  A stage is 2*IPW + 1 loads per wave and loads complete in issue
  // order, so waiting until that many remain leaves exactly the newest stage
  // in flight.  The barrier carries no memory fence (__syncthreads() would
  // also wait for every load in flight): each wave has waited for its own
  // part of the stage to use, and every LDS read of the buffer refilled next
  // has returned its data before the wave reaches the barrier (the tile's
  // products consumed it).  The empty asm statements keep the compiler from
  // moving memory accesses across.
  constexpr int kPerStage = 2 * IPW + 1;
  static_assert(kPerStage < 16, "vmcnt immediate in its low field");
  auto wait_newest = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | kPerStage);  // vmcnt(kPerStage)
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  Cursor cs{0, qt_hi}, ct{0, qt_hi};
  stage(0, cs, sB0);
  advance(cs);
  stage(1, cs, sB1);
  advance(cs);
  wait_newest();
  barrier();
  for (int t = 0;; t += 3) {
    stage(t + 2, cs, sB2);
    advance(cs);
    tile(ct.qt, sB0);
    advance(ct);
    wait_newest();
    barrier();
    if (t + 1 >= T) break;
    stage(t + 3, cs, sB0);
    advance(cs);
    tile(ct.qt, sB1);
    advance(ct);
    wait_newest();
    barrier();
    if (t + 2 >= T) break;
    stage(t + 4, cs, sB1);
    advance(cs);
    tile(ct.qt, sB2);
    advance(ct);
    wait_newest();
    barrier();
    if (t + 3 >= T) break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (!wave_keys) return;
  // dK = scale * acc; lane holds dims 32*db + l32 of keys kw0 + rho(r).
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (kr < n) {
        a.dk[(kvbase + kr) * D + 32 * db + l32] = a.scale * dk[db][r];
        a.dv[(kvbase + kr) * D + 32 * db + l32] = dv[db][r];
      }
    }
}

// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BR = NW * 32, BC = 64;
  constexpr int RB = D * 2, CPR = D / 8, TILE = BC * RB;
  constexpr int IPW = BC * CPR / (64 * NW);
  constexpr int NKB = BC / 32, NDC = D / 16, NDB = D / 32;
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split evenly over waves");
  __shared__ __attribute__((aligned(1024))) char sK0[TILE];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.n;
  const int nqb = (n + BR - 1) / BR;
  // Rounds of B*H workgroups, one query block each (heaviest causal blocks
  // first); inside a round, consecutive heads (those sharing a key/value head)
  // go to the same XCD (workgroups are dealt round-robin over 8 XCDs), so
  // their K/V reads share that XCD's L2.
  const int BH = a.B * a.H;
  const int round = blockIdx.x / BH;
  const int p = blockIdx.x - round * BH;
  const int qblk = a.causal ? nqb - 1 - round : round;
  const int bh = (BH & 7) == 0 ? (p & 7) * (BH >> 3) + (p >> 3) : p;
  const int b = bh / a.H, h = bh % a.H;
  const int g = h / (a.H / a.Hkv);
  const int causal = a.causal, window = a.window;
  auto lo_of = [&](int i) { return window >= 0 ? i - window : 0; };
  auto hi_of = [&](int i) {
    int v = causal ? i : (window >= 0 ? i + window : n - 1);
    return v < n - 1 ? v : n - 1;
  };
  const int q0 = qblk * BR;
  const int qlast = min(q0 + BR, n) - 1;
  const int kt_lo = max(lo_of(q0), 0) / BC;
  const int kt_hi = hi_of(qlast) / BC;

  const int wq0 = q0 + 32 * wave;
  const bool wave_rows = wq0 < n;
  const int wr1 = min(wq0 + 32, n) - 1;
  const int wlo0 = lo_of(wq0), whi0 = hi_of(wq0);
  const int wlo1 = lo_of(wr1), whi1 = hi_of(wr1);
  const int row = wq0 + l32;
  const int rlo = lo_of(row), rhi = hi_of(row);
  const size_t qrow = (size_t)(b * a.H + h) * n + row;
  const __bf16* Kh = a.k + (size_t)(b * a.Hkv + g) * n * D;
  const __bf16* Vh = a.v + (size_t)(b * a.Hkv + g) * n * D;

  bf16x8 qf[NDC], of[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    if (row < n) {
      qf[dc] = *reinterpret_cast<const bf16x8*>(a.q + qrow * D + 16 * dc + 8 * hi);
      of[dc] = *reinterpret_cast<const bf16x8*>(a.dout + qrow * D + 16 * dc + 8 * hi);
    } else {
      qf[dc] = bf16x8{};
      of[dc] = bf16x8{};
    }
  }
  const float pl = row < n ? a.lse[qrow] * kLog2e : 0.f;
  const float dd = row < n ? a.delta[qrow] : 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  unsigned st_off[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int s = (wave * IPW + j) * 64 + lane;
    const int r = s / CPR;
    const int c = (s % CPR) ^ bswz<D>(r);
    st_off[j] = (unsigned)(r * RB + c * 16);
  }
  auto stage = [&](int kt, char* tk, char* tv) {
    const int k0 = kt * BC;
    const int bytes = (n - k0) * RB;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      bwd_load_lds16(Kh + (size_t)k0 * D, bytes, st_off[j], tk + (wave * IPW + j) * 1024);
      bwd_load_lds16(Vh + (size_t)k0 * D, bytes, st_off[j], tv + (wave * IPW + j) * 1024);
    }
  };
  const float c2 = a.scale_log2;

  auto tile = [&](int kt, const char* Ks, const char* Vs) __attribute__((always_inline)) {
    const int k0 = kt * BC, k1 = k0 + BC - 1;
    if (!wave_rows || k1 < wlo0 || k0 > whi1) return;
    const bool full = (k0 >= wlo1) && (k1 <= whi0);
    // Per 32-key half: S^T = K Q^T and dP^T = V dO^T (lane owns a query row and
    // 16 key rows), dS^T, then dQ^T += K^T dS^T with K^T read transposed; the
    // MFMA k index follows the key order of the accumulator.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const bf16x8 ka = row_frag<D>(Ks, 32 * kb, dc, lane);
        const bf16x8 va = row_frag<D>(Vs, 32 * kb, dc, lane);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[dc], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, of[dc], dp, 0, 0, 0);
      }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (kk < rlo || kk > rhi) s[r] = kNegInf;
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(__builtin_fmaf(s[r], c2, -pl));
        dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dd));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 kt_f = tr_frag<D>(Ks, 32 * kb + 16 * c, 32 * db, lane);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_f, dsb[c], acc[db], 0, 0, 0);
        }
    }
  };

  stage(kt_lo, sK0, sV0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
    if (kt + 1 <= kt_hi) stage(kt + 1, sK1, sV1);
    tile(kt, sK0, sV0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 > kt_hi) break;
    if (kt + 2 <= kt_hi) stage(kt + 2, sK0, sV0);
    tile(kt + 1, sK1, sV1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (row >= n) return;
  // dQ = scale * acc: lane holds dims 32*db + 8*(r/4) + 4*hi + r%4 of its row.
  float* out = a.dq + qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = a.scale * acc[db][4 * g4 + j];
      *reinterpret_cast<f32x4*>(out + 32 * db + 8 * g4 + 4 * hi) = x;
    }
}

size_t bwd_workspace_bytes(int B, int H, int n) { return (size_t)B * H * n * sizeof(float); }

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.n;
  hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nkb = (a.n + 127) / 128;
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)(nkb * a.B * a.Hkv)), dim3(256), 0, stream,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Without a window eight waves (256 query rows) share each staged K/V tile,
  // as in the forward kernel (0.8 % faster on the long causal backward);
  // with one, four waves leave fewer partly masked tiles at the band edges.
  if (a.window < 0) {
    const long long nqb = (a.n + 255) / 256;
    hipLaunchKernelGGL((bwd_dq_kernel<D, 8>), dim3((unsigned)(nqb * a.B * a.H)), dim3(512), 0,
                       stream, a);
  } else {
    const long long nqb = (a.n + 127) / 128;
    hipLaunchKernelGGL((bwd_dq_kernel<D, 4>), dim3((unsigned)(nqb * a.B * a.H)), dim3(256), 0,
                       stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* delta, int B, int H, int Hkv, int n, int d, int causal,
                           int window, float scale, hipStream_t stream) {
  BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.lse = lse;
  a.dout = static_cast<const __bf16*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.B = B; a.H = H; a.Hkv = Hkv; a.n = n; a.causal = causal; a.window = window;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  if (d == 128) return launch_bwd_d<128>(a, stream);
  if (d == 64) return launch_bwd_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

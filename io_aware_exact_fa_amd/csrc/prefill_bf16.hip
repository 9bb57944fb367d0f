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
//   * Workgroup = NW waves of 64 lanes (8 for dense, strided or paged
//     layouts whose rows see 16K keys or more, else 4); wave w owns 32 query
//     rows.  Registers are kept under 256 per lane so two waves
//     share each SIMD (one workgroup of 8 or two of 4 per CU): one wave's
//     softmax (vector ALU) overlaps the other's matrix-core work.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims (one ds_read_b128 per
//     lane from LDS), B = Q^T fragment held in VGPRs for the whole loop.  In the
//     32x32 accumulator layout lane l owns query column l%32 and 16 key rows,
//     so the row max / row sum of a query is a 16-value in-lane reduction plus
//     one cross-half swap (v_permlane32_swap) -- no LDS round trip.
//   * The same registers, rounded to bf16, are directly the B operand P^T of
//     the O^T += V^T P^T MFMA: the MFMA's k index is mapped onto the key order
//     the accumulator layout produced.  V stays row-major in LDS and its
//     transposed fragments come from ds_read_b64_tr_b16 (two per fragment).
//   * Softmax runs in the base-2 domain with scale*log2(e) folded into one FMA
//     before v_exp_f32.  A row's reference max moves only when its tile max
//     exceeds it by more than 2^8 (the same reference divides numerator and
//     denominator, so the result is unchanged); most tiles skip the
//     accumulator rescale.
//   * K/V tiles go HBM -> LDS directly (buffer_load_dwordx4 ... lds through
//     one scalar buffer descriptor per tile, no staging registers; the
//     descriptor's range check returns zeros past the sequence end),
//     double-buffered: the next tile's loads are in flight during the current
//     tile; one barrier per tile.  Tiles are dense with an XOR chunk swizzle
//     instead of padding.
//   * Grid order: key/value groups are dealt to the 8 XCDs in turn (dispatch
//     is round-robin), and each XCD runs its groups one after another, a
//     group's query tiles heaviest causal first with its query heads side by
//     side: the workgroups an XCD runs together read the same K/V tiles from
//     its L2, and every XCD gets an equal share of every sequence.  Short
//     causal grids pair query blocks (a workgroup runs block NQ-1-t, then t)
//     so that every workgroup carries the same number of key tiles.

#include "common.hpp"
#include "launch.hpp"

namespace fa {

// Layout of the sequences a launch covers.
//   kDense : q, o [B, H, n, d]; k, v [B, Hkv, n, d]; lse [B, H, n].
//   kVarlen: ragged batch packed per head: q, o [H, total, d]; k, v
//            [Hkv, total, d]; lse [H, total]; sequence b owns rows
//            cu_q[b] .. cu_q[b+1]-1 (xxqk.cn article §8.1: each request's
//            traversal is clipped to its own length, no padding).
//   kPaged : new chunks over paged histories (charles2530 blog §5, §7): q, o
//            [H, total, d] packed like kVarlen; keys and values in pages
//            [num_pages, Hkv, 16, d] behind page_table [B, max_pages];
//            sequence b has seqlens_k[b] keys and its chunk's queries are the
//            last positions among them.
//   kBlockSparse: the dense layout plus a 0/1 layout over blocks of 128 query
//            rows by block_k keys ([layout_heads, ceil(n/128),
//            ceil(n/block_k)], shared by the batch, one per head or one for
//            all); a workgroup visits only its kept key tiles ("Block-Sparse
//            FlashAttention", ruiowl.com deep-dive §四; the band skip of the
//            xxqk.cn article §5 is the case of a band layout).
//   kStrided: the dense problem with caller-given element strides for
//            (batch, head, row) of q, k, v and o, the head dim contiguous (for
//            instance the (batch, seqlen, heads, head_dim) layout of the
//            library call in the xxqk.cn article §7.1); k and v share a row
//            stride.  lse stays [B, H, n].
enum PrefillMode { kDense = 0, kVarlen = 1, kPaged = 2, kBlockSparse = 3, kStrided = 4 };

// Most key tiles a block-sparse workgroup can list (n <= 2048 * 64).
constexpr int kMaxSparseTiles = 2048;

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct PrefillArgs {
  const __bf16* q;
  const __bf16* k;  // kPaged: key pages
  const __bf16* v;  // kPaged: value pages
  __bf16* o;
  float* lse;
  int B, H, Hkv, n, causal, window, nqb;
  float scale_log2;  // scale * log2(e)
  // kVarlen / kPaged
  const int* cu_q;        // [B+1] query (and, kVarlen, key) offsets
  const int* seqlens_k;   // kPaged: [B] keys per sequence
  const int* page_table;  // kPaged: [B, max_pages]
  int total;              // packed rows per head
  int max_seqlen;         // longest query run (grid size)
  int max_pages, num_pages;
  // kBlockSparse
  const unsigned char* layout;
  int layout_heads, layout_cols, tile_shift;  // tile_shift: log2(block_k / 64)
  // kStrided: element strides (batch, head) and row strides
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_ss, kv_ss, o_ss;
  // 1: each workgroup runs query blocks NQ-1-t and t (causal load balance)
  int pair;
  // Counting launches only: [0] += (wave, key tile) pairs whose products are
  // computed, [1] += key/value tiles staged into LDS.
  unsigned long long* counters;
};

// LDS tiles are dense (no padding): row r of a tile holds D bf16 values as
// 16-byte chunks, and logical chunk c of row r sits at physical chunk
// c ^ swz(r).  The swizzle spreads the 16-byte row reads of the K fragments
// (8-16 consecutive rows, one chunk each) and the 8-byte transposed reads of
// the V fragments (4 consecutive rows, 4 chunks each) over distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return row & 7;
}

// 16 bytes per lane from HBM straight into LDS: lane i's bytes land at
// lds + 16*i; the source is base + off, read as zero when off >= nbytes
// (buffer descriptor range check).
__device__ __forceinline__ void buffer_load_lds16(const void* base, int nbytes, unsigned off,
                                                  void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, 0, 0, 0);
}

// Reference-max update threshold (base-2 exponent units).  The reference max
// of a row only moves when the tile max exceeds it by more than this, so
// probabilities stay <= 2^8 and most tiles skip the accumulator rescale.
constexpr float kRescaleThreshold = 8.0f;

template <int D, int NW, int BC, int MODE, bool COUNT = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int BR = NW * 32;         // query rows per workgroup (32 per wave)
  constexpr int RB = D * 2;           // bytes per tile row
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int TILE_BYTES = BC * RB;
  constexpr int IPW = BC * CPR / (64 * NW);  // direct-to-LDS loads per wave per tensor
  constexpr int NKB = BC / 32;        // 32-key MFMA blocks per tile
  constexpr int NDC = D / 16;         // 16-wide head-dim chunks (QK^T contraction)
  constexpr int NDB = D / 32;         // 32-wide head-dim blocks (PV output)
  constexpr int NKC = BC / 16;        // 16-key chunks (PV contraction)
  static_assert(BC * CPR % (64 * NW) == 0, "tile must split evenly over waves");
  static_assert(MODE != kPaged || BC == 64, "a paged key tile is four 16-token pages");

  // Double-buffered K and V tiles (BC x D bf16 each).  Four separate objects,
  // so the compiler can tell the tile being read from the tile being filled
  // by the in-flight HBM->LDS loads and does not wait for those loads.
  __shared__ __attribute__((aligned(1024))) char sK0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;

  // ---- workgroup -> (b, h, query tile) ----
  // Workgroup p runs on XCD p % 8 (round-robin dispatch).  Key/value groups
  // (b, g) are dealt to the XCDs in turn; each XCD then works through its
  // groups one after another, a group's query tiles heaviest (causal) first
  // with the group's G query heads side by side.  The workgroups an XCD runs
  // at once thus read the same K/V tiles from its L2, and every XCD gets an
  // equal share of every sequence (ragged batches stay balanced).
  // With pairing (causal), workgroup t of a head also runs query block t
  // after block NQ-1-t: every workgroup then has the same number of key
  // tiles (2*NQ + 2 for full causal), so the grid ends without a tail of
  // short blocks.
  const int G = a.H / a.Hkv;
  const int NQ = a.nqb;
  const int NT = a.pair ? (NQ + 1) / 2 : NQ;  // workgroups per (b, h)
  const int idx = blockIdx.x;
  int b, h, g, t;
  if (((a.B * a.Hkv) & 7) == 0) {
    const int j = idx >> 3;
    const int per_group = G * NT;
    const int u = (idx & 7) + 8 * (j / per_group);  // (b, g) unit
    const int rest = j - (j / per_group) * per_group;
    t = rest / G;
    b = u / a.Hkv;
    g = u - b * a.Hkv;
    h = g * G + (rest - t * G);
  } else {
    // B*Hkv not a multiple of 8 (the groups cannot be dealt evenly to the
    // XCDs): rounds of B*H workgroups, one query tile each (heaviest causal
    // tiles first), consecutive heads on one XCD when B*H is a multiple of 8.
    t = idx / BH;
    const int p = idx - t * BH;
    const int bh = (BH & 7) == 0 ? (p & 7) * (BH >> 3) + (p >> 3) : p;
    b = bh / a.H;
    h = bh - b * a.H;
    g = h / G;
  }
  const int qb_first = a.causal ? (NQ - 1 - t) : t;
  const int qb_second = (a.pair && t != NQ - 1 - t) ? t : -1;

  // Rows of this (b, h): n_q queries, n_k keys, query i at position i + qoff
  // among the keys.  Offsets read from memory are clamped so every access
  // stays inside the buffers whatever they hold.
  int n_q, n_k, qoff = 0;
  const __bf16 *Qh, *Kh = nullptr, *Vh = nullptr;
  __bf16* Oh;
  float* Lh;
  static_assert(MODE == kDense || MODE == kVarlen || MODE == kPaged || MODE == kBlockSparse ||
                    MODE == kStrided,
                "unknown layout mode");
  // Row strides in elements (the head dim is contiguous in every layout).
  const int q_rs = MODE == kStrided ? a.q_ss : D;
  const int kv_rs = MODE == kStrided ? a.kv_ss : D;
  const int o_rs = MODE == kStrided ? a.o_ss : D;
  if constexpr (MODE == kStrided) {
    n_q = n_k = a.n;
    Qh = a.q + b * a.q_sb + h * a.q_sh;
    Kh = a.k + b * a.k_sb + g * a.k_sh;
    Vh = a.v + b * a.v_sb + g * a.v_sh;
    Oh = a.o + b * a.o_sb + h * a.o_sh;
    Lh = a.lse + (size_t)(b * a.H + h) * a.n;
  } else if constexpr (MODE == kDense || MODE == kBlockSparse) {  // [B, heads, n, d]
    n_q = n_k = a.n;
    Qh = a.q + (size_t)(b * a.H + h) * a.n * D;
    Kh = a.k + (size_t)(b * a.Hkv + g) * a.n * D;
    Vh = a.v + (size_t)(b * a.Hkv + g) * a.n * D;
    Oh = a.o + (size_t)(b * a.H + h) * a.n * D;
    Lh = a.lse + (size_t)(b * a.H + h) * a.n;
  } else {  // kVarlen, kPaged: packed rows located through cu_q
    const int s0 = min(max(a.cu_q[b], 0), a.total);
    n_q = min(max(a.cu_q[b + 1] - s0, 0), min(a.max_seqlen, a.total - s0));
    Qh = a.q + ((size_t)h * a.total + s0) * D;
    Oh = a.o + ((size_t)h * a.total + s0) * D;
    Lh = a.lse + (size_t)h * a.total + s0;
    if constexpr (MODE == kVarlen) {
      n_k = n_q;
      Kh = a.k + ((size_t)g * a.total + s0) * D;
      Vh = a.v + ((size_t)g * a.total + s0) * D;
    } else {
      n_k = min(max(a.seqlens_k[b], 0), a.max_pages * 16);
      qoff = n_k - n_q;
    }
  }

  const int causal = a.causal, window = a.window;
  // Visible keys of row i (at position i + qoff) form the interval
  // [lo(i), hi(i)], both monotone in i.
  auto lo_of = [&](int i) { return window >= 0 ? i + qoff - window : 0; };
  auto hi_of = [&](int i) {
    int v = causal ? i + qoff : (window >= 0 ? i + qoff + window : n_k - 1);
    return v < n_k - 1 ? v : n_k - 1;
  };

  // One query block: its rows' tile loop and epilogue.
  auto query_block = [&](const int qb) __attribute__((always_inline)) {
    const int q0 = qb * BR;
    if (q0 >= n_q) return;  // past this sequence's rows (ragged batches)
    const int qlast = min(q0 + BR, n_q) - 1;
    const int kt_lo = max(lo_of(q0), 0) / BC;
    const int hi_last = hi_of(qlast);
    const int kt_hi = hi_last < 0 ? -1 : hi_last / BC;

    // ---- this wave's 32 query rows; lane owns row wq0 + l32 ----
    const int wq0 = q0 + wave * 32;
    const bool wave_rows = wq0 < n_q;
    const int wr1 = min(wq0 + 32, n_q) - 1;
    const int wlo0 = lo_of(wq0), whi0 = hi_of(wq0);
    const int wlo1 = lo_of(wr1), whi1 = hi_of(wr1);
    const int row = wq0 + l32;
    const int rlo = lo_of(row), rhi = hi_of(row);

    // Q^T fragments (B operand): query row l32, dims 16*dc + 8*hi .. +8.
    bf16x8 qf[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
      qf[dc] = (row < n_q) ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)row * q_rs + dc * 16 +
                                                               hi * 8)
                           : bf16x8{};

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_ref = kNegInf;  // reference max (base-2 scaled units) of this lane's row
    float l_run = 0.f;      // this lane's share of the row sum (pair with lane ^ 32)
    // Counting launches: this wave's visited tiles and (wave 0) staged tiles,
    // added to the device counters once per query block.
    unsigned visited = 0, staged = 0;

    // ---- direct HBM -> LDS staging of one K/V tile ----
    // Wave instruction j writes 64 consecutive 16-byte slots; slot s holds
    // physical chunk s % CPR of tile row s / CPR.  Loads are buffer loads whose
    // descriptor (in scalar registers) starts at the tile and ends at the end of
    // the sequence: each lane's offset is a fixed register, and rows past the
    // end of the sequence read as zeros by the hardware range check (those keys
    // are masked and their zero values contribute nothing).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    unsigned st_off[IPW];  // byte offset of the slot's chunk in a dense tile
    int st_row[IPW];       // tile row of the slot
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int s = (wave_u * IPW + j) * 64 + lane;
      const int r = s / CPR;
      const int c = (s % CPR) ^ swz<D>(r);
      st_off[j] = (unsigned)(r * kv_rs * 2 + c * 16);
      st_row[j] = r;
    }
    // Paged tiles: each slot's byte offset inside its 16-row page.
    unsigned pg_off[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      pg_off[j] = st_off[j] - (unsigned)(st_row[j] & ~15) * (unsigned)RB;
    // Paged tiles: a 64-key tile spans four 16-token pages and wave w's load
    // slots fill page w of the tile (4 waves) or half of page w/2 (8 waves), so
    // each wave needs one page id per tile (pages past the sequence's last one repeat it; an id outside
    // [0, num_pages) reads page 0 instead, so no access leaves the cache
    // whatever the table holds).
    static_assert(MODE != kPaged || BC / NW == 16 || BC / NW == 8,
                  "a wave's load slots fill one 16-token page or half of one");
    constexpr int WPP = MODE == kPaged ? 16 / (BC / NW) : 1;  // waves per page
    // The table is read-only during the kernel: read through the constant
    // address space it is a scalar load, counted apart from the K/V DMAs (a
    // vector load here made the compiler wait for the next tile's DMAs before
    // the current tile's products).
    typedef __attribute__((address_space(4))) const int* const_iptr;
    const_iptr pt = nullptr;
    if constexpr (MODE == kPaged)
      pt = (const_iptr)(uintptr_t)(a.page_table + (size_t)b * a.max_pages);
    const int last_page = (n_k - 1) >> 4;
    // The load is issued a tile ahead; the range check happens at the stage
    // that uses it, so nothing waits for it until then.
    auto page_id = [&](int kt) { return pt[min(kt * 4 + wave_u / WPP, last_page)]; };
    auto stage = [&](int kt, char* tk, char* tv, int pid) {
      const int k0 = kt * BC;
      if constexpr (COUNT) staged += 1;
      if constexpr (MODE != kPaged) {
        (void)pid;
        // the descriptor ends after the tile's last row inside the sequence:
        // later rows read as zero (their offsets lie beyond it, as rows are at
        // least a row apart)
        const int bytes = (min(n_k - k0, BC) - 1) * kv_rs * 2 + RB;
        const __bf16* kb = Kh + (size_t)k0 * kv_rs;
        const __bf16* vb = Vh + (size_t)k0 * kv_rs;
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
          buffer_load_lds16(kb, bytes, st_off[j], tk + (wave_u * IPW + j) * 1024);
          buffer_load_lds16(vb, bytes, st_off[j], tv + (wave_u * IPW + j) * 1024);
        }
      } else {
        // This wave's page is read through a scalar descriptor sized to the
        // page's rows inside the sequence: rows past the last key read as
        // zeros (finite, and the mask gives them zero weight).  A page past the
        // sequence (its id repeats the last page) or an id outside [0,
        // num_pages) (read as page 0) stays in bounds.  Per lane only the
        // fixed offset inside the page is needed, so no address arithmetic is
        // repeated per tile.
        int pg = __builtin_amdgcn_readfirstlane(pid);
        pg = (pg < 0 || pg >= a.num_pages) ? 0 : pg;
        const int p0 = min(kt * 4 + wave_u / WPP, last_page) * 16;  // first key of the page read
        const int rows = min(n_k - p0, 16);
        const size_t base = ((size_t)pg * a.Hkv + g) * 16 * D;
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
          buffer_load_lds16(a.k + base, rows * RB, pg_off[j], tk + (wave_u * IPW + j) * 1024);
          buffer_load_lds16(a.v + base, rows * RB, pg_off[j], tv + (wave_u * IPW + j) * 1024);
        }
      }
    };

    // Per-lane LDS byte offsets of the fragments (tile-relative).
    // K fragment (kb, dc): row kb*32 + l32, logical chunk 2*dc + hi.
    // V^T fragment (db, kc, half): 8-byte transposed read; lane supplies row
    // 16*kc + 8*half + 4*hi + (lane%16)/4 and dims db*32 + 16*((lane/16)%2) + 4*(lane%4).
    const int krow_sw = swz<D>(l32);
    const int vrow = 4 * hi + ((lane & 15) >> 2);
    // swz depends on row bits 0-3: adding 16*kc keeps it, adding 8*half does not.
    const int vrow_sw[2] = {swz<D>(vrow), swz<D>(vrow + 8)};
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    const float c2 = a.scale_log2;

    // One key tile from LDS (Ks, Vs): S^T = K Q^T, masked online softmax,
    // O^T += V^T P^T.
    auto tile = [&](int kt, const char* Ks, const char* Vs) __attribute__((always_inline)) {
      const int k0 = kt * BC, k1 = k0 + BC - 1;
      const bool active = wave_rows && !(k1 < wlo0 || k0 > whi1);
      const bool full = (k0 >= wlo1) && (k1 <= whi0);
      if (!active) return;
      if constexpr (COUNT) visited += 1;
      // S^T = K Q^T; the K fragments of the next head-dim chunk are read while
      // the current chunk's MFMAs run.
      auto kfrag = [&](int dc, int kb) {
        const int off = (kb * 32 + l32) * RB + (((2 * dc + hi) ^ krow_sw) << 4);
        return *reinterpret_cast<const bf16x8*>(Ks + off);
      };
      f32x16 s[NKB];
      bf16x8 kcur[NKB], knext[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        kcur[kb] = kfrag(0, kb);
      }
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        if (dc + 1 < NDC) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) knext[kb] = kfrag(dc + 1, kb);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[kb], qf[dc], s[kb], 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) kcur[kb] = knext[kb];
      }
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key < rlo || key > rhi) s[kb][r] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
      mx = max_xor32(mx) * c2;
      // Move the reference max only when the row max outgrows it by more than
      // the threshold (or on the row's first visible key); wave-uniform branch.
      const bool need = mx > m_ref + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? exp2_fast(m_ref - mx) : 1.f;
        m_ref = need ? mx : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      }
      // A row with nothing visible yet keeps m_ref = -inf and sees only -inf
      // scores here; use 0 so exp2(-inf - m) is 0 rather than NaN.
      const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
      bf16x8 pf[NKC];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2_fast(__builtin_fmaf(s[kb][r], c2, -m_use));
          rs += pv;
          pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)pv;
        }
      l_run += rs;
      // O^T += V^T P^T.  MFMA k index 8*hi + t stands for key
      // 16*kc + 8*(t/4) + 4*hi + t%4, the order the S^T accumulator holds.
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          bf16x8 vf;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int r = 16 * kc + 8 * half + vrow;
            const int cbyte = (db * 32 + vcol) * 2;
            const int off = r * RB + ((((cbyte >> 4) ^ vrow_sw[half]) << 4) | (cbyte & 15));
            typedef short i16x4 __attribute__((ext_vector_type(4)));
            const i16x4 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(
                    (__attribute__((address_space(3))) char*)(Vs) + off));
            const bf16x4 b4 = __builtin_bit_cast(bf16x4, t4);
            vf[4 * half + 0] = b4[0];
            vf[4 * half + 1] = b4[1];
            vf[4 * half + 2] = b4[2];
            vf[4 * half + 3] = b4[3];
          }
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kc], acc[db], 0, 0, 0);
        }
      }
    };

    // The key tiles visited, in order: kt_lo .. kt_hi, or for a block-sparse
    // workgroup the kept ones among them, listed in LDS by wave 0 (ballot +
    // prefix count over 64 tiles at a time).
    int nt = kt_hi - kt_lo + 1;
    unsigned short* tiles = nullptr;
    if constexpr (MODE == kBlockSparse) {
      __shared__ unsigned short sTiles[kMaxSparseTiles];
      __shared__ int sCount;
      tiles = sTiles;
      const int lh = a.layout_heads == 1 ? 0 : h;
      const unsigned char* lay =
          a.layout + ((size_t)lh * a.nqb + qb) * (size_t)a.layout_cols;
      // A paired workgroup builds a second list here: every wave must have
      // read the first block's count before wave 0 overwrites it (a block
      // with no kept tile runs no barrier in its loop).
      if (a.pair) __syncthreads();
      if (wave_u == 0) {
        int cnt = 0;
        for (int c0 = kt_lo; c0 <= kt_hi; c0 += 64) {
          const int kt = c0 + lane;
          // every lane reads an entry of its own row (index clamped to kt_hi)
          const bool on = (lay[min(kt, kt_hi) >> a.tile_shift] != 0) && kt <= kt_hi;
          const unsigned long long m = __builtin_amdgcn_ballot_w64(on);
          const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
          if (on) sTiles[cnt + before] = (unsigned short)kt;
          cnt += __builtin_popcountll(m);
        }
        if (lane == 0) sCount = cnt;
      }
      __syncthreads();
      nt = __builtin_amdgcn_readfirstlane(sCount);
    }
    auto kt_at = [&](int i) {
      if constexpr (MODE == kBlockSparse)
        return (int)__builtin_amdgcn_readfirstlane(tiles[i]);
      else
        return kt_lo + i;
    };

    // Page ids are fetched one tile ahead of their stage.  The fetch is issued
    // whether or not that tile exists (its index is clamped to the sequence's
    // last page): a load under a branch would make the compiler wait for every
    // load in flight, the next tile's DMA included, before the current tile.
    int pid_next = 0;
    if (nt > 0) {
      if constexpr (MODE == kPaged) pid_next = page_id(kt_lo);
      stage(kt_at(0), sK0, sV0, pid_next);
      if constexpr (MODE == kPaged) pid_next = page_id(kt_lo + 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    // Unrolled by two so that each tile's buffer is a fixed LDS object.
    for (int i = 0; i < nt; i += 2) {
      const int kt = kt_at(i);
      if (i + 1 < nt) stage(kt_at(i + 1), sK1, sV1, pid_next);
      if constexpr (MODE == kPaged) pid_next = page_id(kt + 2);
      tile(kt, sK0, sV0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (i + 1 >= nt) break;
      if (i + 2 < nt) stage(kt_at(i + 2), sK0, sV0, pid_next);
      if constexpr (MODE == kPaged) pid_next = page_id(kt + 3);
      tile(kt_at(i + 1), sK1, sV1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    if constexpr (COUNT) {
      if (lane == 0) {
        if (visited) atomicAdd(&a.counters[0], (unsigned long long)visited);
        if (wave_u == 0 && staged) atomicAdd(&a.counters[1], (unsigned long long)staged);
      }
    }
    // ---- epilogue: O = acc / l, lse = ln(2) * (m + log2 l) ----
    if (!wave_rows) return;
    const float lt = sum_xor32(l_run);
    if (row >= n_q) return;
    // lt = 0 only for a row that sees no key (a chunk longer than its
    // sequence's keys): o = 0, lse = -inf.
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    __bf16* orow = Oh + (size_t)row * o_rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(acc[db][4 * g4 + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g4 + 4 * hi) = ov;
      }
    if (hi == 0) {
      const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;
      Lh[row] = lt > 0.f ? (m_use + log2_fast(lt)) * kLn2 : kNegInf;
    }
  };
  query_block(qb_first);
  if (qb_second >= 0) query_block(qb_second);
}

template <int D, int MODE, int NW, bool COUNT = false>
static hipError_t launch_nw(const PrefillArgs& a0, int rows, hipStream_t stream) {
  constexpr int BC = 64;
  constexpr int BR = NW * 32;
  constexpr long long kResident = 256 * (8 / NW);  // workgroups the part holds at once
  PrefillArgs a = a0;
  a.nqb = (rows + BR - 1) / BR;
  // Pair causal query blocks where all sequences share the block count and
  // the grid is short: below 16 rounds of resident workgroups the tail of
  // short blocks costs ~6 % (B4 H16 n4096); above, heaviest-first order
  // leaves little tail and pairing measured 1 % slower.
  a.pair = a.causal && (MODE == kDense || MODE == kStrided || MODE == kBlockSparse) &&
           (long long)a.nqb * a.B * a.H < 16 * kResident;
  const long long grid = (long long)(a.pair ? (a.nqb + 1) / 2 : a.nqb) * a.B * a.H;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, BC, MODE, COUNT>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

// Eight waves (256 query rows, one workgroup per CU) share each staged K/V
// tile when every row sees many keys: half the tile loads and barriers per
// row, 3 % faster on long causal and full attention.  With narrower windows
// four waves (128 rows, two workgroups per CU) leave fewer partly masked
// tiles at the band edges; the two tie near 8K keys per row (causal w 4096,
// band w 4096), 8 waves win from 16K (band w 8192: 2 %, causal w 16384:
// 0.8 %) and lose below (causal w 1024: 7 %).  Chunks over pages follow the
// same rule (2 waves per page: 16 chunks of 2048 over long prefixes 2.9 %
// faster).  Ragged batches measured the same either way (each sequence's
// partly filled last block offsets the gain) and block-sparse layouts are
// defined over 128-row blocks: four waves for both.
template <int D, int MODE, bool COUNT = false>
static hipError_t launch_d(const PrefillArgs& a, int rows, hipStream_t stream) {
  if constexpr (MODE == kDense || MODE == kStrided || MODE == kPaged) {
    const long long keys_per_row =
        a.window < 0 ? (1LL << 62) : (a.causal ? a.window + 1LL : 2LL * a.window + 1);
    if (keys_per_row >= 16384) return launch_nw<D, MODE, 8, COUNT>(a, rows, stream);
  }
  return launch_nw<D, MODE, 4, COUNT>(a, rows, stream);
}

static PrefillArgs base_args(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Hkv, int causal, int window, float scale) {
  PrefillArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.causal = causal;
  a.window = window;
  a.scale_log2 = scale * kLog2e;
  return a;
}

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Hkv, int n, int d, int causal, int window,
                               float scale, hipStream_t stream) {
  PrefillArgs a = base_args(q, k, v, o, lse, B, H, Hkv, causal, window, scale);
  a.n = n;
  if (d == 128) return launch_d<128, kDense>(a, n, stream);
  if (d == 64) return launch_d<64, kDense>(a, n, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16_counted(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int H, int Hkv, int n, int d,
                                       int causal, int window, float scale,
                                       unsigned long long* counters, hipStream_t stream) {
  PrefillArgs a = base_args(q, k, v, o, lse, B, H, Hkv, causal, window, scale);
  a.n = n;
  a.counters = counters;
  if (d == 128) return launch_d<128, kDense, true>(a, n, stream);
  if (d == 64) return launch_d<64, kDense, true>(a, n, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16_varlen(const void* q, const void* k, const void* v, void* o,
                                      float* lse, const int* cu_seqlens, int B, int H, int Hkv,
                                      int total, int max_seqlen, int d, int causal, int window,
                                      float scale, hipStream_t stream) {
  PrefillArgs a = base_args(q, k, v, o, lse, B, H, Hkv, causal, window, scale);
  a.cu_q = cu_seqlens;
  a.total = total;
  a.max_seqlen = max_seqlen;
  if (d == 128) return launch_d<128, kVarlen>(a, max_seqlen, stream);
  if (d == 64) return launch_d<64, kVarlen>(a, max_seqlen, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16_blocksparse(const void* q, const void* k, const void* v, void* o,
                                           float* lse, const unsigned char* layout,
                                           int layout_heads, int B, int H, int Hkv, int n, int d,
                                           int block_k, int causal, int window, float scale,
                                           hipStream_t stream) {
  PrefillArgs a = base_args(q, k, v, o, lse, B, H, Hkv, causal, window, scale);
  a.n = n;
  a.layout = layout;
  a.layout_heads = layout_heads;
  a.layout_cols = (n + block_k - 1) / block_k;
  a.tile_shift = block_k == 128 ? 1 : 0;
  if (d == 128) return launch_d<128, kBlockSparse>(a, n, stream);
  if (d == 64) return launch_d<64, kBlockSparse>(a, n, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16_strided(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const long long* strides, int B, int H,
                                       int Hkv, int n, int d, int causal, int window, float scale,
                                       hipStream_t stream) {
  PrefillArgs a = base_args(q, k, v, o, lse, B, H, Hkv, causal, window, scale);
  a.n = n;
  a.q_sb = strides[0]; a.q_sh = strides[1]; a.q_ss = (int)strides[2];
  a.k_sb = strides[3]; a.k_sh = strides[4]; a.kv_ss = (int)strides[5];
  a.v_sb = strides[6]; a.v_sh = strides[7];
  a.o_sb = strides[9]; a.o_sh = strides[10]; a.o_ss = (int)strides[11];
  if (d == 128) return launch_d<128, kStrided>(a, n, stream);
  if (d == 64) return launch_d<64, kStrided>(a, n, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16_paged(const void* q, const void* kcache, const void* vcache,
                                     const int* page_table, const int* cu_seqlens_q,
                                     const int* seqlens_k, void* o, float* lse, int B, int H,
                                     int Hkv, int d, int total_q, int max_seqlen_q, int num_pages,
                                     int max_pages, int causal, int window, float scale,
                                     hipStream_t stream) {
  PrefillArgs a = base_args(q, kcache, vcache, o, lse, B, H, Hkv, causal, window, scale);
  a.cu_q = cu_seqlens_q;
  a.seqlens_k = seqlens_k;
  a.page_table = page_table;
  a.total = total_q;
  a.max_seqlen = max_seqlen_q;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  if (d == 128) return launch_d<128, kPaged>(a, max_seqlen_q, stream);
  if (d == 64) return launch_d<64, kPaged>(a, max_seqlen_q, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

/*
 * fa.h -- C ABI of libfa.so: exact attention (forward, decode, backward) for
 * AMD MI355X (gfx950).
 *
 * All operations are exact (no approximation of the softmax):
 *
 *   fa_fwd     prefill / self-attention forward over a whole sequence, computed
 *              tile by tile with an online softmax so the n x n score matrix
 *              never exists in device memory; key tiles wholly outside the
 *              causal or sliding-window band are never visited.
 *   fa_decode  one new query token per sequence attending to its whole paged
 *              KV cache, split along the cache (flash decoding) and merged by
 *              log-sum-exp weights.
 *   fa_bwd     gradients dq, dk, dv of fa_fwd's output, recomputing the
 *              probabilities tile by tile from the saved log-sum-exp.
 *   fa_fwd_varlen  fa_fwd over a ragged batch packed without padding.
 *   fa_fwd_paged   chunked prefill: new query chunks over paged KV histories.
 *   fa_fwd_blocksparse  fa_fwd restricted to the kept blocks of a layout.
 *   fa_decode_fp8  fa_decode over an FP8 (E4M3) key/value cache.
 *   fa_fwd_strided fa_fwd over caller-strided tensors (e.g. BSHD).
 *   fa_fwd_tile_count  fa_fwd (bf16) that also counts the key tiles it
 *              visits and stages (the skip, observed on the device).
 *
 * Sources (web pages on IO-aware exact attention):
 *   - charles2530 blog "算子与编译器：FlashAttention 与长上下文": §1 (the
 *     formula softmax(Q Kᵀ/√d) V), §2 (tiling + online softmax, no score
 *     matrix in HBM), §4 and §6 (decode reads a long KV history for a short
 *     query, so it is parallelised along the history), §5 (paged KV).
 *   - xxqk.cn article on FlashAttention for sliding-window prefill: §3.1-§3.2
 *     (tiles and the running max / running sum / rescaled accumulator), §4
 *     (bidirectional band |i-j| <= w; causal range [i-w, i]), §5.1-§5.5 (skip
 *     key blocks outside the band, mask the partly covered ones before the
 *     softmax, skipping an all -inf block is exact), §7.1 (the library call
 *     takes causal and a (left, right) window).
 *   - "FlashAttention 深度解析：大模型长序列的算力解放" (ruiowl.com), §二 (tiles of
 *     64-128 tokens staged in on-chip memory), §三 (the result equals standard
 *     attention).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees, retains or synchronises; work is
 *     enqueued on `stream` (a hipStream_t; NULL means the default stream) and
 *     the call returns at once.  Device-side faults surface at the caller's
 *     next synchronisation.
 *   - Tensors are dense and row-major (C order) with the shapes stated below.
 *   - Return value: FA_OK (0) or a negative fa_status.  Arguments are checked
 *     on the host before anything is launched; on error nothing is enqueued.
 *     No function throws across the ABI.
 *   - Grouped-query attention: query head h uses key/value head
 *     h / (H / Hkv); H must be a multiple of Hkv.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                      */
  FA_ERR_SHAPE = -2,       /* sizes are out of range or inconsistent          */
  FA_ERR_UNSUPPORTED = -3, /* valid request this build does not implement     */
  FA_ERR_WORKSPACE = -4,   /* workspace missing or too small                  */
  FA_ERR_LAUNCH = -5       /* the HIP runtime rejected a kernel launch        */
} fa_status;

typedef enum {
  FA_BF16 = 0, /* bfloat16 storage, fp32 accumulation                  */
  FA_F32 = 1   /* float32 storage and arithmetic throughout             */
} fa_dtype;

/*
 * fa_fwd -- attention forward over whole sequences.
 *
 *   q    [B, H,   n, d]  (dtype)
 *   k, v [B, Hkv, n, d]  (dtype)
 *   o    [B, H,   n, d]  (dtype, written)
 *   lse  [B, H,   n]     float32, written: natural-log log-sum-exp of each
 *                        score row over its visible keys, scale included,
 *                        lse_i = ln sum_{j visible} exp(scale * q_i . k_j)
 *
 * For each row i the visible keys j are (window < 0 means no window):
 *   causal = 0, window < 0 : all 0 <= j < n
 *   causal = 1, window < 0 : j <= i
 *   causal = 0, window >= 0: |i - j| <= window   (bidirectional band)
 *   causal = 1, window >= 0: i - window <= j <= i
 * o_i = sum_{j visible} softmax_j(scale * q_i . k_j) v_j.  Every row sees at
 * least key i, so no row is empty.
 *
 * Limits: B, H, Hkv, n >= 1; H % Hkv == 0; d in {64, 128}; n*d < 2^31;
 * B*H < 2^31 and ceil(n/128)*B*H < 2^31 (workgroups); scale finite.  A
 * tensor may hold more than 2^31 elements (offsets are 64-bit).
 * dtype FA_BF16: MFMA path; FA_F32: float32 path.
 * Errors: FA_ERR_NULL (q, k, v, o or lse NULL), FA_ERR_SHAPE,
 * FA_ERR_UNSUPPORTED (d not 64/128 or unknown dtype), FA_ERR_LAUNCH.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Hkv, int n, int d, int causal, int window,
           float scale, int dtype, void* stream);

/*
 * fa_fwd_tile_count -- fa_fwd with dtype FA_BF16 that also counts, on the
 * device, what the block skip leaves to do.  The pages' sliding-window
 * prefill article (xxqk.cn, §9.1 and §9.3) asks to check which key/value
 * blocks the kernel really computes and reads; this entry point reports
 * both.  The outputs o and lse are bit for bit those of fa_fwd.
 *
 *   counters  DEVICE, two uint64 values, ADDED to (the caller zeroes them):
 *             counters[0] += number of (wave, key tile) pairs whose products
 *                            are computed; a wave owns 32 query rows and a
 *                            key tile is 64 keys, so 2048 (query, key) pairs
 *                            each;
 *             counters[1] += number of 64-key K/V tiles staged into on-chip
 *                            memory (one per workgroup and tile visited).
 *
 * The counting adds one atomic per wave and tile: a diagnostic launch, not
 * for timing.  Limits and errors as fa_fwd with dtype FA_BF16, plus
 * FA_ERR_NULL when counters is NULL.
 */
int fa_fwd_tile_count(const void* q, const void* k, const void* v, void* o,
                      float* lse, int B, int H, int Hkv, int n, int d,
                      int causal, int window, float scale,
                      unsigned long long* counters, void* stream);

/*
 * fa_fwd_varlen -- attention forward over a ragged batch (sequences of
 * different lengths packed without padding).
 *
 * In batched prefill the requests differ in length and share one window; each
 * request's traversal is clipped to its own length instead of computing over
 * padding (xxqk.cn sliding-window prefill article §8.1).  Every sequence is an
 * independent fa_fwd problem, positions counted from its first token.
 *
 *   q, o       [H,   total, d]  bf16 (o written): the packed tokens of all
 *   k, v       [Hkv, total, d]  bf16               sequences, per head
 *   lse        [H,   total]     float32, written (as fa_fwd)
 *   cu_seqlens [B + 1] int32, DEVICE: sequence b owns rows
 *              cu_seqlens[b] .. cu_seqlens[b+1]-1; cu_seqlens[0] = 0,
 *              non-decreasing, cu_seqlens[B] = total, every length at most
 *              max_seqlen.  Empty sequences are allowed.
 *
 * causal, window, scale as in fa_fwd.  Device-side guards: offsets are
 * clamped into [0, total] and lengths into [0, max_seqlen]; they only keep
 * memory accesses in bounds.
 * Limits: B, H, Hkv, total, max_seqlen >= 1; H % Hkv == 0; d in {64, 128};
 * dtype FA_BF16; total*d < 2^31 (tensors of H*total*d elements may be
 * larger: offsets are 64-bit); ceil(max_seqlen/128)*B*H < 2^31.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens, int B, int H, int Hkv, int total,
                  int max_seqlen, int d, int causal, int window, float scale,
                  int dtype, void* stream);

/*
 * fa_fwd_paged -- chunked prefill over paged KV histories (prefix reuse).
 *
 * Requests that share or extend a long prefix should not redo its prefill:
 * the cached keys and values are reused (charles2530 blog "算子与编译器：
 * FlashAttention 与长上下文" §7), held in fixed-size pages (§5).  Each
 * sequence brings a chunk of new queries whose keys and values the caller has
 * already written into its pages; the chunk's queries are the LAST positions
 * of the sequence and attend to its cached prefix and to the chunk itself.
 *
 *   q, o          [H, total_q, d] bf16 (o written), packed chunks
 *   lse           [H, total_q] float32, written
 *   kcache,vcache [num_pages, Hkv, page_size, d] bf16 (as fa_decode)
 *   page_table    [B, max_pages] int32 (as fa_decode)
 *   cu_seqlens_q  [B + 1] int32, DEVICE: chunk b owns rows
 *                 cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (as fa_fwd_varlen,
 *                 lengths at most max_seqlen_q)
 *   seqlens_k     [B] int32, DEVICE: keys of sequence b, its chunk included
 *                 (at least the chunk's length, at most max_pages*page_size)
 *
 * Query i of chunk b sits at position seqlens_k[b] - len_b + i; the keys it
 * sees follow causal / window exactly as in fa_fwd at that position.  A
 * one-query chunk is a decode step; a chunk with no prefix is fa_fwd_varlen.
 * Device-side guards: offsets and lengths are clamped as in fa_fwd_varlen,
 * seqlens_k into [0, max_pages*page_size]; a page id outside [0, num_pages)
 * reads page 0; a query that sees no key (chunk longer than its keys) gives
 * o = 0 and lse = -inf.  They only keep memory accesses in bounds.
 * Limits: B, H, Hkv, total_q, max_seqlen_q, num_pages, max_pages >= 1;
 * total_q*d < 2^31; ceil(max_seqlen_q/128)*B*H < 2^31 (workgroups);
 * H % Hkv == 0; d in {64, 128}; page_size == 16; dtype FA_BF16.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH.
 */
int fa_fwd_paged(const void* q, const void* kcache, const void* vcache,
                 const int32_t* page_table, const int32_t* cu_seqlens_q,
                 const int32_t* seqlens_k, void* o, float* lse, int B, int H, int Hkv,
                 int d, int total_q, int max_seqlen_q, int num_pages, int page_size,
                 int max_pages, int causal, int window, float scale, int dtype,
                 void* stream);

/*
 * fa_fwd_blocksparse -- attention forward with a block-sparse layout.
 *
 * Block-sparse FlashAttention ("FlashAttention 深度解析：大模型长序列的算力解放",
 * ruiowl.com, §四) computes only the kept blocks of the score matrix; the
 * sliding-window block skip (xxqk.cn article §5) is the band case.  The
 * score matrix of each head is cut into blocks of block_q query rows by
 * block_k keys; key j is visible to query i when layout[l, i / block_q,
 * j / block_k] != 0 AND causal / window (as in fa_fwd) allow it.  Dropped
 * blocks are never read.  A row with no visible key gets o = 0, lse = -inf.
 *
 *   q, k, v, o, lse  as fa_fwd (dense [B, heads, n, d] layout)
 *   layout  uint8 [layout_heads, ceil(n/block_q), ceil(n/block_k)], DEVICE,
 *           C order; layout_heads = 1 (one layout for every head) or H (one
 *           per query head, l = h); shared by the whole batch.
 *
 * Limits: as fa_fwd, plus block_q == 128, block_k in {64, 128},
 * layout_heads in {1, H}, n <= 131072; dtype FA_BF16.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH.
 */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       const uint8_t* layout, int layout_heads, int B, int H, int Hkv,
                       int n, int d, int block_q, int block_k, int causal, int window,
                       float scale, int dtype, void* stream);

/*
 * fa_fwd_strided -- fa_fwd with caller-given strides (for instance the
 * (batch, seqlen, heads, head_dim) layout of the library call described in
 * the xxqk.cn sliding-window prefill article §7.1, or q/k/v views into one
 * packed qkv tensor).
 *
 *   strides  HOST array of 12 int64, in ELEMENTS:
 *            q (batch, head, row), k (batch, head, row), v (batch, head, row),
 *            o (batch, head, row); element [b][h][i][t] of q is at
 *            q + b*strides[0] + h*strides[1] + i*strides[2] + t.
 *   lse      [B, H, n] float32, contiguous (as fa_fwd).
 * The head dim is contiguous; k and v must share their row stride; every
 * stride is >= 0, a multiple of 8 elements, and row strides are >= d; base
 * pointers are 16-byte aligned.  q, k and v may share memory (packed qkv);
 * o must not overlap them (it is written while other workgroups still read
 * k and v).  Otherwise as fa_fwd (bf16 only).
 * Errors: FA_ERR_NULL (also strides NULL), FA_ERR_SHAPE (also bad strides),
 * FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH.
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int64_t* strides, int B, int H, int Hkv, int n, int d,
                   int causal, int window, float scale, int dtype, void* stream);

/*
 * fa_decode_workspace_bytes -- device workspace fa_decode needs for these
 * sizes (partial outputs and log-sum-exps of every split).  Depends only on
 * the arguments; 0 if they are out of range.
 */
size_t fa_decode_workspace_bytes(int B, int H, int max_seqlen, int d);

/*
 * fa_decode -- one query token per sequence over a paged KV cache (bf16).
 *
 *   q          [B, H, d]                          bf16
 *   kcache     [num_pages, Hkv, page_size, d]     bf16
 *   vcache     [num_pages, Hkv, page_size, d]     bf16
 *   page_table [B, max_pages] int32: physical page of logical page p of
 *              sequence b; token t of sequence b is slot t % page_size of
 *              page page_table[b, t / page_size]
 *   seqlens    [B] int32: cached tokens of each sequence, the new token's own
 *              key/value already appended; 1 <= seqlens[b] <= max_seqlen and
 *              ceil(seqlens[b] / page_size) <= max_pages
 *   o          [B, H, d] bf16, written;  lse [B, H] float32, written
 *   workspace  device memory of at least
 *              fa_decode_workspace_bytes(B, H, max_seqlen, d) bytes; its
 *              contents on entry do not matter and are overwritten.
 *
 * The query attends to every cached token of its sequence (no mask).
 * Device-side guards: a length outside [1, max_seqlen] is clamped into
 * [0, min(max_seqlen, max_pages*page_size)] and a length of 0 gives o = 0 and
 * lse = -inf; a page id outside [0, num_pages) is never dereferenced (its
 * tokens are left out).  Both only keep memory accesses in bounds: the
 * result for such input is not attention over the intended cache.
 *
 * Limits: B, H, Hkv >= 1; H % Hkv == 0; H / Hkv <= 16; d == 64 or 128;
 * page_size == 16; num_pages >= 1; max_pages >= 1; max_seqlen >= 1;
 * B * H, B * max_pages and max_pages * 16 below 2^31.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (sizes), FA_ERR_UNSUPPORTED (d,
 * page_size or H / Hkv), FA_ERR_WORKSPACE, FA_ERR_LAUNCH.
 */
int fa_decode(const void* q, const void* kcache, const void* vcache,
              const int32_t* page_table, const int32_t* seqlens, void* o,
              float* lse, int B, int H, int Hkv, int d, int num_pages,
              int page_size, int max_pages, int max_seqlen, float scale,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): no workspace argument.  The split partials live in a
 * fixed array inside the library, 32 MiB (FA_DECODE_NOALLOC_MAX_BYTES) on
 * each GPU the library runs on, held until the process ends.  The call makes
 * no allocation of any kind.
 *
 *   Arguments, results and limits as fa_decode, without workspace and
 *   workspace_bytes.  The partials must fit:
 *   fa_decode_workspace_bytes(B, H, max_seqlen, d) <= FA_DECODE_NOALLOC_MAX_BYTES
 *   (for instance B = 64, H = 32, max_seqlen = 32768, d = 128 needs 23 MB);
 *   otherwise FA_ERR_WORKSPACE and nothing is enqueued.
 *
 * Every call on one GPU uses that GPU's one array: calls that overlap on the
 * same GPU (several streams, or several host threads, before the earlier
 * call's kernels have finished) race and give wrong results.  Calls in order
 * on one stream are safe; each call overwrites what the previous one left.
 * Errors: as fa_decode; FA_ERR_LAUNCH also when the array's device address
 * cannot be obtained.
 */
#define FA_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                      const int32_t* page_table, const int32_t* seqlens, void* o,
                      float* lse, int B, int H, int Hkv, int d, int num_pages,
                      int page_size, int max_pages, int max_seqlen, float scale,
                      void* stream);

/*
 * fa_bwd_workspace_bytes -- device workspace fa_bwd needs for these sizes
 * (one float per query row: D_i = <dO_i, O_i>).  0 if out of range.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int n, int d);

/*
 * fa_bwd -- gradients of attention over whole sequences (the backward pass).
 *
 * The score and probability matrices are not read from anywhere: they are
 * recomputed tile by tile from q, k and the forward pass's lse (xxqk.cn
 * sliding-window prefill article §3.3; bomianfm.com Q&A "FlashAttention的原理是
 * 什么？对Agent性能有何提升？" §一), and key tiles outside the band are skipped
 * as in fa_fwd.  With P_ij = exp(scale q_i.k_j - lse_i) on the visible pairs
 * (0 elsewhere) and D_i = <dO_i, O_i>:
 *   dv = P^T dO,  dS = P o (dO v^T - D),  dq = scale dS k,  dk = scale dS^T q,
 * dk and dv summed over the query heads that share a key/value head.
 *
 *   q, o, dout [B, H,   n, d]  bf16   (o and lse exactly as fa_fwd wrote them
 *   k, v       [B, Hkv, n, d]  bf16    for the same q, k, v and mask)
 *   lse        [B, H,   n]     float32 (natural log, as written by fa_fwd)
 *   dq         [B, H,   n, d]  float32, written
 *   dk, dv     [B, Hkv, n, d]  float32, written (not accumulated into)
 *   workspace  device memory of at least fa_bwd_workspace_bytes(B, H, n, d)
 *              bytes; contents on entry do not matter.
 *
 * causal and window select the visible keys exactly as in fa_fwd.  The
 * result is deterministic (no atomics; fixed summation order).
 * Limits: as fa_fwd; dtype must be FA_BF16.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (d not 64/128 or
 * dtype not FA_BF16), FA_ERR_WORKSPACE, FA_ERR_LAUNCH.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, float* dq, float* dk, float* dv,
           int B, int H, int Hkv, int n, int d, int causal, int window,
           float scale, int dtype, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * fa_decode_fp8 -- fa_decode over an FP8 key/value cache (quantised KV,
 * charles2530 blog "算子与编译器：FlashAttention 与长上下文" §9).
 *
 *   kcache, vcache  [num_pages, Hkv, page_size, d] uint8: OCP E4M3 bytes
 *                   (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 *                   infinities; S.1111.111 is NaN)
 *   k_scale, v_scale [Hkv] float32, DEVICE: per key/value head
 *                   dequantisation scales, k = byte * k_scale[g],
 *                   v = byte * v_scale[g]; any finite value, zero included
 *                   (a head quantised from an all-zero cache: its scores are
 *                   all 0 and its softmax uniform) and negative values; a
 *                   non-finite scale gives a non-finite result for its head
 *   everything else as fa_decode (q bf16, page_table, seqlens, o bf16, lse,
 *   workspace of fa_decode_workspace_bytes(B, H, max_seqlen, d) bytes).
 *
 * The result is decode attention over the dequantised keys and values; half
 * the bytes of the bf16 cache are read.  Limits and errors as fa_decode, plus
 * FA_ERR_NULL when k_scale or v_scale is NULL.
 */
int fa_decode_fp8(const void* q, const void* kcache, const void* vcache,
                  const float* k_scale, const float* v_scale,
                  const int32_t* page_table, const int32_t* seqlens, void* o,
                  float* lse, int B, int H, int Hkv, int d, int num_pages,
                  int page_size, int max_pages, int max_seqlen, float scale,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text of a status code (static storage, never NULL). */
const char* fa_strerror(int status);

/* ABI version of this library: (major << 16) | minor. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

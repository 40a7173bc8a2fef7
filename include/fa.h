/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa.so): the
 * forward pass (fused and unfused; bf16, fp32, and FP8 Q/K), the backward pass of
 * the fused forward, and decode attention over a paged key/value cache.
 *
 * The operation.  For every batch item b, head h and query row i:
 *
 *   o[b,h,i,:] = sum_j softmax_j( scale * <q[b,h,i,:], k[b,h,j,:]> + M[b,i,j] ) * v[b,h,j,:]
 *   lse[b,h,i] = log sum_j exp( scale * <q[b,h,i,:], k[b,h,j,:]> + M[b,i,j] )   (natural log)
 *
 * with M = 0 where key j is valid for row i and -inf elsewhere; key j is valid
 * when (kv_limit == NULL or j < kv_limit[b*N + i]) and (causal == 0 or j <= i).
 * A row with no valid key gets o = 0 and lse = -inf.
 *
 *   - O = softmax(Q K^T / sqrt(d)) V, computed exactly: "FlashAttention 1–4: How
 *     IO-Awareness Reshaped the Attention Kernel", section "Why attention is
 *     memory-bound, not compute-bound", and its closing section on what all four
 *     versions share.
 *   - The additive mask M (-inf at future positions for causal attention) and the
 *     [b, h, seq, d] layout: "谁偷走了 5090 的算力和显存", attention section.
 *   - The per-row log-sum-exp L = m + log(l) kept for the backward pass:
 *     "FlashAttention 1–4 ...", section "FlashAttention-2"; "GPU 与 TPU：让硬件不再是
 *     黑魔法" §11.4.
 *   - The fully masked row: "07 GPU、资源估算与 FlashAttention" §7.8 asks only that
 *     -inf minus -inf never be computed; o = 0, lse = -inf is this library's reading
 *     (the log of an empty sum).
 *
 * Layout.  q, k, v, o: contiguous [B, H, N, d] row-major, d fastest.  lse:
 * contiguous [B, H, N] fp32.  kv_limit: NULL or contiguous [B, N] int32, values
 * clamped to [0, N] (negative counts as 0).  Causal masking is top-left aligned
 * with the diagonal included (query i sees keys 0..i).
 *
 * Supported shapes.  d in {64, 128}; B, H, N >= 1; one head of one tensor below
 * 4 GiB (N*d*2 bytes in bf16, N*d*4 in fp32); and B*H*ceil(N/32) < 2^23 row tiles
 * of 32, i.e. B*H*N < 2^28 rows when N is a multiple of 32 (68 GB per bf16
 * tensor at d = 128).  Offsets are 64-bit, so a tensor may exceed 2^31 elements.
 * The unfused path also needs B*H <= 65535 and N <= 32768.  scale may be any finite
 * value: the statement of the problem takes it as a parameter of
 * softmax(scale * Q K^T + M) V ("谁偷走了 5090 的算力和显存", attention section); the
 * pages' workloads use 1/sqrt(d).  scale = 0 gives the mean of the valid values and
 * lse = ln(number of valid keys); a negative scale weights the smallest scores most.
 *
 * Memory and ownership.  Every pointer is device memory owned by the caller.  The
 * library allocates nothing, keeps no pointer after a call returns and has no
 * mutable global state; calls are thread-safe.  o and lse must not overlap any
 * input or each other.  q, k, v, o must be 16-byte aligned; lse and kv_limit 4-byte
 * aligned.
 *
 * Streams and errors.  `stream` is a hipStream_t (NULL = the default stream).
 * Every call validates its arguments on the host before touching the device; an
 * invalid call returns an error code and launches nothing.  A valid call enqueues
 * its kernels on `stream` and returns without synchronising: a fault inside a
 * kernel surfaces at the caller's next synchronisation.  FA_ERR_HIP means a launch
 * was rejected by the HIP runtime.  No C++ exception crosses this boundary.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t fa_bf16; /* raw bf16 bits (the upper half of an IEEE fp32) */

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL                              */
    FA_ERR_SHAPE = 2,     /* B, H or N < 1, or sizes beyond the supported shapes     */
    FA_ERR_HEAD_DIM = 3,  /* d is not 64 or 128                                      */
    FA_ERR_SCALE = 4,     /* scale is NaN or infinite                                */
    FA_ERR_ALIGN = 5,     /* q, k, v, o not 16-byte aligned, or lse / kv_limit not 4-byte aligned */
    FA_ERR_WORKSPACE = 6, /* unfused, backward or decode path: workspace NULL, too small or misaligned */
    FA_ERR_HIP = 7,       /* the HIP runtime rejected a kernel launch or a lookup    */
    FA_ERR_ALIAS = 8,     /* an output overlaps an input, the other output or the workspace */
    FA_ERR_SCRATCH = 9    /* fa_decode_paged_bf16_noalloc: the call needs more than
                             FA_DECODE_SCRATCH_BYTES of scratch */
} fa_status;

/*
 * Fused forward, bf16 inputs and output, fp32 accumulation and statistics.
 * One kernel: Q tile in registers, K/V tiles streamed through LDS, both
 * contractions on bf16 matrix cores, online softmax (an exponent reference per
 * row, running sum, unnormalised accumulator, one normalisation at the end);
 * the N x N score matrix never reaches device memory ("GPU 与 TPU：让硬件不再是
 * 黑魔法" §11.2-§11.4; "FlashAttention 1–4 ...", sections "FlashAttention (v1)"
 * and "FlashAttention-2").  Since O / l does not depend on the reference
 * ("FlashAttention 1–4 ...", section "FlashAttention-4"), without kv_limit each
 * row keeps its first K/V tile's max as the reference; a block whose sum or
 * output then overflows is computed again with the reference following the
 * running max, which kv_limit calls use throughout.  The probabilities feeding
 * P V are rounded to bf16 (nearest-even) and the row sum l is taken over the
 * same rounded values.
 */
fa_status fa_fwd_bf16(const fa_bf16 *q, const fa_bf16 *k, const fa_bf16 *v,
                      fa_bf16 *o, float *lse,
                      int B, int H, int N, int d, int causal, float scale,
                      const int32_t *kv_limit, void *stream);

/*
 * Fused forward, fp32 inputs and output.  Same algorithm as fa_fwd_bf16 with the
 * contractions on fp32 matrix cores and P kept in fp32.
 */
fa_status fa_fwd_f32(const float *q, const float *k, const float *v,
                     float *o, float *lse,
                     int B, int H, int N, int d, int causal, float scale,
                     const int32_t *kv_limit, void *stream);

/*
 * Bytes of workspace the unfused path needs: S in fp32 plus P in the input
 * precision (elem_bytes = 2 for bf16, 4 for fp32), each B*H*N rows of
 * ld = (N rounded up to 64) elements, each part rounded up to 256 bytes.
 * Returns 0 if the size would overflow size_t or an argument is out of range.
 */
size_t fa_unfused_workspace_bytes(int B, int H, int N, int elem_bytes);

/*
 * Unfused three-kernel forward, the standard attention the fused kernel replaces
 * ("FlashAttention 1–4 ...", section "FlashAttention (v1)", the two-panel figure
 * of standard attention: one kernel per step, S and P making a round trip
 * through device memory):
 *   kernel 1 writes S = scale * Q K^T (fp32) for every (query, key) pair;
 *   kernel 2 reads S, applies the mask, runs a safe softmax one row per
 *            workgroup and writes P (bf16, rounded to nearest-even) and lse;
 *   kernel 3 reads P and V and writes O = P V.
 * Same arguments and results as fa_fwd_bf16, plus a caller-owned device
 * workspace of at least fa_unfused_workspace_bytes(B, H, N, 2) bytes, 256-byte
 * aligned, not overlapping any input or output.
 */
fa_status fa_fwd_unfused_bf16(const fa_bf16 *q, const fa_bf16 *k, const fa_bf16 *v,
                              fa_bf16 *o, float *lse,
                              int B, int H, int N, int d, int causal, float scale,
                              const int32_t *kv_limit,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Unfused three-kernel forward in fp32 (P stored in fp32); workspace of at least
 * fa_unfused_workspace_bytes(B, H, N, 4) bytes. */
fa_status fa_fwd_unfused_f32(const float *q, const float *k, const float *v,
                             float *o, float *lse,
                             int B, int H, int N, int d, int causal, float scale,
                             const int32_t *kv_limit,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace the backward pass needs: two fp32 statistics per row
 * (D_i = <dO_i, O_i> and the log-sum-exp in base 2), each B*H*N values rounded up
 * to a multiple of 64.  Returns 0 if an argument is out of range.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * Backward pass of fa_fwd_bf16: given q, k, v, the forward's o and lse, and the
 * gradient dout of a loss with respect to o, writes the gradients dq, dk, dv of
 * that loss (bf16, same layout as q).  Mathematically, with P the attention
 * probabilities of the forward (0 on masked keys and for rows with no valid key):
 *
 *   dv_j = sum_i P_ij dout_i,   dP_ij = <dout_i, v_j>,   D_i = <dout_i, o_i>,
 *   dS_ij = P_ij (dP_ij - D_i),  dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i.
 *
 * P is recomputed tile by tile as exp(S - lse) from the saved statistic, with no
 * online softmax ("GPU 与 TPU：让硬件不再是黑魔法" §11.5, part 3; "FlashAttention
 * 1–4 ...", section "FlashAttention-2": one column block of K/V per thread block,
 * dK and dV accumulated locally).  dq has a pass of its own instead of atomic
 * adds, so results are deterministic.  P and dS are rounded to bf16 (nearest-even)
 * before their contractions; accumulation is fp32.
 *
 * Arguments as for fa_fwd_bf16 (same causal, scale and kv_limit as the forward
 * call that produced o and lse), plus: dout [B, H, N, d] bf16; dq, dk, dv
 * [B, H, N, d] bf16 outputs, 16-byte aligned, overlapping no input, no other
 * output and not the workspace; workspace at least fa_bwd_workspace_bytes(B, H, N)
 * bytes of device memory owned by the caller, 256-byte aligned, overwritten.
 * Errors as for the forward; FA_ERR_WORKSPACE for a missing, small or misaligned
 * workspace.
 */
fa_status fa_bwd_bf16(const fa_bf16 *q, const fa_bf16 *k, const fa_bf16 *v,
                      const fa_bf16 *o, const fa_bf16 *dout, const float *lse,
                      fa_bf16 *dq, fa_bf16 *dk, fa_bf16 *dv,
                      int B, int H, int N, int d, int causal, float scale,
                      const int32_t *kv_limit,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace fa_decode_paged_bf16 needs: per sequence, head and 256-key
 * split an unnormalised fp32 output row (d values) and its (max, sum) pair, with
 * max_pages * 16 / 256 splits (rounded up) per sequence.  Returns 0 if an argument
 * is out of range.
 */
size_t fa_decode_workspace_bytes(int B, int H, int d, int max_pages);

/*
 * Decode attention over a paged key/value cache: one query per sequence (the
 * token being generated) attends to every cached key of its sequence.
 *
 *   key j of sequence b, head h (0 <= j < seq_lens[b]) is
 *     k_cache[page, h, j % 16, :] with page = block_table[b * max_pages + j / 16],
 *   o[b,h,:]  = sum_j softmax_j( scale * <q[b,h,:], key j> ) * value j
 *   lse[b,h]  = log sum_j exp( scale * <q[b,h,:], key j> )   (natural log)
 *
 * and a sequence with no key gets o = 0 and lse = -inf.  The cache is cut into
 * pages of 16 tokens, and the block table maps a sequence's logical pages to
 * physical pages anywhere in the pool ("CS336 第五讲 · GPU 与 GPU 优化", the
 * PagedAttention section).  The key range of each sequence is split into pieces
 * of 256 keys processed in parallel and merged with the online-softmax rescaling
 * ("FlashAttention 1–4 ...", sections "FlashAttention (v1)" and
 * "FlashAttention-2").
 *
 * Layout.  q, o: contiguous [B, H, d] bf16.  k_cache, v_cache: contiguous
 * [num_pages, H, 16, d] bf16 (one page of one head is 16 * d contiguous values).
 * block_table: contiguous [B, max_pages] int32.  seq_lens: [B] int32.  lse:
 * [B, H] fp32.  page_size must be 16; d in {64, 128}; B, H in [1, 65535] with
 * B*H < 2^24; max_pages in [1, 1048560] (at most 65535 splits of 256 keys);
 * num_pages >= 1.
 *
 * Contents.  Lengths are clamped to [0, max_pages * 16].  Block-table entries of
 * pages past a sequence's length are never read; an entry inside the length that
 * lies outside [0, num_pages) is not dereferenced, and its 16 keys and values read
 * as zeros.  Cache slots past a sequence's length in its last page may hold
 * anything.
 *
 * Memory: every pointer is caller-owned device memory; q, k_cache, v_cache, o
 * 16-byte aligned, block_table, seq_lens, lse 4-byte aligned; workspace at least
 * fa_decode_workspace_bytes(B, H, d, max_pages) bytes, 256-byte aligned,
 * overwritten.  o, lse and the workspace must not overlap an input or each other.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (B, H, max_pages, num_pages or page_size out of
 * range), FA_ERR_HEAD_DIM, FA_ERR_SCALE, FA_ERR_ALIGN, FA_ERR_WORKSPACE,
 * FA_ERR_ALIAS, FA_ERR_HIP, as for the forward.
 */
fa_status fa_decode_paged_bf16(const fa_bf16 *q, const fa_bf16 *k_cache, const fa_bf16 *v_cache,
                               const int32_t *block_table, const int32_t *seq_lens,
                               fa_bf16 *o, float *lse,
                               int B, int H, int d, int page_size, int max_pages, int num_pages,
                               float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of the static device buffer fa_decode_paged_bf16_noalloc uses in place of
 * a workspace, on each GPU the library runs on.
 */
#define FA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * fa_decode_paged_bf16 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result and errors as fa_decode_paged_bf16 without the workspace, and
 * the same kernels: the splits' partials go to a buffer of FA_DECODE_SCRATCH_BYTES
 * that the library holds in static device memory, one copy per GPU, until the
 * process ends.  The call allocates nothing.
 *
 * Limit: fa_decode_workspace_bytes(B, H, d, max_pages) <= FA_DECODE_SCRATCH_BYTES,
 * else FA_ERR_SCRATCH (checked on the host before anything is launched).  With
 * n = B * H * ceil(max_pages / 16) splits (d floats and a (max, sum) pair each)
 * that is n <= 32263 for d = 128 and n <= 63550 for d = 64; B = 64, H = 32,
 * max_pages = 128, d = 128 (n = 16384) fits.
 *
 * Every call on one GPU shares that GPU's buffer, and the buffer keeps the last
 * call's contents; nothing in it has to start at zero, since a call reads only
 * what its own first kernel wrote.  Calls on one stream are ordered; calls that
 * may overlap on one GPU (different streams, or host threads without ordering)
 * race on the buffer and must not be made.  The first call on a device looks up
 * the buffer's device address there (FA_ERR_HIP if that fails); a caller that
 * captures the call into a HIP graph makes one call outside the capture first.
 */
fa_status fa_decode_paged_bf16_noalloc(const fa_bf16 *q, const fa_bf16 *k_cache, const fa_bf16 *v_cache,
                                       const int32_t *block_table, const int32_t *seq_lens,
                                       fa_bf16 *o, float *lse,
                                       int B, int H, int d, int page_size, int max_pages, int num_pages,
                                       float scale, void *stream);

/*
 * FP8 forward, step 1: rotate and encode one of Q or K.  Every row x (length d)
 * of the bf16 tensor becomes y = H (signs * x), with H the unnormalised
 * Sylvester-Hadamard matrix (entries +-1, so H H^T = d I) applied as the
 * butterfly in fp32 (stages h = 1, 2, ..., d/2; (a, b) -> (a + b, a - b)); per
 * tile of tile_rows consecutive rows of one head, e = the smallest integer with
 * max |y| <= 448 * 2^e (clamped to [-127, 127]; 0 for an all-zero tile) and the
 * codes are E4M3(y * 2^-e), OCP FP8 with 4 exponent bits (bias 7) and 3 mantissa
 * bits, rounded to nearest even.  This is FlashAttention-3's FP8 recipe: one
 * scale per tile and incoherent processing by random signs plus a Hadamard
 * transform ("FlashAttention 1–4 ...", section "FlashAttention-3"); the scales
 * are powers of two so that encoding is exact up to the E4M3 rounding.
 *
 * x [B, H, N, d] bf16, 16-byte aligned; signs [d] int8, each +1 or -1 (the
 * same vector for Q and K); codes [B, H, N, d] uint8 output, 16-byte aligned;
 * exps [B, H, ceil(N / tile_rows)] int32 output, 4-byte aligned.  tile_rows is
 * 32 for Q and 64 for K (the tiles fa_fwd_fp8 reads); d in {64, 128}.  Inputs
 * must be finite with d * max |x| below the fp32 range.  Outputs must not
 * overlap the inputs or each other.  Errors as for the forward.
 */
fa_status fa_fp8_quantize_bf16(const fa_bf16 *x, const int8_t *signs, uint8_t *codes, int32_t *exps,
                               int B, int H, int N, int d, int tile_rows, void *stream);

/*
 * FP8 forward, step 2: attention with Q and K given as E4M3 codes from
 * fa_fp8_quantize_bf16 (q with tile_rows 32, k with tile_rows 64, both with the
 * same signs) and V in bf16:
 *
 *   s_ij = (scale / d) * sum_c deq(q_i)_c deq(k_j)_c,   deq = E4M3 value * 2^e of the row's tile,
 *
 * then o and lse exactly as fa_fwd_bf16 (masks, layouts, empty rows).  Since
 * (H s q).(H s k) = d q.k, this is attention of the original q and k up to the
 * E4M3 rounding of the rotated rows.  The products run on gfx950's FP8 matrix
 * instructions with the tiles' exponents as block scales; P is rounded to bf16
 * for P V as in the bf16 kernel.  q_codes, k_codes, v, o 16-byte aligned;
 * q_exps, k_exps, lse, kv_limit 4-byte aligned; o and lse must not overlap an
 * input or each other.  Errors as for the forward.
 */
fa_status fa_fwd_fp8(const uint8_t *q_codes, const int32_t *q_exps, const uint8_t *k_codes, const int32_t *k_exps,
                     const fa_bf16 *v, fa_bf16 *o, float *lse, int B, int H, int N, int d, int causal, float scale,
                     const int32_t *kv_limit, void *stream);

/*
 * FP8 forward in one call for Q: the same result as fa_fp8_quantize_bf16 on q
 * (tile_rows 32) followed by fa_fwd_fp8, bit for bit, but q is given in bf16
 * with the rotation's signs, and each group of 32 query rows is rotated and
 * encoded inside the attention kernel, so Q's codes never reach device memory
 * (one launch and one pass over Q fewer).  K still comes as codes and
 * exponents from fa_fp8_quantize_bf16 with tile_rows 64 and the same signs.
 * q [B, H, N, d] bf16, 16-byte aligned; signs [d] int8 (+1 or -1), 16-byte
 * aligned; the other arguments as for fa_fwd_fp8.  Errors as for fa_fwd_fp8.
 */
fa_status fa_fwd_fp8_qbf16(const fa_bf16 *q, const int8_t *signs, const uint8_t *k_codes, const int32_t *k_exps,
                           const fa_bf16 *v, fa_bf16 *o, float *lse, int B, int H, int N, int d, int causal,
                           float scale, const int32_t *kv_limit, void *stream);

/* Static, human-readable name of a status code. */
const char *fa_status_str(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

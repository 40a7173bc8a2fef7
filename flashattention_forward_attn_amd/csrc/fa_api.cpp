// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation on the
// host, then dispatch to the HIP launchers.  No allocation, no synchronisation,
// no exception crosses the boundary; the only global state is the decode path's
// static scratch buffer and its per-device address.
#include "fa.h"

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fa_launch.h"

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

constexpr size_t kWsAlign = 256;
static_assert((int64_t)FA_DECODE_SCRATCH_BYTES == fa::kDecodeScratchBytes, "one scratch size");
constexpr int kUnfusedMaxN = 32768;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Size limits of the [B, H, N, d] paths.  Tensors are addressed with 64-bit
// offsets; two quantities stay 32-bit.  A buffer descriptor spans one head, so
// N * d * elem must fit in 32 bits.  A grid dimension holds at most 2^32 - 1
// work-items, and no launch uses more than 512 threads per 32 rows of a head
// (the row-statistics kernel runs 16 threads per row; the others fewer), so
// B * H * ceil(N / 32) * 512 must fit in 32 bits: at most 2^23 - 1 row tiles,
// e.g. B * H * N < 2^28 when N is a multiple of 32.
constexpr int64_t kMaxThreadsPerTile = 512;

bool shape_ok(int B, int H, int N, int d, int elem) {
    if (B < 1 || H < 1 || N < 1) return false;
    const int64_t tiles = (int64_t)B * H * ((N + 31) / 32);
    if (tiles * kMaxThreadsPerTile > (int64_t)UINT32_MAX) return false;
    return (int64_t)N * d * elem <= (int64_t)UINT32_MAX;
}

// Common checks for every entry point.  elem = bytes per q/k/v/o element.
fa_status validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                   int N, int d, float scale, const int32_t* kv_limit, int elem) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (!shape_ok(B, H, N, d, elem)) return FA_ERR_SHAPE;
    const int64_t elems = (int64_t)B * H * N * d;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        (kv_limit && !aligned(kv_limit, 4)))
        return FA_ERR_ALIGN;
    const int64_t tbytes = elems * elem;
    const Range rq = span(q, tbytes), rk = span(k, tbytes), rv = span(v, tbytes), ro = span(o, tbytes);
    const Range rl = span(lse, (int64_t)B * H * N * 4);
    const Range rm = span(kv_limit, kv_limit ? (int64_t)B * N * 4 : 0);
    for (Range in : {rq, rk, rv, rm}) {
        if (overlap(ro, in) || overlap(rl, in)) return FA_ERR_ALIAS;
    }
    if (overlap(ro, rl)) return FA_ERR_ALIAS;
    return FA_OK;
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

size_t workspace_bytes(int B, int H, int N, int elem) {
    if (B < 1 || H < 1 || N < 1 || (elem != 2 && elem != 4)) return 0;
    typedef unsigned __int128 u128;
    const u128 rows = (u128)B * (u128)H * (u128)N * (u128)fa::unfused_ld(N);
    const u128 total = ((rows * 4 + kWsAlign - 1) / kWsAlign) * kWsAlign +
                       ((rows * (u128)elem + kWsAlign - 1) / kWsAlign) * kWsAlign;
    if (total > (u128)SIZE_MAX) return 0;
    return (size_t)total;
}

fa_status unfused(bool bf16_path, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, int d, int causal, float scale, const int32_t* kv_limit, void* workspace,
                  size_t workspace_bytes_given, void* stream) {
    const int elem = bf16_path ? 2 : 4;
    fa_status st = validate(q, k, v, o, lse, B, H, N, d, scale, kv_limit, elem);
    if (st != FA_OK) return st;
    if ((int64_t)B * H > 65535) return FA_ERR_SHAPE;  // grid y/z limit of the unfused kernels
    if (N > kUnfusedMaxN) return FA_ERR_SHAPE;         // 32-bit offsets into one head's P
    // the softmax launch runs 64, 256 or 512 threads per row (up to 4096, up to
    // 16384, more keys per row); a grid holds fewer than 2^32 work-items
    const int64_t ld = fa::unfused_ld(N), per_row = ld <= 4096 ? 64 : (ld <= 16384 ? 256 : 512);
    if ((int64_t)B * H * N * per_row > (int64_t)UINT32_MAX) return FA_ERR_SHAPE;
    const size_t need = workspace_bytes(B, H, N, elem);
    if (!workspace || need == 0 || workspace_bytes_given < need || !aligned(workspace, kWsAlign))
        return FA_ERR_WORKSPACE;
    const Range rw = span(workspace, (int64_t)need);
    const int64_t tbytes = (int64_t)B * H * N * d * elem;
    for (Range r : {span(q, tbytes), span(k, tbytes), span(v, tbytes), span(o, tbytes),
                    span(lse, (int64_t)B * H * N * 4), span(kv_limit, kv_limit ? (int64_t)B * N * 4 : 0)}) {
        if (overlap(rw, r)) return FA_ERR_ALIAS;
    }
    const size_t rows = (size_t)B * H * N * (size_t)ld;
    float* S = static_cast<float*>(workspace);
    void* P = static_cast<char*>(workspace) + round_up(rows * 4, kWsAlign);
    return hip_status(fa::launch_unfused(bf16_path, q, k, v, o, lse, B, H, N, d, causal != 0, scale, kv_limit, S, P,
                                         static_cast<hipStream_t>(stream)));
}

size_t bwd_workspace_bytes(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1) return 0;
    return (size_t)(2 * fa::bwd_stats_floats(B, H, N) * 4);
}

size_t decode_workspace_bytes(int B, int H, int d, int max_pages) {
    if (B < 1 || H < 1 || max_pages < 1 || (d != 64 && d != 128)) return 0;
    return (size_t)fa::decode_workspace_floats(B, H, d, max_pages) * 4;
}

// Checks shared by the decode entry points, in order: pointers, sizes, head
// dimension, scale, alignment.
fa_status decode_args(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, const void* o, const float* lse, int B, int H, int d, int page_size,
                      int max_pages, int num_pages, float scale) {
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || B > 65535 || H > 65535 || max_pages < 1 || num_pages < 1 || page_size != fa::kDecodePage ||
        fa::decode_max_splits(max_pages) > 65535 ||
        (int64_t)B * H * 256 > (int64_t)UINT32_MAX)  // 256 threads per (sequence, head) in each launch
        return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    return FA_OK;
}

// o, lse and the workspace (if any) overlap no input and no other output.
fa_status decode_alias(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                       const int32_t* seq_lens, const void* o, const float* lse, int B, int H, int d, int max_pages,
                       int num_pages, const void* workspace, size_t workspace_bytes) {
    const int64_t row_bytes = (int64_t)B * H * d * 2;
    const int64_t cache_bytes = (int64_t)num_pages * H * fa::kDecodePage * d * 2;
    const Range ins[] = {span(q, row_bytes), span(k_cache, cache_bytes), span(v_cache, cache_bytes),
                         span(block_table, (int64_t)B * max_pages * 4), span(seq_lens, (int64_t)B * 4)};
    const Range outs[] = {span(o, row_bytes), span(lse, (int64_t)B * H * 4),
                          span(workspace, workspace ? (int64_t)workspace_bytes : 0)};
    for (int i = 0; i < 3; ++i) {
        for (Range in : ins)
            if (overlap(outs[i], in)) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
    }
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd_bf16(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse, int B, int H,
                      int N, int d, int causal, float scale, const int32_t* kv_limit, void* stream) {
    fa_status st = validate(q, k, v, o, lse, B, H, N, d, scale, kv_limit, 2);
    if (st != FA_OK) return st;
    return hip_status(fa::launch_fused_bf16(q, k, v, o, lse, B, H, N, d, causal != 0, scale, kv_limit,
                                            static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                     int d, int causal, float scale, const int32_t* kv_limit, void* stream) {
    fa_status st = validate(q, k, v, o, lse, B, H, N, d, scale, kv_limit, 4);
    if (st != FA_OK) return st;
    return hip_status(fa::launch_fused_f32(q, k, v, o, lse, B, H, N, d, causal != 0, scale, kv_limit,
                                           static_cast<hipStream_t>(stream)));
}

size_t fa_unfused_workspace_bytes(int B, int H, int N, int elem_bytes) {
    return workspace_bytes(B, H, N, elem_bytes);
}

fa_status fa_fwd_unfused_bf16(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                              int B, int H, int N, int d, int causal, float scale, const int32_t* kv_limit,
                              void* workspace, size_t workspace_bytes_given, void* stream) {
    return unfused(true, q, k, v, o, lse, B, H, N, d, causal, scale, kv_limit, workspace, workspace_bytes_given,
                   stream);
}

fa_status fa_fwd_unfused_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                             int N, int d, int causal, float scale, const int32_t* kv_limit, void* workspace,
                             size_t workspace_bytes_given, void* stream) {
    return unfused(false, q, k, v, o, lse, B, H, N, d, causal, scale, kv_limit, workspace, workspace_bytes_given,
                   stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) { return bwd_workspace_bytes(B, H, N); }

fa_status fa_bwd_bf16(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o, const fa_bf16* dout,
                      const float* lse, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv, int B, int H, int N, int d, int causal,
                      float scale, const int32_t* kv_limit, void* workspace, size_t workspace_bytes_given,
                      void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (!shape_ok(B, H, N, d, 2)) return FA_ERR_SHAPE;
    const int64_t elems = (int64_t)B * H * N * d;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)o, (const void*)dout,
                          (const void*)dq, (const void*)dk, (const void*)dv})
        if (!aligned(p, 16)) return FA_ERR_ALIGN;
    if (!aligned(lse, 4) || (kv_limit && !aligned(kv_limit, 4))) return FA_ERR_ALIGN;
    const size_t need = bwd_workspace_bytes(B, H, N);
    if (!workspace || workspace_bytes_given < need || !aligned(workspace, kWsAlign)) return FA_ERR_WORKSPACE;
    const int64_t tbytes = elems * 2;
    const Range ins[] = {span(q, tbytes), span(k, tbytes), span(v, tbytes), span(o, tbytes), span(dout, tbytes),
                         span(lse, (int64_t)B * H * N * 4), span(kv_limit, kv_limit ? (int64_t)B * N * 4 : 0)};
    const Range outs[] = {span(dq, tbytes), span(dk, tbytes), span(dv, tbytes), span(workspace, (int64_t)need)};
    for (int i = 0; i < 4; ++i) {
        for (Range in : ins)
            if (overlap(outs[i], in)) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
    }
    return hip_status(fa::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal != 0, scale,
                                          kv_limit, static_cast<float*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int max_pages) {
    return decode_workspace_bytes(B, H, d, max_pages);
}

fa_status fa_decode_paged_bf16(const fa_bf16* q, const fa_bf16* k_cache, const fa_bf16* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens, fa_bf16* o, float* lse, int B,
                               int H, int d, int page_size, int max_pages, int num_pages, float scale,
                               void* workspace, size_t workspace_bytes_given, void* stream) {
    fa_status st = decode_args(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H, d, page_size, max_pages,
                               num_pages, scale);
    if (st != FA_OK) return st;
    const size_t need = decode_workspace_bytes(B, H, d, max_pages);
    if (!workspace || workspace_bytes_given < need || !aligned(workspace, kWsAlign)) return FA_ERR_WORKSPACE;
    st = decode_alias(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H, d, max_pages, num_pages, workspace,
                      need);
    if (st != FA_OK) return st;
    return hip_status(fa::launch_decode_bf16(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H, d, max_pages,
                                             num_pages, scale, static_cast<float*>(workspace),
                                             static_cast<hipStream_t>(stream)));
}

fa_status fa_decode_paged_bf16_noalloc(const fa_bf16* q, const fa_bf16* k_cache, const fa_bf16* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens, fa_bf16* o, float* lse,
                                       int B, int H, int d, int page_size, int max_pages, int num_pages,
                                       float scale, void* stream) {
    fa_status st = decode_args(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H, d, page_size, max_pages,
                               num_pages, scale);
    if (st != FA_OK) return st;
    if ((int64_t)decode_workspace_bytes(B, H, d, max_pages) > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
    // the static buffer is the library's own: it cannot overlap the caller's memory
    st = decode_alias(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H, d, max_pages, num_pages, nullptr, 0);
    if (st != FA_OK) return st;
    float* scratch = nullptr;
    const hipError_t e = fa::decode_scratch(&scratch);
    if (e != hipSuccess) return FA_ERR_HIP;
    return hip_status(fa::launch_decode_bf16(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H, d, max_pages,
                                             num_pages, scale, scratch, static_cast<hipStream_t>(stream)));
}

fa_status fa_fp8_quantize_bf16(const fa_bf16* x, const int8_t* signs, uint8_t* codes, int32_t* exps, int B, int H,
                               int N, int d, int tile_rows, void* stream) {
    if (!x || !signs || !codes || !exps) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || (tile_rows != fa::kFp8QTile && tile_rows != fa::kFp8KTile)) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (!shape_ok(B, H, N, d, 2)) return FA_ERR_SHAPE;
    const int64_t elems = (int64_t)B * H * N * d;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(exps, 4)) return FA_ERR_ALIGN;
    const int64_t ntile = (int64_t)B * H * ((N + tile_rows - 1) / tile_rows);
    const Range ins[] = {span(x, elems * 2), span(signs, d)};
    const Range outs[] = {span(codes, elems), span(exps, ntile * 4)};
    for (Range out : outs)
        for (Range in : ins)
            if (overlap(out, in)) return FA_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return FA_ERR_ALIAS;
    return hip_status(fa::launch_fp8_quantize(x, signs, codes, exps, B, H, N, d, tile_rows,
                                              static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_fp8(const uint8_t* q_codes, const int32_t* q_exps, const uint8_t* k_codes, const int32_t* k_exps,
                     const fa_bf16* v, fa_bf16* o, float* lse, int B, int H, int N, int d, int causal, float scale,
                     const int32_t* kv_limit, void* stream) {
    if (!q_codes || !q_exps || !k_codes || !k_exps || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (!shape_ok(B, H, N, d, 2)) return FA_ERR_SHAPE;
    const int64_t elems = (int64_t)B * H * N * d;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(q_exps, 4) ||
        !aligned(k_exps, 4) || !aligned(lse, 4) || (kv_limit && !aligned(kv_limit, 4)))
        return FA_ERR_ALIGN;
    const int64_t nqt = (int64_t)B * H * ((N + fa::kFp8QTile - 1) / fa::kFp8QTile);
    const int64_t nkt = (int64_t)B * H * ((N + fa::kFp8KTile - 1) / fa::kFp8KTile);
    const Range ins[] = {span(q_codes, elems), span(k_codes, elems), span(q_exps, nqt * 4), span(k_exps, nkt * 4),
                         span(v, elems * 2), span(kv_limit, kv_limit ? (int64_t)B * N * 4 : 0)};
    const Range ro = span(o, elems * 2), rl = span(lse, (int64_t)B * H * N * 4);
    for (Range in : ins)
        if (overlap(ro, in) || overlap(rl, in)) return FA_ERR_ALIAS;
    if (overlap(ro, rl)) return FA_ERR_ALIAS;
    return hip_status(fa::launch_fused_fp8(q_codes, q_exps, nullptr, nullptr, k_codes, k_exps, v, o, lse, B, H, N, d,
                                           causal != 0, scale, kv_limit, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_fp8_qbf16(const fa_bf16* q, const int8_t* signs, const uint8_t* k_codes, const int32_t* k_exps,
                           const fa_bf16* v, fa_bf16* o, float* lse, int B, int H, int N, int d, int causal,
                           float scale, const int32_t* kv_limit, void* stream) {
    if (!q || !signs || !k_codes || !k_exps || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (!shape_ok(B, H, N, d, 2)) return FA_ERR_SHAPE;
    const int64_t elems = (int64_t)B * H * N * d;
    if (!isfinite(scale)) return FA_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(signs, 16) || !aligned(k_codes, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(k_exps, 4) || !aligned(lse, 4) || (kv_limit && !aligned(kv_limit, 4)))
        return FA_ERR_ALIGN;
    const int64_t nkt = (int64_t)B * H * ((N + fa::kFp8KTile - 1) / fa::kFp8KTile);
    const Range ins[] = {span(q, elems * 2), span(signs, d), span(k_codes, elems), span(k_exps, nkt * 4),
                         span(v, elems * 2), span(kv_limit, kv_limit ? (int64_t)B * N * 4 : 0)};
    const Range ro = span(o, elems * 2), rl = span(lse, (int64_t)B * H * N * 4);
    for (Range in : ins)
        if (overlap(ro, in) || overlap(rl, in)) return FA_ERR_ALIAS;
    if (overlap(ro, rl)) return FA_ERR_ALIAS;
    return hip_status(fa::launch_fused_fp8(nullptr, nullptr, q, signs, k_codes, k_exps, v, o, lse, B, H, N, d,
                                           causal != 0, scale, kv_limit, static_cast<hipStream_t>(stream)));
}

const char* fa_status_str(fa_status s) {
    switch (s) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "a size (B, H, N, pages, tile rows) is out of range";
        case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
        case FA_ERR_SCALE: return "scale must be finite";
        case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned; lse and kv_limit 4-byte aligned";
        case FA_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case FA_ERR_HIP: return "the HIP runtime rejected a kernel launch or a lookup";
        case FA_ERR_ALIAS: return "an output overlaps an input, the other output or the workspace";
        case FA_ERR_SCRATCH: return "the call needs more scratch memory than the library's static buffer holds";
    }
    return "unknown status";
}

}  // extern "C"

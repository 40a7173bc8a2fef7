// fa_launch.h -- host-side launchers behind the C ABI (internal to libfa.so).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

#include "fa_sizes.h"

namespace fa {

// The sign of the softmax scale, folded into the score operand that a kernel
// holds in registers.  The kernels' running max, and their masking (a masked
// score is -inf, and -inf * c must stay -inf), work on c > 0.  A negative scale
// is computed as the positive one with that operand negated: only sign bits
// change, the products are exactly negated and so is their sum, so S' c' equals
// S c bit for bit.  A zero scale is computed with that operand zeroed and
// c = log2(e): every score is then exactly 0, as scale 0 gives.  and_mask and
// xor_mask act on each 32-bit word of the operand (sign_bits marks the sign bit
// of every element packed in a word).
struct ScoreSign {
    uint32_t and_mask, xor_mask;
    float c;  // > 0
};
inline ScoreSign score_sign(float scale, float factor, uint32_t sign_bits) {
    if (scale > 0.f) return ScoreSign{0xffffffffu, 0u, scale * factor};
    if (scale < 0.f) return ScoreSign{0xffffffffu, sign_bits, -scale * factor};
    return ScoreSign{0u, 0u, factor};
}
constexpr uint32_t kSignBf16x2 = 0x80008000u;
constexpr uint32_t kSignF32 = 0x80000000u;
constexpr uint32_t kSignE4m3x4 = 0x80808080u;

// Launch `kernel` on `stream` and return the status of this launch alone.  (The
// runtime's last-error slot, read after a <<<>>> launch, also holds any error an
// earlier, unrelated runtime call left pending, which would then be reported as
// this launch's.)
template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds_bytes, hipStream_t stream,
                                A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<P...> values(static_cast<P>(args)...);
    void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {};
    std::apply(
        [&ptrs](auto&... v) {
            size_t i = 0;
            ((ptrs[i++] = static_cast<void*>(&v)), ...);
        },
        values);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds_bytes, stream);
}

// Grid of a forward launch over `blocks` query blocks: with `walk`, one
// workgroup per CU of the current device (never more than there are blocks),
// each walking several blocks; otherwise one workgroup per block.  Any grid
// size covers every block exactly once, so the CU count only shapes the
// schedule.
inline hipError_t walk_grid(long long blocks, bool walk, unsigned* grid) {
    long long n = blocks;
    if (walk) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (cus > 0 && cus < n) n = cus;
    }
    *grid = (unsigned)n;
    return hipSuccess;
}

hipError_t launch_fused_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                             int N, int d, bool causal, float scale, const int32_t* kv_limit,
                             hipStream_t stream);

hipError_t launch_fused_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                            int N, int d, bool causal, float scale, const int32_t* kv_limit,
                            hipStream_t stream);

// Row stride (elements) of the unfused path's S and P buffers: N rounded up to 64.
inline int64_t unfused_ld(int N) { return ((int64_t)N + 63) / 64 * 64; }

// Three launches: scores, masked row softmax, P V.  S is fp32 [B*H*N, ld];
// P is bf16 (elem 2) or fp32 (elem 4) [B*H*N, ld].
hipError_t launch_unfused(bool bf16_path, const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, bool causal, float scale, const int32_t* kv_limit,
                          float* S, void* P, hipStream_t stream);

// Backward pass: floats per statistic in the workspace (D and the base-2 LSE,
// each B*H*N, the count rounded up to 64 so the second starts 256-byte aligned).
inline int64_t bwd_stats_floats(int B, int H, int N) { return ((int64_t)B * H * N + 63) / 64 * 64; }

// Three launches: row statistics, dK/dV, dQ.  workspace holds 2 * bwd_stats_floats.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, bool causal,
                           float scale, const int32_t* kv_limit, float* workspace, hipStream_t stream);

// Two launches: per-split partials, then the merge into o and lse.
hipError_t launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int B, int H, int d, int max_pages,
                              int num_pages, float scale, float* workspace, hipStream_t stream);

// Device address of the decode path's static scratch buffer (kDecodeScratchBytes)
// on the current device; looked up once per device, on its first use.
hipError_t decode_scratch(float** ptr);

// Rotate (random signs, Hadamard) and encode rows of a bf16 [B, H, N, d] tensor
// to E4M3 codes [B, H, N, d] with per-tile exponents.
hipError_t launch_fp8_quantize(const void* x, const int8_t* signs, uint8_t* codes, int32_t* exps, int B, int H, int N,
                               int d, int tile_rows, hipStream_t stream);

// Fused forward with E4M3 Q and K codes (scores divided by d) and bf16 V.
// Q either as codes and tile exponents (qc, qe; q_bf16 == nullptr) or as bf16
// with the rotation's signs (q_bf16, signs), rotated and encoded in the kernel.
hipError_t launch_fused_fp8(const uint8_t* qc, const int32_t* qe, const void* q_bf16, const int8_t* signs,
                            const uint8_t* kc, const int32_t* ke, const void* v, void* o, float* lse, int B, int H,
                            int N, int d, bool causal, float scale, const int32_t* kv_limit, hipStream_t stream);

}  // namespace fa

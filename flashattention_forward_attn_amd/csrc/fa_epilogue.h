// fa_epilogue.h -- the output stage shared by the kernels whose 32x32 MFMA
// accumulators hold one output row per lane: O in the two fused forward kernels
// (bf16 and FP8 scores) and in the unfused P V, dK, dV and dQ in the backward.
#pragma once
#include "fa_common.h"

namespace fa {

// Lane half h holds dims 8 g + 4 h .. +3 of a 32-dim block of its row in
// acc[4 g .. 4 g + 3] (g = 0..3).
// Scales them by inv, packs them to bf16 and hands back out[p] = dims 16 p + 8 h ..
// +7, ready for one 16-byte store each: for every pair of groups (2 p, 2 p + 1) one
// v_permlane32_swap per word, which trades the upper lanes of its first operand
// with the lower lanes of its second.
__device__ __forceinline__ void o_rows16(const f32x16& acc, float inv, u32x4 (&out)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int g0 = 8 * p + 2 * k, g1 = g0 + 4;
            const uint32_t w0 = pack_bf16x2(acc[g0] * inv, acc[g0 + 1] * inv);
            const uint32_t w1 = pack_bf16x2(acc[g1] * inv, acc[g1 + 1] * inv);
            const auto r = __builtin_amdgcn_permlane32_swap(w0, w1, false, false);
            out[p][k] = (uint32_t)r[0];
            out[p][2 + k] = (uint32_t)r[1];
        }
}

}  // namespace fa

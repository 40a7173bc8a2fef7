// fa_tile.h -- helpers shared by the forward and backward kernels: direct
// global -> LDS loads, the XOR chunk swizzle of a tile row, the transposing LDS
// read, and the forward grids' walk over query blocks.
#pragma once

#include <type_traits>

#include "fa_common.h"

// A build with FA_SINGLE_STAGE=1 streams K/V tiles through one LDS stage and
// loads a tile only after every wave has finished reading the previous one, so
// no load is in flight while a stage is read.  Its results must equal the
// pipelined build's bit for bit: a check that the pipelining has no race.
#ifndef FA_SINGLE_STAGE
#define FA_SINGLE_STAGE 0
#endif

namespace fa {

constexpr bool kSingleStage = FA_SINGLE_STAGE != 0;

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kDmaBytes = kWave * 16;  // one wave-wide 16-byte-per-lane LDS load

// Rows of D bf16 values are stored in LDS as D/8 chunks of 16 bytes; chunk c of
// row `row` sits in slot c ^ swz<D>(row).  With this swizzle a read of one chunk
// from 16 consecutive rows, and a read of 4 chunks from 4 consecutive rows (the
// transposing-read pattern), each touch 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz(int row) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 128) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        const int h = (row >> 1) & 7;
        return ((h & 1) << 2) | (h >> 1);
    }
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr)p; }

// Buffer descriptor over [base, base + bytes) as four scalars: reads past the
// end return zeros.
__device__ __forceinline__ i32x4 dma_desc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// Wave-wide load straight into LDS: lane l's 16 bytes at global offset voff land at
// LDS byte address dst + 16 l (M0 holds dst while the load issues; the load takes
// its LDS address at issue, and M0's previous value is restored afterwards, so
// the compiler's view of M0 is unchanged).  Issued from inline assembly so that
// the compiler does not wait for it before unrelated LDS reads; the caller waits
// with s_waitcnt vmcnt before the barrier that publishes the data.
__device__ __forceinline__ void dma16(const i32x4& desc, uint32_t dst, uint32_t voff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(desc)
        : "memory");
}
// The same with 4 bytes per lane (lane l's word lands at dst + 4 l).
__device__ __forceinline__ void dma4(const i32x4& desc, uint32_t dst, uint32_t voff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(desc)
        : "memory");
}

// ds_read_b64_tr_b16: within each group of 16 lanes, output lane i receives, in
// slot s, element i % 4 of the 8 bytes addressed by lane 4 s + i / 4.
__device__ __forceinline__ u32x2 tr_read(const char* p) {
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    return __builtin_bit_cast(u32x2, r);
}

// Block taken in round r by workgroup g of a grid of P that walks blocks
// r P ... r P + P - 1 per round: block g in even rounds and, in odd rounds, the
// mirror image of g among the workgroups with its residue mod 8 (round-robin
// dispatch puts those on g's XCD), or among all when P is not a multiple of 8.
// With blocks sorted longest first, a long block then pairs with a short one.
__device__ __forceinline__ int walk_block(int r, int g, int P) {
    int j = g;
    if (r & 1) j = (P & 7) ? P - 1 - g : P - 8 - (g & ~7) + (g & 7);
    return r * P + j;
}

}  // namespace fa

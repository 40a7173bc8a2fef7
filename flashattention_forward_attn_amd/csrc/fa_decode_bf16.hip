// fa_decode_bf16.hip -- decode attention over a paged key/value cache for gfx950.
//
// The method: one query per sequence (the token being generated) attends to all
// of its sequence's cached keys.  The cache is cut into pages of 16 tokens and a
// per-sequence block table maps logical pages to physical pages of the pool
// ("CS336 第五讲 · GPU 与 GPU 优化", the PagedAttention section).  With one
// query row, batch x heads alone can be too few independent pieces of work, so
// the key dimension is split too, the way FlashAttention-2 parallelises over the
// sequence ("FlashAttention 1–4: How IO-Awareness Reshaped the Attention
// Kernel", section "FlashAttention-2"), and the per-split results are merged
// with the online-softmax rescaling of partial (m, l, o) ("FlashAttention 1–4",
// section "FlashAttention (v1)").
//
// Every cached key and value is read once and used for one multiply-add per
// element, so the work is bound by HBM bandwidth: no matrix instructions, but
// wide coalesced loads with many bytes in flight.
//
// Two kernels on the caller's stream:
//   1. split: one wave per (sequence, head, 64-key split).  D/8 lanes per key,
//      each loading 16 bytes, so one load instruction covers 512/D consecutive
//      keys of one page (a page of one head is 16 * D * 2 contiguous bytes).
//      Scores by packed bf16 dot products, summed within each lane group by DPP;
//      the wave's max, exponentials, sum and weighted value rows are written as
//      an unnormalised partial (m, l, o) in base 2.
//   2. combine: one wave per (sequence, head) merges its splits:
//      m = max m_s, l = sum 2^(m_s - m) l_s, o = sum 2^(m_s - m) o_s / l.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace decode {

constexpr int kPage = kDecodePage;            // tokens per page
constexpr int kSplitKeys = kDecodeSplitKeys;  // keys per split (one wave)
constexpr int kSplitWaves = 4;                // splits per workgroup
constexpr int kThreads = kSplitWaves * kWave;

// Sum over aligned groups of W lanes (W = 8 or 16); every lane of a group gets
// the group's sum.  Quad swaps, then half-row and row mirrors (within a group
// the pairing does not matter for a sum).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

template <int W>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (W == 16) x += dpp<0x140>(x);  // row_mirror
    return x;
}

// Reduce over the lanes that hold different keys (lane bits at and above log2 W).
template <int W>
__device__ __forceinline__ float cross_max(float x) {
    for (int off = W; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}
template <int W>
__device__ __forceinline__ float cross_sum(float x) {
    for (int off = W; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

__device__ __forceinline__ int clamp_len(int len, int max_pages) {
    const int cap = max_pages * kPage;
    return len < 0 ? 0 : (len > cap ? cap : len);
}

template <int D>
__global__ __launch_bounds__(kThreads) void split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                                                         const bf16* __restrict__ vc,
                                                         const int32_t* __restrict__ block_table,
                                                         const int32_t* __restrict__ seq_lens,
                                                         float* __restrict__ part_o, float* __restrict__ part_ml,
                                                         int H, int max_pages, int num_pages, int max_splits,
                                                         float c) {
    constexpr int LPK = D / 8;           // lanes per key
    constexpr int KPI = kWave / LPK;     // keys per load instruction
    constexpr int NI = kSplitKeys / KPI; // load instructions per split
    static_assert(kPage % KPI == 0, "a load instruction stays inside one page");

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.y, b = blockIdx.z;
    const int split = blockIdx.x * kSplitWaves + w;
    const int len = clamp_len(seq_lens[b], max_pages);
    const int key0 = split * kSplitKeys;
    if (split >= max_splits || key0 >= len) return;

    const int grp = lane / LPK, cidx = lane % LPK;  // key within an instruction, 8-dim chunk
    const size_t bh = (size_t)b * H + h;
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>(q + bh * D + 8 * cidx);

    // Physical pages of this split (uniform); pages past the length are not read.
    constexpr int kPagesPerSplit = kSplitKeys / kPage;
    int page[kPagesPerSplit];
#pragma unroll
    for (int p = 0; p < kPagesPerSplit; ++p) {
        const int lp = key0 / kPage + p;
        page[p] = lp * kPage < len ? block_table[(size_t)b * max_pages + lp] : -1;
    }

    bf16x8 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int pg = page[(i * KPI) / kPage];
        const int slot = (i * KPI) % kPage + grp;
        if (pg >= 0 && pg < num_pages) {
            const size_t off = (((size_t)pg * H + h) * kPage + slot) * D + 8 * cidx;
            kr[i] = *reinterpret_cast<const bf16x8*>(kc + off);
            vr[i] = *reinterpret_cast<const bf16x8*>(vc + off);
        } else {
            kr[i] = bf16x8{};
            vr[i] = bf16x8{};
        }
    }

    // scores (base 2), -inf past the length
    float s[NI];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const u32x4 qa = __builtin_bit_cast(u32x4, qv), ka = __builtin_bit_cast(u32x4, kr[i]);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // (elements copied out first: a bit cast of a vector element reads element 0)
            const uint32_t qe = qa[e], ke = ka[e];
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qe), __builtin_bit_cast(bf16x2, ke), acc,
                                                  false);
        }
        acc = group_sum<LPK>(acc);
        const int key = key0 + i * KPI + grp;
        s[i] = key < len ? acc * c : -INFINITY;
        m = fmaxf(m, s[i]);
    }
    m = cross_max<LPK>(m);  // key0 < len, so m is finite

    float l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int key = key0 + i * KPI + grp;
        const float p = __builtin_amdgcn_exp2f(s[i] - m);
        l += p;
        if (key < len) {  // slots past the length may hold anything
            const u32x4 va = __builtin_bit_cast(u32x4, vr[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = fmaf(p, __builtin_bit_cast(float, va[e] << 16), o[2 * e]);
                o[2 * e + 1] = fmaf(p, __builtin_bit_cast(float, va[e] & 0xffff0000u), o[2 * e + 1]);
            }
        }
    }
    l = cross_sum<LPK>(l);  // one lane per key group: each key counted once
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = cross_sum<LPK>(o[e]);

    const size_t part = bh * max_splits + split;
    if (grp == 0) {
        f32x4* dst = reinterpret_cast<f32x4*>(part_o + part * D + 8 * cidx);
        dst[0] = f32x4{o[0], o[1], o[2], o[3]};
        dst[1] = f32x4{o[4], o[5], o[6], o[7]};
    }
    if (lane == 0) {
        part_ml[2 * part] = m;
        part_ml[2 * part + 1] = l;
    }
}

// One wave per (sequence, head): lane owns dims lane * D / 64 ...
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           const int32_t* __restrict__ seq_lens, bf16* __restrict__ o,
                                                           float* __restrict__ lse, int B, int H, int max_pages,
                                                           int max_splits) {
    constexpr int E = D / kWave;  // dims per lane: 2 or 1
    const int lane = threadIdx.x & (kWave - 1);
    const long long bh = (long long)blockIdx.x * kSplitWaves + (threadIdx.x >> 6);
    if (bh >= (long long)B * H) return;
    const int b = (int)(bh / H);
    const int len = clamp_len(seq_lens[b], max_pages);
    const int n = (len + kSplitKeys - 1) / kSplitKeys;
    bf16* orow = o + bh * D + E * lane;
    if (n == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) orow[e] = (bf16)0.f;
        if (lane == 0) lse[bh] = -INFINITY;
        return;
    }
    const float* ml = part_ml + 2 * bh * max_splits;
    const float* po = part_o + bh * max_splits * D + E * lane;
    float m = -INFINITY;
    for (int s = lane; s < n; s += kWave) m = fmaxf(m, ml[2 * s]);
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    float l = 0.f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int s = 0; s < n; ++s) {
        const float a = __builtin_amdgcn_exp2f(ml[2 * s] - m);
        l = fmaf(a, ml[2 * s + 1], l);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(a, po[(size_t)s * D + e], acc[e]);
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[e] = (bf16)(acc[e] * inv);
    if (lane == 0) lse[bh] = (m + __log2f(l)) * kLn2;
}

}  // namespace decode

hipError_t launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int B, int H, int d, int max_pages,
                              int num_pages, float scale, float* workspace, hipStream_t stream) {
    const int max_splits = (int)decode_max_splits(max_pages);
    float* part_o = workspace;
    float* part_ml = workspace + decode_part_o_floats(B, H, d, max_pages);
    const float c = scale * kLog2e;
    const dim3 grid_split((unsigned)((max_splits + decode::kSplitWaves - 1) / decode::kSplitWaves), (unsigned)H,
                          (unsigned)B);
    const unsigned grid_combine = (unsigned)(((long long)B * H + decode::kSplitWaves - 1) / decode::kSplitWaves);
    const bf16* Q = static_cast<const bf16*>(q);
    const bf16* K = static_cast<const bf16*>(k_cache);
    const bf16* V = static_cast<const bf16*>(v_cache);
    bf16* O = static_cast<bf16*>(o);
    if (max_splits > 0) {
        if (d == 128)
            hipLaunchKernelGGL((decode::split_kernel<128>), grid_split, dim3(decode::kThreads), 0, stream, Q, K, V,
                               block_table, seq_lens, part_o, part_ml, H, max_pages, num_pages, max_splits, c);
        else
            hipLaunchKernelGGL((decode::split_kernel<64>), grid_split, dim3(decode::kThreads), 0, stream, Q, K, V,
                               block_table, seq_lens, part_o, part_ml, H, max_pages, num_pages, max_splits, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (d == 128)
        hipLaunchKernelGGL((decode::combine_kernel<128>), dim3(grid_combine), dim3(decode::kThreads), 0, stream,
                           part_o, part_ml, seq_lens, O, lse, B, H, max_pages, max_splits);
    else
        hipLaunchKernelGGL((decode::combine_kernel<64>), dim3(grid_combine), dim3(decode::kThreads), 0, stream,
                           part_o, part_ml, seq_lens, O, lse, B, H, max_pages, max_splits);
    return hipGetLastError();
}

}  // namespace fa

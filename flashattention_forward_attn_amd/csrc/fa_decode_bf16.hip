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
//   1. split: one workgroup per (sequence, head, 256-key split), one wave per 64
//      keys; the grid runs over (sequence, head) fastest and splits slowest.  D/8 lanes per key, each loading 16 bytes, so one load instruction
//      covers 512/D consecutive keys of one page (a page of one head is
//      16 * D * 2 contiguous bytes).  Scores by packed bf16 dot products, summed
//      within each lane group by DPP; each wave's max, exponentials, sum and
//      weighted value rows form a partial (m, l, o) in base 2, and the four
//      waves' partials are merged through LDS into one unnormalised partial per
//      split.
//   2. combine: one workgroup per (sequence, head) merges its splits:
//      m = max m_s, l = sum 2^(m_s - m) l_s, o = sum 2^(m_s - m) o_s / l.
#include <mutex>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace decode {

constexpr int kPage = kDecodePage;            // tokens per page
constexpr int kSplitKeys = kDecodeSplitKeys;  // keys per split (one workgroup)
constexpr int kWaves = 4;
constexpr int kWaveKeys = kSplitKeys / kWaves;  // keys per wave
constexpr int kThreads = kWaves * kWave;

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
    constexpr int NI = kWaveKeys / KPI;  // load instructions per wave
    static_assert(kPage % KPI == 0, "a load instruction stays inside one page");
    __shared__ float sh_ml[2 * kWaves];
    __shared__ __attribute__((aligned(16))) float sh_o[kWaves * D];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int split = blockIdx.y;
    const int key0 = split * kSplitKeys + w * kWaveKeys;  // this wave's first key

    // Physical pages of this wave's keys, read next to the length (the entries
    // stay inside the table row; they are used only below the length).
    constexpr int kPagesPerWave = kWaveKeys / kPage;
    int page[kPagesPerWave];
#pragma unroll
    for (int p = 0; p < kPagesPerWave; ++p) {
        const int lp = key0 / kPage + p;
        page[p] = lp < max_pages ? block_table[(size_t)b * max_pages + lp] : -1;
    }
    const int len = clamp_len(seq_lens[b], max_pages);
    if (split >= max_splits || split * kSplitKeys >= len) return;  // the whole workgroup
    const bool active = key0 < len;

    const int grp = lane / LPK, cidx = lane % LPK;  // key within an instruction, 8-dim chunk
    const size_t bh = (size_t)b * H + h;
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>(q + bh * D + 8 * cidx);

    bf16x8 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int pg = page[(i * KPI) / kPage];
        const int slot = (i * KPI) % kPage + grp;
        if (active && (key0 + i * KPI) < len && pg >= 0 && pg < num_pages) {
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
    m = cross_max<LPK>(m);  // -inf only for a wave past the length

    float l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int key = key0 + i * KPI + grp;
        const float p = active ? __builtin_amdgcn_exp2f(s[i] - m) : 0.f;
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

    // merge the four waves' partials (a wave past the length has m = -inf, l = 0, o = 0)
    if (grp == 0) {
        f32x4* dst = reinterpret_cast<f32x4*>(sh_o + w * D + 8 * cidx);
        dst[0] = f32x4{o[0], o[1], o[2], o[3]};
        dst[1] = f32x4{o[4], o[5], o[6], o[7]};
    }
    if (lane == 0) {
        sh_ml[2 * w] = m;
        sh_ml[2 * w + 1] = l;
    }
    __syncthreads();
    if (tid < D) {
        float mm = sh_ml[0];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) mm = fmaxf(mm, sh_ml[2 * v]);  // wave 0 is below the length
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float a = __builtin_amdgcn_exp2f(sh_ml[2 * v] - mm);
            acc = fmaf(a, sh_o[v * D + tid], acc);
            lsum = fmaf(a, sh_ml[2 * v + 1], lsum);
        }
        const size_t part = bh * max_splits + split;
        part_o[part * D + tid] = acc;
        if (tid == 0) {
            part_ml[2 * part] = mm;
            part_ml[2 * part + 1] = lsum;
        }
    }
}

// One workgroup per (sequence, head): thread t adds up dim t % D over the
// splits s = t / D (mod 256 / D), the groups are then summed through LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           const int32_t* __restrict__ seq_lens, bf16* __restrict__ o,
                                                           float* __restrict__ lse, int H, int max_pages,
                                                           int max_splits) {
    constexpr int G = kThreads / D;  // split groups
    constexpr int U = 4;             // splits in flight per thread
    __shared__ float sh_m[kWaves];
    __shared__ float sh_acc[kThreads], sh_l[G];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const size_t bh = blockIdx.x;
    const int b = (int)(bh / H);
    const int len = clamp_len(seq_lens[b], max_pages);
    const int n = (len + kSplitKeys - 1) / kSplitKeys;
    if (n == 0) {
        if (tid < D) o[bh * D + tid] = (bf16)0.f;
        if (tid == 0) lse[bh] = -INFINITY;
        return;
    }
    const float* ml = part_ml + 2 * bh * max_splits;
    const float* po = part_o + bh * max_splits * D;
    float m = -INFINITY;
    for (int s = tid; s < n; s += kThreads) m = fmaxf(m, ml[2 * s]);
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) sh_m[w] = m;
    __syncthreads();
    m = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));

    const int dim = tid % D, g = tid / D;
    float acc = 0.f, l = 0.f;
    for (int s0 = g; s0 < n; s0 += G * U) {
        float a[U], x[U], y[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * G;
            a[u] = s < n ? ml[2 * s] : -INFINITY;
            y[u] = s < n ? ml[2 * s + 1] : 0.f;
            x[u] = s < n ? po[(size_t)s * D + dim] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float f = __builtin_amdgcn_exp2f(a[u] - m);
            acc = fmaf(f, x[u], acc);
            l = fmaf(f, y[u], l);
        }
    }
    sh_acc[tid] = acc;
    if (dim == 0) sh_l[g] = l;
    __syncthreads();
    if (tid < D) {
        float t = 0.f, lt = 0.f;
#pragma unroll
        for (int v = 0; v < G; ++v) {
            t += sh_acc[v * D + tid];
            lt += sh_l[v];
        }
        o[bh * D + tid] = (bf16)(t / lt);
        if (tid == 0) lse[bh] = (m + __log2f(lt)) * kLn2;
    }
}

}  // namespace decode

// Workspace of the no-allocation entry point: one copy per GPU, created with the
// code object and held until the process ends.  In host code its name stands for
// a host-side shadow, never a device address: every use goes through the address
// decode_scratch looks up.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / 4];

namespace {
constexpr int kScratchDevices = 64;
std::mutex scratch_mutex;
float* scratch_ptr[kScratchDevices] = {};  // device address per device, once looked up
}  // namespace

hipError_t decode_scratch(float** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = static_cast<float*>(p);
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int B, int H, int d, int max_pages,
                              int num_pages, float scale, float* workspace, hipStream_t stream) {
    const int max_splits = (int)decode_max_splits(max_pages);
    float* part_o = workspace;
    float* part_ml = workspace + decode_part_o_floats(B, H, d, max_pages);
    const float c = scale * kLog2e;
    // (sequence, head) fastest, splits slowest: the first splits, present for
    // every sequence, go out first, and the grid's empty tail (splits past short
    // sequences) comes last.  Measured 243 -> 192 us on ragged lengths.
    const dim3 grid_split((unsigned)((long long)B * H), (unsigned)max_splits);
    const unsigned grid_combine = (unsigned)((long long)B * H);
    const bf16* Q = static_cast<const bf16*>(q);
    const bf16* K = static_cast<const bf16*>(k_cache);
    const bf16* V = static_cast<const bf16*>(v_cache);
    bf16* O = static_cast<bf16*>(o);
    if (max_splits > 0) {
        const hipError_t e =
            d == 128 ? launch_kernel(decode::split_kernel<128>, grid_split, dim3(decode::kThreads), 0, stream, Q, K, V,
                                     block_table, seq_lens, part_o, part_ml, H, max_pages, num_pages, max_splits, c)
                     : launch_kernel(decode::split_kernel<64>, grid_split, dim3(decode::kThreads), 0, stream, Q, K, V,
                                     block_table, seq_lens, part_o, part_ml, H, max_pages, num_pages, max_splits, c);
        if (e != hipSuccess) return e;
    }
    if (d == 128)
        return launch_kernel(decode::combine_kernel<128>, dim3(grid_combine), dim3(decode::kThreads), 0, stream,
                             part_o, part_ml, seq_lens, O, lse, H, max_pages, max_splits);
    return launch_kernel(decode::combine_kernel<64>, dim3(grid_combine), dim3(decode::kThreads), 0, stream, part_o,
                         part_ml, seq_lens, O, lse, H, max_pages, max_splits);
}

}  // namespace fa

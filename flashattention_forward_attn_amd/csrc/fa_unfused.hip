// fa_unfused.hip -- standard (unfused) attention forward: three kernels, with the
// N x N score matrix S and probability matrix P making a round trip through
// device memory.  This is the baseline the fused kernel replaces: "FlashAttention
// 1–4: How IO-Awareness Reshaped the Attention Kernel", section "FlashAttention
// (v1)", the figure contrasting standard attention (one kernel per step, S and P
// out to HBM and back) with the fused kernel; "GPU 与 TPU：让硬件不再是黑魔法"
// §11.1.  The softmax kernel is one row per workgroup with the row held in
// registers, so S is read once and P written once ("GPU 与 Triton 入门" §2.2).
//
//   scores  : S[row, j] = scale * <q_row, k_j>            (fp32, every pair, no mask)
//   softmax : P[row, j] = exp(S - max) / sum over valid j  (mask applied here), lse
//   pv      : O[row, :] = sum_j P[row, j] v_j
//
// S and P rows have stride ld = N rounded up to 64; P is zero in [N, ld) so the
// P V kernel reads whole 64-key tiles.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace unfused {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- scores (bf16)
// Workgroup = 4 waves, a 128 (query) x 128 (key) tile of S.  The K tile is
// staged in LDS once per workgroup; each wave keeps its 32 query rows' Q
// fragments in registers and computes 4 slabs of 32 keys with C = A B,
// A = Q (row = query, k = dims), B = K^T (col = key, k = dims).  S is written
// with streaming stores: it is far larger than any cache.
constexpr int kScoreTile = 128;

template <int D>
__global__ __launch_bounds__(kThreads) void scores_bf16(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                        float* __restrict__ S, int N, int64_t ld, float scale) {
    constexpr int kStride = D + 8;
    __shared__ __attribute__((aligned(16))) bf16 Ks[kScoreTile * kStride];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const size_t head = (size_t)blockIdx.z * N * D;
    const int q0 = blockIdx.y * kScoreTile + w * 32;
    const int k0 = blockIdx.x * kScoreTile;
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(K + head, (uint32_t)N * D * 2u);
#pragma unroll
    for (int i = 0; i < kScoreTile * D / 8 / kThreads; ++i) {
        const int ci = tid + i * kThreads;
        const int row = ci / (D / 8), c8 = ci % (D / 8);
        const uint32_t off = ((uint32_t)(k0 + row) * D + 8 * c8) * 2u;  // rows past N read as zeros
        *reinterpret_cast<u32x4*>(Ks + row * kStride + 8 * c8) =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
    }
    const int qa = q0 + col;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = qa < N ? *reinterpret_cast<const bf16x8*>(Q + head + (size_t)qa * D + 16 * kk + 8 * half) : bf16x8{};
    __syncthreads();
    f32x16 acc[kScoreTile / 32];
#pragma unroll
    for (int sub = 0; sub < kScoreTile / 32; ++sub) acc[sub] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int sub = 0; sub < kScoreTile / 32; ++sub)
            acc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                qf[kk], *reinterpret_cast<const bf16x8*>(Ks + (sub * 32 + col) * kStride + 16 * kk + 8 * half),
                acc[sub], 0, 0, 0);
    float* Sh = S + (size_t)blockIdx.z * N * ld;
#pragma unroll
    for (int sub = 0; sub < kScoreTile / 32; ++sub) {
        const int key = k0 + sub * 32 + col;
        if (key >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int q = q0 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (q < N) __builtin_nontemporal_store(acc[sub][r] * scale, Sh + (size_t)q * ld + key);
        }
    }
}

// ---------------------------------------------------------------- scores (fp32)
template <int D>
__global__ __launch_bounds__(kThreads) void scores_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                       float* __restrict__ S, int N, int64_t ld, float scale) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (int64_t)N * N) return;
    const int q = (int)(idx / N), j = (int)(idx % N);
    const size_t head = (size_t)blockIdx.y * N * D;
    const float* qr = Q + head + (size_t)q * D;
    const float* kr = K + head + (size_t)j * D;
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc = fmaf(qr[c], kr[c], acc);
    S[(size_t)blockIdx.y * N * ld + (size_t)q * ld + j] = acc * scale;
}

// ---------------------------------------------------------------- softmax rows
__device__ __forceinline__ float block_reduce_max(float x, float* red) {
    x = wave_max(x);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_reduce_sum(float x, float* red) {
    x = wave_sum(x);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename PT>
__device__ __forceinline__ PT to_p(float x);
template <>
__device__ __forceinline__ bf16 to_p<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ float to_p<float>(float x) { return x; }

// One workgroup per row.  EPT > 0: the row lives in registers (EPT elements per
// thread, EPT * 256 >= ld).  EPT == 0: long rows, three passes over S.
template <typename PT, int EPT>
__global__ __launch_bounds__(kThreads) void softmax_rows(const float* __restrict__ S, PT* __restrict__ P,
                                                         float* __restrict__ LSE, int H, int N, int64_t ld,
                                                         int causal, const int32_t* __restrict__ kv_limit) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int i = (int)(row % N);
    const int b = (int)(row / N) / H;
    const int lim = row_key_limit(i, N, causal != 0, kv_limit ? kv_limit + (size_t)b * N + i : nullptr);
    const float* srow = S + row * ld;
    PT* prow = P + row * ld;
    const int tid = threadIdx.x;

    if constexpr (EPT > 0) {
        float x[EPT];
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int j = tid + e * kThreads;
            x[e] = j < N ? srow[j] : -INFINITY;
            if (j >= lim) x[e] = -INFINITY;
            m = fmaxf(m, x[e]);
        }
        m = block_reduce_max(m, red);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int j = tid + e * kThreads;
            x[e] = (j < lim) ? __expf(x[e] - m) : 0.f;
            sum += x[e];
        }
        sum = block_reduce_sum(sum, red);
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int j = tid + e * kThreads;
            if (j < ld) prow[j] = to_p<PT>(x[e] * inv);
        }
        if (tid == 0) LSE[row] = sum > 0.f ? m + __logf(sum) : -INFINITY;
    } else {
        float m = -INFINITY;
        for (int j = tid; j < lim; j += kThreads) m = fmaxf(m, srow[j]);
        m = block_reduce_max(m, red);
        float sum = 0.f;
        for (int j = tid; j < lim; j += kThreads) sum += __expf(srow[j] - m);
        sum = block_reduce_sum(sum, red);
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
        for (int j = tid; j < ld; j += kThreads) prow[j] = to_p<PT>(j < lim ? __expf(srow[j] - m) * inv : 0.f);
        if (tid == 0) LSE[row] = sum > 0.f ? m + __logf(sum) : -INFINITY;
    }
}

// ---------------------------------------------------------------- P V (bf16)
// Workgroup = 4 waves x 32 query rows; keys in chunks of 64.  While chunk k is
// multiplied, chunk k+1's P fragments (registers) and V rows (registers, then
// LDS transposed to [dim][key]) are in flight.  C = A B with A = P (row =
// query, k = keys), B = V (col = dim, k = keys).
template <int D>
__global__ __launch_bounds__(kThreads) void pv_bf16(const bf16* __restrict__ P, const bf16* __restrict__ V,
                                                    bf16* __restrict__ O, int N, int64_t ld) {
    constexpr int kBK = 64, kStride = kBK + 8, kUnits = (kBK / 8) * (D / 4);
    __shared__ __attribute__((aligned(16))) bf16 Vt[2][D * kStride];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const size_t head = (size_t)blockIdx.y * N * D;
    const int q0 = blockIdx.x * 128 + w * 32;
    const int qa = q0 + col;
    // rows past N (and keys past N, which P holds as zeros up to ld) read as zeros
    const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(P + (size_t)blockIdx.y * N * ld, (uint32_t)((uint64_t)N * ld * 2u));
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(V + head, (uint32_t)N * D * 2u);
    const int j = tid & 7, c = tid >> 3;  // V unit: 8 consecutive keys x 4 dims

    bf16x8 pa[2][kBK / 16];
    u32x2 vr[8];
    // buffer indices are compile-time constants so pa stays in registers
    auto load = [&](auto buf_c, int k0) {
        constexpr int buf = decltype(buf_c)::value;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks)
            pa[buf][ks] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(prs, ((uint32_t)qa * (uint32_t)ld + k0 + 16 * ks + 8 * half) * 2u, 0, 0));
        if (kUnits == kThreads || tid < kUnits) {
#pragma unroll
            for (int s = 0; s < 8; ++s)
                vr[s] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, ((uint32_t)(k0 + 8 * j + s) * D + 4 * c) * 2u, 0, 0));
        }
    };
    auto stage = [&](auto buf_c) {
        constexpr int buf = decltype(buf_c)::value;
        if (kUnits == kThreads || tid < kUnits) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x4 out;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t a = (e < 2) ? vr[2 * p].x : vr[2 * p].y;
                    const uint32_t bq = (e < 2) ? vr[2 * p + 1].x : vr[2 * p + 1].y;
                    out[p] = (e & 1) ? ((a >> 16) | (bq & 0xffff0000u)) : ((a & 0xffffu) | (bq << 16));
                }
                *reinterpret_cast<u32x4*>(&Vt[buf][(4 * c + e) * kStride + 8 * j]) = out;
            }
        }
    };
    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    const int nchunks = (N + kBK - 1) / kBK;
    auto chunk = [&](auto cur_c, int kc) {
        constexpr int cur = decltype(cur_c)::value;
        const bool more = kc + 1 < nchunks;
        if (more) load(std::integral_constant<int, cur ^ 1>{}, (kc + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks)
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    pa[cur][ks], *reinterpret_cast<const bf16x8*>(&Vt[cur][(32 * t + col) * kStride + 16 * ks + 8 * half]),
                    acc[t], 0, 0, 0);
        if (more) stage(std::integral_constant<int, cur ^ 1>{});
        __syncthreads();
    };
    load(std::integral_constant<int, 0>{}, 0);
    stage(std::integral_constant<int, 0>{});
    __syncthreads();
    for (int kc = 0; kc < nchunks; kc += 2) {
        chunk(std::integral_constant<int, 0>{}, kc);
        if (kc + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, kc + 1);
    }
    bf16* Oh = O + head;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int q = q0 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (q < N) Oh[(size_t)q * D + 32 * t + col] = (bf16)acc[t][r];
        }
}

// ---------------------------------------------------------------- P V (fp32)
template <int D>
__global__ __launch_bounds__(kThreads) void pv_f32(const float* __restrict__ P, const float* __restrict__ V,
                                                   float* __restrict__ O, int N, int64_t ld) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (int64_t)N * D) return;
    const int q = (int)(idx / D), c = (int)(idx % D);
    const size_t head = (size_t)blockIdx.y * N * D;
    const float* prow = P + (size_t)blockIdx.y * N * ld + (size_t)q * ld;
    float acc = 0.f;
    for (int j = 0; j < N; ++j) acc = fmaf(prow[j], V[head + (size_t)j * D + c], acc);
    O[head + (size_t)q * D + c] = acc;
}

template <typename PT>
hipError_t launch_softmax(const float* S, PT* P, float* lse, int B, int H, int N, int64_t ld, bool causal,
                          const int32_t* kv_limit, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)B * H * N)), block(kThreads);
    const int c = causal ? 1 : 0;
    if (ld <= 1 * kThreads)
        return launch_kernel(softmax_rows<PT, 1>, grid, block, 0, stream, S, P, lse, H, N, ld, c, kv_limit);
    if (ld <= 4 * kThreads)
        return launch_kernel(softmax_rows<PT, 4>, grid, block, 0, stream, S, P, lse, H, N, ld, c, kv_limit);
    if (ld <= 16 * kThreads)
        return launch_kernel(softmax_rows<PT, 16>, grid, block, 0, stream, S, P, lse, H, N, ld, c, kv_limit);
    if (ld <= 64 * kThreads)
        return launch_kernel(softmax_rows<PT, 64>, grid, block, 0, stream, S, P, lse, H, N, ld, c, kv_limit);
    return launch_kernel(softmax_rows<PT, 0>, grid, block, 0, stream, S, P, lse, H, N, ld, c, kv_limit);
}

}  // namespace unfused

hipError_t launch_unfused(bool bf16_path, const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, bool causal, float scale, const int32_t* kv_limit,
                          float* S, void* P, hipStream_t stream) {
    using namespace unfused;
    const int64_t ld = unfused_ld(N);
    const unsigned BH = (unsigned)((int64_t)B * H);
    const dim3 block(kThreads);
    hipError_t err;
    if (bf16_path) {
        const bf16 *Q = static_cast<const bf16*>(q), *K = static_cast<const bf16*>(k);
        const dim3 g1((N + kScoreTile - 1) / kScoreTile, (N + kScoreTile - 1) / kScoreTile, BH);
        err = d == 64 ? launch_kernel(scores_bf16<64>, g1, block, 0, stream, Q, K, S, N, ld, scale)
                      : launch_kernel(scores_bf16<128>, g1, block, 0, stream, Q, K, S, N, ld, scale);
        if (err != hipSuccess) return err;
        if ((err = launch_softmax<bf16>(S, (bf16*)P, lse, B, H, N, ld, causal, kv_limit, stream)) != hipSuccess) return err;
        const bf16 *Pb = static_cast<const bf16*>(P), *Vb = static_cast<const bf16*>(v);
        bf16* Ob = static_cast<bf16*>(o);
        const dim3 g3((N + 127) / 128, BH);
        return d == 64 ? launch_kernel(pv_bf16<64>, g3, block, 0, stream, Pb, Vb, Ob, N, ld)
                       : launch_kernel(pv_bf16<128>, g3, block, 0, stream, Pb, Vb, Ob, N, ld);
    }
    const float *Q = static_cast<const float*>(q), *K = static_cast<const float*>(k);
    const dim3 g1((unsigned)(((int64_t)N * N + kThreads - 1) / kThreads), BH);
    err = d == 64 ? launch_kernel(scores_f32<64>, g1, block, 0, stream, Q, K, S, N, ld, scale)
                  : launch_kernel(scores_f32<128>, g1, block, 0, stream, Q, K, S, N, ld, scale);
    if (err != hipSuccess) return err;
    if ((err = launch_softmax<float>(S, (float*)P, lse, B, H, N, ld, causal, kv_limit, stream)) != hipSuccess) return err;
    const float *Pf = static_cast<const float*>(P), *Vf = static_cast<const float*>(v);
    float* Of = static_cast<float*>(o);
    const dim3 g3((unsigned)(((int64_t)N * d + kThreads - 1) / kThreads), BH);
    return d == 64 ? launch_kernel(pv_f32<64>, g3, block, 0, stream, Pf, Vf, Of, N, ld)
                   : launch_kernel(pv_f32<128>, g3, block, 0, stream, Pf, Vf, Of, N, ld);
}

}  // namespace fa

// fa_fwd_f32.hip -- fused exact-attention forward for gfx950, fp32 in/out.
//
// Same method as the bf16 kernel ("GPU 与 TPU：让硬件不再是黑魔法" §11.4; "FlashAttention
// 1–4: How IO-Awareness Reshaped the Attention Kernel", sections "FlashAttention (v1)"
// and "FlashAttention-2"), with both contractions on v_mfma_f32_32x32x2_f32 and
// P kept in fp32.  This path exists for full-precision parity, not throughput:
// one LDS buffer, 32-key tiles, and the plain online recurrence (the reference
// max follows every increase of the row max).
//
// Layout of the contractions (lane l, half = l / 32, col = l % 32):
//   S^T = K Q^T  : A = K[key col][dim 2kk + half] (LDS), B = Q[query col][dim 2kk + half]
//                  (registers); accumulator r of lane l is key 8(r/4) + 4 half + r%4.
//   O^T += V^T P^T: one MFMA per accumulator register r: B = p[r], so hardware k
//                  index `half` stands for key 8(r/4) + 4 half + r%4, and A is V at
//                  that key and dim col of the current 32-dim slab.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace fused_f32 {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kQPW = 32;
constexpr int kBQ = kWaves * kQPW;
constexpr int kBK = 32;

template <int D>
struct Tile {
    static constexpr int kStride = D + 1;  // odd stride: column reads spread over banks
    static constexpr int vStride = D + 4;
};

template <int D, bool CAUSAL, bool MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void fwd_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                float* __restrict__ O, float* __restrict__ LSE, int H, int N, int nqb, float c,
                uint32_t q_and, uint32_t q_xor, const int32_t* __restrict__ kv_limit) {
    using T = Tile<D>;
    __shared__ float Ks[kBK * T::kStride];
    __shared__ float Vs[kBK * T::vStride];
    __shared__ int block_max[kWaves];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
    const int b = bh / H;
    const size_t head = (size_t)bh * N * D;
    const float* Kh = K + head;
    const float* Vh = V + head;

    const int qrow = qb * kBQ + w * kQPW + col;
    const int lim = row_key_limit(qrow, N, CAUSAL, MASK ? kv_limit + (size_t)b * N + qrow : nullptr);
    const int wmax = wave_max_i(lim), wmin = wave_min_i(lim);
    if (lane == 0) block_max[w] = wmax;

    float qf[D / 2];
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
        // the scale's sign folded into Q (see ScoreSign)
        const float x = qrow < N ? Q[head + (size_t)qrow * D + 2 * kk + half] : 0.f;
        qf[kk] = __builtin_bit_cast(float, score_signed(__builtin_bit_cast(uint32_t, x), q_and, q_xor));
    }
    __syncthreads();
    const int kv_end = max(max(block_max[0], block_max[1]), max(block_max[2], block_max[3]));
    const int ntiles = (kv_end + kBK - 1) / kBK;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
    float m_ref = -INFINITY, l_sum = 0.f;

    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = t * kBK;
        __syncthreads();  // previous tile fully consumed
        for (int e = tid; e < kBK * D / 4; e += kThreads) {
            const int row = e / (D / 4), c4 = e % (D / 4);
            const int key = kv0 + row;
            f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (key < N) {
                kx = *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + 4 * c4);
                vx = *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + 4 * c4);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Ks[row * T::kStride + 4 * c4 + i] = kx[i];
                Vs[row * T::vStride + 4 * c4 + i] = vx[i];
            }
        }
        __syncthreads();
        if (kv0 >= wmax) continue;

        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[col * T::kStride + 2 * kk + half], qf[kk], s, 0, 0, 0);
        if (kv0 + kBK > wmin) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (key >= lim) s[r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = halves_max(mx);
        const float mt = mx * c;
        if (__any(mt > m_ref)) {
            const float m_new = fmaxf(m_ref, mt);
            const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            l_sum *= alpha;
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[d32][r] *= alpha;
            m_ref = m_new;
        }
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -m_use));
            l_sum += p[r];
        }
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * half + (r & 3);
                oacc[d32] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * T::vStride + 32 * d32 + col], p[r],
                                                                 oacc[d32], 0, 0, 0);
            }
    }

    const float l_tot = halves_sum(l_sum);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < N) {
        float* orow = O + head + (size_t)qrow * D;
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dim = 32 * d32 + 8 * g + 4 * half;
                f32x4 out = {oacc[d32][4 * g] * inv, oacc[d32][4 * g + 1] * inv, oacc[d32][4 * g + 2] * inv,
                             oacc[d32][4 * g + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + dim) = out;
            }
        if (half == 0)
            LSE[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                  ScoreSign sg, const int32_t* kv_limit, hipStream_t stream) {
    const int nqb = (N + kBQ - 1) / kBQ;
    const dim3 grid((unsigned)((long long)B * H * nqb));
    return launch_kernel(fwd_kernel<D, CAUSAL, MASK>, grid, dim3(kThreads), 0, stream, q, k, v, o, lse, H, N, nqb,
                         sg.c, sg.and_mask, sg.xor_mask, kv_limit);
}

}  // namespace fused_f32

hipError_t launch_fused_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                            int N, int d, bool causal, float scale, const int32_t* kv_limit,
                            hipStream_t stream) {
    using namespace fused_f32;
    const ScoreSign sg = score_sign(scale, kLog2e, kSignF32);
    const bool mask = kv_limit != nullptr;
#define FA_DISPATCH(DD, CC, MM) \
    if (d == DD && causal == CC && mask == MM) return launch<DD, CC, MM>(q, k, v, o, lse, B, H, N, sg, kv_limit, stream);
    FA_DISPATCH(64, false, false)
    FA_DISPATCH(64, false, true)
    FA_DISPATCH(64, true, false)
    FA_DISPATCH(64, true, true)
    FA_DISPATCH(128, false, false)
    FA_DISPATCH(128, false, true)
    FA_DISPATCH(128, true, false)
    FA_DISPATCH(128, true, true)
#undef FA_DISPATCH
    return hipErrorInvalidValue;
}

}  // namespace fa

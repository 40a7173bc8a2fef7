// fa_fwd_bf16.hip -- fused exact-attention forward for gfx950, bf16 in/out.
//
// The method: "GPU 与 TPU：让硬件不再是黑魔法" §11.2-§11.4 and "FlashAttention 1–4:
// How IO-Awareness Reshaped the Attention Kernel", sections "FlashAttention (v1)"
// and "FlashAttention-2".  One workgroup owns one block of query rows of one
// (batch, head); it streams K/V tiles through LDS, keeps the score tile in
// matrix-core accumulators, and carries a running row max m, a running row sum
// l and an unnormalised output accumulator, re-based whenever m moves; O is
// divided by l once at the end and L = m + log l is written per row.  Scores
// never reach device memory.
//
// gfx950 design (not the pages' A100/H100 tiling):
//   * 8 waves x 32 query rows = 256 rows per workgroup, two waves per SIMD
//     (split-Q: each wave owns its rows outright, no cross-wave reduction,
//     "FlashAttention 1–4 ...", section "FlashAttention-2", warp partitioning).
//     Every K/V tile staged in LDS serves 256 queries.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     lane l then holds query (l & 31) and 16 of the 32 keys of a 32-key slab,
//     the other 16 sitting in lane l ^ 32.  Row max and row sum are in-lane
//     reductions plus one exchange between the two lane halves.
//   * O^T = V^T P^T: the exponentiated score accumulators, packed to bf16, are
//     the B operand of the second contraction straight from registers.  V is
//     written into LDS transposed ([dim][key]) with keys permuted so that each
//     lane's 8 keys of a k-step are contiguous (one 16-byte LDS read); the
//     permutation is the accumulator row order of the first contraction.
//   * O accumulates per lane for one query, so the rescale by exp2(m_old - m_new)
//     is a per-lane scalar multiply.  exp2 with log2(e) folded into the scale.
//   * The reference max only moves when a tile's max exceeds it by more than 8
//     (log2 units); O / l is unchanged by the choice of reference and P stays
//     below 2^8 ("FlashAttention 1–4 ...", section "FlashAttention-4",
//     conditional rescaling).  Most tiles skip the O rescale entirely.
//   * K/V tiles are double-buffered in LDS: the next tile's global loads are in
//     flight in registers while the current tile is computed, one barrier per tile.
//   * Causal: tiles past a block's last row are never loaded or computed; a wave
//     whose rows cannot see any key of a tile skips it; element masks are applied
//     only on tiles that cross a wave's smallest key limit (the diagonal, the
//     ragged tail and key padding).  A row that has seen no valid key keeps a
//     finite exponent reference, so -inf - (-inf) is never formed
//     ("07 GPU、资源估算与 FlashAttention" §7.8).
//   * Workgroup order: query-block major, (batch, head) minor, and for causal
//     attention the longest rows first over the whole grid (longest-processing-
//     time-first, "FlashAttention 1–4 ...", section "FlashAttention-4").  With
//     round-robin dispatch over the 8 XCDs, each XCD then sees a fixed subset
//     of heads, and concurrently running workgroups read different heads.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace fused_bf16 {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;  // 512
constexpr int kQPW = 32;                  // query rows per wave
constexpr int kBQ = kWaves * kQPW;        // 256 query rows per workgroup
constexpr int kBK = 64;                   // keys per K/V tile
constexpr int kPad = 8;                   // bf16 padding per LDS row (bank spread)
constexpr float kStaleMax = 8.0f;         // log2 units

template <int D>
struct Tile {
    static constexpr int kStride = D + kPad;   // K: [key][dim] rows
    static constexpr int vStride = kBK + kPad; // V^T: [dim][key position] rows
    static constexpr int kElems = kBK * kStride;
    static constexpr int vElems = D * vStride;
    static constexpr int stageElems = kElems + vElems;
    static constexpr int kChunks = kBK * D / 8;      // 16-byte chunks of a K tile
    static constexpr int kLoads = kChunks / kThreads;
    static constexpr int vUnits = (kBK / 8) * (D / 4); // (key group of 8, 4-dim chunk)
    static_assert(kChunks % kThreads == 0, "K tile must split evenly over the workgroup");
    static_assert(vUnits <= kThreads, "one V unit per thread at most");
};

// Key held at V^T position p: positions 16*ks + 8*g + s (k-step ks, lane half g,
// slot s) carry key 16*ks + 8*(s/4) + 4*g + (s%4), the row order in which the
// 32x32 accumulator of S^T = K Q^T hands keys to lane half g.
__device__ __forceinline__ int group_key(int j, int s) {
    return 16 * (j >> 1) + 4 * (j & 1) + (s < 4 ? s : s + 4);
}

template <int D>
struct Prefetch {
    u32x4 k[Tile<D>::kLoads];
    u32x2 v[8];
};

// Global -> registers for K/V tile starting at key kv0.  Rows past N read as
// zeros through the buffer range check, so no load is predicated.
template <int D>
__device__ __forceinline__ void load_tile(Prefetch<D>& pf, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                          int kv0, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        const int ci = tid + i * kThreads;
        const int row = ci / (D / 8), col8 = ci % (D / 8);
        const uint32_t off = ((uint32_t)(kv0 + row) * D + col8 * 8) * 2u;
        pf.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
    }
    if (tid < T::vUnits) {
        const int j = tid % (kBK / 8), c = tid / (kBK / 8);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t off = ((uint32_t)(kv0 + group_key(j, s)) * D + 4 * c) * 2u;
            pf.v[s] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vr, off, 0, 0));
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const Prefetch<D>& pf, bf16* __restrict__ stage, int tid) {
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        const int ci = tid + i * kThreads;
        const int row = ci / (D / 8), col8 = ci % (D / 8);
        *reinterpret_cast<u32x4*>(stage + row * T::kStride + col8 * 8) = pf.k[i];
    }
    if (tid < T::vUnits) {
        const int j = tid % (kBK / 8), c = tid / (kBK / 8);
        bf16* vt = stage + T::kElems + (4 * c) * T::vStride + 8 * j;
        // 8 keys x 4 dims in registers -> 4 dims x 8 keys in LDS
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u32x4 out;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t a = (e < 2) ? pf.v[2 * p].x : pf.v[2 * p].y;
                const uint32_t b = (e < 2) ? pf.v[2 * p + 1].x : pf.v[2 * p + 1].y;
                out[p] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
            *reinterpret_cast<u32x4*>(vt + e * T::vStride) = out;
        }
    }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                bf16* __restrict__ O, float* __restrict__ LSE,
                int H, int N, int nqb, float c, const int32_t* __restrict__ kv_limit) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * T::stageElems];
    __shared__ int block_max[kWaves];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5, col = lane & 31;

    const int G = gridDim.x, bid = blockIdx.x;
    const int BHn = G / nqb;
    int qb = bid / BHn;
    const int bh = bid - qb * BHn;
    if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first over the whole grid
    const int b = bh / H;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2u;
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(K + head, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(V + head, head_bytes);

    const int q0 = qb * kBQ;
    const int qrow = q0 + w * kQPW + col;
    const int lim = row_key_limit(qrow, N, CAUSAL, MASK ? kv_limit + (size_t)b * N + qrow : nullptr);
    const int wmax = wave_max_i(lim), wmin = wave_min_i(lim);
    if (lane == 0) block_max[w] = wmax;

    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        if (qrow < N)
            qf[kk] = *reinterpret_cast<const bf16x8*>(Q + head + (size_t)qrow * D + 16 * kk + 8 * half);
        else
            qf[kk] = bf16x8{};
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) launder(qf[kk]);
    int kv_end = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) kv_end = max(kv_end, block_max[i]);
    const int ntiles = (kv_end + kBK - 1) / kBK;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
    float m_ref = -INFINITY, l_sum = 0.f;

    Prefetch<D> pf;
    if (ntiles > 0) {
        load_tile<D>(pf, krs, vrs, 0, tid);
        store_tile<D>(pf, smem, tid);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const bool more = t + 1 < ntiles;
        if (more) load_tile<D>(pf, krs, vrs, (t + 1) * kBK, tid);
        const bf16* Ks = smem + (t & 1) * T::stageElems;
        const bf16* Vts = Ks + T::kElems;
        const int kv0 = t * kBK;

        if (kv0 < wmax) {
            // S^T = K Q^T for two 32-key slabs; the two accumulator chains alternate
            f32x16 s[2];
            s[0] = f32x16{};
            s[1] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    const bf16* kp = Ks + (sub * 32 + col) * T::kStride + 8 * half;
                    s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        *reinterpret_cast<const bf16x8*>(kp + 16 * kk), qf[kk], s[sub], 0, 0, 0);
                }
            if (kv0 + kBK > wmin) {  // tile crosses some row's key limit
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                        if (key >= lim) s[sub][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
            mx = halves_max(mx);
            const float mt = mx * c;  // this tile's row max, log2 units
            if (__any(mt > m_ref + kStaleMax)) {
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

            // P = exp2(S c - m), packed to bf16; l sums the same rounded values
            u32x4 pk[4];
            const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int sub = ks >> 1, base = (ks & 1) * 8;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float x0 = __builtin_amdgcn_exp2f(fmaf(s[sub][base + 2 * p], c, -m_use));
                    const float x1 = __builtin_amdgcn_exp2f(fmaf(s[sub][base + 2 * p + 1], c, -m_use));
                    const uint32_t wv = pack_bf16x2(x0, x1);
                    pk[ks][p] = wv;
                    l_sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv), ones, l_sum, false);
                }
            }
            // O^T += V^T P^T; the D/32 accumulator chains alternate
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int d32 = 0; d32 < D / 32; ++d32) {
                    const bf16* vp = Vts + (32 * d32 + col) * T::vStride + 8 * half;
                    oacc[d32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        *reinterpret_cast<const bf16x8*>(vp + 16 * ks), __builtin_bit_cast(bf16x8, pk[ks]),
                        oacc[d32], 0, 0, 0);
                }
        }
        if (more) store_tile<D>(pf, smem + ((t + 1) & 1) * T::stageElems, tid);
        __syncthreads();
    }

    // Epilogue: one division per row; each lane half summed its own keys.
    const float l_tot = halves_sum(l_sum);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < N) {
        bf16* orow = O + head + (size_t)qrow * D;
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dim = 32 * d32 + 8 * g + 4 * half;
                u32x2 out;
                out.x = pack_bf16x2(oacc[d32][4 * g + 0] * inv, oacc[d32][4 * g + 1] * inv);
                out.y = pack_bf16x2(oacc[d32][4 * g + 2] * inv, oacc[d32][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + dim) = out;
            }
        if (half == 0)
            LSE[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const bf16* q, const bf16* k, const bf16* v, bf16* o, float* lse, int B, int H, int N,
                  float c, const int32_t* kv_limit, hipStream_t stream) {
    const int nqb = (N + kBQ - 1) / kBQ;
    const dim3 grid((unsigned)((long long)B * H * nqb));
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, MASK>), grid, dim3(kThreads), 0, stream, q, k, v, o, lse, H, N,
                       nqb, c, kv_limit);
    return hipGetLastError();
}

}  // namespace fused_bf16

hipError_t launch_fused_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                             int N, int d, bool causal, float scale, const int32_t* kv_limit,
                             hipStream_t stream) {
    using namespace fused_bf16;
    const bf16* Q = static_cast<const bf16*>(q);
    const bf16* K = static_cast<const bf16*>(k);
    const bf16* V = static_cast<const bf16*>(v);
    bf16* Ot = static_cast<bf16*>(o);
    const float c = scale * kLog2e;
    const bool mask = kv_limit != nullptr;
#define FA_DISPATCH(DD, CC, MM) \
    if (d == DD && causal == CC && mask == MM) return launch<DD, CC, MM>(Q, K, V, Ot, lse, B, H, N, c, kv_limit, stream);
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

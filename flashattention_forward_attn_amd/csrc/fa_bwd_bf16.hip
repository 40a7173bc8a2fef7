// fa_bwd_bf16.hip -- backward pass of the fused attention for gfx950, bf16 in/out.
//
// The method: the backward pass recomputes the scores and P = exp(S - L) tile by
// tile from the saved Q, K, V, O and the per-row log-sum-exp L, with no online
// softmax ("GPU 与 TPU：让硬件不再是黑魔法" §11.5, part 3; "FlashAttention 1–4: How
// IO-Awareness Reshaped the Attention Kernel", section "FlashAttention-2", where
// one thread block owns one K/V column block and accumulates its dK and dV
// locally).  With dO the gradient of the output and D_i = <dO_i, O_i>:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels on the caller's stream:
//   1. rows:  D_i and the base-2 log-sum-exp L2_i = L_i log2(e) (+inf for a row
//      with no valid key, so that its P is exactly 0), into the workspace.
//   2. dK/dV: one workgroup per 128 keys of one (batch, head), eight waves: per
//      32 keys a score wave and a gradient wave on one SIMD.  Q and dO tiles of 32
//      queries, with their L2 and D values, stream through LDS by direct buffer
//      loads issued two tiles ahead.  Per tile, lane = key:
//        score wave:    S = Q K^T and dP = dO V^T (B operands K and V held in
//                       registers), P = exp2(S c - L2), dS = P (dP - D), packed
//                       to bf16 and handed over through LDS;
//        gradient wave: one tile later, dV^T += dO^T P and dK^T += Q^T dS (A
//                       operands by transposing LDS reads).
//   3. dQ: one workgroup per 256 queries, one wave per 32 queries; K/V tiles stream
//      through LDS as in the forward kernel.  Lane = query:
//        S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// The pages' FA2 design adds into dQ with atomics from the column pass; here dQ
// has its own pass instead, so every result is deterministic, at the cost of
// computing S and dP twice.
#include "fa_common.h"
#include "fa_launch.h"
#include "fa_epilogue.h"
#include "fa_tile.h"

namespace fa {
namespace bwd {

// ---------------------------------------------------------------- 1. row statistics
constexpr int kRowThreads = 256;

template <int D>
__global__ __launch_bounds__(kRowThreads) void rows_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                           const float* __restrict__ LSE, float* __restrict__ Dd,
                                                           float* __restrict__ L2, long long rows) {
    constexpr int E = D / 16;  // bf16 per lane, 16 lanes per row
    const long long t = (long long)blockIdx.x * kRowThreads + threadIdx.x;
    const long long row = t / 16;
    const int part = (int)(t % 16);
    float acc = 0.f;
    if (row < rows) {
        const bf16* o = O + row * D + part * E;
        const bf16* g = dO + row * D + part * E;
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (part == 0 && row < rows) {
        Dd[row] = acc;
        const float l = LSE[row];
        L2[row] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
}

// ---------------------------------------------------------------- 2. dK and dV
namespace kv {
// Two roles per SIMD.  Wave p (p < 4, "score wave") and wave p + 4 ("gradient
// wave") share a SIMD and own the same 32 keys.  The score wave holds K and V of
// its keys as MFMA operands and turns a 32-query tile into P and dS; the
// gradient wave holds the dK and dV accumulators and consumes that tile's P and
// dS one iteration later.  Each wave needs only its role's registers, so two
// fit per SIMD, and one wave's exponentials and conversions overlap the other's
// matrix products.
constexpr int kPairs = 4;
constexpr int kWaves = 2 * kPairs;
constexpr int kThreads = kWaves * kWave;
constexpr int kKPW = 32;                 // keys per wave pair
constexpr int kBKV = kPairs * kKPW;      // 128 keys per workgroup
constexpr int kBQ = 32;                  // queries per streamed tile
constexpr int kStages = 4;               // tile t+2 loads while t (scores) and t-1 (gradients) are read

template <int D>
struct Tile {
    static constexpr int kRow = D * 2;
    static constexpr int kBytes = kBQ * kRow;                // one Q or dO tile
    static constexpr int kStatSlot = kWave * 4;              // one 4-byte-per-lane load
    static constexpr int kStage = 2 * kBytes + 1024;         // Q, dO, then L2, D, key limit slots
    static constexpr int kHand = 4 * kWave * 16;             // P and dS of one pair: 2 + 2 16-byte loads
    static constexpr int kHandOff = kStages * kStage;
    static constexpr int kSmem = kHandOff + 2 * kPairs * kHand;
    static constexpr int kTileBlocks = kBytes / kDmaBytes;   // loads per tensor tile
    static constexpr int kPerWave = 2 * kTileBlocks / kWaves;
    static_assert((2 * kTileBlocks) % kWaves == 0, "Q and dO tiles must split evenly over the waves");
    static_assert(3 * kStatSlot <= 1024, "stats fit their slots");
};

template <int D, bool CAUSAL, bool MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
            const bf16* __restrict__ dO, const float* __restrict__ Dd, const float* __restrict__ L2,
            bf16* __restrict__ dK, bf16* __restrict__ dV, int H, int N, int nkb, float c, float scale,
            uint32_t s_and, uint32_t s_xor, const int32_t* __restrict__ kv_limit) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(1024))) char smem[T::kSmem];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = w & (kPairs - 1);
    const bool scorer = w < kPairs;
    const int half = lane >> 5, col = lane & 31;

    // Key blocks in ascending order: for causal attention the first blocks see
    // the most queries, so the longest work starts first.
    const int BHn = gridDim.x / nkb;
    const int kb = blockIdx.x / BHn;
    const int bh = blockIdx.x - kb * BHn;
    const int b = bh / H;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2u;
    const int k0 = kb * kBKV;
    const int kw0 = k0 + pair * kKPW;        // first key of this wave pair
    const int kcol = kw0 + col;               // this lane's key

    // A key block that no row can see (every row's key limit at or below its
    // first key, as with key padding past a sequence's length) has zero
    // gradients: store them without streaming any query tile.
    if constexpr (MASK) {
        __shared__ int row_limit_max[kWaves];
        int m = 0;
        for (int i = tid; i < N; i += kThreads)
            m = max(m, row_key_limit(i, N, CAUSAL, kv_limit + (size_t)b * N + i));
        m = wave_max_i(m);
        if (lane == 0) row_limit_max[w] = m;
        __syncthreads();
        int seen = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) seen = max(seen, row_limit_max[i]);
        if (seen <= k0) {
            constexpr int kChunks = D / 8;  // 16-byte pieces of a row
            for (int e = tid; e < kBKV * kChunks; e += kThreads) {
                const int key = k0 + e / kChunks;
                if (key < N) {
                    const size_t off = head + (size_t)key * D + 8 * (e % kChunks);
                    *reinterpret_cast<u32x4*>(dK + off) = u32x4{};
                    *reinterpret_cast<u32x4*>(dV + off) = u32x4{};
                }
            }
            return;
        }
    }

    // Direct loads: block g = i * kWaves + w of the stage's Q tile (g < kTileBlocks)
    // or dO tile; lane l's 16 bytes land at LDS position 16 l of the block.
    uint32_t dma_src[T::kPerWave], dma_dst[T::kPerWave];
    bool dma_g[T::kPerWave];
#pragma unroll
    for (int i = 0; i < T::kPerWave; ++i) {
        const int g = i * kWaves + w;
        dma_g[i] = g >= T::kTileBlocks;
        const int blk = dma_g[i] ? g - T::kTileBlocks : g;
        const int p = blk * kDmaBytes + 16 * lane;
        const int row = p / T::kRow, slot = (p % T::kRow) / 16;
        dma_src[i] = (uint32_t)(row * T::kRow + 16 * (slot ^ swz<D>(row)));
        dma_dst[i] = (uint32_t)(dma_g[i] ? T::kBytes : 0) + blk * kDmaBytes;
    }
    const i32x4 qdesc = dma_desc(Q + head, head_bytes), gdesc = dma_desc(dO + head, head_bytes);
    const i32x4 ldesc = dma_desc(L2 + (size_t)bh * N, (uint32_t)N * 4u);
    const i32x4 ddesc = dma_desc(Dd + (size_t)bh * N, (uint32_t)N * 4u);
    const i32x4 mdesc = dma_desc(MASK ? kv_limit + (size_t)b * N : kv_limit, MASK ? (uint32_t)N * 4u : 0u);
    auto dma_tile = [&](int stage, int q0) __attribute__((always_inline)) {
        const uint32_t base = (uint32_t)q0 * T::kRow;
        const uint32_t st = lds_addr(smem + stage * T::kStage);
#pragma unroll
        for (int i = 0; i < T::kPerWave; ++i) dma16(dma_g[i] ? gdesc : qdesc, st + dma_dst[i], base + dma_src[i]);
        const uint32_t soff = (uint32_t)(q0 + lane) * 4u;
        if (w == 0) dma4(ldesc, st + 2 * T::kBytes, soff);
        if (w == 1) dma4(ddesc, st + 2 * T::kBytes + T::kStatSlot, soff);
        if (MASK && w == 2) dma4(mdesc, st + 2 * T::kBytes + 2 * T::kStatSlot, soff);
    };

    // Queries before this block's first key see none of its keys (causal).
    const int q_first = CAUSAL ? k0 : 0;
    const int ntiles = (N - q_first + kBQ - 1) / kBQ;
    // every query of tile u precedes every key of this pair
    auto skipped = [&](int u) __attribute__((always_inline)) {
        return CAUSAL && q_first + u * kBQ + kBQ - 1 < kw0;
    };
    char* const hand0 = smem + T::kHandOff + pair * T::kHand;

    const bool stat_wave = w == 0 || w == 1 || (MASK && w == 2);
    auto wait_next = [&](bool more) __attribute__((always_inline)) {
        if (!more) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (stat_wave) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(T::kPerWave + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(T::kPerWave) : "memory");
    };
    dma_tile(0, q_first);
    if (ntiles > 1) dma_tile(1, q_first + kBQ);
    wait_next(ntiles > 1);
    __syncthreads();

    if (scorer) {
        // K and V rows of this lane's key, as B operands (k = 8 dims per lane half)
        bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            if (kcol < N) {
                // the scale's sign folded into K, the scores' register operand (see ScoreSign)
                u32x4 u = *reinterpret_cast<const u32x4*>(K + head + (size_t)kcol * D + 16 * kk + 8 * half);
#pragma unroll
                for (int e = 0; e < 4; ++e) u[e] = score_signed(u[e], s_and, s_xor);
                kf[kk] = __builtin_bit_cast(bf16x8, u);
                vf[kk] = *reinterpret_cast<const bf16x8*>(V + head + (size_t)kcol * D + 16 * kk + 8 * half);
            } else {
                kf[kk] = bf16x8{};
                vf[kk] = bf16x8{};
            }
        }
        // The loads above complete here, so the loop carries no wait on the memory
        // counter, which also counts the tile loads in flight.
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            launder(kf[kk]);
            launder(vf[kk]);
        }
        // Row-major reads (A of S = Q K^T and dP = dO V^T): query row col, chunk 2 kk + half.
        int koff[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) koff[kk] = col * T::kRow + 16 * ((2 * kk + half) ^ swz<D>(col));

        int st = 0;
        for (int t = 0; t <= ntiles; ++t) {
            const int nst = st == kStages - 1 ? 0 : st + 1;
            if (t + 2 < ntiles) dma_tile((st + 2) & 3, q_first + (t + 2) * kBQ);
            if (t < ntiles && !skipped(t)) {
                const int qc0 = q_first + t * kBQ;
                const char* Qc = smem + st * T::kStage;
                const char* Gc = Qc + T::kBytes;
                const float* Ls = reinterpret_cast<const float*>(Qc + 2 * T::kBytes);
                const float* Ds = reinterpret_cast<const float*>(Qc + 2 * T::kBytes + T::kStatSlot);
                const int* Ms = reinterpret_cast<const int*>(Qc + 2 * T::kBytes + 2 * T::kStatSlot);

                // All operand reads first, then the two product chains interleaved; the
                // score wave's products go ahead of its partner's so that its
                // exponentials overlap the partner's products.
                bf16x8 qa[D / 16], ga[D / 16];
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    qa[kk] = *reinterpret_cast<const bf16x8*>(Qc + koff[kk]);
                    ga[kk] = *reinterpret_cast<const bf16x8*>(Gc + koff[kk]);
                }
                f32x16 s = f32x16{}, dp = f32x16{};
                // (the priority changes are tied to the products' operands and results
                // so that the scheduler keeps the products between them)
                asm volatile("s_setprio 2" : "+v"(kf[0]), "+v"(vf[0]));
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], kf[kk], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[kk], vf[kk], dp, 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16), 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 16), 0);  // products
                asm volatile("s_setprio 0" :: "v"(s[15]), "v"(dp[15]));
                // accumulator r holds query qc0 + 8 (r / 4) + 4 half + r % 4 of this lane's key
                float l2r[16], ddr[16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rq = 8 * i + 4 * half;
                    const f32x4 lv = *reinterpret_cast<const f32x4*>(Ls + rq);
                    const f32x4 dv4 = *reinterpret_cast<const f32x4*>(Ds + rq);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        l2r[4 * i + e] = lv[e];
                        ddr[4 * i + e] = dv4[e];
                    }
                }
                if (MASK) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const u32x4 mv = *reinterpret_cast<const u32x4*>(Ms + 8 * i + 4 * half);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (kcol >= (int)mv[e]) s[4 * i + e] = -INFINITY;
                    }
                }
                if (CAUSAL && qc0 < kw0 + kKPW - 1) {  // tile crosses this pair's diagonal
                    const int rel = kcol - qc0 - 4 * half;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) < rel) s[r] = -INFINITY;
                }

                char* hand = hand0 + (t & 1) * kPairs * T::kHand;
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    u32x4 pk, dsk;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r0 = 8 * kh + 2 * q, r1 = r0 + 1;
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r0], c, -l2r[r0]));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r1], c, -l2r[r1]));
                        pk[q] = pack_bf16x2(p0, p1);
                        dsk[q] = pack_bf16x2(p0 * (dp[r0] - ddr[r0]), p1 * (dp[r1] - ddr[r1]));
                    }
                    *reinterpret_cast<u32x4*>(hand + kh * kDmaBytes + 16 * lane) = pk;
                    *reinterpret_cast<u32x4*>(hand + (2 + kh) * kDmaBytes + 16 * lane) = dsk;
                }
            }
            wait_next(t + 2 < ntiles);
            __syncthreads();
            st = nst;
        }
        return;
    }

    // Gradient wave.  Transposing reads (A of dV^T = dO^T P and dK^T = Q^T dS): lane
    // 16 G + j addresses query 8 hs + 4 (G / 2) + j / 4 at dims
    // 32 d32 + 16 (G % 2) + 4 (j % 4) .. +3.
    int voff[D / 32][2];
    {
        const int G4 = lane >> 4, j = lane & 15;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int row = 8 * hs + 4 * (G4 >> 1) + (j >> 2);
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32) {
                const int dim = 32 * d32 + 16 * (G4 & 1) + 4 * (j & 3);
                voff[d32][hs] = row * T::kRow + 16 * ((dim >> 3) ^ swz<D>(row)) + 2 * (dim & 7);
            }
        }
    }

    f32x16 dvacc[D / 32], dkacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        dvacc[i] = f32x16{};
        dkacc[i] = f32x16{};
    }

    int st = 0, pst = kStages - 1;  // stage of tile t, and of tile t - 1
    for (int t = 0; t <= ntiles; ++t) {
        const int nst = st == kStages - 1 ? 0 : st + 1;
        if (t + 2 < ntiles) dma_tile((st + 2) & 3, q_first + (t + 2) * kBQ);
        if (t > 0 && !skipped(t - 1)) {
            const char* Qc = smem + pst * T::kStage;
            const char* Gc = Qc + T::kBytes;
            const char* hand = hand0 + ((t - 1) & 1) * kPairs * T::kHand;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const u32x4 pk = *reinterpret_cast<const u32x4*>(hand + kh * kDmaBytes + 16 * lane);
#pragma unroll
                for (int d32 = 0; d32 < D / 32; ++d32) {
                    const u32x2 lo = tr_read(Gc + 16 * kh * T::kRow + voff[d32][0]);
                    const u32x2 hi = tr_read(Gc + 16 * kh * T::kRow + voff[d32][1]);
                    const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                    dvacc[d32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pk), dvacc[d32], 0, 0, 0);
                }
            }
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const u32x4 dsk = *reinterpret_cast<const u32x4*>(hand + (2 + kh) * kDmaBytes + 16 * lane);
#pragma unroll
                for (int d32 = 0; d32 < D / 32; ++d32) {
                    const u32x2 lo = tr_read(Qc + 16 * kh * T::kRow + voff[d32][0]);
                    const u32x2 hi = tr_read(Qc + 16 * kh * T::kRow + voff[d32][1]);
                    const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                    dkacc[d32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, dsk), dkacc[d32], 0, 0, 0);
                }
            }
        }
        wait_next(t + 2 < ntiles);
        __syncthreads();
        pst = st;
        st = nst;
    }

    // Epilogue: lane holds key kcol, dims 32 d32 + 8 g + 4 half .. +3 in registers 4 g ..;
    // dK and dV leave in 16-byte stores (8 consecutive dims per lane, see o_rows16)
    u32x4 ko[D / 32][2], vo[D / 32][2];
#pragma unroll
    for (int d32 = 0; d32 < D / 32; ++d32) {
        o_rows16(dkacc[d32], scale, ko[d32]);
        o_rows16(dvacc[d32], 1.0f, vo[d32]);
    }
    if (kcol < N) {
        bf16* krow = dK + head + (size_t)kcol * D;
        bf16* vrow = dV + head + (size_t)kcol * D;
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                *reinterpret_cast<u32x4*>(krow + 32 * d32 + 16 * p + 8 * half) = ko[d32][p];
                *reinterpret_cast<u32x4*>(vrow + 32 * d32 + 16 * p + 8 * half) = vo[d32][p];
            }
    }
}
}  // namespace kv

// ---------------------------------------------------------------- 3. dQ
namespace qd {
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kQPW = 32;
constexpr int kBQ = kWaves * kQPW;  // 256 queries per workgroup
constexpr int kBK = 64;             // keys per streamed K/V tile

template <int D>
struct Tile {
    static constexpr int kRow = D * 2;
    static constexpr int kBytes = kBK * kRow;
    static constexpr int kStage = 2 * kBytes;  // K tile then V tile
    static constexpr int kBlocks = kBytes / kDmaBytes;
    static constexpr int kPerWave = kBlocks / kWaves;
    static_assert(kBlocks % kWaves == 0, "tile must split evenly over the waves");
};

// At d = 64 the kernel fits in 128 registers, so two workgroups share a CU
// (four waves per SIMD); at d = 128 it needs two waves' worth.
template <int D, bool CAUSAL, bool MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(D == 64 ? 4 : 2, D == 64 ? 4 : 2)))
void kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
            const bf16* __restrict__ dO, const float* __restrict__ Dd, const float* __restrict__ L2,
            bf16* __restrict__ dQ, int H, int N, int nqb, float c, float scale, uint32_t s_and, uint32_t s_xor,
            const int32_t* __restrict__ kv_limit) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::kStage];
    __shared__ int block_max[kWaves];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;

    const int BHn = gridDim.x / nqb;
    int qb = blockIdx.x / BHn;
    const int bh = blockIdx.x - qb * BHn;
    if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
    const int b = bh / H;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2u;

    uint32_t dma_off[T::kPerWave];
#pragma unroll
    for (int i = 0; i < T::kPerWave; ++i) {
        const int p = (i * kWaves + w) * kDmaBytes + 16 * lane;
        const int row = p / T::kRow, slot = (p % T::kRow) / 16;
        dma_off[i] = (uint32_t)(row * T::kRow + 16 * (slot ^ swz<D>(row)));
    }
    const i32x4 kdesc = dma_desc(K + head, head_bytes), vdesc = dma_desc(V + head, head_bytes);
    auto dma_tile = [&](int stage, int kv0) {
        const uint32_t base = (uint32_t)kv0 * T::kRow;
#pragma unroll
        for (int i = 0; i < T::kPerWave; ++i) {
            const uint32_t kd = lds_addr(smem + stage * T::kStage + (i * kWaves + w) * kDmaBytes);
            dma16(kdesc, kd, base + dma_off[i]);
            dma16(vdesc, kd + T::kBytes, base + dma_off[i]);
        }
    };

    // With key limits, the row's limit (which the first barrier needs) goes out
    // first: loads complete in order, so the wait before the barrier covers it
    // alone.  Q, dO and the row statistics follow; they stay in flight across that
    // barrier and land together with the first K/V tile.  All go through buffer
    // descriptors, rows past N at an offset past the end (they read zeros), so no
    // load sits in a branch and none waits for another.
    const int qrow = qb * kBQ + w * kQPW + col;
    const bool in = qrow < N;
    int lraw = 0;  // the stored key limit of this row
    if constexpr (MASK)
        lraw = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(kv_limit + (size_t)b * N, (uint32_t)N * 4u),
                                                    in ? qrow * 4 : N * 4, 0, 0);
    const auto qrs = buffer_rsrc(Q + head, head_bytes), grs = buffer_rsrc(dO + head, head_bytes);
    const uint32_t roff = ((uint32_t)qrow * D + 8 * half) * 2u;
    u32x4 qraw[D / 16], graw[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const uint32_t off = in ? roff + 32 * kk : head_bytes;
        qraw[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
        graw[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0));
    }
    const int soff = in ? qrow * 4 : N * 4;
    const float l2_in = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(L2 + (size_t)bh * N, (uint32_t)N * 4u), soff, 0, 0));
    const float dd = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(Dd + (size_t)bh * N, (uint32_t)N * 4u), soff, 0, 0));
    const int lim = row_key_limit(qrow, N, CAUSAL, MASK ? &lraw : nullptr);
    const int wmax = __builtin_amdgcn_readfirstlane(wave_max_i(lim));
    const int wmin = __builtin_amdgcn_readfirstlane(wave_min_i(lim));
    if (lane == 0) block_max[w] = wmax;
    // every wave's block_max entry is written; LDS only (a full __syncthreads
    // would first wait for the loads above)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int kv_end = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) kv_end = max(kv_end, block_max[i]);
    kv_end = __builtin_amdgcn_readfirstlane(kv_end);
    const int ntiles = (kv_end + kBK - 1) / kBK;

    // Row-major reads of K and V (A of S^T = K Q^T and dP^T = V dO^T): key col of a
    // 32-key slab, chunk 2 kk + half.  Transposing reads of K (A of dQ^T = K^T dS^T):
    // lane 16 G + j addresses key 8 hs + 4 (G / 2) + j / 4 at dims
    // 32 d32 + 16 (G % 2) + 4 (j % 4) .. +3.
    int koff[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) koff[kk] = col * T::kRow + 16 * ((2 * kk + half) ^ swz<D>(col));
    int voff[D / 32][2];
    {
        const int G4 = lane >> 4, j = lane & 15;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int key = 8 * hs + 4 * (G4 >> 1) + (j >> 2);
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32) {
                const int dim = 32 * d32 + 16 * (G4 & 1) + 4 * (j & 3);
                voff[d32][hs] = key * T::kRow + 16 * ((dim >> 3) ^ swz<D>(key)) + 2 * (dim & 7);
            }
        }
    }

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{};

    if (ntiles > 0) dma_tile(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the scale's sign folded into Q, the scores' register operand (see ScoreSign)
    bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 u = qraw[kk];
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = score_signed(u[e], s_and, s_xor);
        qf[kk] = __builtin_bit_cast(bf16x8, u);
        gf[kk] = __builtin_bit_cast(bf16x8, graw[kk]);
        launder(qf[kk]);
        launder(gf[kk]);
    }
    const float l2 = in ? l2_in : INFINITY;  // a row past N sees no key
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int st = t & 1;
        if (t + 1 < ntiles) dma_tile(st ^ 1, (t + 1) * kBK);
        const char* Ks = smem + st * T::kStage;
        const char* Vs = Ks + T::kBytes;
        const int kv0 = t * kBK;
        if (kv0 < wmax) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const char* Kc = Ks + 32 * sub * T::kRow;
                const char* Vc = Vs + 32 * sub * T::kRow;
                f32x16 s = f32x16{}, dp = f32x16{};
                // the S and dP chains alternate: 1-5 % faster than the two chains back
                // to back (an explicit schedule of the operand reads gained nothing more)
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(Kc + koff[kk]),
                                                                qf[kk], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(Vc + koff[kk]),
                                                                 gf[kk], dp, 0, 0, 0);
                }
                // accumulator r holds key kv0 + 32 sub + 8 (r / 4) + 4 half + r % 4 of this lane's query
                if (kv0 + 32 * sub + 32 > wmin) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * sub + 8 * (r >> 2) + 4 * half + (r & 3);
                        if (key >= lim) s[r] = -INFINITY;
                    }
                }
                u32x4 dsk[2];
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r0 = 8 * kh + 2 * q, r1 = r0 + 1;
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r0], c, -l2));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r1], c, -l2));
                        dsk[kh][q] = pack_bf16x2(p0 * (dp[r0] - dd), p1 * (dp[r1] - dd));
                    }
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int d32 = 0; d32 < D / 32; ++d32) {
                        const u32x2 lo = tr_read(Kc + 16 * kh * T::kRow + voff[d32][0]);
                        const u32x2 hi = tr_read(Kc + 16 * kh * T::kRow + voff[d32][1]);
                        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                        dqacc[d32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, dsk[kh]), dqacc[d32], 0, 0, 0);
                    }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // dQ leaves in 16-byte stores (8 consecutive dims per lane, see o_rows16)
    u32x4 qo[D / 32][2];
#pragma unroll
    for (int d32 = 0; d32 < D / 32; ++d32) o_rows16(dqacc[d32], scale, qo[d32]);
    if (qrow < N) {
        bf16* row = dQ + head + (size_t)qrow * D;
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
            for (int p = 0; p < 2; ++p) *reinterpret_cast<u32x4*>(row + 32 * d32 + 16 * p + 8 * half) = qo[d32][p];
    }
}
}  // namespace qd

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const bf16* q, const bf16* k, const bf16* v, const bf16* o, const bf16* g, const float* lse,
                  bf16* dq, bf16* dk, bf16* dv, int B, int H, int N, float scale, const int32_t* kv_limit,
                  float* Dd, float* L2, hipStream_t stream) {
    const long long rows = (long long)B * H * N;
    hipError_t e = launch_kernel(rows_kernel<D>, dim3((unsigned)((rows * 16 + kRowThreads - 1) / kRowThreads)),
                                 dim3(kRowThreads), 0, stream, o, g, lse, Dd, L2, rows);
    if (e != hipSuccess) return e;
    // scores use |scale| (or log2(e) at scale 0) with the sign folded into their
    // register operand; the gradients dQ = scale dS K and dK = scale dS^T Q keep the scale
    const ScoreSign sg = score_sign(scale, kLog2e, kSignBf16x2);
    const int nkb = (N + kv::kBKV - 1) / kv::kBKV;
    e = launch_kernel(kv::kernel<D, CAUSAL, MASK>, dim3((unsigned)((long long)B * H * nkb)), dim3(kv::kThreads), 0,
                      stream, q, k, v, g, Dd, L2, dk, dv, H, N, nkb, sg.c, scale, sg.and_mask, sg.xor_mask, kv_limit);
    if (e != hipSuccess) return e;
    const int nqb = (N + qd::kBQ - 1) / qd::kBQ;
    return launch_kernel(qd::kernel<D, CAUSAL, MASK>, dim3((unsigned)((long long)B * H * nqb)), dim3(qd::kThreads), 0,
                         stream, q, k, v, g, Dd, L2, dq, H, N, nqb, sg.c, scale, sg.and_mask, sg.xor_mask, kv_limit);
}

}  // namespace bwd

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, bool causal,
                           float scale, const int32_t* kv_limit, float* workspace, hipStream_t stream) {
    const bf16* Q = static_cast<const bf16*>(q);
    const bf16* K = static_cast<const bf16*>(k);
    const bf16* V = static_cast<const bf16*>(v);
    const bf16* Ob = static_cast<const bf16*>(o);
    const bf16* G = static_cast<const bf16*>(dout);
    bf16* dQ = static_cast<bf16*>(dq);
    bf16* dK = static_cast<bf16*>(dk);
    bf16* dV = static_cast<bf16*>(dv);
    float* Dd = workspace;
    float* L2 = workspace + bwd_stats_floats(B, H, N);
    const bool mask = kv_limit != nullptr;
#define FA_DISPATCH(DD, CC, MM)                                                                                    \
    if (d == DD && causal == CC && mask == MM)                                                                     \
        return bwd::launch<DD, CC, MM>(Q, K, V, Ob, G, lse, dQ, dK, dV, B, H, N, scale, kv_limit, Dd, L2, stream);
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

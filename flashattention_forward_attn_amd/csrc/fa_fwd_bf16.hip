// fa_fwd_bf16.hip -- fused exact-attention forward for gfx950, bf16 in/out.
//
// The method: "GPU 与 TPU：让硬件不再是黑魔法" §11.2-§11.4 and "FlashAttention 1–4:
// How IO-Awareness Reshaped the Attention Kernel", sections "FlashAttention (v1)"
// and "FlashAttention-2".  A workgroup owns one block of query rows of one
// (batch, head) at a time; it streams K/V tiles through LDS, keeps the score tile in
// matrix-core accumulators, and carries an exponent reference m, a running row
// sum l and an unnormalised output accumulator; O is divided by l once at the
// end and L = m + log l is written per row.  Scores never reach device memory.
//
// gfx950 design (not the pages' A100/H100 tiling):
//   * 8 waves x 32 query rows = 256 rows per query block, two waves per SIMD
//     (split-Q: each wave owns its rows outright, no cross-wave reduction,
//     "FlashAttention 1–4 ...", section "FlashAttention-2", warp partitioning).
//     Every K/V tile staged in LDS serves 256 queries.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     lane l then holds query (l & 31) and 16 of the 32 keys of a 32-key slab,
//     the other 16 sitting in lane l ^ 32.  Row max and row sum are in-lane
//     reductions plus one exchange between the two lane halves.
//   * O^T = V^T P^T: the exponentiated score accumulators, packed to bf16, are
//     the B operand of the second contraction straight from registers.  V stays
//     row-major in LDS; its A operand is read with ds_read_b64_tr_b16, which
//     transposes 4x4 blocks of 16-bit values across lanes, and the per-lane source
//     addresses pick the keys in the accumulator row order of the first
//     contraction, so no data is permuted anywhere.
//   * exp2 with log2(e) folded into the scale.  O / l does not depend on the
//     exponent reference ("FlashAttention 1–4 ...", section "FlashAttention-4",
//     conditional rescaling).  Without key limits each row keeps the max of its
//     first tile as its reference: no later tile computes a row max, votes or
//     rescales O.  P then exceeds 1 when later scores are larger; a score 128 or
//     more (log2 units) above the reference overflows P (and a smaller excess can
//     overflow O for huge V), which leaves a non-finite sum or output.  The
//     workgroup checks for that after a block and then computes the block again
//     with the reference following the running max: moved when a tile's max
//     exceeds it by more than 8, so P stays below 2^8, and O rescaled by a
//     per-lane scalar (O accumulates per lane for one query).  With key limits
//     the reference follows the running max from the start.
//   * K/V tiles go from global memory straight into LDS (buffer loads with the
//     LDS bit, 16 bytes per lane, no register staging), double-buffered: the next
//     tile is in flight while the current one is computed, one barrier per tile.
//     The 16-byte chunks of each key row are XOR-swizzled by key so that both the
//     K operand reads (16 keys, one chunk) and the transposing V reads (4 keys, 4
//     chunks) hit distinct LDS banks.
//   * Causal: tiles past a block's last row are never loaded or computed; a wave
//     whose rows cannot see any key of a tile skips it; element masks are applied
//     only on tiles that cross a wave's smallest key limit (the diagonal, the
//     ragged tail and key padding).  A row that has seen no valid key keeps a
//     finite exponent reference, so -inf - (-inf) is never formed
//     ("07 GPU、资源估算与 FlashAttention" §7.8).
//   * Work order: query-block major, (batch, head) minor, and for causal
//     attention the longest rows first (longest-processing-time-first,
//     "FlashAttention 1–4 ...", section "FlashAttention-4").  Without a key
//     limit one workgroup per CU walks the blocks: block g of every even round
//     and the mirror image of g of every odd round, which evens out causal work
//     (a long block pairs with a short one) and saves a workgroup launch and
//     wind-down per block.  The mirror keeps g's residue mod 8, so with round-
//     robin dispatch over the 8 XCDs each XCD still sees a fixed subset of
//     heads.  With a key limit block lengths depend on the data, so every block
//     gets its own workgroup and the hardware balances them.
#include "fa_common.h"
#include "fa_launch.h"
#include "fa_epilogue.h"
#include "fa_tile.h"

namespace fa {
namespace fused_bf16 {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;  // 512
constexpr int kQPW = 32;                  // query rows per wave
constexpr int kBQ = kWaves * kQPW;        // 256 query rows per query block
// Keys per K/V tile: 128 at d = 64 (half the barriers per key; the tile fits
// the registers there), 64 at d = 128.
template <int D>
constexpr int kBKof = D == 64 ? 128 : 64;
constexpr float kStaleMax = 8.0f;         // log2 units (the recomputation pass moves its reference past this)

template <int D>
struct Tile {
    static constexpr int kRow = D * 2;              // bytes per key row
    static constexpr int kBK = kBKof<D>;
    static constexpr int kBytes = kBK * kRow;       // one K or V tile
    static constexpr int kStage = 2 * kBytes;       // K tile then V tile
    static constexpr int kBlocks = kBytes / kDmaBytes;
    static constexpr int kPerWave = kBlocks / kWaves;
    static_assert(kBlocks % kWaves == 0, "tile must split evenly over the waves");
};


template <int D, bool CAUSAL, bool MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                bf16* __restrict__ O, float* __restrict__ LSE,
                int H, int N, int nqb, int items, float c, uint32_t q_and, uint32_t q_xor,
                const int32_t* __restrict__ kv_limit) {
    using T = Tile<D>;
    constexpr int kBK = T::kBK;
    constexpr int kSub = kBK / 32;  // 32-key slabs per tile
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::kStage];
    __shared__ int block_max[2][kWaves];
    __shared__ int redo_flag[2][kWaves];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int P = gridDim.x, g = blockIdx.x;
    const int BHn = items / nqb;
    const uint32_t head_bytes = (uint32_t)N * D * 2u;

    // Item i is query block i / BHn of (batch, head) i mod BHn, the longest rows
    // first for causal attention; the grid walks the items with walk_block.
    struct Item {
        int bh, q0;
    };
    auto decode = [&](int it) -> Item {
        int qb = it / BHn;
        const int bh = it - qb * BHn;
        if (CAUSAL) qb = nqb - 1 - qb;
        return {bh, qb * kBQ};
    };

    // Global offset (relative to the tile's first key) each lane fetches for its DMA blocks.
    uint32_t dma_off[T::kPerWave];
#pragma unroll
    for (int i = 0; i < T::kPerWave; ++i) {
        const int p = (i * kWaves + w) * kDmaBytes + 16 * lane;
        const int row = p / T::kRow, slot = (p % T::kRow) / 16;
        dma_off[i] = (uint32_t)(row * T::kRow + 16 * (slot ^ swz<D>(row)));
    }
    // K/V tiles go to LDS with direct buffer loads (reads past N return zeros).
    auto dma_tile = [&](const i32x4& kdesc, const i32x4& vdesc, int stage, int kv0) __attribute__((always_inline)) {
        const uint32_t base = (uint32_t)kv0 * T::kRow;
#pragma unroll
        for (int i = 0; i < T::kPerWave; ++i) {
            const uint32_t kd = lds_addr(smem + stage * T::kStage + (i * kWaves + w) * kDmaBytes);
            dma16(kdesc, kd, base + dma_off[i]);
            dma16(vdesc, kd + T::kBytes, base + dma_off[i]);
        }
    };

    // LDS byte offsets of this lane's MFMA operands inside a stage.
    // K (A of S^T = K Q^T): key col (+32 per slab), chunk 2 kk + half.
    int koff[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) koff[kk] = col * T::kRow + 16 * ((2 * kk + half) ^ swz<D>(col));
    // V (A of O^T += V^T P^T) through ds_read_b64_tr_b16: lane 16 G + j addresses key
    // 16 ks + 8 hs + 4 (G / 2) + j / 4 at dims 32 d32 + 16 (G % 2) + 4 (j % 4) .. +3; the
    // transposing read hands lane 16 G + i the dim 32 d32 + 16 (G % 2) + i of those 4 keys.
    int voff[D / 32][2];
    {
        const int G4 = lane >> 4, j = lane & 15;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int key = 8 * hs + 4 * (G4 >> 1) + (j >> 2);
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32) {
                const int dim = 32 * d32 + 16 * (G4 & 1) + 4 * (j & 3);
                voff[d32][hs] = T::kBytes + key * T::kRow + 16 * ((dim >> 3) ^ swz<D>(key)) + 2 * (dim & 7);
            }
        }
    }

    for (int r = 0, it = g; it < items; it = MASK ? items : walk_block(++r, g, P)) {
        const Item cur = decode(it);
        const int b = cur.bh / H;
        const size_t head = (size_t)cur.bh * N * D;
        const i32x4 kdesc = dma_desc(K + head, head_bytes), vdesc = dma_desc(V + head, head_bytes);
        const int qrow = cur.q0 + w * kQPW + col;
        // With key limits, this row's limit (which the first barrier needs) goes out
        // first and Q's raw bits right behind it: loads complete in order, so the
        // wait before the barrier covers the limit alone.  Q stays in flight until
        // the first K/V tile lands.  Both go through buffer descriptors, rows past N
        // at an offset past the end (they read as zeros), so no load sits in a
        // branch: with branches the compiler waited for the first loads before
        // issuing the rest.
        int lraw = 0;  // this row's key limit as stored (rows past N read 0)
        if constexpr (MASK)
            lraw = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(kv_limit + (size_t)b * N, (uint32_t)N * 4u),
                                                        qrow < N ? qrow * 4 : N * 4, 0, 0);
        const auto qrs = buffer_rsrc(Q + head, head_bytes);
        const uint32_t qoff = ((uint32_t)qrow * D + 8 * half) * 2u;
        u32x4 qraw[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qraw[kk] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, qrow < N ? qoff + 32 * kk : head_bytes, 0, 0));
        const int lim = row_key_limit(qrow, N, CAUSAL, MASK ? &lraw : nullptr);
        const int wmax = wave_max_i(lim), wmin = wave_min_i(lim);
        // block_max alternates between two rows, so a fast wave writing the next
        // item's entry never meets a slow wave still reading this one's
        if (lane == 0) block_max[r & 1][w] = wmax;

        // After this barrier no wave reads the previous item's stages any more, and
        // every wave's block_max entry is written.  It orders LDS only (a full
        // __syncthreads would first wait for the Q loads and the previous item's
        // output stores); the empty asm statements keep the compiler from moving
        // memory accesses across it.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        int kv_end = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) kv_end = max(kv_end, block_max[r & 1][i]);
        const int ntiles = (kv_end + kBK - 1) / kBK;
        if (ntiles > 0) dma_tile(kdesc, vdesc, 0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        bf16x8 qf[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 u = qraw[kk];
            // the scale's sign folded into Q (see ScoreSign)
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] = score_signed(u[e], q_and, q_xor);
            qf[kk] = __builtin_bit_cast(bf16x8, u);
            launder(qf[kk]);
        }
        __syncthreads();

        f32x16 oacc[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
        float m_ref = -INFINITY;
        float l_sum[4] = {0.f, 0.f, 0.f, 0.f};  // four partial row sums: four short dependency chains

        auto step = [&](auto stage_c, auto rescale_c, auto first_c, int t) __attribute__((always_inline)) {
            constexpr int st = kSingleStage ? 0 : decltype(stage_c)::value;
            constexpr bool RESCALE = decltype(rescale_c)::value;
            constexpr bool FIRST = decltype(first_c)::value;  // tile 0 of a fixed-reference pass
            if (!kSingleStage && t + 1 < ntiles) dma_tile(kdesc, vdesc, st ^ 1, (t + 1) * kBK);
            const char* Sb = smem + st * T::kStage;
            const int kv0 = t * kBK;

            if (kv0 < wmax) {
                // S^T = K Q^T for kSub 32-key slabs; the slabs' accumulator chains alternate
                f32x16 s[kSub];
#pragma unroll
                for (int i = 0; i < kSub; ++i) s[i] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
                    for (int sub = 0; sub < kSub; ++sub)
                        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            *reinterpret_cast<const bf16x8*>(Sb + sub * 32 * T::kRow + koff[kk]), qf[kk], s[sub],
                            0, 0, 0);
                // Schedule: the K operand reads run two MFMA pairs ahead of their use
                // (left to itself the compiler issues them one pair ahead, and the
                // products wait on LDS).  Groups: 4 LDS reads, then (2 MFMAs, 2 LDS
                // reads) repeated, then the last 4 MFMAs.
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int gg = 0; gg < kSub * (D / 16) / 2 - 2; ++gg) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                if (kv0 + kBK > wmin) {  // tile crosses some row's key limit
#pragma unroll
                    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            const int key = kv0 + sub * 32 + 8 * (rr >> 2) + 4 * half + (rr & 3);
                            if (key >= lim) s[sub][rr] = -INFINITY;
                        }
                }
                if constexpr (RESCALE || FIRST) {
                    // four independent partial maxima: a short dependency chain
                    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
                    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) m4[rr & 3] = fmaxf(m4[rr & 3], s[sub][rr]);
                    float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
                    mx = halves_max(mx);
                    const float mt = mx * c;  // this tile's row max, log2 units
                    if constexpr (!RESCALE) {
                        m_ref = mt;  // the reference for the whole block
                    } else if (__any(mt > m_ref + kStaleMax)) {
                        const float m_new = fmaxf(m_ref, mt);
                        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
                        for (int e = 0; e < 4; ++e) l_sum[e] *= alpha;
#pragma unroll
                        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
                            for (int rr = 0; rr < 16; ++rr) oacc[d32][rr] *= alpha;
                        m_ref = m_new;
                    }
                }
                const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;

                // P = exp2(S c - m), packed to bf16; l sums the same rounded values
                u32x4 pk[kBK / 16];
                const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
                for (int ks = 0; ks < kBK / 16; ++ks) {
                    const int sub = ks >> 1, base = (ks & 1) * 8;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[sub][base + 2 * p], c, -m_use));
                        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[sub][base + 2 * p + 1], c, -m_use));
                        const uint32_t wv = pack_bf16x2(x0, x1);
                        pk[ks][p] = wv;
                        l_sum[p] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv), ones, l_sum[p], false);
                    }
                }
                // O^T += V^T P^T; the D/32 accumulator chains alternate
#pragma unroll
                for (int ks = 0; ks < kBK / 16; ++ks)
#pragma unroll
                    for (int d32 = 0; d32 < D / 32; ++d32) {
                        const char* vb = Sb + 16 * ks * T::kRow;
                        const u32x2 lo = tr_read(vb + voff[d32][0]), hi = tr_read(vb + voff[d32][1]);
                        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                        oacc[d32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                            __builtin_bit_cast(bf16x8, pk[ks]),
                                                                            oacc[d32], 0, 0, 0);
                    }
                if constexpr (D == 64) {
                    // V operand reads 8 ahead of their products
                    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
                    for (int gg = 0; gg < D / 32 * (kBK / 16) - 4; ++gg) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                }
            }
            if constexpr (kSingleStage) {
                __syncthreads();  // every wave has finished reading the stage
                if (t + 1 < ntiles) dma_tile(kdesc, vdesc, 0, (t + 1) * kBK);
            }
            if (t + 1 < ntiles) {  // after the last tile, the next item's first barrier serves
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
            }
        };
        auto run = [&](auto rescale_c) __attribute__((always_inline)) {
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            if constexpr (decltype(rescale_c)::value) {
                for (int t = 0; t < ntiles; t += 2) {
                    step(I0{}, rescale_c, std::false_type{}, t);
                    if (t + 1 < ntiles) step(I1{}, rescale_c, std::false_type{}, t + 1);
                }
            } else {
                // tile 0 sets each row's reference (its row max); later tiles take no max
                if (ntiles > 0) step(I0{}, rescale_c, std::true_type{}, 0);
                for (int t = 1; t < ntiles; t += 2) {
                    step(I1{}, rescale_c, std::false_type{}, t);
                    if (t + 1 < ntiles) step(I0{}, rescale_c, std::false_type{}, t + 1);
                }
            }
        };
        // With key limits (the key-padding workload's logits reach ~100 log2 units
        // of spread per row, and most blocks would overflow a fixed reference) the
        // reference follows the running max from the start.
        if constexpr (MASK) run(std::true_type{});
        if constexpr (!MASK) {
            run(std::false_type{});
            // The first pass keeps each row's first-tile max as its reference.  A later
            // score above it by 128 or more (log2 units) overflows P, a smaller excess
            // can still overflow O, and either leaves a non-finite sum or output; then
            // the whole workgroup (its barriers stay matched) computes the block again
            // with the reference following the running max.
            float chk[4] = {l_sum[0], l_sum[1], l_sum[2], l_sum[3]};
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) chk[rr & 3] = fmaf(oacc[d32][rr], 0.f, chk[rr & 3]);
            const bool bad = __any(!__builtin_isfinite((chk[0] + chk[1]) + (chk[2] + chk[3])));
            if (lane == 0) redo_flag[r & 1][w] = bad ? 1 : 0;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            int any_bad = 0;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) any_bad |= redo_flag[r & 1][i];
            if (any_bad) {
#pragma unroll
                for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
                m_ref = -INFINITY;
#pragma unroll
                for (int e = 0; e < 4; ++e) l_sum[e] = 0.f;
                if (ntiles > 0) dma_tile(kdesc, vdesc, 0, 0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                run(std::true_type{});
            }
        }

        // Epilogue: one division per row; each lane half summed its own keys.
        const float l_tot = halves_sum((l_sum[0] + l_sum[1]) + (l_sum[2] + l_sum[3]));
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        // O leaves in 16-byte stores (8 consecutive dims per lane, see o_rows16)
        u32x4 ov[D / 32][2];
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32) o_rows16(oacc[d32], inv, ov[d32]);
        if (qrow < N) {
            bf16* orow = O + head + (size_t)qrow * D;
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    *reinterpret_cast<u32x4*>(orow + 32 * d32 + 16 * p + 8 * half) = ov[d32][p];
            if (half == 0)
                LSE[(size_t)cur.bh * N + qrow] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const bf16* q, const bf16* k, const bf16* v, bf16* o, float* lse, int B, int H, int N,
                  ScoreSign sg, const int32_t* kv_limit, hipStream_t stream) {
    const int nqb = (N + kBQ - 1) / kBQ;
    const long long items = (long long)B * H * nqb;
    // Key limits make block lengths data-dependent: there every block gets its
    // own workgroup and the hardware balances them.
    unsigned grid = 0;
    const hipError_t e = walk_grid(items, !MASK, &grid);
    if (e != hipSuccess) return e;
    return launch_kernel(fwd_kernel<D, CAUSAL, MASK>, dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse, H, N,
                         nqb, (int)items, sg.c, sg.and_mask, sg.xor_mask, kv_limit);
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
    const ScoreSign sg = score_sign(scale, kLog2e, kSignBf16x2);
    const bool mask = kv_limit != nullptr;
#define FA_DISPATCH(DD, CC, MM) \
    if (d == DD && causal == CC && mask == MM) return launch<DD, CC, MM>(Q, K, V, Ot, lse, B, H, N, sg, kv_limit, stream);
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

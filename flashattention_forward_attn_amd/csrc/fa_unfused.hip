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
#include "fa_epilogue.h"
#include "fa_tile.h"

namespace fa {
namespace unfused {

constexpr int kThreads = 256;

// (batch x head, block) of workgroup g in a grid of BH x nb blocks.  Round-robin
// dispatch sends g to XCD g mod 8; with BH a multiple of 8 each XCD takes whole
// heads (those congruent to its index) and walks one head's blocks back to back,
// so the head's K or V stays in that XCD's L2 while its blocks run.
__device__ __forceinline__ void head_block(int g, int BH, int nb, int* bh, int* blk) {
    if (BH % 8 == 0) {
        const int s = g >> 3;
        *bh = 8 * (s / nb) + (g & 7);
        *blk = s % nb;
    } else {
        *bh = g % BH;
        *blk = g / BH;
    }
}

// ---------------------------------------------------------------- scores (bf16)
// One workgroup per 128 query rows of one (batch, head), 4 waves x 32 rows,
// walking every key in tiles of 64.  K tiles go from global memory straight
// into LDS (double-buffered, 16-byte chunks XOR-swizzled by key); each wave
// keeps its rows' Q fragments in registers and forms C = Q K^T with
// v_mfma_f32_32x32x16_bf16, so a lane holds one key of 16 query rows and each
// store instruction writes two 128-byte row segments of S.  A tile's stores go
// out after the barrier that ends it and complete while the next tile is
// multiplied.  Grid: (batch x head) fastest.  Mapping a head's blocks to one
// XCD back to back (head_block) cut the K re-reads from 0.79 to 0.14 GB on the
// causal B2 H32 N4096 d128 workload but made the S writes slower (1065 against
// 935 us), so the writes' order wins here.
constexpr int kScoreRows = 128;
constexpr int kScoreKeys = 64;

template <int D>
__global__ __launch_bounds__(kThreads) void scores_bf16(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                        float* __restrict__ S, int N, int64_t ld, float scale) {
    constexpr int kRow = D * 2, kBytes = kScoreKeys * kRow, kPerWave = kBytes / kDmaBytes / 4;
    static_assert(kBytes % (4 * kDmaBytes) == 0, "tile must split evenly over the waves");
    __shared__ __attribute__((aligned(1024))) char smem[2 * kBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    const size_t bh = blockIdx.x, head = bh * N * D;
    const int q0 = blockIdx.y * kScoreRows + w * 32;
    const i32x4 kdesc = dma_desc(K + head, (uint32_t)N * D * 2u);  // keys past N read as zeros

    uint32_t dma_off[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int p = (i * 4 + w) * kDmaBytes + 16 * lane;
        const int row = p / kRow, slot = (p % kRow) / 16;
        dma_off[i] = (uint32_t)(row * kRow + 16 * (slot ^ swz<D>(row)));
    }
    auto dma_tile = [&](int stage, int kv0) {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i)
            dma16(kdesc, lds_addr(smem + stage * kBytes + (i * 4 + w) * kDmaBytes), (uint32_t)kv0 * kRow + dma_off[i]);
    };
    // B operand (K^T): key col of a 32-key slab, dims 16 kk + 8 half .. + 7
    int koff[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) koff[kk] = col * kRow + 16 * ((2 * kk + half) ^ swz<D>(col));
    const int qa = q0 + col;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = qa < N ? *reinterpret_cast<const bf16x8*>(Q + head + (size_t)qa * D + 16 * kk + 8 * half) : bf16x8{};

    const int ntiles = (N + kScoreKeys - 1) / kScoreKeys;
    dma_tile(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    float* Sh = S + bh * N * ld;
    auto step = [&](auto stage_c, int t) __attribute__((always_inline)) {
        constexpr int st = decltype(stage_c)::value;
        if (t + 1 < ntiles) dma_tile(st ^ 1, (t + 1) * kScoreKeys);
        const char* Kb = smem + st * kBytes;
        f32x16 acc[kScoreKeys / 32];
#pragma unroll
        for (int sub = 0; sub < kScoreKeys / 32; ++sub) acc[sub] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int sub = 0; sub < kScoreKeys / 32; ++sub)
                acc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    qf[kk], *reinterpret_cast<const bf16x8*>(Kb + sub * 32 * kRow + koff[kk]), acc[sub], 0, 0, 0);
        // the wait covers the next tile's loads and the previous tile's stores
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int sub = 0; sub < kScoreKeys / 32; ++sub) {
            const int key = t * kScoreKeys + sub * 32 + col;
            if (key >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = q0 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (q < N) Sh[(size_t)q * ld + key] = acc[sub][r] * scale;
            }
        }
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
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
// W waves per row (W = 1: four rows per workgroup), the row held in registers:
// lane l of wave w holds the 16-byte chunks (c W + w) 64 + l, c < C4, so every
// load instruction reads 1 KB of consecutive S.  S is read once and P written
// once; P is 0 past the row's key limit, up to ld.
// Store P values 4 (chunk 64 + lane) .. + 3 of a row through its descriptor.
template <typename PT>
__device__ __forceinline__ void store_p4(__amdgpu_buffer_rsrc_t r, int lane, int chunk, f32x4 v);
template <>
__device__ __forceinline__ void store_p4<bf16>(__amdgpu_buffer_rsrc_t r, int lane, int chunk, f32x4 v) {
    const u32x2 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(u, r, (chunk * 64 + lane) * 8, 0, 0);
}
template <>
__device__ __forceinline__ void store_p4<float>(__amdgpu_buffer_rsrc_t r, int lane, int chunk, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (chunk * 64 + lane) * 16, 0, 0);
}

template <typename PT, int W, int C4>
__global__ __launch_bounds__(512) void softmax_rows(const float* __restrict__ S, PT* __restrict__ P,
                                                    float* __restrict__ LSE, int H, int N, int64_t ld, int64_t rows,
                                                    int causal, const int32_t* __restrict__ kv_limit) {
    static_assert(W == 1 || W == 4 || W == 8, "waves per row");
    __shared__ float red[2][W];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = W == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
    const int ws = W == 1 ? 0 : wave;  // wave within the row
    if (W == 1 && row >= rows) return;  // (no barrier on this path)
    const int i = (int)(row % N), b = (int)(row / N) / H;
    const int lim = row_key_limit(i, N, causal != 0, kv_limit ? kv_limit + (size_t)b * N + i : nullptr);
    const int ldi = (int)ld;  // at most 32768
    // row descriptors: 32-bit offsets within the row, no 64-bit address per chunk
    const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(S + row * ld, (uint32_t)ldi * 4u);
    const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(P + row * ld, (uint32_t)ldi * (uint32_t)sizeof(PT));

    f32x4 x[C4];
    float m = -INFINITY;
    const int rem = lim - (ws * 64 + lane) * 4;  // keys of chunk c below the limit: c W 256 + e < rem
#pragma unroll
    for (int c = 0; c < C4; ++c) {
        const int j0 = ((c * W + ws) * 64 + lane) * 4;
        x[c] = j0 < ldi ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, 4 * j0, 0, 0))
                        : f32x4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (c * W * 256 + e >= rem) x[c][e] = -INFINITY;
            m = fmaxf(m, x[c][e]);
        }
    }
    m = wave_max(m);
    if constexpr (W > 1) {
        if (lane == 0) red[0][wave] = m;
        __syncthreads();
        m = red[0][0];
#pragma unroll
        for (int v = 1; v < W; ++v) m = fmaxf(m, red[0][v]);
    }
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < C4; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[c][e] = c * W * 256 + e < rem ? __expf(x[c][e] - m) : 0.f;
            sum += x[c][e];
        }
    }
    sum = wave_sum(sum);
    if constexpr (W > 1) {
        if (lane == 0) red[1][wave] = sum;
        __syncthreads();
        sum = red[1][0];
#pragma unroll
        for (int v = 1; v < W; ++v) sum += red[1][v];
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
    for (int c = 0; c < C4; ++c) {
        const int j0 = ((c * W + ws) * 64 + lane) * 4;
        if (j0 < ldi) store_p4<PT>(pr, lane, c * W + ws, x[c] * inv);
    }
    if (ws == 0 && lane == 0) LSE[row] = sum > 0.f ? m + __logf(sum) : -INFINITY;
}

// ---------------------------------------------------------------- P V (bf16)
// One workgroup per 256 query rows of one (batch, head): 8 waves x 32 rows,
// keys in tiles of 64.  Both operands go from global memory straight into LDS
// through three stages (two tiles in flight while one is multiplied): the P
// tile as 256 rows of 128 bytes (each wave-wide load covers 8 whole row
// segments), the V tile as 64 rows of D values, both with XOR-swizzled 16-byte
// chunks.  O^T += V^T P^T as in the fused kernel: V^T through the transposing
// LDS read, P^T as 16-byte reads of a row's 8 keys.  Blocks map to XCDs by
// head (head_block), so each head's V is read from HBM about once (505 against
// about 570 us with (batch x head) fastest).  32-key tiles with up to six
// stages, 128-row blocks (two workgroups per CU), P held in registers per wave
// three to six tiles ahead instead of in LDS, and a three-tile V lead all
// measured within the run-to-run spread of this form.
constexpr int kPvRows = 256;
constexpr int kPvKeys = 64;
constexpr int kPvWaves = kPvRows / 32;
constexpr int kPvThreads = kPvWaves * kWave;
constexpr int kPvStages = 3;

// P tile rows hold kPvChunks 16-byte chunks; chunk c of row `row` sits in slot
// c ^ pswz(row), so 16 consecutive rows reading one chunk each hit 16 distinct
// bank groups.
constexpr int kPvChunks = kPvKeys / 8;
__device__ __forceinline__ int pswz(int row) { return (row / (16 / kPvChunks)) % kPvChunks; }

template <int D>
__global__ __launch_bounds__(kPvThreads) void pv_bf16(const bf16* __restrict__ P, const bf16* __restrict__ V,
                                                      bf16* __restrict__ O, int BH, int N, int64_t ld) {
    constexpr int kPRow = kPvKeys * 2, kPBytes = kPvRows * kPRow;  // 64-byte rows, 16 KB
    constexpr int kVRow = D * 2, kVBytes = kPvKeys * kVRow;
    constexpr int kStage = kPBytes + kVBytes;
    // V blocks: 16 bytes per lane where the tile has a block per wave, else 4 (d = 64)
    constexpr bool kV16 = kVBytes % (kPvWaves * kDmaBytes) == 0;
    constexpr int kVBlock = kV16 ? kDmaBytes : kWave * 4, kVLane = kVBlock / kWave;
    constexpr int kPPerWave = kPBytes / kDmaBytes / kPvWaves, kVPerWave = kVBytes / kVBlock / kPvWaves;
    static_assert(kPBytes % (kPvWaves * kDmaBytes) == 0 && kVBytes % (kPvWaves * kVBlock) == 0,
                  "tiles must split evenly over the waves");
    constexpr int kLoads = kPPerWave + kVPerWave;  // DMA instructions per wave per tile
    __shared__ __attribute__((aligned(1024))) char smem[kPvStages * kStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    int bhi, rb;
    head_block(blockIdx.x, BH, (N + kPvRows - 1) / kPvRows, &bhi, &rb);
    const size_t bh = bhi;
    const int r0 = rb * kPvRows;
    const int nrows = min(N - r0, kPvRows);
    // this block's P rows (rows past them read as zeros) and the head's V rows
    const i32x4 pdesc = dma_desc(P + bh * N * ld + (size_t)r0 * ld, (uint32_t)((int64_t)nrows * ld * 2));
    const i32x4 vdesc = dma_desc(V + bh * N * D, (uint32_t)N * D * 2u);

    // DMA offsets: a P block is 64 / kPvChunks whole rows, a V block kVBlock bytes of key rows
    uint32_t poff[kPPerWave], voff_g[kVPerWave];
#pragma unroll
    for (int i = 0; i < kPPerWave; ++i) {
        const int row = (i * kPvWaves + w) * (kWave / kPvChunks) + lane / kPvChunks, slot = lane % kPvChunks;
        poff[i] = (uint32_t)(row * ld * 2 + 16 * (slot ^ pswz(row)));
    }
#pragma unroll
    for (int i = 0; i < kVPerWave; ++i) {
        const int p = (i * kPvWaves + w) * kVBlock + kVLane * lane;
        const int row = p / kVRow, slot = (p % kVRow) / 16;
        voff_g[i] = (uint32_t)(row * kVRow + 16 * (slot ^ swz<D>(row)) + p % 16);
    }
    auto dma_tile = [&](int stage, int kv0) {
        char* base = smem + stage * kStage;
#pragma unroll
        for (int i = 0; i < kPPerWave; ++i)
            dma16(pdesc, lds_addr(base + (i * kPvWaves + w) * kDmaBytes), (uint32_t)kv0 * 2 + poff[i]);
#pragma unroll
        for (int i = 0; i < kVPerWave; ++i) {
            const uint32_t dst = lds_addr(base + kPBytes + (i * kPvWaves + w) * kVBlock);
            if constexpr (kV16)
                dma16(vdesc, dst, (uint32_t)kv0 * kVRow + voff_g[i]);
            else
                dma4(vdesc, dst, (uint32_t)kv0 * kVRow + voff_g[i]);
        }
    };
    // P^T (B operand): row w 32 + col, keys 16 ks + 8 half .. + 7 = chunk 2 ks + half
    const int prow = w * 32 + col;
    int pk[kPvKeys / 16];
#pragma unroll
    for (int ks = 0; ks < kPvKeys / 16; ++ks) pk[ks] = prow * kPRow + 16 * ((2 * ks + half) ^ pswz(prow));
    // V^T (A operand) through ds_read_b64_tr_b16: lane 16 G + j addresses key
    // 16 ks + 8 (G / 2) + 4 hs + j / 4 at dims 32 d32 + 16 (G % 2) + 4 (j % 4) .. +3, so
    // lane 16 G + i receives dim 32 d32 + 16 (G % 2) + i of keys 16 ks + 8 half + 4 hs + 0..3:
    // the keys of its P^T operand, in order.
    int vo[D / 32][2];
    {
        const int G4 = lane >> 4, j = lane & 15;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int key = 8 * (G4 >> 1) + 4 * hs + (j >> 2);
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32) {
                const int dim = 32 * d32 + 16 * (G4 & 1) + 4 * (j & 3);
                vo[d32][hs] = kPBytes + key * kVRow + 16 * ((dim >> 3) ^ swz<D>(key)) + 2 * (dim & 7);
            }
        }
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    const int ntiles = (int)(ld / kPvKeys);
    // Only DMA loads are outstanding in the loop, and loads complete in order:
    // waiting until at most `newer` tiles' loads remain leaves those in flight.
    static_assert(kPvStages >= 2 && kPvStages <= 6, "wait_tiles covers up to 4 newer tiles");
    auto wait_tiles = [&](int newer) {
        switch (newer) {
            case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
            case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(1 * kLoads) : "memory"); break;
            case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kLoads) : "memory"); break;
            case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kLoads) : "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kLoads) : "memory"); break;
        }
    };
    // prologue: tiles 0 .. kPvStages - 2 in flight, wait for tile 0
    const int pro = min(ntiles, kPvStages - 1);
    for (int u = 0; u < pro; ++u) dma_tile(u, u * kPvKeys);
    wait_tiles(pro - 1);
    __syncthreads();
    auto step = [&](auto stage_c, int t) __attribute__((always_inline)) {
        constexpr int st = decltype(stage_c)::value;
        // stage (st + kPvStages - 1) % kPvStages was last read in the previous step, before its barrier
        if (t + kPvStages - 1 < ntiles) dma_tile((st + kPvStages - 1) % kPvStages, (t + kPvStages - 1) * kPvKeys);
        const char* Sb = smem + st * kStage;
#pragma unroll
        for (int ks = 0; ks < kPvKeys / 16; ++ks) {
            const bf16x8 pb = *reinterpret_cast<const bf16x8*>(Sb + pk[ks]);
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32) {
                const char* vb = Sb + 16 * ks * kVRow;
                const u32x2 lo = tr_read(vb + vo[d32][0]), hi = tr_read(vb + vo[d32][1]);
                const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                acc[d32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb, acc[d32], 0, 0, 0);
            }
        }
        if (t + 1 < ntiles) {
            // tile t + 1 complete; tiles t + 2 .. min(t + kPvStages - 1, ntiles - 1) may still load
            wait_tiles(min(t + kPvStages - 1, ntiles - 1) - (t + 1));
            __syncthreads();
        }
    };
    for (int t = 0; t < ntiles; t += kPvStages) {
        static_for<0, kPvStages>([&](auto u) {
            if (t + decltype(u)::value < ntiles) step(u, t + decltype(u)::value);
        });
    }
    const int q = r0 + prow;
    // O leaves in 16-byte stores (8 consecutive dims per lane, see o_rows16)
    u32x4 ov[D / 32][2];
#pragma unroll
    for (int d32 = 0; d32 < D / 32; ++d32) o_rows16(acc[d32], 1.0f, ov[d32]);
    if (q < N) {
        bf16* orow = O + bh * N * D + (size_t)q * D;
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
            for (int p = 0; p < 2; ++p) *reinterpret_cast<u32x4*>(orow + 32 * d32 + 16 * p + 8 * half) = ov[d32][p];
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
    const int64_t rows = (int64_t)B * H * N;
    const int c = causal ? 1 : 0;
    // one wave per row up to 1024 keys (four rows per workgroup), else 4 or 8 waves per row
    const dim3 g1((unsigned)((rows + 3) / 4)), gw((unsigned)rows);
    if (ld <= 256) return launch_kernel(softmax_rows<PT, 1, 1>, g1, dim3(256), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
    if (ld <= 512) return launch_kernel(softmax_rows<PT, 1, 2>, g1, dim3(256), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
    if (ld <= 1024) return launch_kernel(softmax_rows<PT, 1, 4>, g1, dim3(256), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
    if (ld <= 2048) return launch_kernel(softmax_rows<PT, 4, 2>, gw, dim3(256), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
    if (ld <= 4096) return launch_kernel(softmax_rows<PT, 4, 4>, gw, dim3(256), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
    if (ld <= 8192) return launch_kernel(softmax_rows<PT, 4, 8>, gw, dim3(256), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
    if (ld <= 16384) return launch_kernel(softmax_rows<PT, 4, 16>, gw, dim3(256), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
    return launch_kernel(softmax_rows<PT, 8, 16>, gw, dim3(512), 0, stream, S, P, lse, H, N, ld, rows, c, kv_limit);
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
        const int bhn = (int)BH;
        const dim3 g1(BH, (unsigned)((N + kScoreRows - 1) / kScoreRows));
        err = d == 64 ? launch_kernel(scores_bf16<64>, g1, block, 0, stream, Q, K, S, N, ld, scale)
                      : launch_kernel(scores_bf16<128>, g1, block, 0, stream, Q, K, S, N, ld, scale);
        if (err != hipSuccess) return err;
        if ((err = launch_softmax<bf16>(S, (bf16*)P, lse, B, H, N, ld, causal, kv_limit, stream)) != hipSuccess) return err;
        const bf16 *Pb = static_cast<const bf16*>(P), *Vb = static_cast<const bf16*>(v);
        bf16* Ob = static_cast<bf16*>(o);
        const dim3 g3((unsigned)(BH * ((N + kPvRows - 1) / kPvRows)));
        return d == 64 ? launch_kernel(pv_bf16<64>, g3, dim3(kPvThreads), 0, stream, Pb, Vb, Ob, bhn, N, ld)
                       : launch_kernel(pv_bf16<128>, g3, dim3(kPvThreads), 0, stream, Pb, Vb, Ob, bhn, N, ld);
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

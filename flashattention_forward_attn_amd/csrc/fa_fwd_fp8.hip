// fa_fwd_fp8.hip -- FP8 variant of the fused forward for gfx950: Q and K in E4M3
// with one power-of-two scale per tile, after incoherent processing.
//
// The method ("FlashAttention 1–4: How IO-Awareness Reshaped the Attention
// Kernel", section "FlashAttention-3", FP8 with block quantization and
// incoherent processing): Q and K are multiplied by the same random orthogonal
// matrix -- random sign flips, then a Hadamard transform, O(d log d) per row --
// which leaves Q K^T unchanged but spreads an outlier over every coordinate;
// each tile of rows then gets its own FP8 scale, so an outlier only costs its
// own tile resolution.
//
// Two kernels:
//   1. quantise: one workgroup per tile of 32 (Q) or 64 (K) rows of one head;
//      d/8 lanes per row, 8 values per lane.  y = H (s * x) in fp32 by the
//      butterfly (stages h = 1, 2, 4 inside a lane, then across lanes), the
//      tile's max |y|, the smallest exponent e with max |y| <= 448 * 2^e, and
//      codes E4M3(y * 2^-e) by v_cvt_pk_fp8_f32 (round to nearest even).  H is
//      the unnormalised Sylvester matrix (entries +-1), so scores carry a
//      factor d, removed in the softmax scale.
//   2. attention: the bf16 kernel's structure (8 waves x 32 query rows, K/V
//      tiles of 64 keys at d = 128 and 128 at d = 64 by direct-to-LDS loads,
//      transposed scores, bf16 P V, the same walk over query blocks) with
//      S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 operands, and the
//      two tiles' exponents passed as its E8M0 block scales, so the product
//      comes out already scaled.  V stays bf16.
#include "fa_common.h"
#include "fa_launch.h"
#include "fa_epilogue.h"
#include "fa_tile.h"

namespace fa {
namespace fp8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int8_t i8x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- 1. quantise
constexpr int kQuantThreads = 256;

// Smallest e with a <= 448 * 2^e (a = m 2^k, m in [0.5, 1), 448 = 0.875 2^9),
// clamped to [-127, 127]; 0 for a == 0.  Exact integer logic on the bits.
__device__ __forceinline__ int tile_exponent(float a) {
    const uint32_t u = __builtin_bit_cast(uint32_t, a);
    const int E = (int)((u >> 23) & 0xff);
    const uint32_t M = u & 0x7fffffu;
    if (E == 0) return M == 0 ? 0 : -127;  // subnormal maxima need e below -127
    int e = (E - 126) - 9 + (M > 0x600000u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// The value lane l ^ hb holds (hb = 1, 2, 4 or 8), from within l's 16-lane DPP row:
// quad_perm swaps for 1 and 2; row_half_mirror (l ^ 7) after a quad reversal (l ^ 3)
// for 4, and after row_mirror (l ^ 15) for 8.  No LDS access and no wait.
__device__ __forceinline__ float xor_lanes(float v, int hb) {
    int u = __builtin_bit_cast(int, v);
    switch (hb) {
        case 1: u = __builtin_amdgcn_update_dpp(0, u, 0xB1, 0xF, 0xF, false); break;  // quad_perm 1 0 3 2
        case 2: u = __builtin_amdgcn_update_dpp(0, u, 0x4E, 0xF, 0xF, false); break;  // quad_perm 2 3 0 1
        case 4:
            u = __builtin_amdgcn_update_dpp(0, u, 0x1B, 0xF, 0xF, false);   // quad_perm 3 2 1 0
            u = __builtin_amdgcn_update_dpp(0, u, 0x141, 0xF, 0xF, false);  // row_half_mirror
            break;
        default:
            u = __builtin_amdgcn_update_dpp(0, u, 0x140, 0xF, 0xF, false);  // row_mirror
            u = __builtin_amdgcn_update_dpp(0, u, 0x141, 0xF, 0xF, false);  // row_half_mirror
            break;
    }
    return __builtin_bit_cast(float, u);
}

template <int D, int T>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const bf16* __restrict__ x,
                                                              const int8_t* __restrict__ signs,
                                                              uint8_t* __restrict__ codes, int32_t* __restrict__ exps,
                                                              int N, int nt) {
    constexpr int LPR = D / 8;                  // lanes per row
    constexpr int RPP = kQuantThreads / LPR;    // rows per pass
    constexpr int PASSES = (T + RPP - 1) / RPP;
    static_assert(T % RPP == 0 || RPP % T == 0, "tile and pass shapes");
    __shared__ float wmax[kQuantThreads / kWave];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const long long bh = blockIdx.x / nt;
    const int tile = blockIdx.x % nt;
    const int rp = tid / LPR, cidx = tid % LPR;

    // Every pass's 16 bytes go out at once, through a buffer descriptor over this
    // (batch, head)'s rows; rows past the tile or past N sit at an offset past its
    // end and read zeros, so no load sits in a branch or waits for another.
    const uint32_t head_bytes = (uint32_t)N * D * 2u;
    const auto xrs = buffer_rsrc(x + bh * N * D, head_bytes);
    u32x4 raw[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int rin = p * RPP + rp, row = tile * T + rin;
        const bool ok = rin < T && row < N;
        raw[p] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, ok ? ((uint32_t)row * D + 8 * cidx) * 2u : head_bytes, 0, 0));
    }
    float sg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = (float)signs[8 * cidx + e];

    float y[PASSES][8];
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int rin = p * RPP + rp, row = tile * T + rin;
        const bool ok = rin < T && row < N;
        const bf16x8 v = __builtin_bit_cast(bf16x8, raw[p]);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[p][e] = (float)v[e] * sg[e];
        // butterfly stages inside the lane: dims 8 cidx + i, pairs (i, i + h)
#pragma unroll
        for (int h = 1; h < 8; h <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (!(i & h)) {
                    const float a = y[p][i], b = y[p][i + h];
                    y[p][i] = a + b;
                    y[p][i + h] = a - b;
                }
        // stages across the row's lanes: h = 8 hb; the lane holding the lower dim adds
#pragma unroll
        for (int hb = 1; hb < LPR; hb <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float other = xor_lanes(y[p][i], hb);
                y[p][i] = (cidx & hb) ? other - y[p][i] : y[p][i] + other;
            }
        if (ok)
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[p][i]));
    }
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    if (lane == 0) wmax[tid >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQuantThreads / kWave; ++i) amax = fmaxf(amax, wmax[i]);
    const int e = tile_exponent(amax);
    const float inv = __builtin_ldexpf(1.f, -e);  // exact power of two
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int rin = p * RPP + rp, row = tile * T + rin;
        if (rin < T && row < N) {
            u32x2 out;
            uint32_t w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[p][0] * inv, y[p][1] * inv, 0, false);
            w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[p][2] * inv, y[p][3] * inv, (int)w0, true);
            uint32_t w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[p][4] * inv, y[p][5] * inv, 0, false);
            w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[p][6] * inv, y[p][7] * inv, (int)w1, true);
            out.x = w0;
            out.y = w1;
            *reinterpret_cast<u32x2*>(codes + (bh * N + row) * D + 8 * cidx) = out;
        }
    }
    if (tid == 0) exps[bh * nt + tile] = e;
}

// ---------------------------------------------------------------- 2. attention
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;  // 512
constexpr int kQPW = kFp8QTile;           // query rows per wave = one Q tile
constexpr int kBQ = kWaves * kQPW;        // 256 query rows per query block
// keys per K/V tile: one K code tile at d = 128, two at d = 64 (each 64-key
// half then takes its own exponent)
template <int D>
constexpr int kBKof = D == 64 ? 2 * kFp8KTile : kFp8KTile;
constexpr float kStaleMax = 8.0f;         // log2 units (the recomputation pass moves its reference past this)

// K rows of D E4M3 bytes: chunk c of row r sits in slot c ^ kswz(r), so that
// 16 consecutive rows reading one chunk touch 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int kswz(int row) {
    if constexpr (D == 128) return (row >> 1) & 7;
    else return (row >> 2) & 3;
}

template <int D>
struct Tile {
    static constexpr int kBK = kBKof<D>;
    static constexpr int kSub = kBK / 32;           // 32-key slabs per tile
    static constexpr int kRowK = D;                 // E4M3 key row
    static constexpr int kRowV = 2 * D;             // bf16 value row
    static constexpr int kBytesK = kBK * kRowK;
    static constexpr int kBytesV = kBK * kRowV;
    static constexpr int kStage = kBytesK + kBytesV;
    static constexpr int kBlocksK = kBytesK / kDmaBytes;
    static constexpr int kBlocksV = kBytesV / kDmaBytes;
    static constexpr int kPerWaveK = (kBlocksK + kWaves - 1) / kWaves;
    static constexpr int kPerWaveV = (kBlocksV + kWaves - 1) / kWaves;
};

// QRAW: Q arrives in bf16 (Qb) with the rotation's signs, and each wave rotates
// and encodes its own 32 rows -- exactly one Q tile -- in its prologue, with the
// quantisation kernel's steps in the same order, so the codes and the exponent
// are the ones that kernel would store.  Otherwise Q arrives as codes (Qc, Qe).
template <int D, bool CAUSAL, bool MASK, bool QRAW>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const uint8_t* __restrict__ Qc, const int32_t* __restrict__ Qe, const bf16* __restrict__ Qb,
                const int8_t* __restrict__ signs, const uint8_t* __restrict__ Kc,
                const int32_t* __restrict__ Ke, const bf16* __restrict__ V, bf16* __restrict__ O,
                float* __restrict__ LSE, int H, int N, int nqb, int items, float c, uint32_t q_and,
                uint32_t q_xor, const int32_t* __restrict__ kv_limit) {
    using T = Tile<D>;
    constexpr int kBK = T::kBK, kSub = T::kSub;
    __shared__ __attribute__((aligned(1024))) char smem[2 * T::kStage];
    __shared__ int block_max[2][kWaves];
    __shared__ int redo_flag[2][kWaves];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;

    const int P = gridDim.x, g = blockIdx.x;
    const int BHn = items / nqb;
    // Query blocks in the bf16 kernel's order and walk (walk_block); one block
    // per workgroup when a key limit is given.
    const int nqt = (N + kQPW - 1) / kQPW, nkt = (N + kFp8KTile - 1) / kFp8KTile;

    // Direct-to-LDS loads: block i * kWaves + w of the K tile and of the V tile.
    uint32_t koffd[T::kPerWaveK], voffd[T::kPerWaveV];
#pragma unroll
    for (int i = 0; i < T::kPerWaveK; ++i) {
        const int p = (i * kWaves + w) * kDmaBytes + 16 * lane;
        const int row = p / T::kRowK, slot = (p % T::kRowK) / 16;
        koffd[i] = (uint32_t)(row * T::kRowK + 16 * (slot ^ kswz<D>(row)));
    }
#pragma unroll
    for (int i = 0; i < T::kPerWaveV; ++i) {
        const int p = (i * kWaves + w) * kDmaBytes + 16 * lane;
        const int row = p / T::kRowV, slot = (p % T::kRowV) / 16;
        voffd[i] = (uint32_t)(row * T::kRowV + 16 * (slot ^ swz<D>(row)));
    }
    for (int r = 0, it = g; it < items; it = MASK ? items : walk_block(++r, g, P)) {
        int qb = it / BHn;
        const int bh = it - qb * BHn;
        if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
        const int b = bh / H;
        const i32x4 kdesc = dma_desc(Kc + (size_t)bh * N * D, (uint32_t)N * D);
        const i32x4 vdesc = dma_desc(V + (size_t)bh * N * D, (uint32_t)N * D * 2u);
        auto dma_tile = [&](int stage, int kv0) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(smem + stage * T::kStage);
#pragma unroll
            for (int i = 0; i < T::kPerWaveK; ++i)
                if (i * kWaves + w < T::kBlocksK)
                    dma16(kdesc, st + (i * kWaves + w) * kDmaBytes, (uint32_t)kv0 * T::kRowK + koffd[i]);
#pragma unroll
            for (int i = 0; i < T::kPerWaveV; ++i)
                if (i * kWaves + w < T::kBlocksV)
                    dma16(vdesc, st + T::kBytesK + (i * kWaves + w) * kDmaBytes, (uint32_t)kv0 * T::kRowV + voffd[i]);
        };

        const int q0 = qb * kBQ;
        const int qrow = q0 + w * kQPW + col;
        const int lim = row_key_limit(qrow, N, CAUSAL, MASK ? kv_limit + (size_t)b * N + qrow : nullptr);
        const int wmax = wave_max_i(lim), wmin = wave_min_i(lim);
        // two rows, so consecutive blocks never share one; after this barrier no
        // wave reads the previous block's stages any more
        if (lane == 0) block_max[r & 1][w] = wmax;
        __syncthreads();
        int kv_end = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) kv_end = max(kv_end, block_max[r & 1][i]);
        const int ntiles = (kv_end + kBK - 1) / kBK;
        // the first K/V tile's loads go out before Q is prepared, which hides their latency
        if (ntiles > 0) dma_tile(0, 0);

        // Q codes of this lane's query: 32 bytes per 64 dims (k = 32 half .. +31)
        i32x8 qf[D / 64];
        int qscale;  // E8M0 block scale of this wave's Q tile (uniform)
        if constexpr (QRAW) {
            // y = H (s * q) for this lane's dims 64 kk + 32 half + i (rows past N are zeros)
            float y[D / 64][32];
#pragma unroll
            for (int kk = 0; kk < D / 64; ++kk) {
                const int base = 64 * kk + 32 * half;
                const i8x16 s0 = *reinterpret_cast<const i8x16*>(signs + base);
                const i8x16 s1 = *reinterpret_cast<const i8x16*>(signs + base + 16);
#pragma unroll
                for (int c8 = 0; c8 < 4; ++c8) {
                    bf16x8 x = bf16x8{};
                    if (qrow < N)
                        x = *reinterpret_cast<const bf16x8*>(Qb + ((size_t)bh * N + qrow) * D + base + 8 * c8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int t = 8 * c8 + e;
                        y[kk][t] = (float)x[e] * (float)(t < 16 ? s0[t] : s1[t - 16]);
                    }
                }
            }
            // butterfly stages h = 1 .. 16 inside each 32-dim block of the lane
#pragma unroll
            for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
                for (int h = 1; h < 32; h <<= 1)
#pragma unroll
                    for (int i = 0; i < 32; ++i)
                        if (!(i & h)) {
                            const float a = y[kk][i], b = y[kk][i + h];
                            y[kk][i] = a + b;
                            y[kk][i + h] = a - b;
                        }
            // stage h = 32 across the lane halves: one v_permlane32_swap hands every
            // lane (lower, upper) = the values of lanes l mod 32 and l mod 32 + 32;
            // the lower half keeps lower + upper, the upper half lower - upper
#pragma unroll
            for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    const uint32_t u = __builtin_bit_cast(uint32_t, y[kk][i]);
                    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
                    const float lo = __builtin_bit_cast(float, (uint32_t)r[0]);
                    const float hi = __builtin_bit_cast(float, (uint32_t)r[1]);
                    y[kk][i] = half ? lo - hi : lo + hi;
                }
            // stage h = 64 between the lane's two blocks (d = 128)
            if constexpr (D == 128) {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    const float a = y[0][i], b = y[1][i];
                    y[0][i] = a + b;
                    y[1][i] = a - b;
                }
            }
            float amax = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
                for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[kk][i]));
            for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
            const int e = tile_exponent(amax);
            const float inv = __builtin_ldexpf(1.f, -e);  // exact power of two
#pragma unroll
            for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    uint32_t wv = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[kk][4 * j] * inv, y[kk][4 * j + 1] * inv,
                                                                           0, false);
                    wv = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[kk][4 * j + 2] * inv, y[kk][4 * j + 3] * inv,
                                                                   (int)wv, true);
                    qf[kk][j] = (int)wv;
                }
            qscale = 127 + e;
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 64; ++kk) {
                if (qrow < N) {
                    const u32x4* src =
                        reinterpret_cast<const u32x4*>(Qc + ((size_t)bh * N + qrow) * D + 64 * kk + 32 * half);
                    const u32x4 lo = src[0], hi = src[1];
                    qf[kk] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                } else {
                    qf[kk] = i32x8{};
                }
            }
            const int wq = q0 / kQPW + w;
            qscale = 127 + (wq < nqt ? Qe[(size_t)bh * nqt + wq] : 0);
        }
        // the scale's sign folded into the Q codes (see ScoreSign): E4M3 negates by its
        // sign bit, and the tile exponent is unchanged
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
            for (int j = 0; j < 8; ++j) qf[kk][j] = (int)score_signed((uint32_t)qf[kk][j], q_and, q_xor);
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) launder(qf[kk]);

        // K (A of S^T = K Q^T): key col (+32 per slab), bytes 64 kk + 32 half .. +31,
        // i.e. chunks 4 kk + 2 half and 4 kk + 2 half + 1 of the key row.
        int koff[D / 64][2];
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
            for (int j = 0; j < 2; ++j) koff[kk][j] = col * T::kRowK + 16 * ((4 * kk + 2 * half + j) ^ kswz<D>(col));
        // V (A of O^T += V^T P^T) through ds_read_b64_tr_b16, as in the bf16 kernel.
        int voff[D / 32][2];
        {
            const int G4 = lane >> 4, j = lane & 15;
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const int key = 8 * hs + 4 * (G4 >> 1) + (j >> 2);
#pragma unroll
                for (int d32 = 0; d32 < D / 32; ++d32) {
                    const int dim = 32 * d32 + 16 * (G4 & 1) + 4 * (j & 3);
                    voff[d32][hs] = T::kBytesK + key * T::kRowV + 16 * ((dim >> 3) ^ swz<D>(key)) + 2 * (dim & 7);
                }
            }
        }

        f32x16 oacc[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
        float m_ref = -INFINITY, l_sum = 0.f;
        const int32_t* kexp = Ke + (size_t)bh * nkt;

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        auto step = [&](auto stage_c, auto rescale_c, auto first_c, int t) __attribute__((always_inline)) {
            constexpr int st = kSingleStage ? 0 : decltype(stage_c)::value;
            constexpr bool RESCALE = decltype(rescale_c)::value;
            constexpr bool FIRST = decltype(first_c)::value;  // tile 0 of a fixed-reference pass
            if (!kSingleStage && t + 1 < ntiles) dma_tile(st ^ 1, (t + 1) * kBK);
            const char* Sb = smem + st * T::kStage;
            const int kv0 = t * kBK;

            if (kv0 < wmax) {
                // E8M0 scale of each 64-key half (a half wholly past N has no code tile)
                int kscale[kBK / kFp8KTile];
#pragma unroll
                for (int j = 0; j < kBK / kFp8KTile; ++j) {
                    const int kt = t * (kBK / kFp8KTile) + j;
                    kscale[j] = 127 + (kt < nkt ? kexp[kt] : 0);
                }
                f32x16 s[kSub];
#pragma unroll
                for (int sub = 0; sub < kSub; ++sub) s[sub] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
                    for (int sub = 0; sub < kSub; ++sub) {
                        const char* kb = Sb + sub * 32 * T::kRowK;
                        const u32x4 lo = *reinterpret_cast<const u32x4*>(kb + koff[kk][0]);
                        const u32x4 hi = *reinterpret_cast<const u32x4*>(kb + koff[kk][1]);
                        const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        s[sub] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[kk], s[sub], 0, 0, 0,
                                                                                  kscale[sub / 2], 0, qscale);
                    }
                // Schedule: the K operand reads run one product ahead of their use.
                // Groups: 4 LDS reads, then (1 MFMA, 2 LDS reads) repeated, then the
                // last 2 MFMAs.
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int g = 0; g < kSub * (D / 64) - 2; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (kv0 + kBK > wmin) {  // tile crosses some row's key limit
#pragma unroll
                    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kv0 + sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                            if (key >= lim) s[sub][r] = -INFINITY;
                        }
                }
                if constexpr (RESCALE || FIRST) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
                    mx = halves_max(mx);
                    const float mt = mx * c;  // this tile's row max, log2 units
                    if constexpr (!RESCALE) {
                        m_ref = mt;  // the reference for the whole block
                    } else if (__any(mt > m_ref + kStaleMax)) {
                        const float m_new = fmaxf(m_ref, mt);
                        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                        l_sum *= alpha;
#pragma unroll
                        for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[d32][r] *= alpha;
                        m_ref = m_new;
                    }
                }
                const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;

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
                        l_sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv), ones, l_sum, false);
                    }
                }
#pragma unroll
                for (int ks = 0; ks < kBK / 16; ++ks)
#pragma unroll
                    for (int d32 = 0; d32 < D / 32; ++d32) {
                        const char* vb = Sb + 16 * ks * T::kRowV;
                        const u32x2 lo = tr_read(vb + voff[d32][0]), hi = tr_read(vb + voff[d32][1]);
                        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
                        oacc[d32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                            __builtin_bit_cast(bf16x8, pk[ks]),
                                                                            oacc[d32], 0, 0, 0);
                    }
            }
            if constexpr (kSingleStage) {
                __syncthreads();  // every wave has finished reading the stage
                if (t + 1 < ntiles) dma_tile(0, (t + 1) * kBK);
            }
            if (t + 1 < ntiles) {  // after the last tile, the next block's first barrier serves
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
            // As in the bf16 kernel (without key limits): the first pass keeps each row's first-tile max
            // as its reference; if that overflowed P or O somewhere in the block (a
            // non-finite sum or output), the workgroup computes the block again with
            // the reference following the running max.
            float chk[4] = {l_sum, 0.f, 0.f, 0.f};
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
                l_sum = 0.f;
                if (ntiles > 0) dma_tile(0, 0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                run(std::true_type{});
            }
        }

        const float l_tot = halves_sum(l_sum);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        // O leaves in 16-byte stores (8 consecutive dims per lane, see o_rows16)
        u32x4 ov[D / 32][2];
#pragma unroll
        for (int d32 = 0; d32 < D / 32; ++d32) o_rows16(oacc[d32], inv, ov[d32]);
        if (qrow < N) {
            bf16* orow = O + ((size_t)bh * N + qrow) * D;
#pragma unroll
            for (int d32 = 0; d32 < D / 32; ++d32)
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    *reinterpret_cast<u32x4*>(orow + 32 * d32 + 16 * p + 8 * half) = ov[d32][p];
            if (half == 0)
                LSE[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <int D, bool CAUSAL, bool MASK, bool QRAW>
hipError_t launch(const uint8_t* qc, const int32_t* qe, const bf16* qb, const int8_t* signs, const uint8_t* kc,
                  const int32_t* ke, const bf16* v, bf16* o, float* lse, int B, int H, int N, ScoreSign sg,
                  const int32_t* kv_limit, hipStream_t stream) {
    const int nqb = (N + kBQ - 1) / kBQ;
    const long long items = (long long)B * H * nqb;
    unsigned grid = 0;
    const hipError_t e = walk_grid(items, !MASK, &grid);
    if (e != hipSuccess) return e;
    return launch_kernel(fwd_kernel<D, CAUSAL, MASK, QRAW>, dim3(grid), dim3(kThreads), 0, stream, qc, qe, qb, signs,
                         kc, ke, v, o, lse, H, N, nqb, (int)items, sg.c, sg.and_mask, sg.xor_mask, kv_limit);
}

}  // namespace fp8

hipError_t launch_fp8_quantize(const void* x, const int8_t* signs, uint8_t* codes, int32_t* exps, int B, int H, int N,
                               int d, int tile_rows, hipStream_t stream) {
    const bf16* X = static_cast<const bf16*>(x);
    const int nt = (N + tile_rows - 1) / tile_rows;
    const dim3 grid((unsigned)((long long)B * H * nt));
#define FA_QUANT(DD, TT)                                                                                    \
    if (d == DD && tile_rows == TT) {                                                                       \
        return launch_kernel(fp8::quant_kernel<DD, TT>, grid, dim3(fp8::kQuantThreads), 0, stream, X, signs, \
                             codes, exps, N, nt);                                                           \
    }
    FA_QUANT(64, kFp8QTile)
    FA_QUANT(64, kFp8KTile)
    FA_QUANT(128, kFp8QTile)
    FA_QUANT(128, kFp8KTile)
#undef FA_QUANT
    return hipErrorInvalidValue;
}

hipError_t launch_fused_fp8(const uint8_t* qc, const int32_t* qe, const void* q_bf16, const int8_t* signs,
                            const uint8_t* kc, const int32_t* ke, const void* v, void* o, float* lse, int B, int H,
                            int N, int d, bool causal, float scale, const int32_t* kv_limit, hipStream_t stream) {
    using namespace fp8;
    const bf16* Qb = static_cast<const bf16*>(q_bf16);
    const bf16* Vb = static_cast<const bf16*>(v);
    bf16* Ob = static_cast<bf16*>(o);
    // the rotation multiplies every score by d
    const ScoreSign sg = score_sign(scale, kLog2e / (float)d, kSignE4m3x4);
    const bool mask = kv_limit != nullptr;
    const bool raw = q_bf16 != nullptr;
#define FA_DISPATCH(DD, CC, MM)                                                                                 \
    if (d == DD && causal == CC && mask == MM)                                                                  \
        return raw ? launch<DD, CC, MM, true>(qc, qe, Qb, signs, kc, ke, Vb, Ob, lse, B, H, N, sg, kv_limit, stream) \
                   : launch<DD, CC, MM, false>(qc, qe, Qb, signs, kc, ke, Vb, Ob, lse, B, H, N, sg, kv_limit, stream);
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

// fa_sizes.h -- tile and split sizes shared by kernels and the host-side
// launchers: the decode path's page and split sizes and its workspace layout,
// and the FP8 path's tile sizes.
#pragma once

#include <stdint.h>

namespace fa {

// Decode over a paged cache: pages of kDecodePage tokens; the key range of a
// sequence is split into pieces of kDecodeSplitKeys keys (one workgroup each).
// The workspace holds the splits' unnormalised outputs (fp32 [B*H*max_splits, d], padded to 64
// floats) and then their (max, sum) pairs (fp32 [B*H*max_splits, 2]).
constexpr int kDecodePage = 16;
constexpr int kDecodeSplitKeys = 256;
inline int64_t decode_max_splits(int max_pages) {
    return ((int64_t)max_pages * kDecodePage + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
}
inline int64_t decode_part_o_floats(int B, int H, int d, int max_pages) {
    return ((int64_t)B * H * decode_max_splits(max_pages) * d + 63) / 64 * 64;
}
inline int64_t decode_workspace_floats(int B, int H, int d, int max_pages) {
    return decode_part_o_floats(B, H, d, max_pages) + ((int64_t)B * H * decode_max_splits(max_pages) * 2 + 63) / 64 * 64;
}

// The no-allocation decode entry point keeps its splits' partials in a static
// device buffer of this many bytes per GPU instead of a caller's workspace.
constexpr int64_t kDecodeScratchBytes = (int64_t)16 << 20;

// FP8 forward: Q codes come in tiles of kFp8QTile rows, K codes in tiles of
// kFp8KTile rows, one int32 exponent per tile ([B, H, ceil(N / tile)]).
constexpr int kFp8QTile = 32;
constexpr int kFp8KTile = 64;

}  // namespace fa

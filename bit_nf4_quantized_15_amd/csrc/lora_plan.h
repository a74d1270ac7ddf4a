// Host-side work split of the LoRA reduction kernels; shared by the launchers
// and by the workspace-size queries so that both always agree.
#pragma once

#include <algorithm>
#include <cstdint>

namespace qlora {

struct SplitPlan {
    int splits;  // number of partial sums
    int chunk;   // reduction length per split (multiple of 64)
};

// Splits of a reduction of length len (a multiple of 64 per split, at most
// max_chunk) over `tiles` independent output tiles: enough splits for about
// 256 workgroups, as few as the chunk limit allows otherwise.
inline SplitPlan plan_split(int64_t tiles, int64_t len, int64_t max_chunk) {
    const int64_t steps = (len + 63) / 64;
    int64_t s = std::max<int64_t>((steps + max_chunk / 64 - 1) / (max_chunk / 64), (256 + tiles - 1) / tiles);
    s = std::max<int64_t>(1, std::min<int64_t>(s, steps));
    const int64_t chunk = (steps + s - 1) / s * 64;
    return SplitPlan{(int)((len + chunk - 1) / chunk), (int)chunk};
}

// out[M, r] = X[M, C] * Yt[r, C]^T : one workgroup per 128 rows of M and split of C;
// all of a split's X loads are in flight at once, so ranks above 96 (4 column
// tiles of accumulators) take half the columns per split
inline int nt_max_chunk(int r) { return r <= 96 ? 512 : 256; }
inline SplitPlan plan_nt(int64_t M, int64_t C, int r) { return plan_split((M + 127) / 128, C, nt_max_chunk(r)); }

// out[D, r] = X[M, D]^T * S[M, r] : one workgroup per 128 columns of X and split of M;
// the split's slice of S (32 * ceil(r / 32) rows) must fit next to the X tiles
inline int tn_max_chunk(int r) { return r <= 96 ? 512 : 256; }
inline SplitPlan plan_tn(int64_t M, int64_t D, int r) { return plan_split((D + 127) / 128, M, tn_max_chunk(r)); }

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Workspace of one split contraction: a 64-bit publication tag per (output tile,
// split), then the fp32 partial tiles of every split but the last (128 rows x
// 32 * ceil(r / 32) columns each).  Nothing in it has to start at zero.
inline size_t split_tags_bytes(int64_t tiles, const SplitPlan& sp) { return align256((size_t)tiles * sp.splits * 8); }
inline size_t split_ws_bytes(int64_t tiles, const SplitPlan& sp, int r) {
    const size_t tile_bytes = (size_t)128 * 32 * ((r + 31) / 32) * 4;
    return split_tags_bytes(tiles, sp) + align256((size_t)(sp.splits - 1) * tiles * tile_bytes);
}
inline size_t nt_ws_bytes(int64_t M, int64_t C, int r) { return split_ws_bytes((M + 127) / 128, plan_nt(M, C, r), r); }
inline size_t tn_ws_bytes(int64_t M, int64_t D, int r) { return split_ws_bytes((D + 127) / 128, plan_tn(M, D, r), r); }

}  // namespace qlora

// Host-side work split of the LoRA reduction kernels; shared by the launchers
// and by the workspace-size queries so that both always agree.
#pragma once

#include <algorithm>
#include <cstdint>

namespace qlora {

struct SplitPlan {
    int splits;  // number of partial sums
    int chunk;   // reduction length per split (multiple of 16)
};

constexpr int kGroupTarget = 512;  // workgroups (2 per CU) for an HBM-bound pass

inline SplitPlan make_plan(int64_t tiles, int64_t len, int min_len) {
    int64_t want = std::max<int64_t>(1, kGroupTarget / std::max<int64_t>(1, tiles));
    int64_t maxs = std::max<int64_t>(1, len / min_len);
    int64_t s = std::min(want, maxs);
    int64_t chunk = ((len + s - 1) / s + 15) / 16 * 16;
    if (chunk < 16) chunk = 16;
    s = (len + chunk - 1) / chunk;
    if (s < 1) s = 1;
    return SplitPlan{(int)s, (int)chunk};
}

// out[M, r] = X[M, C] * Yt[r, C]^T : one workgroup per 128 rows of M and split of C;
// a split is a multiple of 64 columns, at most 512 (the kernel's LDS slice), and
// there are enough splits for about 256 workgroups
inline SplitPlan plan_nt(int64_t M, int64_t C) {
    const int64_t tiles = (M + 127) / 128;
    const int64_t steps = (C + 63) / 64;
    int64_t s = std::max<int64_t>((steps + 7) / 8, (256 + tiles - 1) / tiles);
    s = std::min<int64_t>(s, steps);
    const int64_t chunk = (steps + s - 1) / s * 64;
    return SplitPlan{(int)((C + chunk - 1) / chunk), (int)chunk};
}

// out[D, r] = X[M, D]^T * S[M, r] : one workgroup per 128 columns of X and split of M
inline SplitPlan plan_tn(int64_t M, int64_t D) { return make_plan((D + 127) / 128, M, 128); }

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace qlora

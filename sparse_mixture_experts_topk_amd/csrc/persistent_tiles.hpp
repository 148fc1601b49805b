// Work split of the persistent tiled GEMM launches (bf16 and fp8).
#pragma once
#include <algorithm>

#include "device_common.hpp"

namespace moe {

// The expert-major tile list (token tiles fastest) is cut into 8 contiguous
// shares, one per XCD; the `slots` workgroups of XCD x (blockIdx = slot * 8 +
// x) take its full tiles in rounds: tiles share_begin + slot + i * slots,
// i < R.  The share's last `tail` < slots tiles are either taken whole by the
// first `tail` slots (data-parallel), or (split) cut along K into `slots`
// near-equal runs of P slices, one per workgroup, each covering parts of at
// most two tiles; the parts are written as fp32 partial tiles and summed by a
// second kernel in K order, which keeps the result independent of timing.
struct TileSplit {
  int share_begin, R, tail, P;

  // Tiles of `rows` tokens x n_tiles channel tiles over every expert group.
  __device__ static int total_tiles(const int32_t* offs, int E, int n_tiles, int rows) {
    int total = 0;
    for (int e = 0; e < E; ++e)
      total += (__builtin_amdgcn_readfirstlane(offs[e + 1]) -
                __builtin_amdgcn_readfirstlane(offs[e]) + rows - 1) / rows;
    return total * n_tiles;
  }
  __device__ static TileSplit of(int total, int xcd, int slots, int KT) {
    TileSplit t;
    const int per_xcd = (total + 7) >> 3;
    t.share_begin = xcd * per_xcd;
    const int len = max(0, min(t.share_begin + per_xcd, total) - t.share_begin);
    t.R = len / slots;
    t.tail = len - t.R * slots;
    t.P = (t.tail * KT + slots - 1) / slots;
    return t;
  }
};

constexpr int kMaxPersistentGroups = 256;

int device_cu_count();

// Workgroups of a persistent launch: one per CU, at most kMaxPersistentGroups,
// a multiple of the 8 XCDs, and no more than there are tiles.
inline int64_t persistent_grid(int64_t max_tiles) {
  const int64_t cus = std::min<int64_t>(device_cu_count(), kMaxPersistentGroups);
  return std::max<int64_t>(8, std::min<int64_t>((max_tiles + 7) / 8 * 8, cus / 8 * 8));
}

}  // namespace moe

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
// A split kernel still takes the tail whole (`whole_tail`, P = 0) when whole
// tiles would leave less than an eighth of the share's workgroup time idle:
// the runs' partial tiles, their sum, and workgroups that no longer read the
// same K slices at the same time cost more than that (down projection,
// MI355X: Mixtral prefill, a last round 92% full, 1.81 -> 1.67 ms whole;
// 256 experts, a 17th round 6% full, 1.69 -> 1.65 ms; a Zipf-skewed batch
// with a second round 7% full needs the split, 0.68 against 1.07 ms).
struct TileSplit {
  int share_begin, R, tail, P;
  bool whole_tail;

  __device__ static TileSplit of(int total, int xcd, int slots, int KT) {
    TileSplit t;
    const int per_xcd = (total + 7) >> 3;
    t.share_begin = xcd * per_xcd;
    const int len = max(0, min(t.share_begin + per_xcd, total) - t.share_begin);
    t.R = len / slots;
    t.tail = len - t.R * slots;
    t.whole_tail = t.tail > 0 && 8 * (slots - t.tail) < slots * (t.R + 1);
    t.P = t.whole_tail ? 0 : (t.tail * KT + slots - 1) / slots;
    return t;
  }
};

// Cumulative token tiles of the expert groups: pre[e] = the sum over e' < e
// of ceil(rows of e' / rows_per_tile), for e = 0 .. E (so pre[E] is the
// number of token tiles).  Built in LDS from the group offsets (in LDS) by
// one wavefront, 64 groups per step with a wavefront prefix sum; the caller
// synchronises before reading it.
__device__ inline void build_tile_prefix(const int32_t* offs, int E, int rows_per_tile, int32_t* pre,
                                         int lane) {
  int carry = 0;
  for (int base = 0; base <= E; base += 64) {
    const int e = base + lane;
    const int m = e < E ? (offs[e + 1] - offs[e] + rows_per_tile - 1) / rows_per_tile : 0;
    int v = m;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(v, d);
      if (lane >= d) v += u;
    }
    if (e <= E) pre[e] = carry + v - m;
    carry += __shfl(v, 63);
  }
}

// Tile t of the expert-major tile list (token tiles fastest, n_tiles channel
// tiles per token tile), t < pre[E] * n_tiles: its group e (a binary search
// of the prefix for the last group whose first tile is <= t, which is never
// empty), the group's rows [r0, r1), and its token tile m and channel tile n.
// Every argument and result is uniform.
__device__ inline void find_tile(const int32_t* offs, const int32_t* pre, int E, int n_tiles, int t, int& e,
                                 int& r0, int& r1, int& m, int& n) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(pre[mid]) * n_tiles <= t) lo = mid;
    else hi = mid;
  }
  e = lo;
  const int p0 = __builtin_amdgcn_readfirstlane(pre[lo]);
  const int mt = __builtin_amdgcn_readfirstlane(pre[lo + 1]) - p0;
  const int l = t - p0 * n_tiles;
  r0 = __builtin_amdgcn_readfirstlane(offs[lo]);
  r1 = __builtin_amdgcn_readfirstlane(offs[lo + 1]);
  m = l % mt;
  n = l / mt;
}

constexpr int kMaxPersistentGroups = 256;

int device_cu_count();

// Workgroups of a persistent launch: one per CU, at most kMaxPersistentGroups,
// a multiple of the 8 XCDs, and no more than there are tiles.
inline int64_t persistent_grid(int64_t max_tiles) {
  const int64_t cus = std::min<int64_t>(device_cu_count(), kMaxPersistentGroups);
  return std::max<int64_t>(8, std::min<int64_t>((max_tiles + 7) / 8 * 8, cus / 8 * 8));
}

}  // namespace moe

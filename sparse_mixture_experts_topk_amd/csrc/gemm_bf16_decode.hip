// bf16 grouped expert GEMMs for few tokens per expert (decode): weight streaming.
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x);
// "Mixtral and Mixture-of-Experts, Explained" notes the extra memory loads of
// running more than one expert per device -- at decode the layer is bound by
// reading the touched experts' weights once.
//
// A row group is 16 output channels (dual: 16 rows of w1 and the same 16 of
// w3) of one expert against one tile of up to 16 of its tokens; each
// wavefront owns one row group and streams all of K.  The matrix-core
// operand layout (lane = row, 4 lanes per row) would read only 64 contiguous
// bytes per row per load instruction, which measured 3.5 TB/s on MI355X for a
// pure read of this pattern; loading ROWS rows x (1024 / ROWS) contiguous
// bytes per instruction reached 6.2-6.5 TB/s.  So each K stage is read in the
// wide pattern (non-temporal: read once), written to the wavefront's own LDS
// tile (16-byte chunks XOR-swizzled by row, no bank conflicts), and read back
// in the v_mfma_f32_16x16x32_bf16 layout.  The LDS tile is private to the
// wavefront: LDS operations of one wavefront execute in order, so no barrier
// is needed.  The token operand (a few rows, L2-resident) is read directly.
//
// Workgroups are dispatched round-robin over the 8 XCDs.  In that order every
// XCD streams row groups spread over all of w1 and w3 at once, and the gate/up
// time then depended on where the weights were allocated: 289-336 us on four
// copies of the same weights in one process (MI355X, Mixtral decode batch).
// With the workgroups of each XCD on one contiguous eighth of the row groups it
// was 276-287 us on all four.  For down (one matrix) an eighth of every
// expert's channel groups per XCD measured the same as round-robin on boxes
// where neither was slow (138-140 us), and a contiguous eighth of all of w2
// (one expert per XCD) was slower (150 us).  With many experts, gate/up takes
// the persistent form (grouped_gemm_bf16_decode_tiles), which spreads the
// touched experts' groups evenly over the XCDs, and down a contiguous eighth.
#include "device_common.hpp"
#include "launch.hpp"
#include "lane_ops.hpp"
#include "lds_stream.hpp"
#include "persistent_tiles.hpp"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

// A K stage of a row group: ROWS rows x (1024 / ROWS) contiguous bytes per load
// instruction, KB elements per row per stage.
template <bool DUAL, int ROWS>
struct StreamGeom {
  static constexpr int KB = 512 / ROWS;        // elements per row per stage
  static constexpr int CPR = KB / 8;           // 16-byte chunks per row per stage
  static constexpr int NL = 16 / ROWS;         // load instructions per matrix per stage
  static constexpr int NM = DUAL ? 2 : 1;
  static constexpr int ROW_BYTES = KB * 2;
  static constexpr int KEY_MASK = (CPR < 16 ? CPR : 16) - 1;
  static constexpr int WAVE_LDS = NM * 16 * ROW_BYTES;   // one wavefront's private tile
  static constexpr int LPR = kWave / ROWS;     // lanes per row (== CPR)
};

// One row group streamed over all of K into acc: the 16 weight rows at pw[m]
// (dual: w1 and w3) against the token operand, through the wavefront's private
// LDS tile `lds`.  Matrix instruction j of a stage takes, in lane (t, g), K
// elements 32 j + 8 g .. + 7 of token t.  One token load carries P of them:
// lane (t, g) with t = s (16 / P) + u reads token u at px (its row, plus
// 8 g + 32 s; lanes with u past the tile's rows have tok_ok false and read
// zeros), operands s, P + s, ...; a row rotation brings operand j to lanes
// (u, g).  The other lanes then hold other operands: columns u >= 16 / P,
// past the tile's rows, which are never stored (a column depends only on its
// own token), so the stored result does not depend on P.
template <bool DUAL, int ROWS, int P>
__device__ __forceinline__ void stream_row_group(const uint16_t* const* pw, const uint16_t* px, bool tok_ok,
                                                 int K, uint8_t* lds, f32x4_t* acc) {
  using S = StreamGeom<DUAL, ROWS>;
  constexpr int NOP = S::KB / 32;              // token operands per stage
  static_assert(NOP % P == 0, "whole token loads per stage");
  const int lane = threadIdx.x & 63;
  const int lrow = lane / S::LPR, lch = lane % S::LPR;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int m = 0; m < S::NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nst = K / S::KB;
  for (int st = 0; st < nst; ++st) {
    const int k0 = st * S::KB;
    uint4 v[S::NM][S::NL];
#pragma unroll
    for (int m = 0; m < S::NM; ++m)
#pragma unroll
      for (int i = 0; i < S::NL; ++i)
        v[m][i] = load_stream16(pw[m] + (int64_t)(i * ROWS + lrow) * K + k0 + lch * 8);
    uint4 xv[NOP / P];
#pragma unroll
    for (int i = 0; i < NOP / P; ++i)
      xv[i] = tok_ok ? *reinterpret_cast<const uint4*>(px + k0 + i * P * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < S::NM; ++m)
#pragma unroll
      for (int i = 0; i < S::NL; ++i) {
        const int row = i * ROWS + lrow;
        const int pc = lch ^ (row & S::KEY_MASK);
        *reinterpret_cast<uint4*>(&lds[(m * 16 + row) * S::ROW_BYTES + pc * 16]) = v[m][i];
      }
#pragma unroll
    for (int j = 0; j < NOP; ++j) {
      const int pc = (4 * j + g) ^ (r & S::KEY_MASK);
      const uint4 xj = from_lane_above_even(xv[j / P], j % P * (16 / P));
#pragma unroll
      for (int m = 0; m < S::NM; ++m) {
        const uint4 a = *reinterpret_cast<const uint4*>(&lds[(m * 16 + r) * S::ROW_BYTES + pc * 16]);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(xj), acc[m], 0, 0, 0);
      }
    }
  }
}

// Calls run(IntC<P>) with the most token operands per load (4, 2 or 1) that a
// tile of `rows` rows allows at this stage width.
template <int NOP, class F>
__device__ __forceinline__ void with_token_packing(int rows, F&& run) {
  if constexpr (NOP % 4 == 0) {
    if (rows <= 4) return run(IntC<4>{});
  }
  if constexpr (NOP % 2 == 0) {
    if (rows <= 8) return run(IntC<2>{});
  }
  run(IntC<1>{});
}

// One output group: 16 rows of expert e's weights (dual: w1 and w3, channels
// cg * 16 ..) against the token tile of `rows` permuted rows from row0; writes
// h (dual: SwiGLU, bf16) or y_perm (fp32) for the tile's rows.
template <bool DUAL, int ROWS>
__device__ __forceinline__ void decode_group(const uint16_t* __restrict__ act, const uint16_t* __restrict__ wa,
                                             const uint16_t* __restrict__ wb, int N, int K, void* __restrict__ out,
                                             const int32_t* __restrict__ gather, int k, int Tk, int e, int cg,
                                             int row0, int rows, uint8_t* lds) {
  using S = StreamGeom<DUAL, ROWS>;
  const int lane = threadIdx.x & 63;
  const uint16_t* pw[S::NM];
  pw[0] = wa + ((int64_t)e * N + cg * 16) * K;
  if constexpr (DUAL) pw[1] = wb + ((int64_t)e * N + cg * 16) * K;
  // matrix-core operand: lane (r, g) feeds row r, chunk 4 j + g of MFMA j
  const int r = lane & 15, g = lane >> 4;
  f32x4_t acc[S::NM];
  with_token_packing<S::KB / 32>(rows, [&](auto pc) __attribute__((always_inline)) {
    constexpr int TPL = 16 / decltype(pc)::value;     // token lanes per row of 16 lanes
    const int u = r % TPL;
    const bool tok_ok = u < rows;
    // token operand row: a permuted row, or (gather) the token row of x that
    // permuted row copies (slot t*k + s -> token t; the shared expert's T*k + t -> t)
    int arow = row0 + (tok_ok ? u : 0);
    if (gather != nullptr) {
      const int src = gather[arow];
      arow = src < Tk ? src / k : src - Tk;
    }
    const uint16_t* px = act + (int64_t)arow * K + g * 8 + r / TPL * 32;
    stream_row_group<DUAL, ROWS, decltype(pc)::value>(pw, px, tok_ok, K, lds, acc);
  });

  // 16x16 accumulator: lane holds token column (lane & 15), channels 4 * (lane >> 4) + 0..3.
  const int tcol = lane & 15;
  if (tcol >= rows) return;
  const int c = cg * 16 + (lane >> 4) * 4;
  const int64_t orow = row0 + tcol;
  if constexpr (DUAL) {
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = swiglu_fast(acc[0][i], acc[1][i]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * N + c) =
        make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * N + c) =
        make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
  }
}

template <bool DUAL, int ROWS, int MIN_WAVES, bool CONTIG>
__global__ __launch_bounds__(kWavesPerBlock * kWave, MIN_WAVES) void grouped_gemm_bf16_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int N, int K,
    void* __restrict__ out, int tok_tiles, const int32_t* __restrict__ gather, int k, int Tk) {
  using S = StreamGeom<DUAL, ROWS>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWavesPerBlock][S::WAVE_LDS];

  const int w = threadIdx.x >> 6;
  const int groups = N / 16;
  // Each XCD streams its own part of the weights (the grid is whole rounds of
  // the 8 XCDs): CONTIG (gate/up) one contiguous eighth of all row groups,
  // otherwise the same eighth of every expert's channel groups.
  int cg, rest;
  if constexpr (CONTIG) {
    const int gid = xcd_remap(blockIdx.x, gridDim.x) * kWavesPerBlock + w;
    cg = gid % groups;
    rest = gid / groups;
  } else {
    const int gx = (groups + 7) / 8;                           // channel groups per XCD
    const int lw = (blockIdx.x >> 3) * kWavesPerBlock + w;     // wavefront within its XCD
    cg = (blockIdx.x & 7) * gx + lw % gx;
    rest = lw / gx;
    if (cg >= groups) return;
  }
  const int tt = rest % tok_tiles;
  const int e = rest / tok_tiles;
  if (e >= E) return;
  const int row0 = offsets[e] + tt * 16;
  const int rows = min(16, offsets[e + 1] - row0);
  if (rows <= 0) return;
  decode_group<DUAL, ROWS>(act, wa, wb, N, K, out, gather, k, Tk, e, cg, row0, rows, lds[w]);
}

// Many experts (at most a few rows each, most of them untouched; gate/up): a grid of the
// resident capacity.  Each workgroup builds the token-tile prefix of the expert
// groups once (from the offsets, in LDS); the output groups are numbered over
// the token tiles that exist only (expert-major, channel groups fastest), each
// XCD takes a contiguous eighth of them, and its wavefronts take every
// (grid / 8 * 4)-th group of that eighth.  With the whole grid laid over all
// E + S groups instead, each XCD's share of real work was set by how many
// touched experts fell in its eighth (1.22 x the mean for the busiest XCD at
// 256 experts top-8 + shared, 16 tokens).
template <bool DUAL, int ROWS, int MIN_WAVES>
__global__ __launch_bounds__(kWavesPerBlock * kWave, MIN_WAVES) void grouped_gemm_bf16_decode_tiles(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int N, int K,
    void* __restrict__ out, const int32_t* __restrict__ gather, int k, int Tk) {
  using S = StreamGeom<DUAL, ROWS>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWavesPerBlock][S::WAVE_LDS];
  __shared__ int32_t offs[kMaxExpertGroups + 1];
  __shared__ int32_t pre[kMaxExpertGroups + 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i <= E; i += kWavesPerBlock * kWave) offs[i] = offsets[i];
  __syncthreads();
  if (w == 0) build_tile_prefix(offs, E, 16, pre, lane);
  __syncthreads();
  const int groups = N / 16;
  const int total = __builtin_amdgcn_readfirstlane(pre[E]) * groups;   // output groups that exist
  const int per_xcd = (total + 7) / 8;
  const int x = blockIdx.x & 7;
  const int nslots = (gridDim.x >> 3) * kWavesPerBlock;
  for (int li = (blockIdx.x >> 3) * kWavesPerBlock + w; li < per_xcd; li += nslots) {
    const int t = x * per_xcd + li;
    if (t >= total) break;
    int e, r0, r1, m, cg;
    find_tile(offs, pre, E, groups, t, e, r0, r1, m, cg);
    const int row0 = r0 + m * 16;
    decode_group<DUAL, ROWS>(act, wa, wb, N, K, out, gather, k, Tk, e, cg, row0, min(16, r1 - row0),
                             lds[w]);
  }
}

// Down projection and combine in one launch, for a decode batch whose experts
// hold one token tile each (T <= 16, top-2, nothing dropped, E <= 16).  A
// workgroup owns 16 output channels; its wavefront w streams expert w's 16
// rows of w2 against that expert's h rows (the same row group as the down
// kernel above).  The fp32 results meet in LDS, indexed by permuted row, and
// the workgroup then forms y[t] = fma(G1, y_e1, G0 * y_e0) for its channels in
// the order the combine kernel uses, so the result equals the separate down +
// combine calls bit for bit, without the y_perm round trip or the extra launch.
constexpr int kFusedMaxExperts = 16;
constexpr int kFusedMaxRows = 32;     // T * top_k

template <int ROWS>
__global__ __launch_bounds__(kFusedMaxExperts * kWave) void down_combine_bf16_decode(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets, const uint16_t* __restrict__ w2,
    int N, int K, const int32_t* __restrict__ slot_to_row, const float* __restrict__ gw, int T,
    uint16_t* __restrict__ y) {
  using S = StreamGeom<false, ROWS>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFusedMaxExperts][S::WAVE_LDS];
  __shared__ float4 yrow[kFusedMaxRows][4];          // [permuted row][channel quad], fp32

  const int lane = threadIdx.x & 63, e = threadIdx.x >> 6;   // wavefront = expert (blockDim = 64 E)
  const int cg = xcd_remap(blockIdx.x, gridDim.x);   // an eighth of the channels per XCD
  if (cg >= N / 16) return;                           // the whole workgroup: no barrier reached
  const int row0 = offsets[e];
  const int rows = min(16, offsets[e + 1] - row0);
  if (rows > 0) {
    const uint16_t* pw[1] = {w2 + ((int64_t)e * N + cg * 16) * K};
    const int r = lane & 15, g = lane >> 4;
    f32x4_t acc[1];
    with_token_packing<S::KB / 32>(rows, [&](auto pc) __attribute__((always_inline)) {
      constexpr int TPL = 16 / decltype(pc)::value;
      const int u = r % TPL;
      const bool tok_ok = u < rows;
      const uint16_t* px = h + (int64_t)(row0 + (tok_ok ? u : 0)) * K + g * 8 + r / TPL * 32;
      stream_row_group<false, ROWS, decltype(pc)::value>(pw, px, tok_ok, K, lds[e], acc);
    });
    if (r < rows) yrow[row0 + r][g] = make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
  }
  __syncthreads();
  for (int o = threadIdx.x; o < T * 4; o += blockDim.x) {
    const int t = o >> 2, q = o & 3;
    const int2 rr = reinterpret_cast<const int2*>(slot_to_row)[t];
    const float2 gg = reinterpret_cast<const float2*>(gw)[t];
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (rr.x >= 0) {
      const float4 a = yrow[rr.x][q];
      v = make_float4(gg.x * a.x, gg.x * a.y, gg.x * a.z, gg.x * a.w);
    }
    if (rr.y >= 0) {
      const float4 b = yrow[rr.y][q];
      v = make_float4(fmaf(gg.y, b.x, v.x), fmaf(gg.y, b.y, v.y), fmaf(gg.y, b.z, v.z), fmaf(gg.y, b.w, v.w));
    }
    *reinterpret_cast<uint2*>(y + (int64_t)t * N + cg * 16 + q * 4) =
        make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

// Gate/up with 32 or more expert groups: the persistent form above (256
// experts top-8 + shared, 16 tokens: 0.528 -> 0.518 ms); otherwise a grid over
// all groups, a contiguous eighth of the row groups per XCD.  Down: a
// contiguous eighth with 32 or more expert groups, several whole experts per
// XCD (0.287 -> 0.264 ms; the persistent form: 0.271 ms); with fewer, an
// eighth of every expert's channel groups (Mixtral decode batch: 138-140 us
// against 150 us with one expert per XCD).
constexpr int kManyExpertGroups = 32;
constexpr int kWgPerCuTiles = 4;     // resident workgroups per CU of the persistent form

template <bool DUAL, int ROWS, int MIN_WAVES, bool CONTIG>
hipError_t launch_mapped(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                         const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                         hipStream_t st, const int32_t* gather) {
  const int tok_tiles = (int)((max_rows_per_expert(s) + 15) / 16);
  const int64_t groups = (int64_t)expert_groups(s) * tok_tiles * (N / 16);
  if (groups <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  // whole rounds of the 8 XCDs (waves past the work exit)
  const int64_t per_xcd = CONTIG ? (groups + 8 * kWavesPerBlock - 1) / (8 * kWavesPerBlock)
                                 : ((int64_t)(N / 16 + 7) / 8 * expert_groups(s) * tok_tiles + kWavesPerBlock - 1) /
                                       kWavesPerBlock;
  const int64_t blocks = 8 * per_xcd;
  hipLaunchKernelGGL((grouped_gemm_bf16_decode<DUAL, ROWS, MIN_WAVES, CONTIG>), dim3((unsigned)blocks),
                     dim3(kWavesPerBlock * kWave), 0, st, act, offsets, expert_groups(s), wa, wb, N, K,
                     out, tok_tiles, gather, s.top_k, s.T * s.top_k);
  return hipGetLastError();
}

template <bool DUAL, int ROWS, int MIN_WAVES>
hipError_t launch_variant(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                          hipStream_t st, const int32_t* gather = nullptr) {
  if (max_rows_per_expert(s) <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  if (DUAL && expert_groups(s) >= kManyExpertGroups) {
    static_assert(kManyExpertGroups <= kMaxExpertGroups, "offset table in LDS");
    const int64_t blocks = (int64_t)device_cu_count() * kWgPerCuTiles / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_bf16_decode_tiles<DUAL, ROWS, MIN_WAVES>), dim3((unsigned)blocks),
                       dim3(kWavesPerBlock * kWave), 0, st, act, offsets, expert_groups(s), wa, wb, N, K, out,
                       gather, s.top_k, s.T * s.top_k);
    return hipGetLastError();
  }
  if (DUAL || expert_groups(s) >= kManyExpertGroups)
    return launch_mapped<DUAL, ROWS, MIN_WAVES, true>(s, act, offsets, wa, wb, N, K, out, st, gather);
  if constexpr (!DUAL)
    return launch_mapped<DUAL, ROWS, MIN_WAVES, false>(s, act, offsets, wa, wb, N, K, out, st, gather);
  return hipErrorInvalidValue;   // not reached
}

}  // namespace

hipError_t launch_decode_bf16(const moe_shape_t& s, bool dual, const uint16_t* act,
                              const int32_t* offsets, const uint16_t* wa, const uint16_t* wb,
                              int N, int K, void* out, hipStream_t st) {
  // 4 rows x 256 B per load instruction where K allows it.  At the Mixtral
  // decode batch (MI355X) gate/up streams 6.9 TB/s and down 6.8 TB/s; with
  // 8 rows x 128 B gate/up was 0.2-3% slower, down 13% slower, and with
  // 2 rows x 512 B down was 18% slower.
  if (dual && K % 128 == 0) return launch_variant<true, 4, 4>(s, act, offsets, wa, wb, N, K, out, st);
  if (dual) return launch_variant<true, 8, 4>(s, act, offsets, wa, wb, N, K, out, st);
  if (K % 128 == 0) return launch_variant<false, 4, 4>(s, act, offsets, wa, wb, N, K, out, st);
  return launch_variant<false, 8, 4>(s, act, offsets, wa, wb, N, K, out, st);
}

bool down_combine_fused(const moe_shape_t& s) {
  return s.act_dtype == MOE_BF16 && s.w_dtype == MOE_BF16 && s.top_k == 2 && s.n_shared == 0 &&
         s.capacity < 0 && s.T <= 16 && s.n_experts <= kFusedMaxExperts && s.d_model % 16 == 0;
}

hipError_t launch_down_combine_bf16(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                                    const uint16_t* w2, const int32_t* slot_to_row, const float* gw,
                                    uint16_t* y, hipStream_t st) {
  if (!down_combine_fused(s)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((s.d_model / 16 + 7) / 8 * 8)), block((unsigned)(s.n_experts * kWave));
  // the down kernel's choice: 4 rows x 256 B per load instruction when K allows it
  if (s.d_ff % 128 == 0)
    hipLaunchKernelGGL((down_combine_bf16_decode<4>), grid, block, 0, st, h, offsets, w2, s.d_model,
                       s.d_ff, slot_to_row, gw, s.T, y);
  else
    hipLaunchKernelGGL((down_combine_bf16_decode<8>), grid, block, 0, st, h, offsets, w2, s.d_model,
                       s.d_ff, slot_to_row, gw, s.T, y);
  return hipGetLastError();
}

hipError_t launch_gate_up_bf16_gather(const moe_shape_t& s, const uint16_t* x, const int32_t* perm_src,
                                      const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                                      uint16_t* h, hipStream_t st) {
  if (s.d_model % 128 == 0)
    return launch_variant<true, 4, 4>(s, x, offsets, w1, w3, s.d_ff, s.d_model, h, st, perm_src);
  return launch_variant<true, 8, 4>(s, x, offsets, w1, w3, s.d_ff, s.d_model, h, st, perm_src);
}

}  // namespace moe

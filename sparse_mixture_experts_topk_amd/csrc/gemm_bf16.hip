// bf16 grouped expert GEMMs on the gfx950 matrix cores (fp32 accumulate).
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x)
// (nn.Linear weights [out, in], no biases) and section "SwiGLU Experts";
// "How Mixtral 8x7B uses mixture of experts": tokens are batched by expert
// and the experts run in parallel.
//
// Both GEMMs are "NT": the token rows (x_perm or h) and the weight rows are
// contiguous along the contraction K.  The matrix-core operand A is the
// weight block (output channels) and B the token block, so an accumulator
// tile is [channel][token]; each lane then holds one token and runs of 4
// consecutive channels, which the epilogue stores as 8-byte (bf16 h) or
// 16-byte (fp32 y_perm) vectors.
//
// Prefill kernel (many tokens per expert): 256 lanes, a 256 x 256 tile
// (weights x tokens; the dual gate/up variant holds 128 w1 rows and the same
// 128 w3 rows so silu(g) * u is formed in registers), K staged 64 at a time
// through two LDS buffers of 2 x 32 KiB.  Rows are 128 bytes in LDS with the
// 16-byte chunks XOR-swizzled by (row & 7), so the fragment reads of 8
// consecutive rows hit distinct banks.  The next K slice is fetched into
// registers while the current one feeds v_mfma_f32_32x32x16_bf16; one
// barrier per slice.  Each wavefront owns 128 x 128 of the tile: 16
// accumulator blocks, 256 fp32 per lane.  Tiles are scheduled expert by
// expert with token tiles fastest and remapped so that consecutive tiles run
// on the same XCD and share its L2 copy of the weight tile.
//
// Decode kernel (few tokens per expert): weight streaming.  One wavefront
// owns 16 output channels (dual: of w1 and of w3) x up to 16 tokens over all
// of K, reading each weight row once in 16-byte vectors (lane = row r,
// K-quarter g), with the next K block prefetched into registers while
// v_mfma_f32_16x16x32_bf16 consumes the current one.  Any permutation of K
// is valid for a dot product as long as both operands use the same one, so
// each lane reads contiguous 64-byte runs.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------ prefill ---

constexpr int PF_ROWS = 256;         // rows of each LDS operand tile
constexpr int PF_BK = 64;            // K per stage (128 bytes per row)
constexpr int PF_TILE_BYTES = PF_ROWS * PF_BK * 2;
constexpr int PF_THREADS = 256;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <bool DUAL>
__global__ __launch_bounds__(PF_THREADS, 1) void grouped_gemm_bf16_prefill(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int N, int K,
    void* __restrict__ out, int n_tiles, int grid_padded) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][PF_TILE_BYTES];  // [stage][weights/tokens]

  constexpr int CH_TILE = DUAL ? 128 : 256;
  int e, r0, r1, mt, nt;
  const int tile = xcd_remap(blockIdx.x, grid_padded);
  if (!locate_tile(offsets, E, PF_ROWS, n_tiles, tile, e, r0, r1, mt, nt)) return;
  const int tok0 = r0 + mt * PF_ROWS;
  const int tok_rows = min(PF_ROWS, r1 - tok0);
  const int ch0 = nt * CH_TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // ---- global -> register loader: 8 chunks of each operand per lane ----
  const int lrow = tid >> 3, lchunk = tid & 7;   // rows lrow + 32 j, j = 0..7
  const int64_t rowstride = K;
  const uint16_t* pw0;   // weight rows 0..127 (dual: w1) at row lrow
  const uint16_t* pw1;   // weight rows 128..255 (dual: w3 rows 0..127)
  if constexpr (DUAL) {
    pw0 = wa + ((int64_t)e * N + ch0 + lrow) * rowstride + lchunk * 8;
    pw1 = wb + ((int64_t)e * N + ch0 + lrow) * rowstride + lchunk * 8;
  } else {
    pw0 = wa + ((int64_t)e * N + ch0 + lrow) * rowstride + lchunk * 8;
    pw1 = pw0 + (int64_t)128 * rowstride;
  }
  const uint16_t* pt = act + (int64_t)(tok0 + lrow) * rowstride + lchunk * 8;
  uint32_t wmask = 0, tmask = 0;   // bit j: row lrow + 32 j is in range
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int wrow = (DUAL ? (j & 3) * 32 : j * 32) + lrow;
    if (ch0 + wrow < N) wmask |= 1u << j;
    if (j * 32 + lrow < tok_rows) tmask |= 1u << j;
  }
  const int st_off = swz(lrow, lchunk);          // + j * 32 * 128

  uint4 rw[8], rt[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t* p = (j < 4 ? pw0 : pw1) + (int64_t)((j & 3) * 32) * rowstride + k0;
      rw[j] = (wmask >> j) & 1 ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
      const uint16_t* q = pt + (int64_t)(j * 32) * rowstride + k0;
      rt[j] = (tmask >> j) & 1 ? *reinterpret_cast<const uint4*>(q) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<uint4*>(&smem[buf][0][st_off + j * 32 * 128]) = rw[j];
      *reinterpret_cast<uint4*>(&smem[buf][1][st_off + j * 32 * 128]) = rt[j];
    }
  };

  // ---- fragment addressing ----
  const int fi = lane & 31, fg = lane >> 5;
  int frag_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) frag_off[s] = fi * 128 + (((2 * s + fg) ^ (fi & 7)) << 4);
  int arow[4], brow[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if constexpr (DUAL) arow[a] = (a >> 1) * 128 + wr * 64 + (a & 1) * 32;  // a: 0,1 = w1; 2,3 = w3
    else arow[a] = wr * 128 + a * 32;
    brow[a] = wc * 128 + a * 32;
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int KT = K / PF_BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * PF_BK);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        fa[a] = as_bf16x8(*reinterpret_cast<const uint4*>(&smem[buf][0][arow[a] * 128 + frag_off[s]]));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        fb[b] = as_bf16x8(*reinterpret_cast<const uint4*>(&smem[buf][1][brow[b] * 128 + frag_off[s]]));
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane = token (fi), registers = channels ----
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int tl = wc * 128 + b * 32 + fi;      // token row within the tile
    if (tl >= tok_rows) continue;
    const int64_t orow = tok0 + tl;
    if constexpr (DUAL) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = ch0 + wr * 64 + a * 32 + q * 8 + fg * 4;
          if (c >= N) continue;
          float hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[r] = silu_f32(acc[a][b][q * 4 + r]) * acc[a + 2][b][q * 4 + r];
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * N + c) =
              make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = ch0 + wr * 128 + a * 32 + q * 8 + fg * 4;
          if (c >= N) continue;
          *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * N + c) =
              make_float4(acc[a][b][q * 4 + 0], acc[a][b][q * 4 + 1], acc[a][b][q * 4 + 2],
                          acc[a][b][q * 4 + 3]);
        }
    }
  }
}

// ------------------------------------------------------------- decode ---

template <bool DUAL, int KB>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int N, int K,
    void* __restrict__ out, int tok_tiles) {
  constexpr int NC = KB / 32;          // 16-byte chunks per lane per K block
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int groups = N / 16;
  const int cg = wid % groups;
  const int rest = wid / groups;
  const int tt = rest % tok_tiles;
  const int e = rest / tok_tiles;
  if (e >= E) return;
  const int row0 = offsets[e] + tt * 16;
  const int rows = min(16, offsets[e + 1] - row0);
  if (rows <= 0) return;

  const int r = lane & 15, g = lane >> 4;
  const int64_t kofs = (int64_t)g * (KB / 4);
  const uint16_t* pa = wa + ((int64_t)e * N + cg * 16 + r) * K + kofs;
  const uint16_t* pb = DUAL ? wb + ((int64_t)e * N + cg * 16 + r) * K + kofs : nullptr;
  const bool tok_ok = r < rows;
  const uint16_t* px = act + (int64_t)(row0 + (tok_ok ? r : 0)) * K + kofs;

  f32x4_t acc_a = {0.f, 0.f, 0.f, 0.f}, acc_b = {0.f, 0.f, 0.f, 0.f};
  uint4 ca[NC], cb[NC], cx[NC], na[NC], nb[NC], nx[NC];
  auto load = [&](int k0, uint4* A, uint4* B, uint4* X) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      A[j] = *reinterpret_cast<const uint4*>(pa + k0 + j * 8);
      if constexpr (DUAL) B[j] = *reinterpret_cast<const uint4*>(pb + k0 + j * 8);
      X[j] = tok_ok ? *reinterpret_cast<const uint4*>(px + k0 + j * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  load(0, ca, cb, cx);
  for (int k0 = 0; k0 < K; k0 += KB) {
    const bool more = k0 + KB < K;
    if (more) load(k0 + KB, na, nb, nx);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ca[j]), as_bf16x8(cx[j]), acc_a, 0, 0, 0);
      if constexpr (DUAL)
        acc_b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cb[j]), as_bf16x8(cx[j]), acc_b, 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        ca[j] = na[j];
        if constexpr (DUAL) cb[j] = nb[j];
        cx[j] = nx[j];
      }
    }
  }

  // 16x16 accumulator: lane holds token column (lane & 15), channels 4 * (lane >> 4) + 0..3.
  const int tcol = lane & 15;
  if (tcol >= rows) return;
  const int c = cg * 16 + (lane >> 4) * 4;
  const int64_t orow = row0 + tcol;
  if constexpr (DUAL) {
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_f32(acc_a[i]) * acc_b[i];
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * N + c) =
        make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * N + c) =
        make_float4(acc_a[0], acc_a[1], acc_a[2], acc_a[3]);
  }
}

template <bool DUAL, int KB>
hipError_t launch_decode(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                         const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                         hipStream_t st) {
  const int tok_tiles = (int)((max_rows_per_expert(s) + 15) / 16);
  const int64_t waves = (int64_t)s.n_experts * tok_tiles * (N / 16);
  const int64_t blocks = (waves + 3) / 4;
  if (blocks <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  hipLaunchKernelGGL((grouped_gemm_bf16_decode<DUAL, KB>), dim3((unsigned)blocks), dim3(256), 0,
                     st, act, offsets, s.n_experts, wa, wb, N, K, out, tok_tiles);
  return hipGetLastError();
}

template <bool DUAL>
hipError_t launch_prefill(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                          hipStream_t st) {
  constexpr int CH_TILE = DUAL ? 128 : 256;
  const int n_tiles = (N + CH_TILE - 1) / CH_TILE;
  const int64_t grid = max_token_tiles(s, PF_ROWS) * n_tiles;
  const int64_t padded = (grid + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_bf16_prefill<DUAL>, dim3((unsigned)padded), dim3(PF_THREADS),
                     0, st, act, offsets, s.n_experts, wa, wb, N, K, out, n_tiles, (int)padded);
  return hipGetLastError();
}

// Decode (weight streaming) while no expert can hold more than this many rows.
constexpr int kDecodeMaxRows = 64;

template <bool DUAL>
hipError_t launch_bf16(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                       const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                       hipStream_t st) {
  if (max_rows_per_expert(s) <= kDecodeMaxRows) {
    // 8 (single) or 8 + 8 (dual) 16-byte weight loads in flight per lane.
    if (!DUAL && K % 256 == 0) return launch_decode<DUAL, 256>(s, act, offsets, wa, wb, N, K, out, st);
    if (K % 128 == 0) return launch_decode<DUAL, 128>(s, act, offsets, wa, wb, N, K, out, st);
    return launch_decode<DUAL, 64>(s, act, offsets, wa, wb, N, K, out, st);
  }
  return launch_prefill<DUAL>(s, act, offsets, wa, wb, N, K, out, st);
}

}  // namespace

hipError_t launch_gate_up_bf16(const moe_shape_t& s, const uint16_t* x_perm,
                               const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                               uint16_t* h, hipStream_t st) {
  return launch_bf16<true>(s, x_perm, offsets, w1, w3, s.d_ff, s.d_model, h, st);
}

hipError_t launch_down_bf16(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                            const uint16_t* w2, float* y_perm, hipStream_t st) {
  return launch_bf16<false>(s, h, offsets, w2, nullptr, s.d_model, s.d_ff, y_perm, st);
}

}  // namespace moe

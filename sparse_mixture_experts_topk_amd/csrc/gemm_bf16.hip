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
// consecutive rows hit distinct banks.  Global reads use buffer resources
// bounded to the tile's valid rows: rows past the expert's last token or the
// last channel read as zero without a branch.  The next K slice is fetched
// into registers while the current one feeds v_mfma_f32_32x32x16_bf16, LDS
// fragments are read one 16-wide substep ahead of the matrix instructions,
// and there is one barrier per slice.  Each wavefront owns 128 x 128 of the
// tile: 16 accumulator blocks, 256 fp32 per lane.  Tiles are scheduled expert
// by expert with token tiles fastest and remapped so that consecutive tiles
// run on the same XCD and share its L2 copy of the weight tile.
//
// Decode kernel (few tokens per expert): weight streaming.  One wavefront
// owns 16 output channels (dual: of w1 and of w3) x up to 16 tokens over all
// of K, reading each weight row once with non-temporal 16-byte loads, the
// next K block prefetched into registers while v_mfma_f32_16x16x32_bf16
// consumes the current one.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// silu(g) * u for a bf16 result: hardware exp2 and reciprocal (about 1 ulp
// in fp32, far below the bf16 rounding that follows).
__device__ __forceinline__ float swiglu_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufferFlags);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

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
  // Lane reads 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 j.
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int64_t rowbytes = (int64_t)K * 2;
  const __amdgpu_buffer_rsrc_t rs_t = make_rsrc(act + (int64_t)tok0 * K, tok_rows * rowbytes);
  const __amdgpu_buffer_rsrc_t rs_w0 =
      make_rsrc(wa + ((int64_t)e * N + ch0) * K, (int64_t)(N - ch0) * rowbytes);
  const __amdgpu_buffer_rsrc_t rs_w1 =
      DUAL ? make_rsrc(wb + ((int64_t)e * N + ch0) * K, (int64_t)(N - ch0) * rowbytes) : rs_w0;
  int voff_w[8], voff_t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // dual: tile rows 0..127 are w1 rows, 128..255 the same w3 rows
    const int wrow = (DUAL ? (j & 3) * 32 : j * 32) + lrow;
    voff_w[j] = (int)(wrow * rowbytes) + lchunk * 16;
    voff_t[j] = (int)((j * 32 + lrow) * rowbytes) + lchunk * 16;
  }
  const int st_off = swz(lrow, lchunk);          // + j * 32 * 128

  uint4 rw[8], rt[8];
  auto gload = [&](int k0) {
    const int soff = k0 * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rw[j] = buf_load16((DUAL && j >= 4) ? rs_w1 : rs_w0, voff_w[j], soff);
      rt[j] = buf_load16(rs_t, voff_t[j], soff);
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

  auto read_frags = [&](int buf, int s, bf16x8_t* fa, bf16x8_t* fb) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
      fa[a] = as_bf16x8(*reinterpret_cast<const uint4*>(&smem[buf][0][arow[a] * 128 + frag_off[s]]));
#pragma unroll
    for (int b = 0; b < 4; ++b)
      fb[b] = as_bf16x8(*reinterpret_cast<const uint4*>(&smem[buf][1][brow[b] * 128 + frag_off[s]]));
  };

  auto mfmas = [&](const bf16x8_t* fa, const bf16x8_t* fb) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
  };

  // Software pipeline of one K slice (64 MFMAs per wavefront), one basic
  // block: the next slice's 16 global reads and the next substep's 8
  // fragment reads are spread between the matrix instructions, the LDS
  // writes of the next slice fill the last substep, then one barrier.  The
  // read of slice KT (past the end) is bounded by the buffer resources and
  // its LDS copy is never consumed.
  const int KT = K / PF_BK;
  gload(0);
  sstore(0);
  __syncthreads();
  bf16x8_t fa0[4], fb0[4], fa1[4], fb1[4];
  read_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    gload((kt + 1) * PF_BK);
    read_frags(buf, 1, fa1, fb1);
    mfmas(fa0, fb0);
    read_frags(buf, 2, fa0, fb0);
    mfmas(fa1, fb1);
    read_frags(buf, 3, fa1, fb1);
    mfmas(fa0, fb0);
    sstore(buf ^ 1);
    mfmas(fa1, fb1);
    // substep 0: 16 MFMA, 16 global reads, 8 fragment reads
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // VMEM read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    // substeps 1, 2: 16 MFMA and 8 fragment reads each
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // substep 3: 16 MFMA and the 16 LDS writes of the next slice
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __syncthreads();
    read_frags(buf ^ 1, 0, fa0, fb0);
  }

  // ---- epilogue: lane = token (fi), registers = channels ----
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int tl = wc * 128 + b * 32 + fi;      // token row within the tile
    const bool tok_in = tl < tok_rows;
    const int64_t orow = tok0 + tl;
    if constexpr (DUAL) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = ch0 + wr * 64 + a * 32 + q * 8 + fg * 4;
          float hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[r] = swiglu_fast(acc[a][b][q * 4 + r], acc[a + 2][b][q * 4 + r]);
          if (tok_in && c < N)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * N + c) =
                make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = ch0 + wr * 128 + a * 32 + q * 8 + fg * 4;
          if (tok_in && c < N)
            *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * N + c) =
                make_float4(acc[a][b][q * 4 + 0], acc[a][b][q * 4 + 1], acc[a][b][q * 4 + 2],
                            acc[a][b][q * 4 + 3]);
        }
    }
  }
}

// ------------------------------------------------------------- decode ---

template <bool DUAL, int KB, int MIN_WAVES>
__global__ __launch_bounds__(256, MIN_WAVES) void grouped_gemm_bf16_decode(
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

  // Lane (r, g) feeds row r; MFMA j of a K block takes the 32 consecutive
  // elements k0 + 32 j .. + 31, lane group g its 8-element chunk g, so the 4
  // lanes of a row read 64 contiguous bytes per load instruction.
  const int r = lane & 15, g = lane >> 4;
  const int64_t kofs = (int64_t)g * 8;
  const uint16_t* pa = wa + ((int64_t)e * N + cg * 16 + r) * K + kofs;
  const uint16_t* pb = DUAL ? wb + ((int64_t)e * N + cg * 16 + r) * K + kofs : nullptr;
  const bool tok_ok = r < rows;
  const uint16_t* px = act + (int64_t)(row0 + (tok_ok ? r : 0)) * K + kofs;

  f32x4_t acc_a = {0.f, 0.f, 0.f, 0.f}, acc_b = {0.f, 0.f, 0.f, 0.f};
  uint4 ca[NC], cb[NC], cx[NC], na[NC], nb[NC], nx[NC];
  auto load = [&](int k0, uint4* A, uint4* B, uint4* X) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      A[j] = load_stream16(pa + k0 + j * 32);
      if constexpr (DUAL) B[j] = load_stream16(pb + k0 + j * 32);
      X[j] = tok_ok ? *reinterpret_cast<const uint4*>(px + k0 + j * 32) : make_uint4(0, 0, 0, 0);
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
    for (int i = 0; i < 4; ++i) hv[i] = swiglu_fast(acc_a[i], acc_b[i]);
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
  // dual, 64-wide K blocks: 7 wavefronts per SIMD (no spills) keep a whole
  // Mixtral-size grid (8 experts x 896 channel groups) resident at once
  constexpr int MIN_WAVES = (DUAL && KB == 64) ? 7 : 2;
  hipLaunchKernelGGL((grouped_gemm_bf16_decode<DUAL, KB, MIN_WAVES>), dim3((unsigned)blocks), dim3(256), 0,
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
    // dual: 2 + 2 weight loads per K block, few registers, so every wavefront
    // of the grid is resident at once; single: 8 loads in flight per lane.
    if (!DUAL && K % 256 == 0) return launch_decode<DUAL, 256>(s, act, offsets, wa, wb, N, K, out, st);
    if (!DUAL && K % 128 == 0) return launch_decode<DUAL, 128>(s, act, offsets, wa, wb, N, K, out, st);
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

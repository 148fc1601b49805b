// bf16 grouped expert GEMMs on the gfx950 matrix cores (fp32 accumulate):
// the many-tokens-per-expert (prefill) kernel and the bf16 dispatch.
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
// Prefill kernel: 256 lanes, a 256 x 256 tile (weights x tokens; the dual
// gate/up variant holds 128 w1 rows and the same 128 w3 rows so silu(g) * u
// is formed in registers), K staged 64 at a time through two LDS buffers of
// 2 x 32 KiB.  Rows are 128 bytes in LDS with the 16-byte chunks XOR-swizzled
// (lds_swizzle_key), so the fragment reads of 16 consecutive rows are free of
// bank conflicts.  Global reads use buffer resources bounded to the tile's valid rows:
// rows past the expert's last token or the last channel read as zero without
// a branch.  The next K slice is fetched into registers while the current one
// feeds v_mfma_f32_32x32x16_bf16, LDS fragments are read one 16-wide substep
// ahead of the matrix instructions, and there is one barrier per slice.  Each
// wavefront owns 128 x 128 of the tile: 16 accumulator blocks, 256 fp32 per
// lane.  Tiles are scheduled expert by expert with token tiles fastest and
// remapped so that consecutive tiles run on the same XCD and share its L2
// copy of the weight tile.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

hipError_t launch_decode_bf16(const moe_shape_t& s, bool dual, const uint16_t* act,
                              const int32_t* offsets, const uint16_t* wa, const uint16_t* wb,
                              int N, int K, void* out, hipStream_t st);

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

constexpr int PF_ROWS = 256;         // rows of each LDS operand tile
constexpr int PF_BK = 64;            // K per stage (128 bytes per row)
constexpr int PF_TILE_BYTES = PF_ROWS * PF_BK * 2;
constexpr int PF_THREADS = 256;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ lds_swizzle_key(row)) << 4);
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
  for (int s = 0; s < 4; ++s) frag_off[s] = fi * 128 + (((2 * s + fg) ^ lds_swizzle_key(fi)) << 4);
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

// Weight streaming (decode kernels) while no expert can hold more than this many rows.
constexpr int kDecodeMaxRows = 64;

}  // namespace

hipError_t launch_gate_up_bf16(const moe_shape_t& s, const uint16_t* x_perm,
                               const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                               uint16_t* h, hipStream_t st) {
  if (max_rows_per_expert(s) <= kDecodeMaxRows)
    return launch_decode_bf16(s, true, x_perm, offsets, w1, w3, s.d_ff, s.d_model, h, st);
  return launch_prefill<true>(s, x_perm, offsets, w1, w3, s.d_ff, s.d_model, h, st);
}

hipError_t launch_down_bf16(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                            const uint16_t* w2, float* y_perm, hipStream_t st) {
  if (max_rows_per_expert(s) <= kDecodeMaxRows)
    return launch_decode_bf16(s, false, h, offsets, w2, nullptr, s.d_model, s.d_ff, y_perm, st);
  return launch_prefill<false>(s, h, offsets, w2, nullptr, s.d_model, s.d_ff, y_perm, st);
}

}  // namespace moe

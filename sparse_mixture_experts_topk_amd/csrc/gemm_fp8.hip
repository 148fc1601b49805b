// fp8 (OCP e4m3) grouped expert GEMMs on the gfx950 matrix cores, fp32 accumulate.
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x);
// "How Mixtral 8x7B uses mixture of experts", section "Quantization
// asymmetry": experts are the quantised part, the router stays 16-bit.
//
// Formats.  Expert weights are e4m3 codes with one fp32 scale per output
// channel.  The token operand (x_perm, h) is e4m3 codes with one E8M0
// (power-of-two) scale per row and per 32-element block along K.  One
// v_mfma_scale_f32_32x32x64_f8f6f4 covers K = 64 (two scale blocks) with
// 32 bytes per lane; measured on gfx950, the scale that lane (i, h) supplies
// multiplies bytes 16 h .. 16 h + 15 of both lanes (i, 0) and (i, 1).  So
// lane half h holds the h-th 16-element half of each of the two blocks and
// supplies the scale of block h: the token operand's block scales are
// applied in hardware with no extra VALU work.  The weight operand's scale
// is 1 (E8M0 127) and its per-channel fp32 scale is applied in the epilogue.  The gate/up epilogue forms h = silu(g) * u in
// fp32 and block-quantises it per (token, 32 channels): the amax of a block
// lives in two lanes (16 channels each) and is completed with one lane swap.
//
// Tile structure follows the bf16 prefill kernel: 256 lanes, 256 weight rows
// (dual: 128 w1 + the same 128 w3) x 256 token rows, K staged 128 at a time
// (128 bytes per LDS row, 16-byte chunks XOR-swizzled by row), buffer-
// resource loads bounded to the valid rows, the next slice fetched into
// registers during the current one, fragment reads one substep ahead, one
// barrier per slice, XCD-aware grouped tile schedule.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufferFlags);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

__device__ __forceinline__ float swiglu_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// E8M0 exponent of a block: ceil(log2(fp32(amax / 448))) clamped to [-127, 127];
// 0 for an all-zero block.
__device__ __forceinline__ int block_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t bits = __float_as_uint(amax / 448.0f);
  const int ex = (int)((bits >> 23) & 255u);
  const uint32_t man = bits & 0x7fffffu;
  if (ex == 0) return man > (1u << 22) ? -126 : -127;
  return man == 0 ? ex - 127 : ex - 126;
}

constexpr int F8_ROWS = 256;
constexpr int F8_BK = 128;                    // K per stage: 128 fp8 = 128 bytes per row
constexpr int F8_TILE_BYTES = F8_ROWS * F8_BK;
constexpr int F8_THREADS = 256;
constexpr int kF8GroupN = 8;                  // channel tiles per group of the tile order

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ lds_swizzle_key(row)) << 4);
}

template <bool DUAL>
__global__ __launch_bounds__(F8_THREADS, 1) void grouped_gemm_fp8_prefill(
    const uint8_t* __restrict__ act, const uint8_t* __restrict__ act_scale,
    const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ wa,
    const uint8_t* __restrict__ wb, const float* __restrict__ sa, const float* __restrict__ sb,
    int N, int K, void* __restrict__ out, uint8_t* __restrict__ out_scale, int n_tiles,
    int grid_padded) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][F8_TILE_BYTES];

  constexpr int CH_TILE = DUAL ? 128 : 256;
  int e, r0, r1, mt, nt;
  const int tile = xcd_remap(blockIdx.x, grid_padded);
  if (!locate_tile(offsets, E, F8_ROWS, n_tiles, tile, e, r0, r1, mt, nt)) return;
  {
    // Order of an expert's tiles: groups of kF8GroupN channel tiles, channel
    // tile fastest inside a group, so the tiles one XCD runs at a time (its 32
    // consecutive ones) are 8 channel tiles x 4 token tiles, each weight and
    // token slice fetched into its L2 once for several of them.
    const int mtc = (r1 - r0 + F8_ROWS - 1) / F8_ROWS;
    const int l = nt * mtc + mt;                      // tile index inside the expert
    const int gi = l / (mtc * kF8GroupN);
    const int nt0 = gi * kF8GroupN;
    const int gsz = min(kF8GroupN, n_tiles - nt0);
    const int idx = l - gi * mtc * kF8GroupN;
    nt = nt0 + idx % gsz;
    mt = idx / gsz;
  }
  const int tok0 = r0 + mt * F8_ROWS;
  const int tok_rows = min(F8_ROWS, r1 - tok0);
  const int ch0 = nt * CH_TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  const int lrow = tid >> 3, lchunk = tid & 7;
  const int64_t rowbytes = K;
  const int nblk = K / 32;                    // scale blocks per row
  const __amdgpu_buffer_rsrc_t rs_t = make_rsrc(act + (int64_t)tok0 * K, tok_rows * rowbytes);
  const __amdgpu_buffer_rsrc_t rs_ts = make_rsrc(act_scale + (int64_t)tok0 * nblk,
                                                 (int64_t)tok_rows * nblk);
  const __amdgpu_buffer_rsrc_t rs_w0 =
      make_rsrc(wa + ((int64_t)e * N + ch0) * K, (int64_t)(N - ch0) * rowbytes);
  const __amdgpu_buffer_rsrc_t rs_w1 =
      DUAL ? make_rsrc(wb + ((int64_t)e * N + ch0) * K, (int64_t)(N - ch0) * rowbytes) : rs_w0;
  int voff_w[8], voff_t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int wrow = (DUAL ? (j & 3) * 32 : j * 32) + lrow;
    voff_w[j] = (int)(wrow * rowbytes) + lchunk * 16;
    voff_t[j] = (int)((j * 32 + lrow) * rowbytes) + lchunk * 16;
  }
  const int st_off = swz(lrow, lchunk);

  uint4 rw[8], rt[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rw[j] = buf_load16((DUAL && j >= 4) ? rs_w1 : rs_w0, voff_w[j], k0);
      rt[j] = buf_load16(rs_t, voff_t[j], k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<uint4*>(&smem[buf][0][st_off + j * 32 * 128]) = rw[j];
      *reinterpret_cast<uint4*>(&smem[buf][1][st_off + j * 32 * 128]) = rt[j];
    }
  };

  // fragment addressing.  The scale a lane supplies covers bytes 16 h .. 16 h + 15
  // of BOTH lanes of its row (h = its lane half), so a 32-element scale block
  // is split across the halves: for MFMA step s, lane half fg holds 16-byte
  // chunk 4 s + fg (block 2 s) in its low half and chunk 4 s + 2 + fg
  // (block 2 s + 1) in its high half, and supplies the scale of block 2 s + fg.
  const int fi = lane & 31, fg = lane >> 5;
  int frag_off[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      frag_off[s][c] = fi * 128 + (((4 * s + 2 * c + fg) ^ lds_swizzle_key(fi)) << 4);
  int arow[4], brow[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if constexpr (DUAL) arow[a] = (a >> 1) * 128 + wr * 64 + (a & 1) * 32;
    else arow[a] = wr * 128 + a * 32;
    brow[a] = wc * 128 + a * 32;
  }
  // token-operand scales: 4 E8M0 bytes (blocks 4 kt .. 4 kt + 3) per token row per slice;
  // shifted so that the byte of this lane's half sits at position 2 s
  int voff_sc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) voff_sc[b] = (brow[b] + fi) * nblk;
  const int sc_shift = 8 * fg;

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  auto read_frags = [&](int buf, int s, i32x8_t* fa, i32x8_t* fb) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint4 lo = *reinterpret_cast<const uint4*>(&smem[buf][0][arow[a] * 128 + frag_off[s][0]]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&smem[buf][0][arow[a] * 128 + frag_off[s][1]]);
      fa[a] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint4 lo = *reinterpret_cast<const uint4*>(&smem[buf][1][brow[b] * 128 + frag_off[s][0]]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&smem[buf][1][brow[b] * 128 + frag_off[s][1]]);
      fb[b] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
  constexpr int kOne = 0x7f7f7f7f;            // E8M0 127 = 1.0 in every byte
  auto mfmas = [&](const i32x8_t* fa, const i32x8_t* fb, const int* sc, int s) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (s == 0)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a], fb[b], acc[a][b], 0, 0,
                                                                      0, kOne, 0, sc[b]);
        else
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a], fb[b], acc[a][b], 0, 0,
                                                                      0, kOne, 2, sc[b]);
      }
  };

  const int KT = K / F8_BK;
  gload(0);
  sstore(0);
  int sc_cur[4], sc_next[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) sc_cur[b] = (int)(buf_load4(rs_ts, voff_sc[b], 0) >> sc_shift);
  __syncthreads();
  i32x8_t fa0[4], fb0[4], fa1[4], fb1[4];
  read_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    gload((kt + 1) * F8_BK);
#pragma unroll
    for (int b = 0; b < 4; ++b) sc_next[b] = (int)buf_load4(rs_ts, voff_sc[b], (kt + 1) * 4);
    read_frags(buf, 1, fa1, fb1);
    mfmas(fa0, fb0, sc_cur, 0);
    sstore(buf ^ 1);
    mfmas(fa1, fb1, sc_cur, 1);
    // step 0: 16 MFMA with 16 global + 4 scale reads and 16 fragment reads
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
    }
    // step 1: 16 MFMA with the 16 LDS writes of the next slice
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __syncthreads();
    read_frags(buf ^ 1, 0, fa0, fb0);
#pragma unroll
    for (int b = 0; b < 4; ++b) sc_cur[b] = sc_next[b] >> sc_shift;
  }

  // ---- epilogue: lane = token (fi), registers = channels ----
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int tl = wc * 128 + b * 32 + fi;
    const bool tok_in = tl < tok_rows;
    const int64_t orow = tok0 + tl;
    if constexpr (DUAL) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int cbase = ch0 + wr * 64 + a * 32;      // one 32-channel quantisation block
        float hv[16];
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = cbase + q * 8 + fg * 4;
          const bool cin = c < N;
          const float4 s1 = cin ? *reinterpret_cast<const float4*>(sa + (int64_t)e * N + c) : make_float4(0, 0, 0, 0);
          const float4 s3 = cin ? *reinterpret_cast<const float4*>(sb + (int64_t)e * N + c) : make_float4(0, 0, 0, 0);
          const float w1s[4] = {s1.x, s1.y, s1.z, s1.w}, w3s[4] = {s3.x, s3.y, s3.z, s3.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = swiglu_fast(acc[a][b][q * 4 + r] * w1s[r], acc[a + 2][b][q * 4 + r] * w3s[r]);
            hv[q * 4 + r] = v;
            amax = fmaxf(amax, fabsf(v));
          }
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int ex = block_exponent(amax);
        const float inv = __uint_as_float((uint32_t)(127 - ex) << 23);
        if (tok_in && cbase < N) {
          uint8_t* hrow = static_cast<uint8_t*>(out) + orow * N;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int packed = 0;
            packed = __builtin_amdgcn_cvt_pk_fp8_f32(hv[q * 4 + 0] * inv, hv[q * 4 + 1] * inv, packed, false);
            packed = __builtin_amdgcn_cvt_pk_fp8_f32(hv[q * 4 + 2] * inv, hv[q * 4 + 3] * inv, packed, true);
            *reinterpret_cast<int*>(hrow + cbase + q * 8 + fg * 4) = packed;
          }
          if (fg == 0) out_scale[orow * (N / 32) + cbase / 32] = (uint8_t)(ex + 127);
        }
      }
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = ch0 + wr * 128 + a * 32 + q * 8 + fg * 4;
          if (tok_in && c < N) {
            const float4 s2 = *reinterpret_cast<const float4*>(sa + (int64_t)e * N + c);
            *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * N + c) =
                make_float4(acc[a][b][q * 4 + 0] * s2.x, acc[a][b][q * 4 + 1] * s2.y,
                            acc[a][b][q * 4 + 2] * s2.z, acc[a][b][q * 4 + 3] * s2.w);
          }
        }
    }
  }
}

template <bool DUAL>
hipError_t launch_fp8(const moe_shape_t& s, const uint8_t* act, const uint8_t* act_scale,
                      const int32_t* offsets, const uint8_t* wa, const uint8_t* wb, const float* sa,
                      const float* sb, int N, int K, void* out, uint8_t* out_scale, hipStream_t st) {
  constexpr int CH_TILE = DUAL ? 128 : 256;
  const int n_tiles = (N + CH_TILE - 1) / CH_TILE;
  const int64_t grid = max_token_tiles(s, F8_ROWS) * n_tiles;
  const int64_t padded = (grid + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_fp8_prefill<DUAL>, dim3((unsigned)padded), dim3(F8_THREADS), 0,
                     st, act, act_scale, offsets, expert_groups(s), wa, wb, sa, sb, N, K, out,
                     out_scale, n_tiles, (int)padded);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_fp8(const moe_shape_t& s, const uint8_t* x_perm, const uint8_t* x_scale,
                              const int32_t* offsets, const uint8_t* w1, const uint8_t* w3,
                              const float* w1_scale, const float* w3_scale, uint8_t* h,
                              uint8_t* h_scale, hipStream_t st) {
  return launch_fp8<true>(s, x_perm, x_scale, offsets, w1, w3, w1_scale, w3_scale, s.d_ff,
                          s.d_model, h, h_scale, st);
}

hipError_t launch_down_fp8(const moe_shape_t& s, const uint8_t* h, const uint8_t* h_scale,
                           const int32_t* offsets, const uint8_t* w2, const float* w2_scale,
                           float* y_perm, hipStream_t st) {
  return launch_fp8<false>(s, h, h_scale, offsets, w2, nullptr, w2_scale, nullptr, s.d_model,
                           s.d_ff, y_perm, nullptr, st);
}

}  // namespace moe

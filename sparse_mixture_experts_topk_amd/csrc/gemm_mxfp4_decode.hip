// Grouped expert GEMMs with MXFP4 (4-bit) expert weights and bf16 activations,
// for few tokens per expert (decode): weight streaming.
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x);
// "How Mixtral 8x7B uses mixture of experts", section "Quantization
// asymmetry": the router stays in bf16 and the experts are quantised to 4
// bits.  Format: OCP Microscaling FP4 -- E2M1 codes, two per byte (even
// element in the low nibble), one E8M0 scale byte per 32 consecutive
// elements of a weight row.
//
// At decode the layer reads each touched expert's weights once, so 4-bit
// weights cut the dominant traffic to a quarter of bf16 (plus 1/64 for the
// scales).  Dequantisation is one v_cvt_scalef32_pk_bf16_fp4 per two weights:
// it turns two E2M1 codes into two bf16 values times a power-of-two scale,
// exactly (every E2M1 value times 2^e is a bf16 value), so the matrix cores
// (v_mfma_f32_16x16x32_bf16) see the exact dequantised weights.
//
// A wavefront owns RB blocks of 16 output channels (dual: the same channels
// of w1 and w3) of one expert against one tile of up to 16 of its tokens, and
// streams all of K in stages of 256 elements (128 bytes per row).  Weights
// are read in a wide pattern (8 rows x 128 contiguous bytes per load
// instruction, non-temporal), written to the wavefront's own LDS tile
// (16-byte chunks XOR-swizzled by row) and read back one 16-byte chunk --
// one whole 32-element scale block -- per lane.  The K order inside a matrix
// instruction is free as long as both operands follow it: lane (r, g) feeds
// row r with elements 32 (4 j + g) + 8 q .. + 7 of the stage to instruction
// (j, q), and the token operand lane (t, g) feeds the same elements of token
// t, so a lane's chunk covers four instructions and one scale.  The next
// stage's weights and scales are loaded while the current one is multiplied.
#include "device_common.hpp"
#include "launch.hpp"
#include "lds_stream.hpp"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr int kMx4Waves = 4;           // wavefronts per workgroup
constexpr int kMx4StageK = 256;        // K elements per stage
constexpr int kMx4RowBytes = kMx4StageK / 2;

// E8M0 scale byte -> fp32 2^(b - 127); byte 0 is the subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b == 0 ? 0x00400000u : (b << 23));
}

// Eight E2M1 codes (one dword, element 2i in bits 8i..8i+3) -> eight bf16
// values times `scale` (a power of two).
__device__ __forceinline__ bf16x8_t dequant8(uint32_t codes, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                             __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
  return as_bf16x8(u);
}

template <bool DUAL, int RB, int MIN_WAVES>
__global__ __launch_bounds__(kMx4Waves * kWave, MIN_WAVES) void grouped_gemm_mxfp4_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ wa, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ wb,
    const uint8_t* __restrict__ sb, int N, int K, void* __restrict__ out, int tok_tiles) {
  constexpr int NM = DUAL ? 2 : 1;
  constexpr int CH = 16 * RB;                       // output channels per wavefront
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMx4Waves][NM][RB][16 * kMx4RowBytes];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int groups = N / CH;
  const int gid = blockIdx.x * kMx4Waves + w;
  const int cg = gid % groups;
  const int rest = gid / groups;
  const int tt = rest % tok_tiles;
  const int e = rest / tok_tiles;
  if (e >= E) return;
  const int row0 = offsets[e] + tt * 16;
  const int rows = min(16, offsets[e + 1] - row0);
  if (rows <= 0) return;

  const int64_t kb = K / 2;                         // bytes per weight row
  const int nblk = K / 32;                          // scale bytes per weight row
  // wide loader: lane -> row lrow (+ 8 for the second instruction), 16-byte chunk lch
  const int lrow = lane >> 3, lch = lane & 7;
  const uint8_t* pw[NM];
  const uint8_t* ps[NM];
  pw[0] = wa + ((int64_t)e * N + cg * CH) * kb;
  ps[0] = sa + ((int64_t)e * N + cg * CH) * nblk;
  if constexpr (DUAL) {
    pw[1] = wb + ((int64_t)e * N + cg * CH) * kb;
    ps[1] = sb + ((int64_t)e * N + cg * CH) * nblk;
  }
  // matrix-core operands: lane (r, g) = row / token r, element group g
  const int r = lane & 15, g = lane >> 4;
  const bool tok_ok = r < rows;
  const uint16_t* px = act + (int64_t)(row0 + (tok_ok ? r : 0)) * K + g * 32;

  f32x4_t acc[NM][RB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[m][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // stage st: weight chunks (2 wide loads per 16-row block) and this lane's
  // 8 scale bytes of row r (blocks 8 st .. 8 st + 7)
  uint4 wv[NM][RB][2];
  uint2 sv[NM][RB];
  auto load_stage = [&](int st, uint4 (&wd)[NM][RB][2], uint2 (&sd)[NM][RB]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          wd[m][b][i] = load_stream16(pw[m] + (int64_t)(b * 16 + i * 8 + lrow) * kb +
                                      st * kMx4RowBytes + lch * 16);
        sd[m][b] = *reinterpret_cast<const uint2*>(ps[m] + (int64_t)(b * 16 + r) * nblk + st * 8);
      }
  };

  const int nst = K / kMx4StageK;
  load_stage(0, wv, sv);
  for (int st = 0; st < nst; ++st) {
    uint4 wn[NM][RB][2];
    uint2 sn[NM][RB];
    if (st + 1 < nst) load_stage(st + 1, wn, sn);
    // token operand of instruction (j, q): 8 bf16 at element 32 (4 j + g) + 8 q of the stage
    uint4 xv[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[j][q] = tok_ok ? *reinterpret_cast<const uint4*>(px + st * kMx4StageK + j * 128 + q * 8)
                          : make_uint4(0, 0, 0, 0);
    // wavefront-private transpose: LDS operations of one wavefront execute in order
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = i * 8 + lrow;
          *reinterpret_cast<uint4*>(&lds[w][m][b][row * kMx4RowBytes + ((lch ^ lds_swizzle_key(row)) & 7) * 16]) =
              wv[m][b][i];
        }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = 4 * j + g;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const uint4 c = *reinterpret_cast<const uint4*>(
              &lds[w][m][b][r * kMx4RowBytes + ((chunk ^ lds_swizzle_key(r)) & 7) * 16]);
          const uint32_t sbyte = ((j ? sv[m][b].y : sv[m][b].x) >> (8 * g)) & 255u;
          const float scale = e8m0_to_f32(sbyte);
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(cw[q], scale),
                                                                 as_bf16x8(xv[j][q]), acc[m][b], 0, 0, 0);
        }
    }
    if (st + 1 < nst) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          wv[m][b][0] = wn[m][b][0];
          wv[m][b][1] = wn[m][b][1];
          sv[m][b] = sn[m][b];
        }
    }
  }

  // 16x16 accumulators: lane holds token column (lane & 15), channels 4 (lane >> 4) + 0..3.
  const int tcol = lane & 15;
  if (tcol >= rows) return;
  const int64_t orow = row0 + tcol;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int c = cg * CH + b * 16 + (lane >> 4) * 4;
    if constexpr (DUAL) {
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = swiglu_fast(acc[0][b][i], acc[1][b][i]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * N + c) =
          make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * N + c) =
          make_float4(acc[0][b][0], acc[0][b][1], acc[0][b][2], acc[0][b][3]);
    }
  }
}

template <bool DUAL, int RB, int MIN_WAVES>
hipError_t launch_variant(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint8_t* wa, const uint8_t* sa, const uint8_t* wb,
                          const uint8_t* sb, int N, int K, void* out, hipStream_t st) {
  const int tok_tiles = (int)((max_rows_per_expert(s) + 15) / 16);
  const int64_t groups = (int64_t)s.n_experts * tok_tiles * (N / (16 * RB));
  if (groups <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  const int64_t blocks = (groups + kMx4Waves - 1) / kMx4Waves;
  hipLaunchKernelGGL((grouped_gemm_mxfp4_decode<DUAL, RB, MIN_WAVES>), dim3((unsigned)blocks),
                     dim3(kMx4Waves * kWave), 0, st, act, offsets, s.n_experts, wa, sa, wb, sb, N,
                     K, out, tok_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_mxfp4(const moe_shape_t& s, const uint16_t* x_perm,
                                const int32_t* offsets, const uint8_t* w1, const uint8_t* w1_scale,
                                const uint8_t* w3, const uint8_t* w3_scale, uint16_t* h,
                                hipStream_t st) {
  return launch_variant<true, 2, 2>(s, x_perm, offsets, w1, w1_scale, w3, w3_scale, s.d_ff,
                                    s.d_model, h, st);
}

hipError_t launch_down_mxfp4(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                             const uint8_t* w2, const uint8_t* w2_scale, float* y_perm,
                             hipStream_t st) {
  return launch_variant<false, 2, 2>(s, h, offsets, w2, w2_scale, nullptr, nullptr, s.d_model,
                                     s.d_ff, y_perm, st);
}

}  // namespace moe

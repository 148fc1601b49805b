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
// streams its part of K (KS wavefronts of a workgroup split K) in stages of
// 256 elements (128 bytes per row), PD stages ahead.  Weights
// are read in a wide pattern (8 rows x 128 contiguous bytes per load
// instruction, non-temporal), written to the wavefront's own LDS tile
// (16-byte chunks XOR-swizzled by row) and read back one 16-byte chunk --
// one whole 32-element scale block -- per lane.  The K order inside a matrix
// instruction is free as long as both operands follow it: lane (r, g) feeds
// row r with elements 32 (4 j + g) + 8 q .. + 7 of the stage to instruction
// (j, q), and the token operand lane (t, g) feeds the same elements of token
// t, so a lane's chunk covers four instructions and one scale.
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

// KS wavefronts of a workgroup share one output group and split its K range
// (more wavefronts in flight for a long K); their partial sums are added
// through LDS in K order, so the result does not depend on timing.
template <bool DUAL, int RB, int MIN_WAVES, int PD, int KS>
__global__ __launch_bounds__(kMx4Waves * kWave, MIN_WAVES) void grouped_gemm_mxfp4_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ wa, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ wb,
    const uint8_t* __restrict__ sb, int N, int K, void* __restrict__ out, int tok_tiles) {
  constexpr int NM = DUAL ? 2 : 1;
  constexpr int CH = 16 * RB;                       // output channels per wavefront
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMx4Waves][NM][RB][16 * kMx4RowBytes];

  static_assert(kMx4Waves % KS == 0, "K split");
  // wavefront index and everything derived from it are uniform: kept in
  // scalar registers (the token descriptor must be, or every buffer load
  // would become a loop over the lanes' distinct descriptors)
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kpart = w % KS;
  const int groups = N / CH;
  const int gid = blockIdx.x * (kMx4Waves / KS) + w / KS;
  const int cg = gid % groups;
  const int rest = gid / groups;
  const int tt = rest % tok_tiles;
  const int e = rest / tok_tiles;
  int row0 = 0, rows = 0;
  if (e < E) {
    row0 = __builtin_amdgcn_readfirstlane(offsets[e] + tt * 16);
    rows = __builtin_amdgcn_readfirstlane(min(16, offsets[e + 1] - row0));
  }
  // the KS wavefronts of a group share this flag; a workgroup only returns as a whole
  const bool active = rows > 0;
  if constexpr (KS == 1) {
    if (!active) return;
  } else {
    if (__syncthreads_or(active) == 0) return;
  }

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
  // matrix-core operands: lane (r, g) = row / token r, element group g.  The
  // token operand is read through a buffer descriptor bounded to the tile's
  // rows: lanes of rows past the tile get an out-of-range offset, load zeros
  // and fetch nothing (at decode most of the 16 rows are empty, and every
  // weight byte here meets four token bytes).
  const int r = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(act) + (int64_t)row0 * K, 0,
                                        rows * K * 2, 0x00020000);
  const int xoff = r < rows ? (r * K + g * 32) * 2 : 0x7ff00000;

  f32x4_t acc[NM][RB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[m][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Stage st's weight chunks (2 wide loads per 16-row block) and this lane's
  // 8 scale bytes of row r (blocks 8 st .. 8 st + 7).
  struct WOps {
    uint4 w[NM][RB][2];
    uint2 s[NM][RB];
  };
  auto load_weights = [&](int st, WOps& o) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          o.w[m][b][i] = load_stream16(pw[m] + (int64_t)(b * 16 + i * 8 + lrow) * kb +
                                       st * kMx4RowBytes + lch * 16);
        o.s[m][b] = *reinterpret_cast<const uint2*>(ps[m] + (int64_t)(b * 16 + r) * nblk + st * 8);
      }
  };
  // One stage:
  //  1. the token operand of instruction (j, q): 8 bf16 at element
  //     32 (4 j + g) + 8 q of the stage (zeros for rows past the tile);
  //  2. this stage's weights (loaded PD stages earlier) to the wavefront-private
  //     LDS tile (LDS operations of one wavefront execute in order);
  //  3. the weights of stage st + PD into `nxt`, the slot stage st - 1 used:
  //     issued after the token loads, so waiting for the tokens leaves them in
  //     flight.  Unconditional (past the end they reload the last stage): a
  //     branch would make the compiler's wait counts assume they may be absent;
  //  4. read back, dequantise, multiply.
  // The PD + 1 weight sets rotate without copies, so no register move waits
  // for a load in flight.
  const int nst_all = K / kMx4StageK;
  const int st_begin = nst_all * kpart / KS, st_end = nst_all * (kpart + 1) / KS;
  const int nst = st_end;                           // stages are numbered globally
  auto stage = [&](int st, WOps& cur, WOps& nxt) __attribute__((always_inline)) {
    uint4 x[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        x[j][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                      xrs, xoff, (st * kMx4StageK + j * 128 + q * 8) * 2, 0));
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = i * 8 + lrow;
          *reinterpret_cast<uint4*>(&lds[w][m][b][row * kMx4RowBytes + ((lch ^ lds_swizzle_key(row)) & 7) * 16]) =
              cur.w[m][b][i];
        }
    load_weights(min(st + PD, nst - 1), nxt);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = 4 * j + g;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const uint4 c = *reinterpret_cast<const uint4*>(
              &lds[w][m][b][r * kMx4RowBytes + ((chunk ^ lds_swizzle_key(r)) & 7) * 16]);
          const uint32_t sbyte = ((j ? cur.s[m][b].y : cur.s[m][b].x) >> (8 * g)) & 255u;
          const float scale = e8m0_to_f32(sbyte);
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(cw[q], scale),
                                                                 as_bf16x8(x[j][q]), acc[m][b], 0, 0, 0);
        }
    }
  };
  if (active && st_end > st_begin) {          // a K part can be empty when K is short
    WOps ring[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) load_weights(min(st_begin + i, nst - 1), ring[i]);
    // full rounds of PD + 1 stages, then the remaining stages one by one
    const int nfull = st_begin + (st_end - st_begin) / (PD + 1) * (PD + 1);
    for (int st0 = st_begin; st0 < nfull; st0 += PD + 1) {
#pragma unroll
      for (int u = 0; u <= PD; ++u) stage(st0 + u, ring[u], ring[(u + PD) % (PD + 1)]);
    }
#pragma unroll
    for (int u = 0; u < PD; ++u)
      if (nfull + u < nst) stage(nfull + u, ring[u], ring[(u + PD) % (PD + 1)]);
  }
  if constexpr (KS > 1) {
    // partial sums through LDS: each wavefront's own tile region holds its
    // 16x16 accumulators; the group's first wavefront adds the others in K order
    static_assert(NM * RB * 16 * 16 * 4 <= NM * RB * 16 * kMx4RowBytes, "partials fit the LDS tile");
    float* part = reinterpret_cast<float*>(&lds[w][0][0][0]);
    __syncthreads();                                // every wavefront is done with its LDS tile
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b)
        *reinterpret_cast<f32x4_t*>(&part[((m * RB + b) * 64 + lane) * 4]) = acc[m][b];
    __syncthreads();
    if (kpart != 0 || !active) return;
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      const float* other = reinterpret_cast<const float*>(&lds[w + k][0][0][0]);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < RB; ++b)
          acc[m][b] += *reinterpret_cast<const f32x4_t*>(&other[((m * RB + b) * 64 + lane) * 4]);
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

template <bool DUAL, int RB, int MIN_WAVES, int PD, int KS>
hipError_t launch_variant(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint8_t* wa, const uint8_t* sa, const uint8_t* wb,
                          const uint8_t* sb, int N, int K, void* out, hipStream_t st) {
  const int tok_tiles = (int)((max_rows_per_expert(s) + 15) / 16);
  const int64_t groups = (int64_t)expert_groups(s) * tok_tiles * (N / (16 * RB));
  if (groups <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  constexpr int GPB = kMx4Waves / KS;   // output groups per workgroup
  const int64_t blocks = (groups + GPB - 1) / GPB;
  hipLaunchKernelGGL((grouped_gemm_mxfp4_decode<DUAL, RB, MIN_WAVES, PD, KS>), dim3((unsigned)blocks),
                     dim3(kMx4Waves * kWave), 0, st, act, offsets, expert_groups(s), wa, sa, wb, sb, N,
                     K, out, tok_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_mxfp4(const moe_shape_t& s, const uint16_t* x_perm,
                                const int32_t* offsets, const uint8_t* w1, const uint8_t* w1_scale,
                                const uint8_t* w3, const uint8_t* w3_scale, uint16_t* h,
                                hipStream_t st) {
  // Measured at the Mixtral decode shape (4 rows per expert): 32 channels per
  // wavefront and K split in two streams 4.8 TB/s; 16 channels, no split, 4.3.
  return launch_variant<true, 2, 2, 2, 2>(s, x_perm, offsets, w1, w1_scale, w3, w3_scale, s.d_ff,
                                    s.d_model, h, st);
}

hipError_t launch_down_mxfp4(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                             const uint8_t* w2, const uint8_t* w2_scale, float* y_perm,
                             hipStream_t st) {
  // 64 channels per wavefront, K (14336) split in four: 4.7 TB/s; 16, no split: 3.7.
  return launch_variant<false, 4, 2, 2, 4>(s, h, offsets, w2, w2_scale, nullptr, nullptr, s.d_model,
                                     s.d_ff, y_perm, st);
}

}  // namespace moe

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
// An output group is RB blocks of 16 output channels (dual: the same channels
// of w1 and w3) of one expert against one tile of up to 16 of its tokens; the
// KS wavefronts of a workgroup split its K range.  The launch is persistent:
// each wavefront works through a sequence of groups and streams its part of
// K of each in stages of 256 elements (128 bytes per row), PD stages ahead
// without a break between groups (so no wavefront is a short stream that
// starts and drains on its own).  Weights
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
#include "lane_ops.hpp"
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

// Element offset, inside a 256-element stage, of matrix-instruction operand
// c = 4 j + q of lane group g = 0 (j = c / 4 selects the 128-element half).
__device__ __forceinline__ constexpr int operand_elem(int c) { return (c >> 2) * 128 + (c & 3) * 8; }

// Persistent form.  The grid is the resident capacity; workgroup b takes
// rounds r = 0, 1, ... of GPW output groups (the KS wavefronts of a group
// split its K range), groups numbered over the experts' token tiles only, so
// no workgroup streams an empty expert.  Each wavefront's weight loads form
// one stream across its groups: the ring keeps PD stages in flight through
// group boundaries.  KS must divide the stage count K / 256.
//
// Packed token loads.  When every token tile of the launch has at most 16 / P
// rows (P = 2, 4, 8; decided in the kernel from the offsets), one token load
// instruction carries P of a stage's eight operands: lane (t, g) with
// t = s (16 / P) + u loads operand i P + s of token u, and a row rotation brings
// it to lane (u, g) for its matrix instruction.  Lanes u >= 16 / P then hold
// other operands: columns past the tile's rows, which are never stored (a
// column of the product depends only on its own token).  Same operands in the
// stored columns, same instruction order: the result is the unpacked one, bit
// for bit, with a half to an eighth of the token load instructions.
//
// Scale bytes.  Each stage needs the 8 scale bytes of each of the wavefront's
// 64 weight rows, 64 cache lines for 512 bytes.  So a lane reads Q stages of
// one row at once (Q = 2; four spill the gate/up form): lane (r, c) holds
// Q * 8 contiguous bytes of row r of block
// c = m RB + b, read once every Q stages, and
// lane (t, g) takes its row's bytes of each block from lane (t, c) through the
// cross-lane permute.  Q divides the stages of a K part, and the stage loop is
// unrolled to a multiple of Q, so no load is conditional.  The next cycle's
// bytes are read in the last stage of a cycle, once that stage has taken its
// own: the two register sets are never live together.
template <bool DUAL, int RB, int MIN_WAVES, int PD, int KS, int Q>
__global__ __launch_bounds__(kMx4Waves * kWave, MIN_WAVES) void grouped_gemm_mxfp4_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ wa, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ wb,
    const uint8_t* __restrict__ sb, int N, int K, void* __restrict__ out,
    const int32_t* __restrict__ gather, int k, int Tk, int xrows) {
  constexpr int NM = DUAL ? 2 : 1;
  constexpr int CH = 16 * RB;                       // output channels per wavefront
  constexpr int GPW = kMx4Waves / KS;               // output groups per workgroup round
  constexpr int PART = NM * RB * 64 * 4;            // fp32 partial sums per wavefront
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMx4Waves][NM][RB][16 * kMx4RowBytes];
  __shared__ __attribute__((aligned(16))) float parts[kMx4Waves][PART];
  __shared__ int32_t s_offs[kMaxExpertGroups + 1];
  static_assert(kMx4Waves % KS == 0, "K split");

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kpart = w % KS, slot = w / KS;
  for (int i = threadIdx.x; i <= E; i += kMx4Waves * kWave) s_offs[i] = offsets[i];
  __syncthreads();
  const int CGN = N / CH;
  int A = 0;                                        // output groups over all token tiles
  int mrows = 0;                                    // most rows in a token tile
  for (int e = 0; e < E; ++e) {
    const int cnt = __builtin_amdgcn_readfirstlane(s_offs[e + 1] - s_offs[e]);
    A += (cnt + 15) / 16 * CGN;
    mrows = max(mrows, min(cnt, 16));
  }
  const int per_round = gridDim.x * GPW;
  const int first = blockIdx.x * GPW;
  if (first >= A) return;                           // uniform over the workgroup
  const int R = (A - first + per_round - 1) / per_round;
  auto run = [&](auto pc) __attribute__((always_inline)) {
  constexpr int P = decltype(pc)::value;            // token operands per load instruction
  constexpr int TPL = 16 / P;                       // token lanes per row of 16 lanes

  struct Grp { int e, cg, row0, rows; };            // rows == 0: no group (loads stay valid)
  auto locate = [&](int rd) __attribute__((always_inline)) -> Grp {
    int a = rd * per_round + first + slot;
    Grp gp{0, 0, 0, 0};
    if (a >= A) return gp;
    for (int e = 0; e < E; ++e) {
      const int cnt = __builtin_amdgcn_readfirstlane(s_offs[e + 1] - s_offs[e]);
      const int t = (cnt + 15) / 16 * CGN;
      if (a < t) {
        const int tt = a / CGN;
        gp.e = e;
        gp.cg = a - tt * CGN;
        gp.row0 = __builtin_amdgcn_readfirstlane(s_offs[e]) + tt * 16;
        gp.rows = min(16, cnt - tt * 16);
        break;
      }
      a -= t;
    }
    return gp;
  };

  const int64_t kb = K / 2;                         // bytes per weight row
  const int nblk = K / 32;                          // scale bytes per weight row
  const int lrow = lane >> 3, lch = lane & 7;
  const int tr = lane & 15, g = lane >> 4;
  const int nsp = K / kMx4StageK / KS;              // stages per K part
  const int st_begin = kpart * nsp;
  const int S = R * nsp;                            // stages of this wavefront's stream

  static_assert(NM * RB == 4, "one scale row per lane: four 16-row blocks per wavefront");
  static_assert(Q == 1 || Q == 2, "scale stages per load");
  const int s_blk = lane >> 4;                      // the block whose scale row this lane reads
  struct WOps {
    uint4 w[NM][RB][2];
  };
  // load cursor
  int lr = 0, lst = st_begin;
  Grp lg = locate(0);
  auto load_weights = [&](WOps& o) __attribute__((always_inline)) {
    const int64_t wrow0 = (int64_t)lg.e * N + lg.cg * CH;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint8_t* pw = (m == 0 ? wa : wb) + wrow0 * kb;
      const uint8_t* ps = (m == 0 ? sa : sb) + wrow0 * nblk;
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          o.w[m][b][i] = load_stream16(pw + (int64_t)(b * 16 + i * 8 + lrow) * kb + lst * kMx4RowBytes + lch * 16);
    }
    if (++lst == st_begin + nsp) {                  // past the stream's end: reload its last group
      lst = st_begin;
      if (lr + 1 < R) lg = locate(++lr);
    }
  };
  // scale cursor: Q stages per load
  int sr = 0, sst = st_begin;
  Grp sg = locate(0);
  uint32_t s_cur[2 * Q], s_nxt[2 * Q];
  auto load_scales = [&](uint32_t (&d)[2 * Q]) __attribute__((always_inline)) {
    const int m = s_blk / RB, b = s_blk % RB;
    const uint8_t* ps = (m == 0 ? sa : sb) + ((int64_t)sg.e * N + sg.cg * CH + b * 16 + tr) * nblk + sst * 8;
    if constexpr (Q == 1) {
      const uint2 v = *reinterpret_cast<const uint2*>(ps);
      d[0] = v.x;
      d[1] = v.y;
    } else {                                        // 16-byte aligned: K is a multiple of 512
      const uint4 v = *reinterpret_cast<const uint4*>(ps);
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    }
    sst += Q;
    if (sst == st_begin + nsp) {                    // past the stream's end: reload its last group
      sst = st_begin;
      if (sr + 1 < R) sg = locate(++sr);
    }
  };
  // compute cursor
  int cr = 0, cst = st_begin;
  Grp cgp = locate(0);
  // Token operand: the group's permuted rows, or (gather) the rows of x those
  // rows copy (slot t*k + s -> token t; the shared expert's T*k + t -> t).
  // Lanes past the group's rows read beyond the range: zeros.
  auto token_rsrc = [&]() __attribute__((always_inline)) {
    if (gather != nullptr)
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(act), 0, xrows * K * 2, 0x00020000);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(act) + (int64_t)cgp.row0 * K, 0,
                                             cgp.rows * K * 2, 0x00020000);
  };
  auto token_off = [&]() __attribute__((always_inline)) -> int {
    const int u = tr % TPL, sp = tr / TPL;          // token, operand within the instruction
    if (u >= cgp.rows) return 0x7ff00000;
    int row = u;
    if (gather != nullptr) {
      const int src = gather[cgp.row0 + u];
      row = src < Tk ? src / k : src - Tk;
    }
    return (row * K + g * 32 + (P == 8 ? operand_elem(sp) : sp * 8)) * 2;
  };
  __amdgpu_buffer_rsrc_t xrs = token_rsrc();
  int xoff_cur = token_off();

  f32x4_t acc[NM][RB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[m][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // End of a group: partial sums of its KS wavefronts through LDS in K order,
  // the first wavefront stores, every wavefront moves to its next group.
  auto finish = [&]() __attribute__((always_inline)) {
    if constexpr (KS > 1) {
      __syncthreads();                              // the previous group's partials are read
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < RB; ++b)
          *reinterpret_cast<f32x4_t*>(&parts[w][((m * RB + b) * 64 + lane) * 4]) = acc[m][b];
      __syncthreads();
      if (kpart == 0) {
#pragma unroll
        for (int k = 1; k < KS; ++k)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int b = 0; b < RB; ++b)
              acc[m][b] += *reinterpret_cast<const f32x4_t*>(&parts[w + k][((m * RB + b) * 64 + lane) * 4]);
      }
    }
    if (kpart == 0 && tr < cgp.rows) {
      const int64_t orow = cgp.row0 + tr;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int c = cgp.cg * CH + b * 16 + g * 4;
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
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b) acc[m][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    cst = st_begin;
    if (cr + 1 < R) {
      cgp = locate(++cr);
      xrs = token_rsrc();
      xoff_cur = token_off();
    }
  };

  // ph: the stage's place in its cycle of Q (a constant once the loop is unrolled)
  auto stage = [&](WOps& cur, WOps& nxt, int ph) __attribute__((always_inline)) {
    const int xoff = xoff_cur;
    uint4 xv[8 / P];
#pragma unroll
    for (int i = 0; i < 8 / P; ++i)
      xv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                  xrs, xoff, (cst * kMx4StageK + operand_elem(i * P)) * 2, 0));
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
    uint32_t sc[NM][RB][2];                         // this lane's row: the stage's 8 scale bytes per block
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int src = ((m * RB + b) * 16 + tr) * 4;
        sc[m][b][0] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)s_cur[2 * ph]);
        sc[m][b][1] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)s_cur[2 * ph + 1]);
      }
    // The next cycle's scale bytes, a stage ahead (this cycle's are all taken),
    // issued before the weight prefetch: loads complete in order, so waiting
    // for them next stage does not wait for weights PD stages ahead.
    if (ph == Q - 1) load_scales(s_nxt);
    load_weights(nxt);
    uint4 x[2][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      x[c >> 2][c & 3] = from_lane_above_even(xv[c / P], c % P * TPL);   // operand c: TPL (c % P) lanes above
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = 4 * j + g;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const uint4 c = *reinterpret_cast<const uint4*>(
              &lds[w][m][b][tr * kMx4RowBytes + ((chunk ^ lds_swizzle_key(tr)) & 7) * 16]);
          const uint32_t sbyte = (sc[m][b][j] >> (8 * g)) & 255u;
          const float scale = e8m0_to_f32(sbyte);
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(cw[q], scale),
                                                                 as_bf16x8(x[j][q]), acc[m][b], 0, 0, 0);
        }
    }
    if (ph == Q - 1) {
#pragma unroll
      for (int i = 0; i < 2 * Q; ++i) s_cur[i] = s_nxt[i];
    }
    if (++cst == st_begin + nsp) finish();
  };

  WOps ring[PD + 1];
#pragma unroll
  for (int i = 0; i < PD; ++i) load_weights(ring[i]);
  load_scales(s_cur);
  // U stages per iteration: whole turns of the ring and whole scale cycles
  constexpr int U = (PD + 1) % Q == 0 ? PD + 1 : Q % (PD + 1) == 0 ? Q : (PD + 1) * Q;
  const int nfull = S / U * U;
  for (int p0 = 0; p0 < nfull; p0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) stage(ring[u % (PD + 1)], ring[(u + PD) % (PD + 1)], u % Q);
  }
#pragma unroll
  for (int u = 0; u < U - 1; ++u)
    if (nfull + u < S) stage(ring[u % (PD + 1)], ring[(u + PD) % (PD + 1)], u % Q);
  };
  if (mrows <= 2) run(IntC<8>{});
  else if (mrows <= 4) run(IntC<4>{});
  else if (mrows <= 8) run(IntC<2>{});
  else run(IntC<1>{});
}

// Workgroups per CU = MIN_WAVES wavefronts per SIMD; KS is the largest of 4, 2, 1
// that divides the stage count; Q = 2 when the stages per part are even.
template <bool DUAL, int RB, int MIN_WAVES, int PD, int KS, int Q>
hipError_t launch_kq(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                     const uint8_t* wa, const uint8_t* sa, const uint8_t* wb, const uint8_t* sb,
                     int N, int K, void* out, hipStream_t st, const int32_t* gather) {
  constexpr int kWgPerCu = MIN_WAVES * 4 / kMx4Waves;
  static_assert(kWgPerCu >= 1, "resident workgroups");
  const int64_t grid = (int64_t)device_cu_count() * kWgPerCu;
  hipLaunchKernelGGL((grouped_gemm_mxfp4_decode<DUAL, RB, MIN_WAVES, PD, KS, Q>), dim3((unsigned)grid),
                     dim3(kMx4Waves * kWave), 0, st, act, offsets, expert_groups(s), wa, sa, wb, sb, N,
                     K, out, gather, s.top_k, s.T * s.top_k, s.T);
  return hipGetLastError();
}

template <bool DUAL, int RB, int MIN_WAVES, int PD, int KS>
hipError_t launch_ks(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                     const uint8_t* wa, const uint8_t* sa, const uint8_t* wb, const uint8_t* sb,
                     int N, int K, void* out, hipStream_t st, const int32_t* gather) {
  const int nsp = K / kMx4StageK / KS;
  if (nsp % 2 == 0)
    return launch_kq<DUAL, RB, MIN_WAVES, PD, KS, 2>(s, act, offsets, wa, sa, wb, sb, N, K, out, st, gather);
  return launch_kq<DUAL, RB, MIN_WAVES, PD, KS, 1>(s, act, offsets, wa, sa, wb, sb, N, K, out, st, gather);
}

template <bool DUAL, int RB, int MIN_WAVES, int PD>
hipError_t launch_variant(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint8_t* wa, const uint8_t* sa, const uint8_t* wb,
                          const uint8_t* sb, int N, int K, void* out, hipStream_t st,
                          const int32_t* gather = nullptr) {
  if (max_rows_per_expert(s) <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  const int nst = K / kMx4StageK;
  if (nst % 4 == 0)
    return launch_ks<DUAL, RB, MIN_WAVES, PD, 4>(s, act, offsets, wa, sa, wb, sb, N, K, out, st, gather);
  if (nst % 2 == 0)
    return launch_ks<DUAL, RB, MIN_WAVES, PD, 2>(s, act, offsets, wa, sa, wb, sb, N, K, out, st, gather);
  return launch_ks<DUAL, RB, MIN_WAVES, PD, 1>(s, act, offsets, wa, sa, wb, sb, N, K, out, st, gather);
}

}  // namespace

hipError_t launch_gate_up_mxfp4(const moe_shape_t& s, const uint16_t* x_perm,
                                const int32_t* offsets, const uint8_t* w1, const uint8_t* w1_scale,
                                const uint8_t* w3, const uint8_t* w3_scale, uint16_t* h,
                                hipStream_t st) {
  // Measured at the Mixtral decode shape (up to 6 rows per expert): 32 channels
  // per wavefront, K split in four, one stage ahead, three workgroups per CU
  // (the one-group-per-workgroup form was 12% slower, 64 channels per
  // wavefront at two workgroups per CU 14% slower).
  return launch_variant<true, 2, 3, 1>(s, x_perm, offsets, w1, w1_scale, w3, w3_scale, s.d_ff,
                                       s.d_model, h, st);
}

hipError_t launch_gate_up_mxfp4_gather(const moe_shape_t& s, const uint16_t* x, const int32_t* perm_src,
                                       const int32_t* offsets, const uint8_t* w1, const uint8_t* w1_scale,
                                       const uint8_t* w3, const uint8_t* w3_scale, uint16_t* h,
                                       hipStream_t st) {
  return launch_variant<true, 2, 3, 1>(s, x, offsets, w1, w1_scale, w3, w3_scale, s.d_ff, s.d_model, h,
                                       st, perm_src);
}

hipError_t launch_down_mxfp4(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                             const uint8_t* w2, const uint8_t* w2_scale, float* y_perm,
                             hipStream_t st) {
  // 64 channels per wavefront, K (14336) split in four, one stage ahead (two
  // ahead was 5% slower once the scale bytes came two stages per load).
  return launch_variant<false, 4, 2, 1>(s, h, offsets, w2, w2_scale, nullptr, nullptr, s.d_model,
                                        s.d_ff, y_perm, st);
}

}  // namespace moe

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
#include "device_common.hpp"
#include "launch.hpp"
#include "lds_stream.hpp"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

template <bool DUAL, int ROWS, int MIN_WAVES>
__global__ __launch_bounds__(kWavesPerBlock * kWave, MIN_WAVES) void grouped_gemm_bf16_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int N, int K,
    void* __restrict__ out, int tok_tiles) {
  constexpr int KB = 512 / ROWS;        // elements per row per stage
  constexpr int CPR = KB / 8;           // 16-byte chunks per row per stage
  constexpr int NL = 16 / ROWS;         // load instructions per matrix per stage
  constexpr int NM = DUAL ? 2 : 1;
  constexpr int ROW_BYTES = KB * 2;
  constexpr int KEY_MASK = (CPR < 16 ? CPR : 16) - 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWavesPerBlock][NM][16 * ROW_BYTES];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int groups = N / 16;
  const int gid = blockIdx.x * kWavesPerBlock + w;
  const int cg = gid % groups;
  const int rest = gid / groups;
  const int tt = rest % tok_tiles;
  const int e = rest / tok_tiles;
  if (e >= E) return;
  const int row0 = offsets[e] + tt * 16;
  const int rows = min(16, offsets[e + 1] - row0);
  if (rows <= 0) return;

  // wide loader: instruction i covers rows ROWS i .. ROWS i + ROWS - 1
  constexpr int LPR = kWave / ROWS;     // lanes per row (== CPR)
  const int lrow = lane / LPR, lch = lane % LPR;
  const uint16_t* pw[NM];
  pw[0] = wa + ((int64_t)e * N + cg * 16) * K;
  if constexpr (DUAL) pw[1] = wb + ((int64_t)e * N + cg * 16) * K;
  // matrix-core operand: lane (r, g) feeds row r, chunk 4 j + g of MFMA j
  const int r = lane & 15, g = lane >> 4;
  const bool tok_ok = r < rows;
  const uint16_t* px = act + (int64_t)(row0 + (tok_ok ? r : 0)) * K + g * 8;

  f32x4_t acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nst = K / KB;
  for (int st = 0; st < nst; ++st) {
    const int k0 = st * KB;
    uint4 v[NM][NL];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < NL; ++i)
        v[m][i] = load_stream16(pw[m] + (int64_t)(i * ROWS + lrow) * K + k0 + lch * 8);
    uint4 xv[KB / 32];
#pragma unroll
    for (int j = 0; j < KB / 32; ++j)
      xv[j] = tok_ok ? *reinterpret_cast<const uint4*>(px + k0 + j * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int row = i * ROWS + lrow;
        const int pc = lch ^ (row & KEY_MASK);
        *reinterpret_cast<uint4*>(&lds[w][m][row * ROW_BYTES + pc * 16]) = v[m][i];
      }
#pragma unroll
    for (int j = 0; j < KB / 32; ++j) {
      const int pc = (4 * j + g) ^ (r & KEY_MASK);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 a = *reinterpret_cast<const uint4*>(&lds[w][m][r * ROW_BYTES + pc * 16]);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(xv[j]), acc[m],
                                                         0, 0, 0);
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
    for (int i = 0; i < 4; ++i) hv[i] = swiglu_fast(acc[0][i], acc[1][i]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * N + c) =
        make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * N + c) =
        make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
  }
}

template <bool DUAL, int ROWS, int MIN_WAVES>
hipError_t launch_variant(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                          hipStream_t st) {
  const int tok_tiles = (int)((max_rows_per_expert(s) + 15) / 16);
  const int64_t groups = (int64_t)expert_groups(s) * tok_tiles * (N / 16);
  if (groups <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  const int64_t blocks = (groups + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((grouped_gemm_bf16_decode<DUAL, ROWS, MIN_WAVES>), dim3((unsigned)blocks),
                     dim3(kWavesPerBlock * kWave), 0, st, act, offsets, expert_groups(s), wa, wb, N, K,
                     out, tok_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const moe_shape_t& s, bool dual, const uint16_t* act,
                              const int32_t* offsets, const uint16_t* wa, const uint16_t* wb,
                              int N, int K, void* out, hipStream_t st) {
  // Measured at the Mixtral shape (4 rows per expert): dual with 8 rows x 128 B
  // per load instruction streams 6.5 TB/s; single with 4 rows x 256 B, 6.3 TB/s.
  if (dual) return launch_variant<true, 8, 4>(s, act, offsets, wa, wb, N, K, out, st);
  if (K % 128 == 0) return launch_variant<false, 4, 4>(s, act, offsets, wa, wb, N, K, out, st);
  return launch_variant<false, 8, 4>(s, act, offsets, wa, wb, N, K, out, st);
}

}  // namespace moe

// bf16 grouped expert GEMMs for few tokens per expert (decode): weight streaming.
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x);
// "Mixtral and Mixture-of-Experts, Explained" notes the extra memory loads of
// running more than one expert per device -- at decode the layer is bound by
// reading the touched experts' weights once.
//
// A row group is 16 output channels (dual: 16 rows of w1 and the same 16 of
// w3) of one expert against one tile of up to 16 of its tokens.  S wavefronts
// of a workgroup share a row group and each streams one K slice of it, so the
// 8 KB rows are read by neighbouring wavefronts at the same time; the S
// partial 16x16 tiles are summed through LDS in a fixed order (deterministic).
// With S = 1 each of the 4 wavefronts of a workgroup owns its own row group.
// Each wavefront starts its K walk at a block rotated by its row group, so
// wavefronts that run together do not all hit the same address offset of
// rows spaced by a power of two.  Lane (r, g) feeds row r; MFMA j of a K
// block takes elements k0 + 32 j .. + 31, lane group g its 8-element chunk g,
// so the 4 lanes of a row read 64 contiguous bytes per load instruction;
// weights use non-temporal loads (read once) and the next block is prefetched
// into registers while v_mfma_f32_16x16x32_bf16 consumes the current one.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

__device__ __forceinline__ float swiglu_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

template <bool DUAL, int S, int KB, int MIN_WAVES>
__global__ __launch_bounds__(S == 1 ? 256 : S * 64, MIN_WAVES) void grouped_gemm_bf16_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int N, int K,
    void* __restrict__ out, int tok_tiles) {
  constexpr int NC = KB / 32;
  __shared__ f32x4_t part[S > 1 ? S : 1][2][kWave];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int groups = N / 16;
  const int gid = S == 1 ? blockIdx.x * 4 + w : blockIdx.x;
  const int cg = gid % groups;
  const int rest = gid / groups;
  const int tt = rest % tok_tiles;
  const int e = rest / tok_tiles;
  if (e >= E) return;
  const int row0 = offsets[e] + tt * 16;
  const int rows = min(16, offsets[e + 1] - row0);
  if (rows <= 0) return;   // uniform across the workgroup (same row group)

  const int r = lane & 15, g = lane >> 4;
  const int kslice = K / S;
  const int nblk = kslice / KB;
  const int64_t kofs = (int64_t)(S == 1 ? 0 : w) * kslice + g * 8;
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
  int blk = (int)(((unsigned)cg * 7u + (unsigned)e * 13u) % (unsigned)nblk);
  load(blk * KB, ca, cb, cx);
  for (int i = 0; i < nblk; ++i) {
    const bool more = i + 1 < nblk;
    const int next = blk + 1 == nblk ? 0 : blk + 1;
    if (more) load(next * KB, na, nb, nx);
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
    blk = next;
  }
  if constexpr (S > 1) {
    part[w][0][lane] = acc_a;
    if constexpr (DUAL) part[w][1][lane] = acc_b;
    __syncthreads();
    if (w != 0) return;
    acc_a = part[0][0][lane];
    if constexpr (DUAL) acc_b = part[0][1][lane];
#pragma unroll
    for (int i = 1; i < S; ++i) {
      acc_a += part[i][0][lane];
      if constexpr (DUAL) acc_b += part[i][1][lane];
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

template <bool DUAL, int S, int KB, int MIN_WAVES>
hipError_t launch_variant(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                          hipStream_t st) {
  const int tok_tiles = (int)((max_rows_per_expert(s) + 15) / 16);
  const int64_t groups = (int64_t)s.n_experts * tok_tiles * (N / 16);
  if (groups <= 0) return hipSuccess;   // no expert can hold a row (capacity 0)
  const int64_t blocks = S == 1 ? (groups + 3) / 4 : groups;
  hipLaunchKernelGGL((grouped_gemm_bf16_decode<DUAL, S, KB, MIN_WAVES>), dim3((unsigned)blocks),
                     dim3(S == 1 ? 256 : S * 64), 0, st, act, offsets, s.n_experts, wa, wb, N, K,
                     out, tok_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const moe_shape_t& s, bool dual, const uint16_t* act,
                              const int32_t* offsets, const uint16_t* wa, const uint16_t* wb,
                              int N, int K, void* out, hipStream_t st) {
  // Measured on MI355X at the Mixtral shape (4 rows per expert): dual with a
  // 4-way K split reads 5.3 TB/s, single with 128-wide blocks 4.8 TB/s.
  if (dual) {
    if (K % (4 * 128) == 0) return launch_variant<true, 4, 128, 1>(s, act, offsets, wa, wb, N, K, out, st);
    return launch_variant<true, 1, 64, 7>(s, act, offsets, wa, wb, N, K, out, st);
  }
  if (K % 128 == 0) return launch_variant<false, 1, 128, 4>(s, act, offsets, wa, wb, N, K, out, st);
  return launch_variant<false, 1, 64, 8>(s, act, offsets, wa, wb, N, K, out, st);
}

}  // namespace moe

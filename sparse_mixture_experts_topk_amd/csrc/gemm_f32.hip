// fp32 grouped expert GEMMs (activation and weight dtype fp32).
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x)
// and section "SwiGLU Experts".
//
// A plain LDS-tiled VALU GEMM: a 256-lane workgroup owns 64 rows (tokens of
// one expert) x 64 output channels, stages 16-wide K slices of the token rows
// and the weight rows in LDS, and each lane accumulates a 4 x 4 block in fp32
// with fma.  The dual variant keeps the w1 and w3 blocks side by side and
// applies silu(g) * u before storing h.  Sized for small layers; the same
// grouped tile schedule as the matrix-core kernels (token tiles of one
// expert fastest) is used.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int F32_TM = 64;   // token rows per tile
constexpr int F32_TN = 64;   // channels per tile
constexpr int F32_TK = 16;   // K per stage

template <bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const float* __restrict__ wa, const float* __restrict__ wb, int N, int K,
    float* __restrict__ out, int n_tiles) {
  __shared__ float s_act[F32_TK][F32_TM + 4];
  __shared__ float s_wa[F32_TK][F32_TN + 4];
  __shared__ float s_wb[DUAL ? F32_TK : 1][F32_TN + 4];

  int e, r0, r1, mt, nt;
  if (!locate_tile(offsets, E, F32_TM, n_tiles, blockIdx.x, e, r0, r1, mt, nt)) return;
  const int row0 = r0 + mt * F32_TM;
  const int rows = min(F32_TM, r1 - row0);
  const int ch0 = nt * F32_TN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float* wae = wa + (int64_t)e * N * K;
  const float* wbe = DUAL ? wb + (int64_t)e * N * K : nullptr;

  float acc[4][4], acc3[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc3[i][j] = 0.f;

  // Loader: 64 rows x 16 k per operand = 1024 floats = 4 per lane.
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  for (int k0 = 0; k0 < K; k0 += F32_TK) {
    float4 va = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lr < rows) va = *reinterpret_cast<const float4*>(act + (int64_t)(row0 + lr) * K + k0 + lk);
    float4 vw = make_float4(0.f, 0.f, 0.f, 0.f), vw3 = vw;
    if (ch0 + lr < N) {
      vw = *reinterpret_cast<const float4*>(wae + (int64_t)(ch0 + lr) * K + k0 + lk);
      if constexpr (DUAL) vw3 = *reinterpret_cast<const float4*>(wbe + (int64_t)(ch0 + lr) * K + k0 + lk);
    }
    s_act[lk + 0][lr] = va.x; s_act[lk + 1][lr] = va.y; s_act[lk + 2][lr] = va.z; s_act[lk + 3][lr] = va.w;
    s_wa[lk + 0][lr] = vw.x; s_wa[lk + 1][lr] = vw.y; s_wa[lk + 2][lr] = vw.z; s_wa[lk + 3][lr] = vw.w;
    if constexpr (DUAL) {
      s_wb[lk + 0][lr] = vw3.x; s_wb[lk + 1][lr] = vw3.y; s_wb[lk + 2][lr] = vw3.z; s_wb[lk + 3][lr] = vw3.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F32_TK; ++kk) {
      float a[4], w[4], w3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = s_act[kk][ty * 4 + i];
        w[i] = s_wa[kk][tx * 4 + i];
        if constexpr (DUAL) w3[i] = s_wb[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
          if constexpr (DUAL) acc3[i][j] = fmaf(a[i], w3[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    const int c = ch0 + tx * 4;
    if (r >= rows || c >= N) continue;
    float4 o;
    if constexpr (DUAL) {
      o = make_float4(silu_f32(acc[i][0]) * acc3[i][0], silu_f32(acc[i][1]) * acc3[i][1],
                      silu_f32(acc[i][2]) * acc3[i][2], silu_f32(acc[i][3]) * acc3[i][3]);
    } else {
      o = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
    *reinterpret_cast<float4*>(out + (int64_t)(row0 + r) * N + c) = o;
  }
}

template <bool DUAL>
hipError_t launch_f32(const moe_shape_t& s, const float* act, const int32_t* offsets,
                      const float* wa, const float* wb, int N, int K, float* out, hipStream_t st) {
  const int n_tiles = (N + F32_TN - 1) / F32_TN;
  const int64_t grid = max_token_tiles(s, F32_TM) * n_tiles;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<DUAL>, dim3((unsigned)grid), dim3(256), 0, st, act,
                     offsets, expert_groups(s), wa, wb, N, K, out, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_f32(const moe_shape_t& s, const float* x_perm, const int32_t* offsets,
                              const float* w1, const float* w3, float* h, hipStream_t st) {
  return launch_f32<true>(s, x_perm, offsets, w1, w3, s.d_ff, s.d_model, h, st);
}

hipError_t launch_down_f32(const moe_shape_t& s, const float* h, const int32_t* offsets,
                           const float* w2, float* y_perm, hipStream_t st) {
  return launch_f32<false>(s, h, offsets, w2, nullptr, s.d_model, s.d_ff, y_perm, st);
}

}  // namespace moe

// Gate-weighted combine back to token order.
//
// Pages: "Mixtral and Mixture-of-Experts, Explained", y = sum_i G(x)_i *
// Expert_i(x); "Mixtral" study notes, MoE forward (the output starts at zero
// in x's shape, then each expert's rows are accumulated with their gate weight).
//
// One workgroup per token row: y[t] = G0 * y_perm[row0] + G1 * y_perm[row1]
// over the kept slots (a dropped slot has row -1 and adds nothing), computed
// in fp32 as fma(G1, b, G0 * a) and rounded once to the activation dtype.
// Top-k with a shared expert (DeepSeek-V3 remark on the "Mixtral 8x7B"
// interview page): the same fma chain over the k slots in slot order, then
// the shared expert's row with weight 1.
// Gathers instead of scatter-adds, so there are no atomics and the result is
// deterministic.  HBM-bound: reads the kept y_perm rows, writes y once.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_to_row,
                                                      const float* __restrict__ gw, int d,
                                                      void* __restrict__ y) {
  const int t = blockIdx.x;
  const int2 rows = reinterpret_cast<const int2*>(slot_to_row)[t];
  const float2 g = reinterpret_cast<const float2*>(gw)[t];
  const float4* a = rows.x >= 0 ? reinterpret_cast<const float4*>(y_perm + (int64_t)rows.x * d) : nullptr;
  const float4* b = rows.y >= 0 ? reinterpret_cast<const float4*>(y_perm + (int64_t)rows.y * d) : nullptr;
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a != nullptr) {
      const float4 v = a[c];
      r = make_float4(g.x * v.x, g.x * v.y, g.x * v.z, g.x * v.w);
    }
    if (b != nullptr) {
      const float4 v = b[c];
      r = make_float4(fmaf(g.y, v.x, r.x), fmaf(g.y, v.y, r.y), fmaf(g.y, v.z, r.z),
                      fmaf(g.y, v.w, r.w));
    }
    if constexpr (BF16) {
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (int64_t)t * d)[c] =
          make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(y) + (int64_t)t * d)[c] = r;
    }
  }
}

// K slots and S (0 or 1) shared rows (slot T*K + t).  Every row's load is
// issued unconditionally (a dropped slot reads row 0 and is selected away),
// so the K + S gathers of a lane are in flight together.
template <bool BF16, int K, int S>
__global__ __launch_bounds__(256) void combine_topk_kernel(const float* __restrict__ y_perm,
                                                           const int32_t* __restrict__ slot_to_row,
                                                           const float* __restrict__ gw, int d, int T,
                                                           void* __restrict__ y) {
  constexpr int N = K + S;
  const int t = blockIdx.x;
  int rows[N];
  float g[N];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = slot_to_row[(int64_t)t * K + j];
    g[j] = gw[(int64_t)t * K + j];
  }
  if constexpr (S == 1) {
    rows[K] = slot_to_row[(int64_t)T * K + t];
    g[K] = 1.0f;
  }
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    float4 v[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float4 a = reinterpret_cast<const float4*>(y_perm + (int64_t)(rows[j] >= 0 ? rows[j] : 0) * d)[c];
      v[j] = rows[j] >= 0 ? a : z;
    }
    float4 r = z;
#pragma unroll
    for (int j = 0; j < N; ++j)
      r = make_float4(fmaf(g[j], v[j].x, r.x), fmaf(g[j], v[j].y, r.y), fmaf(g[j], v[j].z, r.z),
                      fmaf(g[j], v[j].w, r.w));
    if constexpr (BF16) {
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (int64_t)t * d)[c] =
          make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(y) + (int64_t)t * d)[c] = r;
    }
  }
}

template <int K, int S>
hipError_t launch_topk(const moe_shape_t& s, const float* y_perm, const int32_t* slot_to_row,
                       const float* weights, void* y, hipStream_t st) {
  if (s.act_dtype == MOE_BF16)
    hipLaunchKernelGGL((combine_topk_kernel<true, K, S>), dim3(s.T), dim3(256), 0, st, y_perm,
                       slot_to_row, weights, s.d_model, s.T, y);
  else
    hipLaunchKernelGGL((combine_topk_kernel<false, K, S>), dim3(s.T), dim3(256), 0, st, y_perm,
                       slot_to_row, weights, s.d_model, s.T, y);
  return hipGetLastError();
}

template <int S>
hipError_t launch_k(const moe_shape_t& s, const float* y_perm, const int32_t* slot_to_row,
                    const float* weights, void* y, hipStream_t st) {
  static_assert(kMaxTopK == 8, "one instance per k");
  switch (s.top_k) {
    case 1: return launch_topk<1, S>(s, y_perm, slot_to_row, weights, y, st);
    case 2: return launch_topk<2, S>(s, y_perm, slot_to_row, weights, y, st);
    case 3: return launch_topk<3, S>(s, y_perm, slot_to_row, weights, y, st);
    case 4: return launch_topk<4, S>(s, y_perm, slot_to_row, weights, y, st);
    case 5: return launch_topk<5, S>(s, y_perm, slot_to_row, weights, y, st);
    case 6: return launch_topk<6, S>(s, y_perm, slot_to_row, weights, y, st);
    case 7: return launch_topk<7, S>(s, y_perm, slot_to_row, weights, y, st);
    default: return launch_topk<8, S>(s, y_perm, slot_to_row, weights, y, st);
  }
}

}  // namespace

hipError_t launch_combine(const moe_shape_t& s, const float* y_perm, const int32_t* slot_to_row,
                          const float* weights, void* y, hipStream_t st) {
  if (s.n_shared != 0) return launch_k<1>(s, y_perm, slot_to_row, weights, y, st);
  if (s.top_k != 2) return launch_k<0>(s, y_perm, slot_to_row, weights, y, st);
  if (s.act_dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(s.T), dim3(256), 0, st, y_perm, slot_to_row,
                       weights, s.d_model, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(s.T), dim3(256), 0, st, y_perm, slot_to_row,
                       weights, s.d_model, y);
  return hipGetLastError();
}

}  // namespace moe

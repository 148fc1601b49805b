// Router GEMV fused with top-2 selection and the two-way softmax.
//
// Pages: "Mixtral" study notes, MixtralMoE.forward (gate -> topk -> softmax of
// the kept logits); "Mixtral and Mixture-of-Experts, Explained", gate equation
// G(x) = Softmax(TopK(x . W_g)) with non-selected logits at -inf, so the kept
// pair's weights are w0 = 1 / (1 + exp(l1 - l0)) and w1 = 1 - w0.
//
// Mapping: one wavefront owns TPW = 64 / EP tokens (EP = n_experts rounded up
// to 8, 16, 32 or 64).  Each lane strides over d in 16-byte vectors of x and
// of every router row, accumulating TPW * EP = 64 fp32 partial sums.  A
// recursive-halving exchange (6 shuffle rounds, 63 exchanges) then leaves lane
// L holding the full logit of (token L / EP, expert L % EP); the top-2 is a
// butterfly arg-max inside each EP-lane group, ties going to the lower index.
// W_g (64 KiB at d = 4096, E = 8) stays L2-resident; x is read once.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <bool BF16>
__device__ __forceinline__ void load_vec(const void* base, int64_t off, float* out) {
  if constexpr (BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
}

template <int EP, bool BF16>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const void* __restrict__ x, const void* __restrict__ wg, const float* __restrict__ bias, int T,
    int d, int E, int32_t* __restrict__ ids, float* __restrict__ wout, float* __restrict__ logits) {
  constexpr int TPW = kWave / EP;
  constexpr int VEC = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int tok0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * TPW;
  if (tok0 >= T) return;  // whole wavefront leaves; the kernel has no barrier

  float acc[TPW * EP];
#pragma unroll
  for (int i = 0; i < TPW * EP; ++i) acc[i] = 0.f;

  for (int k = lane * VEC; k < d; k += kWave * VEC) {
    float xv[TPW][VEC];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (tok0 + t < T) {
        load_vec<BF16>(x, (int64_t)(tok0 + t) * d + k, xv[t]);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) xv[t][v] = 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      if (e < E) {
        float wv[VEC];
        load_vec<BF16>(wg, (int64_t)e * d + k, wv);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[t * EP + e] = fmaf(xv[t][v], wv[v], acc[t * EP + e]);
      }
    }
  }

  // Recursive halving across the wavefront: after the round with offset o,
  // a lane keeps the half of its values whose index bit log2(o) equals its
  // own lane bit, and adds the partner's copy of that half.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const bool upper = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < o; ++i) {
      const float send = upper ? acc[i] : acc[i + o];
      const float keep = upper ? acc[i + o] : acc[i];
      acc[i] = keep + __shfl_xor(send, o);
    }
  }

  const int t = lane / EP, e = lane % EP;
  const int tok = tok0 + t;
  const bool real = e < E;
  float l = acc[0];
  if (real && bias != nullptr) l += bias[e];
  if (logits != nullptr && real && tok < T) logits[(int64_t)tok * E + e] = l;

  // Top-2 inside each group of EP lanes: (value desc, index asc).
  float v0 = real ? l : -INFINITY;
  int i0 = e;
#pragma unroll
  for (int o = EP / 2; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v0, o);
    const int oi = __shfl_xor(i0, o);
    if (ov > v0 || (ov == v0 && oi < i0)) { v0 = ov; i0 = oi; }
  }
  float v1 = (real && e != i0) ? l : -INFINITY;
  int i1 = e;
#pragma unroll
  for (int o = EP / 2; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v1, o);
    const int oi = __shfl_xor(i1, o);
    if (ov > v1 || (ov == v1 && oi < i1)) { v1 = ov; i1 = oi; }
  }
  if (e == 0 && tok < T) {
    const float w0 = 1.0f / (1.0f + expf(v1 - v0));
    reinterpret_cast<int2*>(ids)[tok] = make_int2(i0, i1);
    reinterpret_cast<float2*>(wout)[tok] = make_float2(w0, 1.0f - w0);
  }
}

template <int EP, bool BF16>
hipError_t launch_ep(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                     int32_t* ids, float* w, float* logits, hipStream_t st) {
  constexpr int TPW = kWave / EP;
  const int waves = (s.T + TPW - 1) / TPW;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((route_topk_kernel<EP, BF16>), dim3(blocks), dim3(256), 0, st, x, wg, bias,
                     s.T, s.d_model, s.n_experts, ids, w, logits);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                        int32_t* ids, float* w, float* logits, hipStream_t st) {
  if (s.n_experts <= 8) return launch_ep<8, BF16>(s, x, wg, bias, ids, w, logits, st);
  if (s.n_experts <= 16) return launch_ep<16, BF16>(s, x, wg, bias, ids, w, logits, st);
  if (s.n_experts <= 32) return launch_ep<32, BF16>(s, x, wg, bias, ids, w, logits, st);
  return launch_ep<64, BF16>(s, x, wg, bias, ids, w, logits, st);
}

}  // namespace

hipError_t launch_route_topk(const moe_shape_t& s, const void* x, const void* w_gate,
                             const float* bias, int32_t* ids, float* weights, float* logits,
                             hipStream_t st) {
  if (s.act_dtype == MOE_BF16)
    return launch_dtype<true>(s, x, w_gate, bias, ids, weights, logits, st);
  return launch_dtype<false>(s, x, w_gate, bias, ids, weights, logits, st);
}

}  // namespace moe

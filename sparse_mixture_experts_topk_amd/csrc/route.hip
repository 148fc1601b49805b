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
// On request the two best experts outside the top-2 (ranks 3 and 4, the
// targets of the overflow fallback) follow with the same arg-max.
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
    int d, int E, int32_t* __restrict__ ids, float* __restrict__ wout, float* __restrict__ logits,
    int32_t* __restrict__ next) {
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
  if (next != nullptr) {   // ranks 3 and 4: the same arg-max outside the top-2
    float v2 = (real && e != i0 && e != i1) ? l : -INFINITY;
    int i2 = e;
#pragma unroll
    for (int o = EP / 2; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(v2, o);
      const int oi = __shfl_xor(i2, o);
      if (ov > v2 || (ov == v2 && oi < i2)) { v2 = ov; i2 = oi; }
    }
    float v3 = (real && e != i0 && e != i1 && e != i2) ? l : -INFINITY;
    int i3 = e;
#pragma unroll
    for (int o = EP / 2; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(v3, o);
      const int oi = __shfl_xor(i3, o);
      if (ov > v3 || (ov == v3 && oi < i3)) { v3 = ov; i3 = oi; }
    }
    // logits are finite, so -inf marks a rank past n_experts
    if (e == 0 && tok < T)
      reinterpret_cast<int2*>(next)[tok] = make_int2(v2 == -INFINITY ? -1 : i2, v3 == -INFINITY ? -1 : i3);
  }
}

// ---------------------------------------------------------------------------
// bf16 router on the matrix cores.  A 512-lane workgroup owns 16 tokens; its
// 8 wavefronts split K, each accumulating D[expert][token] = W_g . x^T with
// v_mfma_f32_16x16x32_bf16 (A = 16 router rows, B = 16 token rows, zero rows
// past E / T), for EB blocks of 16 experts.  Partial tiles are summed through
// LDS in a fixed order; wavefront 0 then holds, per lane, token (lane & 15)
// and experts 16 eb + 4 (lane >> 4) + r.  Each lane keeps its local top-2
// and two xor-shuffle merges (16, 32) give the token's top-2 (on request a
// second such pass outside the top-2 gives ranks 3 and 4).  Exact in the
// sense that matters: bf16 products are exact in fp32 and accumulate in fp32.
constexpr int kRouteWaves = 8;

// (value, index) a ranks before b: larger value, or equal value and lower index.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Merge two sorted top-2 lists (v0,i0 >= v1,i1) and (w0,j0 >= w1,j1) into the first.
// Plain scalars and selects, so everything stays in registers.
__device__ __forceinline__ void merge2(float& v0, int& i0, float& v1, int& i1, float w0, int j0,
                                       float w1, int j1) {
  const bool a_first = better(v0, i0, w0, j0);
  const float fv = a_first ? v0 : w0;
  const int fi = a_first ? i0 : j0;
  // runner-up: best of the loser's head and the winner's second
  const float cv = a_first ? w0 : v0;
  const int ci = a_first ? j0 : i0;
  const float sv2 = a_first ? v1 : w1;
  const int si2 = a_first ? i1 : j1;
  const bool c_second = better(cv, ci, sv2, si2);
  v1 = c_second ? cv : sv2;
  i1 = c_second ? ci : si2;
  v0 = fv;
  i0 = fi;
}

template <int EB>
__global__ __launch_bounds__(kRouteWaves * 64) void route_topk_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias,
    int T, int d, int E, int32_t* __restrict__ ids, float* __restrict__ wout,
    float* __restrict__ logits, int32_t* __restrict__ next) {
  __shared__ f32x4_t part[kRouteWaves - 1][EB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const bool tok_ok = tok0 + r < T;
  const uint16_t* px = x + (int64_t)(tok_ok ? tok0 + r : 0) * d + g * 8;
  const uint16_t* pw[EB];
  bool w_ok[EB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    w_ok[eb] = eb * 16 + r < E;
    pw[eb] = wg + (int64_t)(w_ok[eb] ? eb * 16 + r : 0) * d + g * 8;
  }
  f32x4_t acc[EB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) acc[eb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nblk = d / 32;
  const int b0 = wave * nblk / kRouteWaves, b1 = (wave + 1) * nblk / kRouteWaves;
  // all of a wavefront's K blocks in flight at once at d = 4096 (16 per wavefront)
  constexpr int U = 16 / EB;
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int b = b0; b < b1; b += U) {
    // Unconditional 16-byte loads from clamped (always valid) addresses, then a
    // select: a conditional load would be split into guarded dword loads.
    uint4 xa[U], wa[U][EB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = b + u < b1;
      const int blk = in ? b + u : b0;
      const uint4 xv = *reinterpret_cast<const uint4*>(px + blk * 32);
      xa[u] = (in && tok_ok) ? xv : z;
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        const uint4 wv = *reinterpret_cast<const uint4*>(pw[eb] + blk * 32);
        wa[u][eb] = (in && w_ok[eb]) ? wv : z;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
        acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[u][eb]), as_bf16x8(xa[u]),
                                                           acc[eb], 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) part[wave - 1][eb][lane] = acc[eb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kRouteWaves - 1; ++w)
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) acc[eb] += part[w][eb][lane];

  const int tok = tok0 + r;
  // local top-2 over this lane's experts, visited in increasing index order
  float v0 = -INFINITY, v1 = -INFINITY;
  int i0 = 1 << 30, i1 = 1 << 30;
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    const int ebase = eb * 16 + 4 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = ebase + q;
      const bool real = e < E;
      float l = acc[eb][q];
      if (real && bias != nullptr) l += bias[e];
      acc[eb][q] = l;
      const float lv = real ? l : -INFINITY;
      const int li = real ? e : (1 << 30);
      const bool top = better(lv, li, v0, i0);
      const bool sec = !top && better(lv, li, v1, i1);
      v1 = top ? v0 : (sec ? lv : v1);
      i1 = top ? i0 : (sec ? li : i1);
      v0 = top ? lv : v0;
      i0 = top ? li : i0;
    }
    if (logits != nullptr && tok < T) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (ebase + q < E) logits[(int64_t)tok * E + ebase + q] = acc[eb][q];
    }
  }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float w0 = __shfl_xor(v0, o), w1 = __shfl_xor(v1, o);
    const int j0 = __shfl_xor(i0, o), j1 = __shfl_xor(i1, o);
    merge2(v0, i0, v1, i1, w0, j0, w1, j1);
  }
  if (g == 0 && tok < T) {
    const float w0 = 1.0f / (1.0f + expf(v1 - v0));
    reinterpret_cast<int2*>(ids)[tok] = make_int2(i0, i1);
    reinterpret_cast<float2*>(wout)[tok] = make_float2(w0, 1.0f - w0);
  }
  if (next != nullptr) {   // ranks 3 and 4: top-2 of the experts outside the top-2
    float u0 = -INFINITY, u1 = -INFINITY;
    int j0 = 1 << 30, j1 = 1 << 30;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = eb * 16 + 4 * g + q;
        const bool cand = e < E && e != i0 && e != i1;
        const float lv = cand ? acc[eb][q] : -INFINITY;
        const int li = cand ? e : (1 << 30);
        const bool top = better(lv, li, u0, j0);
        const bool sec = !top && better(lv, li, u1, j1);
        u1 = top ? u0 : (sec ? lv : u1);
        j1 = top ? j0 : (sec ? li : j1);
        u0 = top ? lv : u0;
        j0 = top ? li : j0;
      }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float w0 = __shfl_xor(u0, o), w1 = __shfl_xor(u1, o);
      const int k0 = __shfl_xor(j0, o), k1 = __shfl_xor(j1, o);
      merge2(u0, j0, u1, j1, w0, k0, w1, k1);
    }
    // logits are finite, so -inf marks a rank past n_experts
    if (g == 0 && tok < T)
      reinterpret_cast<int2*>(next)[tok] = make_int2(u0 == -INFINITY ? -1 : j0, u1 == -INFINITY ? -1 : j1);
  }
}

template <int EB>
hipError_t launch_mfma(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                       int32_t* ids, float* w, float* logits, int32_t* next, hipStream_t st) {
  const int blocks = (s.T + 15) / 16;
  hipLaunchKernelGGL((route_topk_mfma_kernel<EB>), dim3(blocks), dim3(kRouteWaves * 64), 0, st,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), bias, s.T,
                     s.d_model, s.n_experts, ids, w, logits, next);
  return hipGetLastError();
}

template <int EP, bool BF16>
hipError_t launch_ep(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                     int32_t* ids, float* w, float* logits, int32_t* next, hipStream_t st) {
  constexpr int TPW = kWave / EP;
  const int waves = (s.T + TPW - 1) / TPW;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((route_topk_kernel<EP, BF16>), dim3(blocks), dim3(256), 0, st, x, wg, bias,
                     s.T, s.d_model, s.n_experts, ids, w, logits, next);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                        int32_t* ids, float* w, float* logits, int32_t* next, hipStream_t st) {
  if (s.n_experts <= 8) return launch_ep<8, BF16>(s, x, wg, bias, ids, w, logits, next, st);
  if (s.n_experts <= 16) return launch_ep<16, BF16>(s, x, wg, bias, ids, w, logits, next, st);
  if (s.n_experts <= 32) return launch_ep<32, BF16>(s, x, wg, bias, ids, w, logits, next, st);
  return launch_ep<64, BF16>(s, x, wg, bias, ids, w, logits, next, st);
}

}  // namespace

hipError_t launch_route_topk(const moe_shape_t& s, const void* x, const void* w_gate,
                             const float* bias, int32_t* ids, float* weights, float* logits,
                             int32_t* next_ids, hipStream_t st) {
  if (s.act_dtype == MOE_BF16) {
    if (s.n_experts <= 16) return launch_mfma<1>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
    if (s.n_experts <= 32) return launch_mfma<2>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
    return launch_mfma<4>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
  }
  return launch_dtype<false>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
}

}  // namespace moe

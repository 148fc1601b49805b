// Router GEMV fused with top-k selection and the softmax of the kept logits.
//
// Pages: "Mixtral" study notes, MixtralMoE.forward (gate -> topk -> softmax of
// the kept logits); "Mixtral and Mixture-of-Experts, Explained", gate equation
// G(x) = Softmax(TopK(x . W_g)) with non-selected logits at -inf, so a kept
// pair's weights are w0 = 1 / (1 + exp(l1 - l0)) and w1 = 1 - w0, and k kept
// logits get w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).  Many experts and
// k up to 8: the DeepSeek-V3 remark on the "Mixtral 8x7B" interview page
// (256 routed experts, 8 active per token).
//
// Up to 64 experts the router is one fused kernel (below); more experts
// (bf16) take two: logits over a token x expert grid, then selection.
//
// Selection, every kernel: k rounds of an arg-max (value descending, index
// ascending) over the experts not yet taken, so slot j holds the j-th largest
// logit and equal logits go to the lower index; on request two more rounds
// give the experts ranked k+1 and k+2 (the targets of the overflow fallback).
//
// Mapping: one wavefront owns TPW = 64 / EP tokens (EP = n_experts rounded up
// to 8, 16, 32 or 64).  Each lane strides over d in 16-byte vectors of x and
// of every router row, accumulating TPW * EP = 64 fp32 partial sums.  A
// recursive-halving exchange (6 shuffle rounds, 63 exchanges) then leaves lane
// L holding the full logit of (token L / EP, expert L % EP); each selection
// round is a butterfly arg-max inside the EP-lane group.
// W_g (64 KiB at d = 4096, E = 8) stays L2-resident; x is read once.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// Selection rounds at most: k, then ranks k+1 and k+2.
constexpr int kMaxRounds = kMaxTopK + 2;

// (value, index) a ranks before b: larger value, or equal value and lower index.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Gate weights of one token from its k kept logits v[0] >= v[1] >= ...:
// k == 2 keeps the logistic form (w0 + w1 == 1 exactly), otherwise the
// softmax relative to the largest logit.
__device__ __forceinline__ void gate_weights(const float (&v)[kMaxRounds], int k, float (&w)[kMaxTopK]) {
  if (k == 2) {
    w[0] = 1.0f / (1.0f + expf(v[1] - v[0]));
    w[1] = 1.0f - w[0];
    return;
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    w[j] = j < k ? expf(v[j] - v[0]) : 0.f;
    sum += w[j];
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) w[j] *= inv;
}

// One token's outputs: ids and weights [k], next [2] (-inf marks a rank past
// n_experts: logits are finite).
__device__ __forceinline__ void store_token(const float (&v)[kMaxRounds], const int (&id)[kMaxRounds],
                                            int k, int64_t tok, int32_t* __restrict__ ids,
                                            float* __restrict__ wout, int32_t* __restrict__ next) {
  float w[kMaxTopK];
  gate_weights(v, k, w);
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) {
      ids[tok * k + j] = id[j];
      wout[tok * k + j] = w[j];
    }
  if (next != nullptr) {
#pragma unroll
    for (int j = 0; j < kMaxRounds; ++j)
      if (j == k || j == k + 1) next[tok * 2 + (j - k)] = v[j] == -INFINITY ? -1 : id[j];
  }
}

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
    int d, int E, int k, int32_t* __restrict__ ids, float* __restrict__ wout,
    float* __restrict__ logits, int32_t* __restrict__ next) {
  constexpr int TPW = kWave / EP;
  constexpr int VEC = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int tok0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * TPW;
  if (tok0 >= T) return;  // whole wavefront leaves; the kernel has no barrier

  float acc[TPW * EP];
#pragma unroll
  for (int i = 0; i < TPW * EP; ++i) acc[i] = 0.f;

  for (int kk = lane * VEC; kk < d; kk += kWave * VEC) {
    float xv[TPW][VEC];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (tok0 + t < T) {
        load_vec<BF16>(x, (int64_t)(tok0 + t) * d + kk, xv[t]);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) xv[t][v] = 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      if (e < E) {
        float wv[VEC];
        load_vec<BF16>(wg, (int64_t)e * d + kk, wv);
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

  // Selection rounds inside each group of EP lanes: butterfly arg-max over the
  // lanes whose expert is not taken yet; the winner's lane leaves later rounds.
  const int rounds = k + (next != nullptr ? 2 : 0);
  bool taken = !real;
  float v[kMaxRounds];
  int id[kMaxRounds];
#pragma unroll
  for (int j = 0; j < kMaxRounds; ++j) {
    v[j] = -INFINITY;
    id[j] = 0;
    if (j < rounds) {
      float bv = taken ? -INFINITY : l;
      int bi = e;
#pragma unroll
      for (int o = EP / 2; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (bv != -INFINITY && bi == e) taken = true;
      v[j] = bv;
      id[j] = bi;
    }
  }
  if (e == 0 && tok < T) store_token(v, id, k, tok, ids, wout, next);
}

// ---------------------------------------------------------------------------
// bf16 router on the matrix cores.  A 512-lane workgroup owns 16 tokens; its
// 8 wavefronts split K, each accumulating D[expert][token] = W_g . x^T with
// v_mfma_f32_16x16x32_bf16 (A = 16 router rows, B = 16 token rows, zero rows
// past E / T), for EB blocks of 16 experts (E <= 64).  Partial tiles are
// summed through LDS in a fixed order;
// wavefront 0 then holds, per lane, token (lane & 15) and experts
// 16 eb + 4 (lane >> 4) + q.  A selection round takes each lane's best
// expert not yet taken (a 64-bit mask per lane) and two xor-shuffle merges
// (16, 32) give the token's winner.  Exact in the sense that matters: bf16
// products are exact in fp32 and accumulate in fp32.
constexpr int kRouteWaves = 8;

// Pointers of lane (r, g) into the 16-token tile at tok0 and the EB blocks of
// 16 router rows (rows past T or E read row 0 and are zeroed after the load).
template <int EB>
struct RouteLanes {
  const uint16_t* px;
  const uint16_t* pw[EB];
  bool tok_ok;
  bool w_ok[EB];
  __device__ __forceinline__ RouteLanes(const uint16_t* x, const uint16_t* wg, int T, int d, int E,
                                        int tok0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    tok_ok = tok0 + r < T;
    px = x + (int64_t)(tok_ok ? tok0 + r : 0) * d + g * 8;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      w_ok[eb] = eb * 16 + r < E;
      pw[eb] = wg + (int64_t)(w_ok[eb] ? eb * 16 + r : 0) * d + g * 8;
    }
  }
};

// One wavefront's share of the router product: K blocks [b0, b1) of 32
// elements, accumulated in block order into acc (every block's loads of a
// group are issued before the first is used).
template <int EB>
__device__ __forceinline__ void route_kloop(const RouteLanes<EB>& L, int b0, int b1, f32x4_t* acc) {
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) acc[eb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // all of a wavefront's K blocks in flight at once at d = 4096 (16 per wavefront)
  constexpr int U = 16 / EB;
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int b = b0; b < b1; b += U) {
    // Unconditional 16-byte loads from clamped (always valid) addresses, then a
    // select: a conditional load would be split into guarded dword loads.
    // Every load of the group is issued before the first is used (left to
    // itself the scheduler waited for each pair before the next, one memory
    // round trip per matrix instruction).
    uint4 xa[U], wa[U][EB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = b + u < b1 ? b + u : b0;
      xa[u] = *reinterpret_cast<const uint4*>(L.px + blk * 32);
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) wa[u][eb] = *reinterpret_cast<const uint4*>(L.pw[eb] + blk * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = b + u < b1;
      const uint4 xv = (in && L.tok_ok) ? xa[u] : z;
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        const uint4 wv = (in && L.w_ok[eb]) ? wa[u][eb] : z;
        acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv), as_bf16x8(xv), acc[eb], 0, 0, 0);
      }
    }
  }
}

// Everything after the K sum, in wavefront 0: acc holds, per lane (r, g),
// token tok0 + r and experts 16 eb + 4 g + q.  Bias, optional logits, the
// selection rounds and the token's outputs; with INDEX (one tile: T <= 16,
// E <= 16, top-2, nothing dropped, no shared expert) also the grouping that
// the permute index kernel would write (counts, offsets, the rows of each
// expert in ascending token order, perm_src and slot_to_row).
template <int EB, bool INDEX>
__device__ __forceinline__ void route_finish(f32x4_t* acc, int lane, int tok0, const float* __restrict__ bias,
                                             int T, int E, int k, int32_t* __restrict__ ids,
                                             float* __restrict__ wout, float* __restrict__ logits,
                                             int32_t* __restrict__ next, int32_t* __restrict__ counts,
                                             int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
                                             int32_t* __restrict__ slot_to_row) {
  const int r = lane & 15, g = lane >> 4;
  const int tok = tok0 + r;
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    const int ebase = eb * 16 + 4 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ebase + q < E && bias != nullptr) acc[eb][q] += bias[ebase + q];
    if (logits != nullptr && tok < T) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (ebase + q < E) logits[(int64_t)tok * E + ebase + q] = acc[eb][q];
    }
  }
  // taken: bit 4 eb + q = expert 16 eb + 4 g + q of this lane is out (taken or past E)
  uint64_t taken = 0;
#pragma unroll
  for (int eb = 0; eb < EB; ++eb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (eb * 16 + 4 * g + q >= E) taken |= 1ull << (4 * eb + q);
  const int rounds = k + (next != nullptr ? 2 : 0);
  float v[kMaxRounds];
  int id[kMaxRounds];
#pragma unroll
  for (int j = 0; j < kMaxRounds; ++j) {
    v[j] = -INFINITY;
    id[j] = 0;
    if (j < rounds) {
      float bv = -INFINITY;
      int bi = 1 << 30;
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {       // increasing expert index within the lane
          const bool cand = ((taken >> (4 * eb + q)) & 1ull) == 0;
          const float lv = cand ? acc[eb][q] : -INFINITY;
          const int li = cand ? eb * 16 + 4 * g + q : (1 << 30);
          const bool win = better(lv, li, bv, bi);
          bv = win ? lv : bv;
          bi = win ? li : bi;
        }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (bi < E && ((bi >> 2) & 3) == g) taken |= 1ull << (4 * (bi >> 4) + (bi & 3));
      v[j] = bv;
      id[j] = bi;
    }
  }
  if (g == 0 && tok < T) store_token(v, id, k, tok, ids, wout, next);
  if constexpr (INDEX) {
    // lane r (< 16) is token r; a token's two experts are distinct.  The rank
    // of a token among an expert's tokens counts the lower tokens that chose it.
    const bool me = g == 0 && tok < T;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int run = 0, row0 = 0, row1 = 0;
    for (int e = 0; e < E; ++e) {
      const uint64_t b = __ballot(me && (id[0] == e || id[1] == e));
      const int c = __popcll(b);
      if (lane == 0) {
        offsets[e] = run;
        counts[e] = c;
      }
      const int rk = run + __popcll(b & lt_mask);
      if (id[0] == e) row0 = rk;
      if (id[1] == e) row1 = rk;
      run += c;
    }
    if (lane == 0) offsets[E] = run;
    if (me) {
      perm_src[row0] = 2 * tok;
      perm_src[row1] = 2 * tok + 1;
      reinterpret_cast<int2*>(slot_to_row)[tok] = make_int2(row0, row1);
    }
  }
}

template <int EB>
__global__ __launch_bounds__(kRouteWaves * 64) void route_topk_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias,
    int T, int d, int E, int k, int32_t* __restrict__ ids, float* __restrict__ wout,
    float* __restrict__ logits, int32_t* __restrict__ next) {
  static_assert(EB * 4 <= 64, "one bit per expert of a lane in the taken mask");
  __shared__ f32x4_t part[kRouteWaves - 1][EB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * 16;
  const RouteLanes<EB> L(x, wg, T, d, E, tok0, lane);
  const int nblk = d / 32;
  f32x4_t acc[EB];
  route_kloop<EB>(L, wave * nblk / kRouteWaves, (wave + 1) * nblk / kRouteWaves, acc);
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
  route_finish<EB, false>(acc, lane, tok0, bias, T, E, k, ids, wout, logits, next, nullptr, nullptr,
                          nullptr, nullptr);
}

// The decode form (one tile of at most 16 tokens, up to 16 experts) in two
// launches, so that the router rows and tokens are read by eight CUs instead
// of one: workgroup w of route_partial_kernel (one wavefront) computes
// exactly what wavefront w of route_topk_mfma_kernel computes and stores it;
// route_finish_kernel adds the eight partial tiles in the order that kernel
// adds them (wavefront 0's, then 1 .. 7), so the logits are the same bit for
// bit, and finishes with the selection and the grouping.
__global__ __launch_bounds__(64) void route_partial_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wg, int T, int d,
                                                           int E, f32x4_t* __restrict__ part) {
  const int lane = threadIdx.x, w = blockIdx.x;
  const RouteLanes<1> L(x, wg, T, d, E, 0, lane);
  const int nblk = d / 32;
  f32x4_t acc[1];
  route_kloop<1>(L, w * nblk / kRouteWaves, (w + 1) * nblk / kRouteWaves, acc);
  part[w * 64 + lane] = acc[0];
}

__global__ __launch_bounds__(64) void route_finish_kernel(
    const f32x4_t* __restrict__ part, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wout, float* __restrict__ logits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_to_row) {
  const int lane = threadIdx.x;
  f32x4_t p[kRouteWaves];
#pragma unroll
  for (int w = 0; w < kRouteWaves; ++w) p[w] = part[w * 64 + lane];
  f32x4_t acc[1] = {p[0]};
#pragma unroll
  for (int w = 1; w < kRouteWaves; ++w) acc[0] += p[w];
  route_finish<1, true>(acc, lane, 0, bias, T, E, k, ids, wout, logits, nullptr, counts, offsets, perm_src,
                        slot_to_row);
}

// ---------------------------------------------------------------------------
// Many experts (E > 64, bf16): logits, then selection, in two kernels.
//
// route_logits: one workgroup of 4 wavefronts per tile of 16 TM tokens x
// 16 EN experts; the wavefronts split K and sum their partial tiles through
// LDS in a fixed order.  The grid spans tokens and experts, so at decode
// (one token tile) the router matrix is read by E / (16 EN) workgroups in
// parallel instead of one.  Logits (+ bias) go to an fp32 [T, E] buffer.
// route_select: one wavefront per token; lane l holds experts l + 64 j; a
// selection round is a local arg-max then a 6-step butterfly over the lanes.
constexpr int kLogitWaves = 4;

template <int TM, int EN>
__global__ __launch_bounds__(kLogitWaves * 64) void route_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias,
    int T, int d, int E, float* __restrict__ logits) {
  __shared__ f32x4_t part[kLogitWaves - 1][TM * EN][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * 16 * TM, e0 = blockIdx.y * 16 * EN;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* px[TM];
  const uint16_t* pw[EN];
  bool x_ok[TM], w_ok[EN];
#pragma unroll
  for (int m = 0; m < TM; ++m) {
    x_ok[m] = tok0 + 16 * m + r < T;
    px[m] = x + (int64_t)(x_ok[m] ? tok0 + 16 * m + r : 0) * d + g * 8;
  }
#pragma unroll
  for (int n = 0; n < EN; ++n) {
    w_ok[n] = e0 + 16 * n + r < E;
    pw[n] = wg + (int64_t)(w_ok[n] ? e0 + 16 * n + r : 0) * d + g * 8;
  }
  f32x4_t acc[TM][EN];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < EN; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nblk = d / 32;
  const int b0 = wave * nblk / kLogitWaves, b1 = (wave + 1) * nblk / kLogitWaves;
  // 16-byte loads in flight per lane: 32 for small tiles, 16 for the 4 x 4 tile
  // (whose accumulators leave room for no more at three wavefronts per SIMD)
  constexpr int NLD = TM + EN >= 8 ? 16 : 32;
  constexpr int U = NLD / (TM + EN) > 0 ? NLD / (TM + EN) : 1;
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int b = b0; b < b1; b += U) {
    // every load of the group is issued before the first is used (clamped,
    // always valid addresses; out-of-range operands are zeroed afterwards)
    uint4 xa[U][TM], wa[U][EN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = b + u < b1 ? b + u : b0;
#pragma unroll
      for (int m = 0; m < TM; ++m) xa[u][m] = *reinterpret_cast<const uint4*>(px[m] + blk * 32);
#pragma unroll
      for (int n = 0; n < EN; ++n) wa[u][n] = *reinterpret_cast<const uint4*>(pw[n] + blk * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = b + u < b1;
#pragma unroll
      for (int m = 0; m < TM; ++m) {
        const uint4 xv = (in && x_ok[m]) ? xa[u][m] : z;
#pragma unroll
        for (int n = 0; n < EN; ++n) {
          const uint4 wv = (in && w_ok[n]) ? wa[u][n] : z;
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv), as_bf16x8(xv), acc[m][n], 0, 0, 0);
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int n = 0; n < EN; ++n) part[wave - 1][m * EN + n][lane] = acc[m][n];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < TM; ++m) {
    const int tok = tok0 + 16 * m + r;
#pragma unroll
    for (int n = 0; n < EN; ++n) {
#pragma unroll
      for (int w = 0; w < kLogitWaves - 1; ++w) acc[m][n] += part[w][m * EN + n][lane];
      // lane (r, g) holds token r and experts 4 g + q of the 16 x 16 tile
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + 16 * n + 4 * g + q;
        if (tok < T && e < E) logits[(int64_t)tok * E + e] = acc[m][n][q] + (bias != nullptr ? bias[e] : 0.f);
      }
    }
  }
}

constexpr int kSelectTokensPerBlock = 4;

__global__ __launch_bounds__(kSelectTokensPerBlock * 64) void route_select_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ next) {
  constexpr int J = kMaxExperts / kWave;       // logits per lane
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * kSelectTokensPerBlock + (threadIdx.x >> 6);
  if (tok >= T) return;   // whole wavefront leaves; the kernel has no barrier
  float l[J];
  uint32_t taken = 0;      // bit j: expert lane + 64 j is out (taken or past E)
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + kWave * j;
    l[j] = e < E ? logits[(int64_t)tok * E + e] : -INFINITY;
    if (e >= E) taken |= 1u << j;
  }
  const int rounds = k + (next != nullptr ? 2 : 0);
  float v[kMaxRounds];
  int id[kMaxRounds];
#pragma unroll
  for (int jr = 0; jr < kMaxRounds; ++jr) {
    v[jr] = -INFINITY;
    id[jr] = 0;
    if (jr < rounds) {
      float bv = -INFINITY;
      int bi = 1 << 30;
#pragma unroll
      for (int j = 0; j < J; ++j) {          // increasing expert index within the lane
        const bool cand = ((taken >> j) & 1u) == 0;
        const float lv = cand ? l[j] : -INFINITY;
        const int li = cand ? lane + kWave * j : (1 << 30);
        const bool win = better(lv, li, bv, bi);
        bv = win ? lv : bv;
        bi = win ? li : bi;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (bi < E && (bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
      v[jr] = bv;
      id[jr] = bi;
    }
  }
  if (lane == 0) store_token(v, id, k, tok, ids, wout, next);
}

template <int TM, int EN>
hipError_t launch_logits(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                         float* logits, hipStream_t st) {
  const dim3 grid((unsigned)((s.T + 16 * TM - 1) / (16 * TM)), (unsigned)((s.n_experts + 16 * EN - 1) / (16 * EN)));
  hipLaunchKernelGGL((route_logits_kernel<TM, EN>), grid, dim3(kLogitWaves * 64), 0, st,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), bias, s.T,
                     s.d_model, s.n_experts, logits);
  return hipGetLastError();
}

hipError_t launch_two_pass(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                           int32_t* ids, float* w, float* logits, int32_t* next, hipStream_t st) {
  // one token tile: spread the router matrix over as many workgroups as possible
  hipError_t e = s.T <= 16 ? launch_logits<1, 1>(s, x, wg, bias, logits, st)
                           : launch_logits<4, 4>(s, x, wg, bias, logits, st);
  if (e != hipSuccess) return e;
  const int blocks = (s.T + kSelectTokensPerBlock - 1) / kSelectTokensPerBlock;
  hipLaunchKernelGGL(route_select_kernel, dim3(blocks), dim3(kSelectTokensPerBlock * 64), 0, st,
                     logits, s.T, s.n_experts, s.top_k, ids, w, next);
  return hipGetLastError();
}

template <int EB>
hipError_t launch_mfma(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                       int32_t* ids, float* w, float* logits, int32_t* next, hipStream_t st) {
  const int blocks = (s.T + 15) / 16;
  hipLaunchKernelGGL((route_topk_mfma_kernel<EB>), dim3(blocks), dim3(kRouteWaves * 64), 0, st,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wg), bias, s.T,
                     s.d_model, s.n_experts, s.top_k, ids, w, logits, next);
  return hipGetLastError();
}

template <int EP, bool BF16>
hipError_t launch_ep(const moe_shape_t& s, const void* x, const void* wg, const float* bias,
                     int32_t* ids, float* w, float* logits, int32_t* next, hipStream_t st) {
  constexpr int TPW = kWave / EP;
  const int waves = (s.T + TPW - 1) / TPW;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((route_topk_kernel<EP, BF16>), dim3(blocks), dim3(256), 0, st, x, wg, bias,
                     s.T, s.d_model, s.n_experts, s.top_k, ids, w, logits, next);
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

bool route_index_fused(const moe_shape_t& s) {
  return s.act_dtype == MOE_BF16 && s.n_experts <= 16 && s.top_k == 2 && s.T <= 16 &&
         s.capacity < 0 && s.n_shared == 0;
}

hipError_t launch_route_index(const moe_shape_t& s, const void* x, const void* w_gate,
                              const float* bias, int32_t* ids, float* weights, float* logits,
                              int32_t* counts, int32_t* offsets, int32_t* perm_src,
                              int32_t* slot_to_row, void* part, hipStream_t st) {
  hipLaunchKernelGGL(route_partial_kernel, dim3(kRouteWaves), dim3(64), 0, st,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_gate), s.T, s.d_model,
                     s.n_experts, static_cast<f32x4_t*>(part));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_finish_kernel, dim3(1), dim3(64), 0, st, static_cast<const f32x4_t*>(part), bias,
                     s.T, s.n_experts, s.top_k, ids, weights, logits, counts, offsets, perm_src, slot_to_row);
  return hipGetLastError();
}

size_t route_index_part_bytes() { return (size_t)kRouteWaves * 64 * sizeof(f32x4_t); }

size_t route_workspace_bytes(const moe_shape_t& s) {
  return route_two_pass(s) ? (size_t)s.T * s.n_experts * 4 : 0;
}

hipError_t launch_route_topk(const moe_shape_t& s, const void* x, const void* w_gate,
                             const float* bias, int32_t* ids, float* weights, float* logits,
                             int32_t* next_ids, void* workspace, hipStream_t st) {
  if (route_two_pass(s))
    return launch_two_pass(s, x, w_gate, bias, ids, weights,
                           logits != nullptr ? logits : static_cast<float*>(workspace), next_ids, st);
  if (s.act_dtype == MOE_BF16) {
    if (s.n_experts <= 16) return launch_mfma<1>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
    if (s.n_experts <= 32) return launch_mfma<2>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
    return launch_mfma<4>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
  }
  return launch_dtype<false>(s, x, w_gate, bias, ids, weights, logits, next_ids, st);
}

}  // namespace moe

// Grouping of token assignments by expert, with the optional capacity limit.
//
// Pages: "How Mixtral 8x7B uses mixture of experts" -- capacity-limited
// dispatch ("Routing without auxiliary loss": over-capacity tokens are
// dropped), the per-expert bincount of the top-2 ids (expert activation
// listing) and "batch tokens by expert, run experts in parallel, scatter
// back" (simplified forward pass).
//
// capacity_select: one workgroup per expert.  Each assignment gets the
//   64-bit key (fp32 bits of its gate weight) << 32 | (0xffffffff - token),
//   unique inside an expert and ordered exactly like "higher weight first,
//   lower token on ties".  The expert's keys are gathered into LDS and sorted
//   (bitonic network, descending); the key of rank `capacity` is the cutoff
//   and assignments with a key at or above it are kept.  Experts with more
//   keys than fit use an MSB-first radix select (8 passes of 8-bit digits,
//   LDS histograms) over global memory instead.  Index-only,
//   order-independent and therefore deterministic.
//   Overflow fallback ("Routing without auxiliary loss": the excess goes to
//   the next-best expert): a second launch of the same selection in which
//   an assignment belongs to its fallback expert if the first round dropped
//   it (the 3rd-ranked expert; with both slots of the token dropped, 3rd for
//   slot 0 and 4th for slot 1), and each expert's capacity is what the first
//   round left free.  Taken assignments are marked 2.  The round only turns
//   marks 1 into 2, so "dropped in the first round" (mark != 0) reads the
//   same in every workgroup while others write.
// permute_index (top-2, up to 64 experts, no shared expert): one workgroup
//   of 1024 lanes.  Pass 1 counts kept assignments per expert with LDS
//   atomics (order-free).  Pass 2 walks the tokens in chunks of 1024; per
//   expert a wavefront ballot + popcount gives each assignment its rank among
//   earlier tokens of the chunk, and a scan over the 16 wavefronts places the
//   chunk after the previous ones, so rows inside an expert follow ascending
//   token order (stable, deterministic).
// expert_count + expert_place (any top-k, up to 256 experts, shared expert;
//   the many-expert form of the DeepSeek-V3 remark on the "Mixtral 8x7B"
//   interview page): one workgroup per expert.  The first kernel counts the
//   expert's kept assignments; the second sums the counts of the experts
//   before it (its offset) and walks the tokens in chunks of 1024, a token
//   per lane, placing the token's assignment to this expert with a ballot
//   rank plus a scan over the 16 wavefronts -- ascending token order again.
//   The shared expert's workgroup writes its T rows (slot T*k + t) after
//   the routed ones.
// permute_scatter: one wavefront per permuted row copies x[token] in 16-byte
//   vectors; for fp8 experts each lane quantises 32-element blocks to e4m3
//   with a power-of-two (E8M0) block scale.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t capacity_key(const float* w, int i, int k) {
  const uint32_t gbits = __float_as_uint(w[i]);  // gate weights are >= +0: bits are monotone
  const uint32_t tok = (uint32_t)(i / k);
  return ((uint64_t)gbits << 32) | (uint64_t)(0xffffffffu - tok);
}

// Keys of one expert held in LDS by the capacity selection (larger experts
// read their keys from global memory in every pass).
constexpr int kCapKeysInLds = 8192;   // a power of two

// Fallback expert of assignment i = 2 t + s that the capacity round dropped
// (the fallback round is defined for top-2 only):
// the token's 3rd-ranked expert, or its 4th for slot 1 when slot 0 was
// dropped too (-1 where there is no such expert).
__device__ __forceinline__ int fallback_expert(const uint8_t* drop, const int32_t* next, int i) {
  const int t = i >> 1;
  const int j = ((i & 1) && drop[2 * t] != 0) ? 1 : 0;
  return next[2 * t + j];
}

// Token of slot index i: t * k + s for routed slots, T * k + t for the shared expert's.
__device__ __forceinline__ int slot_token(int i, int k, int Tk) { return i < Tk ? i / k : i - Tk; }

// Expert that finally processes assignment i (-1: dropped).
__device__ __forceinline__ int final_expert(const int32_t* ids, const uint8_t* drop,
                                            const int32_t* next, int i) {
  if (drop == nullptr) return ids[i];
  const uint8_t m = drop[i];
  return m == 0 ? ids[i] : m == 2 ? fallback_expert(drop, next, i) : -1;
}

// FALLBACK = false: the capacity round over the top-k assignments (marks 0/1).
// FALLBACK = true: the fallback round over the assignments the first marked 1.
template <bool FALLBACK>
__global__ __launch_bounds__(1024) void capacity_select_kernel(const int32_t* __restrict__ ids,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ next,
                                                               int n_assign, int k, int capacity_in,
                                                               uint8_t* __restrict__ drop) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ uint32_t hist[256];
  __shared__ int s_count;
  __shared__ int s_digit;
  __shared__ int s_remaining;
  __shared__ int s_kept;
  __shared__ uint64_t keys[kCapKeysInLds];
  // the expert this round offers assignment i to (-1: none)
  auto expert_of = [&](int i) -> int {
    if constexpr (!FALLBACK) return ids[i];
    return drop[i] != 0 ? fallback_expert(drop, next, i) : -1;
  };
  constexpr uint8_t kKept = FALLBACK ? 2 : 0;
  int capacity = capacity_in;
  if constexpr (FALLBACK) {
    // slots left free by the first round: capacity minus what it kept
    if (tid == 0) s_kept = 0;
    __syncthreads();
    int mine = 0;
    for (int i = tid; i < n_assign; i += blockDim.x) mine += (ids[i] == e && drop[i] == 0) ? 1 : 0;
    for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o);
    if ((tid & 63) == 0) atomicAdd(&s_kept, mine);
    __syncthreads();
    capacity = capacity_in - s_kept;
  }

  // pass 0: this expert's assignments; their keys go to LDS (any order: the
  // selection below depends only on the set of keys)
  // (one LDS atomic per wavefront: ballot, then each lane's rank among the
  // matching lanes below it)
  if (tid == 0) s_count = 0;
  __syncthreads();
  const int lane = tid & 63;
  constexpr int kBatch = 4;                    // loads issued together per lane
  for (int i0 = tid - lane; i0 < n_assign; i0 += kBatch * blockDim.x) {
    int id[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = i0 + q * blockDim.x + lane;
      id[q] = i < n_assign ? expert_of(i) : -1;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = i0 + q * blockDim.x + lane;
      const bool m = id[q] == e;
      const uint64_t bal = __ballot(m);
      if (bal == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_count, (int)__popcll(bal));
      base = __shfl(base, 0);
      const int pos = base + (int)__popcll(bal & ((1ull << lane) - 1));
      if (m && pos < kCapKeysInLds) keys[pos] = capacity_key(w, i, k);
    }
  }
  __syncthreads();
  const int n_e = s_count;
  const bool in_lds = n_e <= kCapKeysInLds;

  if (n_e <= capacity) {
    for (int i = tid; i < n_assign; i += blockDim.x)
      if (expert_of(i) == e) drop[i] = kKept;
    return;
  }
  if (capacity == 0) {
    for (int i = tid; i < n_assign; i += blockDim.x)
      if (expert_of(i) == e) drop[i] = 1;
    return;
  }

  uint64_t prefix = 0;
  if (in_lds) {
    // Bitonic sort of the keys, descending, padded with zero keys (below every
    // real key) to a power of two; the kept set is the first `capacity`.
    int n = 1;
    while (n < n_e) n <<= 1;
    for (int i = n_e + tid; i < n; i += blockDim.x) keys[i] = 0;
    __syncthreads();
    // Each step compares n / 2 pairs (i, i + j), i with bit j clear; a thread
    // takes pairs tid, tid + 1024, ... (at most 4), loading all of them first.
    constexpr int kPairsPerThread = kCapKeysInLds / 2 / 1024;
    for (int k = 2; k <= n; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        uint64_t a[kPairsPerThread], b[kPairsPerThread];
        int lo[kPairsPerThread];
#pragma unroll
        for (int q = 0; q < kPairsPerThread; ++q) {
          const int pr = tid + q * 1024;
          lo[q] = ((pr & ~(j - 1)) << 1) | (pr & (j - 1));
          if (pr < n / 2) {
            a[q] = keys[lo[q]];
            b[q] = keys[lo[q] + j];
          }
        }
#pragma unroll
        for (int q = 0; q < kPairsPerThread; ++q) {
          const int pr = tid + q * 1024;
          if (pr < n / 2) {
            const bool desc = (lo[q] & k) == 0;
            if (desc ? a[q] < b[q] : a[q] > b[q]) {
              keys[lo[q]] = b[q];
              keys[lo[q] + j] = a[q];
            }
          }
        }
        __syncthreads();
      }
    prefix = keys[capacity - 1];
  } else {
    // MSB-first radix select over the keys read from global memory.
    __shared__ uint32_t above[256];
    uint64_t mask = 0;
    int remaining = capacity;  // rank (1-based, from the top) still to locate
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n_assign; i += blockDim.x) {
        if (expert_of(i) != e) continue;
        const uint64_t key = capacity_key(w, i, k);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // above[b] = keys of this prefix with a digit > b (parallel suffix sum)
      if (tid < 256) above[tid] = tid < 255 ? hist[tid + 1] : 0;
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        const uint32_t add = (tid < 256 && tid + off < 256) ? above[tid + off] : 0;
        __syncthreads();
        if (tid < 256) above[tid] += add;
        __syncthreads();
      }
      if (tid < 256 && (int)above[tid] < remaining && (int)(above[tid] + hist[tid]) >= remaining) {
        s_digit = tid;
        s_remaining = remaining - (int)above[tid];
      }
      __syncthreads();
      prefix |= (uint64_t)s_digit << shift;
      mask |= (uint64_t)255 << shift;
      remaining = s_remaining;
      __syncthreads();
    }
  }
  // `prefix` is now the exact key of rank `capacity`; keys are unique.
  for (int i0 = tid; i0 < n_assign; i0 += kBatch * blockDim.x) {
    int id[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = i0 + q * blockDim.x;
      id[q] = i < n_assign ? expert_of(i) : -1;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = i0 + q * blockDim.x;
      if (id[q] == e) drop[i] = capacity_key(w, i, k) >= prefix ? kKept : 1;
    }
  }
}

constexpr int kIndexThreads = 1024;
constexpr int kIndexWaves = kIndexThreads / kWave;

__global__ __launch_bounds__(kIndexThreads) void permute_index_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ drop,
    const int32_t* __restrict__ next, int T, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_to_row) {
  __shared__ int s_count[64];
  __shared__ int s_base[64];
  __shared__ int s_wave[kIndexWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (tid < 64) s_count[tid] = 0;
  __syncthreads();
  for (int i = tid; i < 2 * T; i += kIndexThreads) {
    const int fe = final_expert(ids, drop, next, i);
    if (fe >= 0) atomicAdd(&s_count[fe], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = run;
      s_base[e] = run;
      counts[e] = s_count[e];
      run += s_count[e];
    }
    offsets[E] = run;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < T; c0 += kIndexThreads) {
    const int t = c0 + tid;
    int e0 = -1, e1 = -1;
    if (t < T) {
      e0 = final_expert(ids, drop, next, 2 * t);
      e1 = final_expert(ids, drop, next, 2 * t + 1);
    }
    int rank0 = 0, rank1 = 0;
    for (int e = 0; e < E; ++e) {
      const uint64_t b = __ballot(e0 == e || e1 == e);
      if (lane == 0) s_wave[wave][e] = __popcll(b);
      const int r = __popcll(b & lt_mask);
      if (e0 == e) rank0 = r;
      if (e1 == e) rank1 = r;
    }
    __syncthreads();
    if (tid < E) {
      int run = s_base[tid];
      for (int w = 0; w < kIndexWaves; ++w) {
        const int c = s_wave[w][tid];
        s_wave[w][tid] = run;
        run += c;
      }
      s_base[tid] = run;
    }
    __syncthreads();
    if (t < T) {
      int row0 = -1, row1 = -1;
      if (e0 >= 0) {
        row0 = s_wave[wave][e0] + rank0;
        perm_src[row0] = 2 * t;
      }
      if (e1 >= 0) {
        row1 = s_wave[wave][e1] + rank1;
        perm_src[row1] = 2 * t + 1;
      }
      reinterpret_cast<int2*>(slot_to_row)[t] = make_int2(row0, row1);
    }
    __syncthreads();
  }
}

constexpr int kPlaceThreads = 1024;
constexpr int kPlaceWaves = kPlaceThreads / kWave;

// Sum over the workgroup of one int per lane (every lane gets the total).
__device__ __forceinline__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < kPlaceWaves; ++w) total += red[w];
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kPlaceThreads) void expert_count_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ drop,
    const int32_t* __restrict__ next, int n_assign, int32_t* __restrict__ counts) {
  __shared__ int red[kPlaceWaves];
  const int e = blockIdx.x;
  int mine = 0;
  for (int i = threadIdx.x; i < n_assign; i += kPlaceThreads)
    mine += final_expert(ids, drop, next, i) == e ? 1 : 0;
  const int total = block_sum(mine, red);
  if (threadIdx.x == 0) counts[e] = total;
}

// Workgroup e < E: rows of routed expert e; workgroup E: the shared expert.
__global__ __launch_bounds__(kPlaceThreads) void expert_place_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ drop,
    const int32_t* __restrict__ next, int T, int k, int E, int S, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_to_row) {
  __shared__ int red[kPlaceWaves];
  __shared__ int s_wave[kPlaceWaves];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int part = 0;
  for (int j = tid; j < e && j < E; j += kPlaceThreads) part += counts[j];
  const int base = block_sum(part, red);
  const int64_t Tk = (int64_t)T * k;
  if (e == E) {   // shared expert: every token, after the routed rows
    for (int t = tid; t < T; t += kPlaceThreads) {
      perm_src[base + t] = (int32_t)(Tk + t);
      slot_to_row[Tk + t] = base + t;
    }
    if (tid == 0) {
      counts[E] = T;
      offsets[E] = base;
      offsets[E + 1] = base + T;
    }
    return;
  }
  if (tid == 0) {
    offsets[e] = base;
    if (e == E - 1 && S == 0) offsets[E] = base + counts[e];
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int chunk_base = base;
  for (int c0 = 0; c0 < T; c0 += kPlaceThreads) {
    const int t = c0 + tid;
    int slot = -1;
    if (t < T) {
      for (int s = 0; s < k; ++s) {
        const int i = t * k + s;
        const int fe = final_expert(ids, drop, next, i);
        if (fe == e) slot = s;
        else if (fe < 0 && ids[i] == e) slot_to_row[i] = -1;   // dropped: its router expert writes it
      }
    }
    const uint64_t b = __ballot(slot >= 0);
    if (lane == 0) s_wave[wave] = __popcll(b);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kPlaceWaves; ++w) {
      before += w < wave ? s_wave[w] : 0;
      total += s_wave[w];
    }
    if (slot >= 0) {
      const int row = chunk_base + before + __popcll(b & lt_mask);
      perm_src[row] = t * k + slot;
      slot_to_row[t * k + slot] = row;
    }
    chunk_base += total;
    __syncthreads();
  }
}

// One wavefront per row; 16-byte vectors.
__global__ __launch_bounds__(256) void permute_scatter_copy_kernel(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ offsets, int G,
    const int32_t* __restrict__ perm_src, int k, int Tk, int row_bytes, uint8_t* __restrict__ x_perm,
    int max_rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= max_rows || row >= offsets[G]) return;
  const int tok = slot_token(perm_src[row], k, Tk);
  const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)tok * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(x_perm + (int64_t)row * row_bytes);
  for (int c = lane; c < row_bytes / 16; c += kWave) dst[c] = src[c];
}

// E8M0 exponent of a block: ceil(log2(fp32(amax / 448))) clamped to [-127, 127];
// 0 for an all-zero block.
__device__ __forceinline__ int block_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t bits = __float_as_uint(amax / 448.0f);
  const int ex = (int)((bits >> 23) & 255u);
  const uint32_t man = bits & 0x7fffffu;
  if (ex == 0) return man > (1u << 22) ? -126 : -127;  // subnormal quotient
  return man == 0 ? ex - 127 : ex - 126;
}

// 32 bf16 values -> 32 e4m3 codes with scale 2^e (exact multiply by 2^-e, one rounding).
__device__ __forceinline__ void quantize_block32_bf16(const uint4* src, uint4* dst, uint8_t* sc) {
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[i];
  const uint32_t* w = reinterpret_cast<const uint32_t*>(v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  const int e = block_exponent(amax);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, a normal float for e in [-127, 126]
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int packed = 0;
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w[2 * i]) * inv, bf16_hi(w[2 * i]) * inv, packed, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w[2 * i + 1]) * inv, bf16_hi(w[2 * i + 1]) * inv, packed, true);
    out[i] = (uint32_t)packed;
  }
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  *sc = (uint8_t)(e + 127);
}

__global__ __launch_bounds__(256) void permute_scatter_fp8_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets, int G,
    const int32_t* __restrict__ perm_src, int k, int Tk, int d, uint8_t* __restrict__ x_perm,
    uint8_t* __restrict__ x_scale, int max_rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= max_rows || row >= offsets[G]) return;
  const int tok = slot_token(perm_src[row], k, Tk);
  const int nblk = d / 32;
  for (int b = lane; b < nblk; b += kWave) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)tok * d + b * 32);
    uint4* dst = reinterpret_cast<uint4*>(x_perm + (int64_t)row * d + b * 32);
    quantize_block32_bf16(src, dst, x_scale + (int64_t)row * nblk + b);
  }
}

__global__ void fill_u8_kernel(uint8_t* __restrict__ p, int64_t n, uint8_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_capacity_select(const moe_shape_t& s, const int32_t* ids, const float* weights,
                                  const int32_t* next_ids, uint8_t* drop_mask, hipStream_t st) {
  const int n_assign = s.T * s.top_k;
  hipLaunchKernelGGL(capacity_select_kernel<false>, dim3(s.n_experts), dim3(1024), 0, st, ids,
                     weights, nullptr, n_assign, s.top_k, s.capacity, drop_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s.overflow != MOE_OVERFLOW_NEXT_BEST) return e;
  hipLaunchKernelGGL(capacity_select_kernel<true>, dim3(s.n_experts), dim3(1024), 0, st, ids,
                     weights, next_ids, n_assign, s.top_k, s.capacity, drop_mask);
  return hipGetLastError();
}

hipError_t launch_permute_index(const moe_shape_t& s, const int32_t* ids, const uint8_t* drop_mask,
                                const int32_t* next_ids, int32_t* counts, int32_t* offsets,
                                int32_t* perm_src, int32_t* slot_to_row, hipStream_t st) {
  if (s.top_k == 2 && s.n_experts <= 64 && s.n_shared == 0) {
    hipLaunchKernelGGL(permute_index_kernel, dim3(1), dim3(kIndexThreads), 0, st, ids, drop_mask,
                       next_ids, s.T, s.n_experts, counts, offsets, perm_src, slot_to_row);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(expert_count_kernel, dim3(s.n_experts), dim3(kPlaceThreads), 0, st, ids,
                     drop_mask, next_ids, s.T * s.top_k, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(expert_place_kernel, dim3(expert_groups(s)), dim3(kPlaceThreads), 0, st, ids,
                     drop_mask, next_ids, s.T, s.top_k, s.n_experts, s.n_shared, counts, offsets,
                     perm_src, slot_to_row);
  return hipGetLastError();
}

hipError_t launch_permute_scatter(const moe_shape_t& s, const void* x, const int32_t* offsets,
                                  const int32_t* perm_src, void* x_perm, uint8_t* x_perm_scale,
                                  hipStream_t st) {
  const int max_rows = (int)total_slots(s);
  const int blocks = (max_rows + 3) / 4;
  const int G = expert_groups(s), k = s.top_k, Tk = s.T * s.top_k;
  if (s.w_dtype == MOE_FP8_E4M3) {
    hipLaunchKernelGGL(permute_scatter_fp8_kernel, dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), offsets, G, perm_src, k, Tk, s.d_model,
                       static_cast<uint8_t*>(x_perm), x_perm_scale, max_rows);
  } else {
    const int es = s.act_dtype == MOE_F32 ? 4 : 2;
    hipLaunchKernelGGL(permute_scatter_copy_kernel, dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint8_t*>(x), offsets, G, perm_src, k, Tk,
                       s.d_model * es, static_cast<uint8_t*>(x_perm), max_rows);
  }
  return hipGetLastError();
}

hipError_t launch_fill_u8(uint8_t* p, int64_t n, uint8_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_u8_kernel, dim3(blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace moe

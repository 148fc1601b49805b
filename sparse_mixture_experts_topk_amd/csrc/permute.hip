// Grouping of token assignments by expert, with the optional capacity limit.
//
// Pages: "How Mixtral 8x7B uses mixture of experts" -- capacity-limited
// dispatch ("Routing without auxiliary loss": over-capacity tokens are
// dropped), the per-expert bincount of the top-2 ids (expert activation
// listing) and the simplified forward pass, which gathers each expert's
// tokens into one batch, runs the experts on their batches and writes the
// results back in token order.
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
//   of 1024 lanes per chunk of 1024 tokens.  Each counts every kept
//   assignment per expert with LDS atomics (the eight chunks of a batch
//   loaded before any is counted), those of the tokens before its chunk
//   apart from the rest; a scan over the experts gives the offsets and the chunk's start
//   inside each expert.  Per expert a ballot + popcount ranks a token among
//   the earlier tokens of its wavefront, and a scan over the 16 wavefronts
//   places the wavefronts, so rows inside an expert follow ascending token
//   order (stable; every workgroup derives the same totals, so deterministic).
// group_chunks (any top-k, up to 256 experts, shared expert; the many-expert
//   form of the DeepSeek-V3 remark on the "Mixtral 8x7B" interview page): one
//   workgroup per chunk of 1024 tokens.  Each histograms every assignment
//   with LDS atomics (the part before its chunk apart from the rest; their
//   sum is the total) and sets bit
//   (token - chunk start) in a 1024-bit mask of the final expert for each of
//   its own tokens' assignments; prefix popcounts of the mask words give a
//   token its rank among the chunk's earlier tokens of that expert --
//   ascending token order again.  The shared expert's T rows (slot T*k + t)
//   follow the routed ones.
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

// The expert that finally processes an assignment: its router expert when
// kept (mark 0, or no drop marks at all), its fallback expert when the
// fallback round took it (mark 2), none (-1) when dropped (mark 1).
//
// Final experts of top-2 token t from values already loaded: its two ids,
// its two drop marks (byte s = slot s; 0 when nothing is dropped) and its two
// fallback ids (the rule of fallback_expert).
__device__ __forceinline__ int2 final_pair(int2 id, uint32_t marks, int2 nx) {
  const uint32_t m0 = marks & 255u, m1 = (marks >> 8) & 255u;
  const int e0 = m0 == 0 ? id.x : m0 == 2 ? nx.x : -1;
  const int e1 = m1 == 0 ? id.y : m1 == 2 ? (m0 != 0 ? nx.y : nx.x) : -1;
  return make_int2(e0, e1);
}

// Loads of token t (< T) for final_pair: every load unconditional, so a
// batch of them is in flight together.
__device__ __forceinline__ int2 load_final_pair(const int32_t* ids, const uint8_t* drop,
                                                const int32_t* next, int t) {
  const int2 id = reinterpret_cast<const int2*>(ids)[t];
  uint32_t marks = 0;
  int2 nx = make_int2(-1, -1);
  if (drop != nullptr) {
    marks = reinterpret_cast<const uint16_t*>(drop)[t];
    if (next != nullptr) nx = reinterpret_cast<const int2*>(next)[t];
  }
  return final_pair(id, marks, nx);
}

// Final experts of N assignments i[0..N) with every load issued before any
// is used (the fallback exists for top-2 only: next != nullptr implies k == 2).
template <int N>
__device__ __forceinline__ void load_final_experts(const int32_t* ids, const uint8_t* drop,
                                                   const int32_t* next, const int* i, int* fe) {
  uint32_t m[N], m0[N];
  int2 nx[N];
#pragma unroll
  for (int q = 0; q < N; ++q) fe[q] = ids[i[q]];
  if (drop != nullptr) {
#pragma unroll
    for (int q = 0; q < N; ++q) m[q] = drop[i[q]];
    if (next != nullptr) {
#pragma unroll
      for (int q = 0; q < N; ++q) {
        m0[q] = drop[i[q] & ~1];
        nx[q] = reinterpret_cast<const int2*>(next)[i[q] >> 1];
      }
    }
#pragma unroll
    for (int q = 0; q < N; ++q) {
      int fb = -1;
      if (next != nullptr) fb = ((i[q] & 1) && m0[q] != 0) ? nx[q].y : nx[q].x;
      fe[q] = m[q] == 0 ? fe[q] : m[q] == 2 ? fb : -1;
    }
  }
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
constexpr int kIndexBatch = 8;     // chunks whose assignments are loaded before any is counted

// Grouping for top-2 with up to 64 experts, no shared expert: one workgroup
// per chunk of 1024 tokens, a token per lane.  Every workgroup counts all
// assignments (the totals fix the experts' offsets) and, apart, those of the
// tokens before its chunk (where its rows start inside each expert); then it
// ranks its own tokens with one ballot per expert and a scan over its 16
// wavefronts.  Every workgroup derives the same totals from the same data, so
// the rows do not depend on timing; workgroup 0 writes counts and offsets.
__global__ __launch_bounds__(kIndexThreads) void permute_index_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ drop,
    const int32_t* __restrict__ next, int T, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_to_row) {
  __shared__ int s_rest[64];     // assignments of the own and later chunks, per expert
  __shared__ int s_before[64];   // assignments of earlier chunks, per expert
  __shared__ int s_base[64];
  __shared__ int s_wave[kIndexWaves][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x, n_chunks = gridDim.x;

  if (tid < 64) {
    s_rest[tid] = 0;
    s_before[tid] = 0;
  }
  __syncthreads();
  // count: chunks in batches, all of a batch's loads issued before any is
  // counted; one LDS atomic per kept assignment, into the histogram of the
  // earlier chunks or into that of the rest (their sum is the total)
  int m0 = -1, m1 = -1;                       // this lane's token of the own chunk
  for (int c0 = 0; c0 < n_chunks; c0 += kIndexBatch) {
    // loads from clamped (valid) tokens, then a select: no load waits for another
    int e0[kIndexBatch], e1[kIndexBatch];
#pragma unroll
    for (int q = 0; q < kIndexBatch; ++q) {
      const int t = (c0 + q) * kIndexThreads + tid;
      const int2 f = load_final_pair(ids, drop, next, t < T ? t : T - 1);
      const bool in = c0 + q < n_chunks && t < T;
      e0[q] = in ? f.x : -1;
      e1[q] = in ? f.y : -1;
    }
#pragma unroll
    for (int q = 0; q < kIndexBatch; ++q) {
      if (c0 + q == chunk) {
        m0 = e0[q];
        m1 = e1[q];
      }
      // chunks past the last and wavefronts past the last token count nothing
      if ((c0 + q) * kIndexThreads + wave * kWave >= T) continue;
      int* const h = c0 + q < chunk ? s_before : s_rest;
      if (e0[q] >= 0) atomicAdd(&h[e0[q]], 1);
      if (e1[q] >= 0) atomicAdd(&h[e1[q]], 1);
    }
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the totals over the experts, lane e = expert e
    const int v = lane < E ? s_before[lane] + s_rest[lane] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    const int excl = incl - v;
    if (lane < E) {
      s_base[lane] = excl + s_before[lane];
      if (chunk == 0) {
        offsets[lane] = excl;
        counts[lane] = v;
      }
    }
    if (chunk == 0 && lane == 63) offsets[E] = incl;
  }
  __syncthreads();

  // rank the own chunk's tokens: a token's two experts are distinct
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int t = chunk * kIndexThreads + tid;
  int rank0 = 0, rank1 = 0;
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(m0 == e || m1 == e);
    if (lane == 0) s_wave[wave][e] = __popcll(b);
    const int r = __popcll(b & lt_mask);
    if (m0 == e) rank0 = r;
    if (m1 == e) rank1 = r;
  }
  __syncthreads();
  if (tid < E) {
    int run = s_base[tid];
    for (int w = 0; w < kIndexWaves; ++w) {
      const int c = s_wave[w][tid];
      s_wave[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  if (t < T) {
    int row0 = -1, row1 = -1;
    if (m0 >= 0) {
      row0 = s_wave[wave][m0] + rank0;
      perm_src[row0] = 2 * t;
    }
    if (m1 >= 0) {
      row1 = s_wave[wave][m1] + rank1;
      perm_src[row1] = 2 * t + 1;
    }
    reinterpret_cast<int2*>(slot_to_row)[t] = make_int2(row0, row1);
  }
}

constexpr int kGroupTokens = 1024;                // tokens per chunk: one per lane
constexpr int kGroupWords = kGroupTokens / 32;      // mask words per expert
constexpr int kGroupBatch = 8;                      // assignments loaded before any is counted

// Grouping for any top-k, many experts and the shared expert: one workgroup
// per chunk of 1024 tokens.  Every workgroup histograms all assignments with
// LDS atomics, those of tokens before its chunk apart from the rest: the
// totals (their sum) fix the experts' offsets, the earlier part where its rows
// start inside each expert.  For its own
// tokens it sets bit (token - chunk start) of the final expert's 1024-bit mask
// (a token has at most one assignment per expert), so a row's rank inside
// the chunk is the number of bits below its own: ascending token order, the
// same as walking the tokens, without depending on timing.  Dropped
// assignments get row -1; the shared expert's rows follow the routed ones in
// token order.  Workgroup 0 writes counts and offsets.
__global__ __launch_bounds__(kGroupTokens) void group_chunks_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ drop,
    const int32_t* __restrict__ next, int T, int k, int E, int S, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_to_row) {
  __shared__ int s_rest[kMaxExpertGroups];     // own and later chunks
  __shared__ int s_before[kMaxExpertGroups];   // earlier chunks
  __shared__ int s_base[kMaxExpertGroups];
  __shared__ uint32_t s_mask[kMaxExperts][kGroupWords];
  __shared__ uint16_t s_pre[kMaxExperts][kGroupWords];   // bits of the expert's earlier words
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kGroupTokens;
  const int G = E + S;
  const int64_t n_assign = (int64_t)T * k;
  const int a0 = t0 * k;                              // first assignment of the own chunk
  const int64_t a1_full = (int64_t)(t0 + kGroupTokens) * k;
  const int a1 = (int)(a1_full < n_assign ? a1_full : n_assign);

  for (int j = tid; j < kMaxExpertGroups; j += kGroupTokens) {
    s_rest[j] = 0;
    s_before[j] = 0;
  }
  for (int j = tid; j < kMaxExperts * kGroupWords; j += kGroupTokens) (&s_mask[0][0])[j] = 0u;
  __syncthreads();
  for (int64_t i0 = tid; i0 < n_assign; i0 += (int64_t)kGroupBatch * kGroupTokens) {
    // loads from clamped (valid) assignments, then a select: no load waits for another
    int fe[kGroupBatch], ic[kGroupBatch];
#pragma unroll
    for (int q = 0; q < kGroupBatch; ++q) {
      const int64_t i = i0 + (int64_t)q * kGroupTokens;
      ic[q] = i < n_assign ? (int)i : (int)n_assign - 1;
    }
    load_final_experts<kGroupBatch>(ids, drop, next, ic, fe);
#pragma unroll
    for (int q = 0; q < kGroupBatch; ++q)
      if (i0 + (int64_t)q * kGroupTokens >= n_assign) fe[q] = -1;
#pragma unroll
    for (int q = 0; q < kGroupBatch; ++q) {
      const int i = (int)(i0 + (int64_t)q * kGroupTokens);
      if (fe[q] < 0) continue;
      if (i < a0) {
        atomicAdd(&s_before[fe[q]], 1);
      } else {
        atomicAdd(&s_rest[fe[q]], 1);
        if (i < a1) {
          const int lt = i / k - t0;
          atomicOr(&s_mask[fe[q]][lt >> 5], 1u << (lt & 31));
        }
      }
    }
  }
  __syncthreads();
  if (S > 0 && tid == 0) {
    s_rest[E] = T - t0;
    s_before[E] = t0;
  }
  // per expert, the bits of its earlier mask words: 4 lanes per expert, 8 words each
  {
    const int e = tid >> 2, part = tid & 3;
    int run = 0;
    uint16_t local[kGroupWords / 4];
    if (e < E) {
#pragma unroll
      for (int w = 0; w < kGroupWords / 4; ++w) {
        local[w] = (uint16_t)run;
        run += __popc(s_mask[e][part * (kGroupWords / 4) + w]);
      }
    }
    // exclusive sum of the 4 parts' counts (lanes 4e .. 4e + 3 of one wavefront)
    const int p1 = __shfl_up(run, 1, 4), p2 = __shfl_up(run, 2, 4), p3 = __shfl_up(run, 3, 4);
    const int off = (part >= 1 ? p1 : 0) + (part >= 2 ? p2 : 0) + (part >= 3 ? p3 : 0);
    if (e < E) {
#pragma unroll
      for (int w = 0; w < kGroupWords / 4; ++w)
        s_pre[e][part * (kGroupWords / 4) + w] = (uint16_t)(local[w] + off);
    }
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the G totals: lane l sums groups 5 l .. 5 l + 4
    constexpr int PER = (kMaxExpertGroups + 63) / 64;
    int v[PER], sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int g = lane * PER + j;
      v[j] = g < G ? s_before[g] + s_rest[g] : 0;
      sum += v[j];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    int run = incl - sum;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int g = lane * PER + j;
      if (g < G) {
        s_base[g] = run + s_before[g];
        if (blockIdx.x == 0) {
          offsets[g] = run;
          counts[g] = v[j];
        }
      }
      run += v[j];
    }
    if (blockIdx.x == 0 && lane == 63) offsets[G] = incl;
  }
  __syncthreads();
  const int t = t0 + tid;
  if (t < T) {
    const int lt = tid;
    int fes[kMaxTopK], ic[kMaxTopK];
#pragma unroll
    for (int sl = 0; sl < kMaxTopK; ++sl) ic[sl] = t * k + (sl < k ? sl : k - 1);
    load_final_experts<kMaxTopK>(ids, drop, next, ic, fes);
#pragma unroll
    for (int sl = 0; sl < kMaxTopK; ++sl) {
      if (sl >= k) break;
      const int i = t * k + sl;
      const int fe = fes[sl];
      int row = -1;
      if (fe >= 0) {
        const uint32_t below = s_mask[fe][lt >> 5] & ((1u << (lt & 31)) - 1u);
        row = s_base[fe] + s_pre[fe][lt >> 5] + __popc(below);
        perm_src[row] = i;
      }
      slot_to_row[i] = row;
    }
    if (S > 0) {
      const int row = s_base[E] + lt;                 // routed rows, then the shared rows
      perm_src[row] = (int32_t)(n_assign + t);
      slot_to_row[n_assign + t] = row;
    }
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
  if (s.T <= 0) return hipSuccess;     // every entry point returns before this; loads clamp to T - 1
  if (s.top_k == 2 && s.n_experts <= 64 && s.n_shared == 0) {
    const int chunks = (s.T + kIndexThreads - 1) / kIndexThreads;
    hipLaunchKernelGGL(permute_index_kernel, dim3(chunks), dim3(kIndexThreads), 0, st, ids, drop_mask,
                       next_ids, s.T, s.n_experts, counts, offsets, perm_src, slot_to_row);
    return hipGetLastError();
  }
  const int chunks = (s.T + kGroupTokens - 1) / kGroupTokens;
  hipLaunchKernelGGL(group_chunks_kernel, dim3(chunks), dim3(kGroupTokens), 0, st, ids, drop_mask,
                     next_ids, s.T, s.top_k, s.n_experts, s.n_shared, counts, offsets, perm_src,
                     slot_to_row);
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

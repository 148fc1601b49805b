// fp8 (OCP e4m3) grouped expert GEMMs on the gfx950 matrix cores, fp32 accumulate.
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x);
// "How Mixtral 8x7B uses mixture of experts", section "Quantization
// asymmetry": experts are the quantised part, the router stays 16-bit.
//
// Formats.  Expert weights are e4m3 codes with one fp32 scale per output
// channel.  The token operand (x_perm, h) is e4m3 codes with one E8M0
// (power-of-two) scale per row and per 32-element block along K.  One
// v_mfma_scale_f32_32x32x64_f8f6f4 covers K = 64 (two scale blocks) with
// 32 bytes per lane; measured on gfx950, the scale that lane (i, h) supplies
// multiplies bytes 16 h .. 16 h + 15 of both lanes (i, 0) and (i, 1).  So
// lane half h holds the h-th 16-element half of each of the two blocks and
// supplies the scale of block h: the token operand's block scales are
// applied in hardware with no extra VALU work.  The weight operand's scale
// is 1 (E8M0 127) and its per-channel fp32 scale is applied in the epilogue.
// The gate/up epilogue forms h = silu(g) * u in fp32 and block-quantises it
// per (token, 32 channels): the amax of a block lives in two lanes (16
// channels each) and is completed with one lane swap.
//
// The kernel below runs the bf16 prefill kernel's pipeline (persistent
// workgroups, one load stream through a ring of LDS stages filled by loads
// that write LDS directly, 384 x 256 tiles, 8 wavefronts) on fp8 operands.
#include "device_common.hpp"
#include "launch.hpp"
#include "lds_stream.hpp"
#include "persistent_tiles.hpp"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Persistent tile kernel: the bf16 prefill kernel's pipeline with fp8 operands.
//
// 512 lanes (two wavefronts per SIMD), a 384 x 256 tile (weights x tokens;
// gate/up: 192 rows of w1 and the same 192 of w3).  K advances 64 at a time:
// a slice row is 64 fp8 bytes, so an LDS stage holds 24 + 16 KiB as in the
// bf16 kernel and is filled the same way, by buffer loads that write LDS
// directly, two slices in flight while one is multiplied.  One
// v_mfma_scale_f32_32x32x64_f8f6f4 per block pair covers a slice.  The token
// operand's E8M0 scales (one byte per row and 32-element block) come by the
// same kind of load, 64 bytes of every token row at once -- the scales of 32
// slices -- into one of two LDS slots, at the first slice of each group of
// 32: lanes run along a row so that a dword load touches 4 rows, not 64
// (the scale loads of a row-per-lane layout made the tile's load requests
// 1.4x as many).  The wait for a slice allows the five weight and token loads
// of the slice after it to be pending; when that slice also carries scale
// loads (or, in a tile's first slice, its weight scales) the wait is
// stricter than needed, never looser.  Each wavefront owns 6 x 2
// accumulator blocks (192 fp32 per lane); a slice's 12 matrix instructions
// run in two halves of 3 weight blocks: the first carries the slice loads,
// the second follows the wait and the barrier and reads the next slice's
// first fragments.  Weight fragments are double-buffered one block ahead.
// Tiles are scheduled as in the bf16 kernel (persistent workgroups, one load
// stream across tiles).
constexpr int F8T_BK = 64;                          // K (bytes) per slice
constexpr int F8T_NS = 3;                           // LDS ring stages
constexpr int F8T_WR = 2, F8T_WC = 4, F8T_WA = 6, F8T_WB = 2;
constexpr int F8T_NW = F8T_WR * F8T_WC;
constexpr int F8T_THREADS = 64 * F8T_NW;
constexpr int F8T_TA = 32 * F8T_WR * F8T_WA;        // 384 weight rows
constexpr int F8T_TB = 32 * F8T_WC * F8T_WB;        // 256 token rows
constexpr int F8T_CPR = F8T_BK / 16;                // 16-byte chunks per row slice
constexpr int F8T_RPI = 64 / F8T_CPR;               // rows per 1 KiB load instruction
constexpr int F8T_JA = F8T_TA / F8T_RPI / F8T_NW;   // weight loads per wavefront per slice
constexpr int F8T_JB = F8T_TB / F8T_RPI / F8T_NW;   // token loads per wavefront per slice
constexpr int F8T_DMA = F8T_JA + F8T_JB;            // weight and token loads per slice
constexpr int F8T_OPA = F8T_TA * F8T_BK;
constexpr int F8T_STAGE = (F8T_TA + F8T_TB) * F8T_BK;
constexpr int F8T_SCG = 32;                         // slices per scale group (64 bytes per row)
constexpr int F8T_SCQ = F8T_TB / 4 / F8T_NW;        // scale loads per wavefront per group (4 rows each)
constexpr int F8T_SLOTS = 3 * F8T_WB;               // load slots of a slice (the first half's instructions)
constexpr int F8T_OOB = 0x7ff00000;                 // offset past every descriptor
constexpr int kF8GroupN = 4;                        // channel tiles per group of the tile order
static_assert(F8T_JA * F8T_RPI * F8T_NW == F8T_TA && F8T_JB * F8T_RPI * F8T_NW == F8T_TB, "whole loads");
static_assert(F8T_DMA + 1 <= F8T_SLOTS, "one load slot per matrix instruction of the first half");
static_assert((F8T_NW * F8T_RPI) % 16 == 0, "loads of a wavefront are whole swizzle periods apart");

template <bool DUAL>
__global__ __launch_bounds__(F8T_THREADS, 1) void grouped_gemm_fp8_tiles(
    const uint8_t* __restrict__ act, const uint8_t* __restrict__ act_scale,
    const int32_t* __restrict__ offsets, int E, const uint8_t* __restrict__ wa,
    const uint8_t* __restrict__ wb, const float* __restrict__ sa, const float* __restrict__ sb,
    int N, int K, void* __restrict__ out, uint8_t* __restrict__ out_scale, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[F8T_NS * F8T_STAGE];
  __shared__ __attribute__((aligned(1024))) uint32_t scs[2][F8T_TB * 16];   // [slot][row][16 dwords]
  __shared__ int32_t offs[kMaxExpertGroups + 1];
  __shared__ int32_t tpre[kMaxExpertGroups + 1];
  // per-channel weight scales of the tile (gate/up: 192 of w1, then the same
  // 192 of w3), one slot per tile in a ring of 3
  __shared__ __attribute__((aligned(16))) float wsc[3][F8T_TA];
  constexpr int WA = F8T_WA, WB = F8T_WB, NS = F8T_NS;
  constexpr int HA = WA / 2;                        // dual: w1 (or w3) blocks per wavefront
  constexpr int CH_TILE = DUAL ? F8T_TA / 2 : F8T_TA;
  constexpr int kOne = 0x7f7f7f7f;                  // E8M0 127 = 1.0: the weight operand's scale
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / F8T_WC, wc = wave % F8T_WC;
  // lane index the compiler cannot keep in a register through the K loop
  auto lane_now = [&]() __attribute__((always_inline)) {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  auto key = [](int row) { return (row / (16 / F8T_CPR)) & (F8T_CPR - 1); };

  if (tid <= E) offs[tid] = offsets[tid];
  __syncthreads();
  if (wave == 0) build_tile_prefix(offs, E, F8T_TB, tpre, lane);
  __syncthreads();
  const int KT = K / F8T_BK;                        // even: K is a multiple of 128
  const int slots = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const TileSplit sp = TileSplit::of(__builtin_amdgcn_readfirstlane(tpre[E]) * n_tiles, xcd, slots, KT);
  const int n_items = sp.R + (slot < sp.tail ? 1 : 0);
  if (n_items == 0) return;

  struct Tile { int e, tok0, tok_rows, ch0; };
  auto tile_of = [&](int i) __attribute__((always_inline)) -> Tile {
    int e, r0, r1, mt, nt;
    find_tile(offs, tpre, E, n_tiles, sp.share_begin + slot + i * slots, e, r0, r1, mt, nt);
    {
      // an expert's tiles in groups of kF8GroupN channel tiles, channel tile
      // fastest: the tiles an XCD's workgroups run at a time share weight and
      // token slices in its L2
      const int mtc = (r1 - r0 + F8T_TB - 1) / F8T_TB;
      const int l = nt * mtc + mt;
      const int gi = l / (mtc * kF8GroupN);
      const int nt0 = gi * kF8GroupN;
      const int gsz = min(kF8GroupN, n_tiles - nt0);
      const int idx = l - gi * mtc * kF8GroupN;
      nt = nt0 + idx % gsz;
      mt = idx / gsz;
    }
    Tile t;
    t.e = __builtin_amdgcn_readfirstlane(e);
    t.tok0 = __builtin_amdgcn_readfirstlane(r0 + mt * F8T_TB);
    t.tok_rows = __builtin_amdgcn_readfirstlane(min(F8T_TB, r1 - t.tok0));
    t.ch0 = __builtin_amdgcn_readfirstlane(nt * CH_TILE);
    return t;
  };

  // ---- global -> LDS loads (as in the bf16 kernel, one byte per element) ----
  const int64_t rowbytes = K;
  const int nblk = K / 32;                          // scale bytes per token row
  auto voff_base = [&]() __attribute__((always_inline)) {
    const int l = lane_now();
    const int r = wave * F8T_RPI + l / F8T_CPR;
    return (int)(r * rowbytes) + (((l % F8T_CPR) ^ key(r)) << 4);
  };
  const int vstep = F8T_NW * F8T_RPI * (int)rowbytes;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const uint32_t sc_base = (uint32_t)(uintptr_t)&scs[0][0];
  const uint32_t wsc_base = (uint32_t)(uintptr_t)&wsc[0][0];

  i32x4_t d_tok, d_w0, d_w1, d_sc;
  int li = 0, lkt = 0, lgrp = 0;                   // lgrp: scale groups loaded so far
  auto load_tile = [&]() __attribute__((always_inline)) {
    if (li < n_items) {
      const Tile t = tile_of(li);
      lkt = 0;
      d_tok = make_desc(act + (int64_t)t.tok0 * K, t.tok_rows * rowbytes);
      d_sc = make_desc(act_scale + (int64_t)t.tok0 * nblk, (int64_t)t.tok_rows * nblk);
      d_w0 = make_desc(wa + ((int64_t)t.e * N + t.ch0) * K, (int64_t)(N - t.ch0) * rowbytes);
      d_w1 = DUAL ? make_desc(wb + ((int64_t)t.e * N + t.ch0 - F8T_TA / 2) * K,
                              (int64_t)(N - t.ch0 + F8T_TA / 2) * rowbytes)
                  : d_w0;
    }
  };
  load_tile();
  // Load j of the cursor's slice (stream slice ls): JA weight blocks, JB
  // token blocks, then, at the first slice of a scale group, this
  // wavefront's F8T_SCQ scale loads (load q: rows 4 q .. 4 q + 3, lane l
  // the dword l % 16 of row 4 q + l / 16).
  auto dma = [&](int ls, int j, int vb) __attribute__((always_inline)) {
    const bool live = li < n_items;
    const int soff = live ? lkt * F8T_BK : F8T_OOB;
    const uint32_t stg = lds_base + (uint32_t)((ls % NS) * F8T_STAGE);
    if (j < F8T_JA) {
      const int blk = F8T_NW * j + wave;
      const bool w3 = DUAL && blk * F8T_RPI >= F8T_TA / 2;
      dma_to_lds(w3 ? d_w1 : d_w0, vb + j * vstep, soff, __builtin_amdgcn_readfirstlane(stg + blk * 1024));
    } else if (j < F8T_JA + F8T_JB) {
      const int q = j - F8T_JA;
      dma_to_lds(d_tok, vb + q * vstep, soff,
                 __builtin_amdgcn_readfirstlane(stg + F8T_OPA + (F8T_NW * q + wave) * 1024));
    } else {
      if (live && lkt % F8T_SCG == 0) {
        const uint32_t slot = sc_base + (uint32_t)((lgrp & 1) * F8T_TB * 64);
        const int l = lane_now();
#pragma unroll
        for (int i = 0; i < F8T_SCQ; ++i) {
          const int q = wave * F8T_SCQ + i;
          dma4_to_lds(d_sc, (4 * q + l / 16) * nblk + (l % 16) * 4, (lkt / F8T_SCG) * 64,
                      __builtin_amdgcn_readfirstlane(slot + q * 256));
        }
        ++lgrp;
      }
      // With the tile's first slice, its weight scales: wavefront w < 6 brings
      // 64 of them into slot li % 3 (channels past N read as zero), so that
      // the epilogue reads LDS and issues no vector-memory load, which would
      // have to wait for every load of the next slices issued before it.
      if (live && lkt == 0 && wave < F8T_TA / 64) {
        const Tile t = tile_of(li);
        constexpr int HW = DUAL ? F8T_TA / 128 : F8T_TA / 64;   // wavefronts per scale array
        const float* src = (DUAL && wave >= HW) ? sb : sa;
        const i32x4_t d = make_desc(src + (int64_t)t.e * N + t.ch0, (int64_t)(N - t.ch0) * 4);
        dma4_to_lds(d, ((wave % HW) * 64 + lane_now()) * 4, 0,
                    __builtin_amdgcn_readfirstlane(wsc_base + (uint32_t)((li % 3) * F8T_TA * 4 + wave * 256)));
      }
    }
  };
  auto advance_load = [&]() __attribute__((always_inline)) {
    if (++lkt == KT) {
      ++li;
      load_tile();
    }
  };

  // ---- fragments (v_mfma_scale_f32_32x32x64_f8f6f4: lane (fi, fg) holds row
  //      fi, chunk fg in its low and chunk 2 + fg in its high 16 bytes, and
  //      supplies the scale of block fg of the slice) ----
  int arow[WA], bfrow[WB];
#pragma unroll
  for (int a = 0; a < WA; ++a) {
    if constexpr (DUAL) arow[a] = (a / HA) * (F8T_TA / 2) + wr * (HA * 32) + (a % HA) * 32;
    else arow[a] = wr * (WA * 32) + a * 32;
  }
#pragma unroll
  for (int b = 0; b < WB; ++b) bfrow[b] = wc * (WB * 32) + b * 32;
  auto read_frag = [&](int g, int f) __attribute__((always_inline)) -> i32x8_t {
    const int l = lane_now(), fi = l & 31, fg = l >> 5;
    const int row = f < WA ? arow[f] + fi : bfrow[f - WA] + fi;
    const int base = (g % NS) * F8T_STAGE + (f < WA ? 0 : F8T_OPA) + row * F8T_BK;
    const uint4 lo = *reinterpret_cast<const uint4*>(&smem[base + ((fg ^ key(fi)) << 4)]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&smem[base + (((2 + fg) ^ key(fi)) << 4)]);
    return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // The E8M0 byte of this lane's token row and block for tile slice kt (scale
  // slot cs), in the low byte.
  int cgrp = 0;                                     // scale groups read so far
  auto read_scale = [&](int cs, int kt, int b) __attribute__((always_inline)) -> int {
    const int l = lane_now(), fi = l & 31, fg = l >> 5;
    const uint32_t w = scs[cs][(bfrow[b] + fi) * 16 + (kt % F8T_SCG) / 2];
    return (int)(w >> (8 * ((kt & 1) * 2 + fg)));
  };
  // slot of tile slice kt's scales (a new group starts every F8T_SCG slices)
  int cslot = 0;
  auto scale_slot = [&](int kt) __attribute__((always_inline)) {
    if (kt % F8T_SCG == 0) cslot = cgrp++ & 1;
    return cslot;
  };

  f32x16_t acc[WA][WB];
  i32x8_t fa[2], fb[WB];
  int sc[WB];

  // Half h of slice g: weight blocks a = 3 h .. 3 h + 2 against both token
  // blocks.  Before the instructions of block a, block a + 1's fragment is
  // read into the other buffer.  With `loads`, the six loads of stream slice
  // ls ride along; with `reads` (second half), the next slice gn's token
  // fragments, scales and first weight fragment are read after their last use.
  auto half = [&](int h, int g, bool loads, int ls, bool reads, int gn, int ktn) __attribute__((always_inline)) {
    const int cs = reads ? scale_slot(ktn) : 0;
    const int vb = loads ? voff_base() : 0;
#pragma unroll
    for (int ai = 0; ai < 3; ++ai) {
      const int a = 3 * h + ai;
      if (a + 1 < WA) fa[(a + 1) & 1] = read_frag(g, a + 1);
#pragma unroll
      for (int b = 0; b < WB; ++b) {
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a & 1], fb[b], acc[a][b], 0, 0, 0,
                                                                     kOne, 0, sc[b]);
        if (loads && ai * WB + b <= F8T_DMA) dma(ls, ai * WB + b, vb);
        if (reads && a == WA - 1) {
          fb[b] = read_frag(gn, WA + b);
          sc[b] = read_scale(cs, ktn, b);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (reads) fa[0] = read_frag(gn, 0);
  };

  // One slice: the first half with the loads of slice g + NS - 1 (into the
  // stage slice g - 1 used); wait for this wavefront's loads of slice g + 1,
  // finish its LDS reads, barrier; the second half.
  auto iteration = [&](int g, int kt, bool last) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    half(0, g, true, g + NS - 1, false, 0, 0);
    advance_load();
    wait_vmcnt<F8T_DMA * (NS - 2)>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    half(1, g, false, 0, !last, g + 1, kt + 1);
  };

  // Results: lane = token (fi), registers = channels; stores through
  // descriptors bounded to the tile's rows, columns past N get an offset
  // beyond them.
  auto epilogue = [&](const Tile& t, int ws) __attribute__((always_inline)) {
    // Every accumulator is final here: the matrix instructions of the last
    // slice are not moved down into the epilogue, where their fragments would
    // be spilled to scratch and the reload would wait for every load in flight.
#pragma unroll
    for (int a = 0; a < WA; ++a)
#pragma unroll
      for (int b = 0; b < WB; ++b) asm volatile("" : "+v"(acc[a][b]));
    int fi = lane & 31, fg = lane >> 5;
    asm volatile("" : "+v"(fi), "+v"(fg));
    if constexpr (DUAL) {
      const i32x4_t ro = make_desc(static_cast<uint8_t*>(out) + (int64_t)t.tok0 * N, (int64_t)t.tok_rows * N);
      const i32x4_t rs = make_desc(out_scale + (int64_t)t.tok0 * (N / 32), (int64_t)t.tok_rows * (N / 32));
#pragma unroll
      for (int b = 0; b < WB; ++b) {
        const int tl = wc * (WB * 32) + b * 32 + fi;
#pragma unroll
        for (int a = 0; a < HA; ++a) {
          const int cbase = t.ch0 + wr * (HA * 32) + a * 32;      // one 32-channel quantisation block
          const bool cin = cbase < N;
          float hv[16];
          float amax = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cl = wr * (HA * 32) + a * 32 + q * 8 + fg * 4;   // channel within the tile
            const float4 s1 = *reinterpret_cast<const float4*>(&wsc[ws][cl]);
            const float4 s3 = *reinterpret_cast<const float4*>(&wsc[ws][F8T_TA / 2 + cl]);
            const float w1s[4] = {s1.x, s1.y, s1.z, s1.w}, w3s[4] = {s3.x, s3.y, s3.z, s3.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = swiglu_fast(acc[a][b][q * 4 + r] * w1s[r], acc[a + HA][b][q * 4 + r] * w3s[r]);
              hv[q * 4 + r] = v;
              amax = fmaxf(amax, fabsf(v));
            }
          }
          amax = fmaxf(amax, __shfl_xor(amax, 32));   // the block's other 16 channels
          const int ex = block_exponent(amax);
          const float inv = __uint_as_float((uint32_t)(127 - ex) << 23);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int packed = 0;
            packed = __builtin_amdgcn_cvt_pk_fp8_f32(hv[q * 4 + 0] * inv, hv[q * 4 + 1] * inv, packed, false);
            packed = __builtin_amdgcn_cvt_pk_fp8_f32(hv[q * 4 + 2] * inv, hv[q * 4 + 3] * inv, packed, true);
            store_b32(ro, cin ? tl * N + cbase + q * 8 + fg * 4 : 0x7fffffff, (uint32_t)packed);
          }
          store_b8(rs, (cin && fg == 0) ? tl * (N / 32) + cbase / 32 : 0x7fffffff, (uint32_t)(ex + 127));
          __builtin_amdgcn_sched_barrier(0);
          acc[a][b] = acc[a + HA][b] = f32x16_t{};   // the next tile starts from zero
        }
      }
    } else {
      const i32x4_t ro = make_desc(static_cast<float*>(out) + (int64_t)t.tok0 * N, (int64_t)t.tok_rows * N * 4);
#pragma unroll
      for (int b = 0; b < WB; ++b) {
        const int tl = wc * (WB * 32) + b * 32 + fi;
#pragma unroll
        for (int a = 0; a < WA; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cl = wr * (WA * 32) + a * 32 + q * 8 + fg * 4;   // channel within the tile
            const int c = t.ch0 + cl;
            const bool cin = c < N;
            const float4 s2 = *reinterpret_cast<const float4*>(&wsc[ws][cl]);
            const u32x4_t v = {__float_as_uint(acc[a][b][q * 4 + 0] * s2.x), __float_as_uint(acc[a][b][q * 4 + 1] * s2.y),
                               __float_as_uint(acc[a][b][q * 4 + 2] * s2.z), __float_as_uint(acc[a][b][q * 4 + 3] * s2.w)};
            store_b128(ro, cin ? (tl * N + c) * 4 : 0x7fffffff, v);
            __builtin_amdgcn_sched_barrier(0);
            if (q == 3) acc[a][b] = f32x16_t{};
          }
      }
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    const int vb = voff_base();
#pragma unroll
    for (int j = 0; j <= F8T_DMA; ++j) dma(s, j, vb);
    advance_load();
  }
  wait_vmcnt<F8T_DMA * (NS - 2)>();
  __builtin_amdgcn_s_barrier();

#pragma unroll
  for (int a = 0; a < WA; ++a)
#pragma unroll
    for (int b = 0; b < WB; ++b) acc[a][b] = f32x16_t{};
  int g = 0;                      // stream index of the slice being multiplied
  for (int ci = 0; ci < n_items; ++ci) {
    const Tile t = tile_of(ci);
    fa[0] = read_frag(g, 0);
    const int cs = scale_slot(0);
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      fb[b] = read_frag(g, WA + b);
      sc[b] = read_scale(cs, 0, b);
    }
    for (int kt = 0; kt < KT - 1; ++kt) iteration(g++, kt, false);
    iteration(g++, KT - 1, true);
    epilogue(t, ci % 3);
  }
  wait_vmcnt<0>();   // the loads past the end land before the workgroup's LDS is released
}

template <bool DUAL>
hipError_t launch_fp8_tiles(const moe_shape_t& s, const uint8_t* act, const uint8_t* act_scale,
                            const int32_t* offsets, const uint8_t* wa, const uint8_t* wb,
                            const float* sa, const float* sb, int N, int K, void* out,
                            uint8_t* out_scale, hipStream_t st) {
  constexpr int CH_TILE = DUAL ? F8T_TA / 2 : F8T_TA;
  const int n_tiles = (N + CH_TILE - 1) / CH_TILE;
  const int64_t max_tiles = max_token_tiles(s, F8T_TB) * n_tiles;
  if (max_tiles <= 0) return hipSuccess;
  const int64_t grid = persistent_grid(max_tiles);
  hipLaunchKernelGGL(grouped_gemm_fp8_tiles<DUAL>, dim3((unsigned)grid), dim3(F8T_THREADS), 0, st, act,
                     act_scale, offsets, expert_groups(s), wa, wb, sa, sb, N, K, out, out_scale, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_fp8(const moe_shape_t& s, const uint8_t* x_perm, const uint8_t* x_scale,
                              const int32_t* offsets, const uint8_t* w1, const uint8_t* w3,
                              const float* w1_scale, const float* w3_scale, uint8_t* h,
                              uint8_t* h_scale, hipStream_t st) {
  return launch_fp8_tiles<true>(s, x_perm, x_scale, offsets, w1, w3, w1_scale, w3_scale, s.d_ff,
                                s.d_model, h, h_scale, st);
}

hipError_t launch_down_fp8(const moe_shape_t& s, const uint8_t* h, const uint8_t* h_scale,
                           const int32_t* offsets, const uint8_t* w2, const float* w2_scale,
                           float* y_perm, hipStream_t st) {
  return launch_fp8_tiles<false>(s, h, h_scale, offsets, w2, nullptr, w2_scale, nullptr, s.d_model,
                                 s.d_ff, y_perm, nullptr, st);
}

}  // namespace moe

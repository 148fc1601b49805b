// bf16 grouped expert GEMMs on the gfx950 matrix cores (fp32 accumulate):
// the many-tokens-per-expert (prefill) kernel and the bf16 dispatch.
//
// Pages: "Mixtral" study notes, MixtralExpert.forward = w2(silu(w1 x) * w3 x)
// (nn.Linear weights [out, in], no biases) and section "SwiGLU Experts";
// "How Mixtral 8x7B uses mixture of experts": tokens are batched by expert
// and the experts run in parallel.
//
// Both GEMMs are "NT": the token rows (x_perm or h) and the weight rows are
// contiguous along the contraction K.  The matrix-core operand A is the
// weight block (output channels) and B the token block, so an accumulator
// tile is [channel][token]; each lane then holds one token and runs of 4
// consecutive channels, which the epilogue stores as 8-byte (bf16 h) or
// 16-byte (fp32 y_perm) vectors.
//
// Prefill kernel: 512 lanes (two wavefronts per SIMD), a 384 x 256 tile
// (weights x tokens; the dual gate/up variant holds 192 w1 rows and the same
// 192 w3 rows so silu(g) * u is formed in registers).  K advances 32 at a
// time through a ring of three LDS stages of 24 + 16 KiB, filled by buffer
// loads that write LDS directly (no staging registers), so two slices are in
// flight while one is multiplied.  Rows are 64 bytes in LDS with the 16-byte
// chunks XOR-swizzled, so the fragment reads of 16 consecutive rows are free
// of bank conflicts.  The buffer descriptors are bounded to the tile's valid
// rows: rows past the expert's last token or the last channel load as zero
// without a branch.  Each wavefront owns 12 accumulator blocks of
// v_mfma_f32_32x32x16_bf16 (192 fp32 per lane); fragments are read ahead of
// the matrix instructions that use them and there is one barrier per slice.
// The larger weight tile cuts the bytes moved per flop (the global -> LDS
// path bounds this kernel) by a sixth against a 256 x 256 tile.  Tiles are
// scheduled expert by expert with token tiles fastest and remapped so that
// consecutive tiles run on the same XCD and share its L2 copy of the weight
// tile.
#include "device_common.hpp"
#include "launch.hpp"
#include "lds_stream.hpp"
#include "persistent_tiles.hpp"

namespace moe {

hipError_t launch_decode_bf16(const moe_shape_t& s, bool dual, const uint16_t* act,
                              const int32_t* offsets, const uint16_t* wa, const uint16_t* wb,
                              int N, int K, void* out, hipStream_t st);

namespace {


// Layout of a tile: WR x WC wavefronts, wavefront (wr, wc) owning WA 32-row
// weight blocks of wavefront row wr against WB 32-token blocks of column wc.
// The weight operand has TA = 32 WR WA rows, the token operand TB = 32 WC WB
// rows (the token tile).  One K slice of BK elements is an LDS row of BK * 2 bytes
// made of CPR 16-byte chunks; chunk c of row r sits at chunk position
// c ^ key(r), which spreads the fragment reads of 16 consecutive rows (one
// LDS phase, same logical chunk) over all 64 banks.  A 1 KiB load
// instruction covers RPI whole rows.
template <int BK, int WR, int WC, int WA, int WB>
struct TileGeom {
  static constexpr int NW = WR * WC;
  static constexpr int THREADS = 64 * NW;
  static constexpr int CPR = BK / 8;
  static constexpr int ROW_B = BK * 2;
  static constexpr int TA = 32 * WR * WA;
  static constexpr int TB = 32 * WC * WB;
  static constexpr int OPA_BYTES = TA * ROW_B;
  static constexpr int OPB_BYTES = TB * ROW_B;
  static constexpr int STAGE_BYTES = OPA_BYTES + OPB_BYTES;
  static constexpr int RPI = 64 / CPR;
  static constexpr int SUB = BK / 16;                  // 16-wide matrix substeps
  __device__ static __forceinline__ int key(int row) { return (row / (16 / CPR)) & (CPR - 1); }
};


// Tile: TA weight rows x 256 tokens.  The dual (gate/up) kernel's weight rows
// are TA / 2 rows of w1 followed by the same TA / 2 rows of w3, and a
// wavefront's WA blocks are WA / 2 blocks of w1 and the matching blocks of
// w3, so it forms silu(g) * u in registers.
//
// The kernel is persistent: the grid is a multiple of 8 workgroups, one per
// CU at most, and workgroup b works through tiles of XCD b % 8's share of
// the tile list (consecutive tiles, so the workgroups of one XCD share
// weight and token tiles in its L2), b / 8, b / 8 + grid / 8, ...  The K
// slices of all its tiles form one stream through the LDS ring, so the
// first slices of the next tile load while the current one finishes and
// stores its results.  Split K-runs go to fp32 partial tiles [token][TA].
//
// GATHER (gate/up only): the token operand rows are read straight from x, row
// perm_src[row] / k of it for a routed slot (slot - T k for the shared
// expert's), instead of from a permuted copy; each loading lane keeps the byte
// offsets of its JB token rows of the load cursor's tile in registers.
template <bool DUAL, int BK, int NS, int WR, int WC, int WA, int WB, int LW, bool SPLIT, bool GATHER>
__global__ __launch_bounds__(64 * WR * WC, 1) void grouped_gemm_bf16_prefill(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int N, int K,
    void* __restrict__ out, float* __restrict__ partials, int n_tiles,
    const int32_t* __restrict__ gather, int k, int Tk, int xrows) {
  using G = TileGeom<BK, WR, WC, WA, WB>;
  constexpr int TR = G::TB;                  // token rows of a tile
  static_assert(G::SUB % 2 == 0 && NS >= 2 && (!DUAL || WA % 2 == 0) && WB >= 2, "pipeline shape");
  static_assert(!SPLIT || !DUAL, "split runs: single GEMM");
  static_assert(!GATHER || DUAL, "gathered token rows: gate/up only");
  static_assert(!DUAL || (G::TA / 2) % 16 == 0, "w3 rows start on a swizzle period");
  // The expert-group tables (offsets and token-tile prefix) follow the LDS
  // ring when they fit in the 160 KiB; otherwise (the 2-stage ring of 64-wide
  // slices fills it) the offsets are read with scalar loads, which the load
  // stream's waits do not count, and a tile is found by a linear scan, for
  // at most kWideMaxGroups groups.
  constexpr int RING = NS * G::STAGE_BYTES;
  constexpr bool LDS_TABLES = RING + 2 * (kMaxExpertGroups + 1) * 4 <= 160 * 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RING + (LDS_TABLES ? 2 * (kMaxExpertGroups + 1) * 4 : 0)];
  int32_t* const offs = reinterpret_cast<int32_t*>(smem + RING);
  int32_t* const tpre = offs + (kMaxExpertGroups + 1);
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* const goffs = (const_i32*)offsets;   // generic -> constant address space

  constexpr int HA = WA / 2;                 // dual: w1 (or w3) blocks per wavefront
  constexpr int CH_TILE = DUAL ? G::TA / 2 : G::TA;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index is uniform
  const int wr = wave / WC, wc = wave % WC;
  // With two wavefronts per SIMD the accumulators and fragments leave few
  // registers: lane-derived offsets are then formed afresh where they are
  // used (from a lane index the compiler cannot reuse) rather than being
  // kept live through the K loop.
  constexpr bool LEAN = G::NW > 4 || WA * WB > 16;
  auto lane_now = [&]() __attribute__((always_inline)) {
    if constexpr (!LEAN) return lane;
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };

  // Expert offsets and their token-tile prefix go to LDS once (or stay in
  // memory, read by scalar loads), so that locating a tile in the middle of
  // the load stream issues no vector-memory read (the stream's waits count
  // its own loads).
  int n_token_tiles = 0;
  if constexpr (LDS_TABLES) {
    if (tid <= E) offs[tid] = offsets[tid];
    __syncthreads();
    if (wave == 0) build_tile_prefix(offs, E, TR, tpre, lane);
    __syncthreads();
    n_token_tiles = __builtin_amdgcn_readfirstlane(tpre[E]);
  } else {
    for (int e = 0; e < E; ++e) n_token_tiles += (goffs[e + 1] - goffs[e] + TR - 1) / TR;
  }
  const int KT = K / BK;
  const int slots = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const TileSplit sp = TileSplit::of(n_token_tiles * n_tiles, xcd, slots, KT);
  // this workgroup's items: whole tiles, then (split) up to two K-runs of tail tiles
  const int n_whole = sp.R + (((!SPLIT || sp.whole_tail) && slot < sp.tail) ? 1 : 0);
  const int run0 = slot * sp.P, run1 = min(run0 + sp.P, sp.tail * KT);
  const int n_runs = (SPLIT && run0 < run1) ? (run1 - 1) / KT - run0 / KT + 1 : 0;
  const int n_items = n_whole + n_runs;
  if (n_items == 0) return;

  // Item i: its tile, K-slice range [kb, ke) and partial slot (-1: whole tile).
  struct Tile { int e, tok0, tok_rows, ch0, kb, ke, part; };
  auto tile_of = [&](int i) __attribute__((always_inline)) -> Tile {
    int t_idx, kb = 0, ke = KT, part = -1;
    if (i < n_whole) {
      t_idx = sp.share_begin + slot + i * slots;
    } else {
      const int j = run0 / KT + (i - n_whole);        // tail tile
      t_idx = sp.share_begin + sp.R * slots + j;
      kb = max(run0, j * KT) - j * KT;
      ke = min(run1, (j + 1) * KT) - j * KT;
      part = (int)blockIdx.x * 2 + (i - n_whole);
    }
    int e, r0, r1, mt, nt;
    if constexpr (LDS_TABLES) {
      find_tile(offs, tpre, E, n_tiles, t_idx, e, r0, r1, mt, nt);
    } else {
      e = r0 = r1 = mt = nt = 0;
      for (int g = 0, tt = t_idx; g < E; ++g) {
        const int a0 = goffs[g], a1 = goffs[g + 1];
        const int m = (a1 - a0 + TR - 1) / TR;
        if (tt < m * n_tiles) {
          e = g; r0 = a0; r1 = a1; mt = tt % m; nt = tt / m;
          break;
        }
        tt -= m * n_tiles;
      }
    }
    Tile t;   // uniform values, kept in scalar registers
    t.e = __builtin_amdgcn_readfirstlane(e);
    t.tok0 = __builtin_amdgcn_readfirstlane(r0 + mt * TR);
    t.tok_rows = __builtin_amdgcn_readfirstlane(min(TR, r1 - t.tok0));
    t.ch0 = __builtin_amdgcn_readfirstlane(nt * CH_TILE);
    t.kb = __builtin_amdgcn_readfirstlane(kb);
    t.ke = __builtin_amdgcn_readfirstlane(ke);
    t.part = __builtin_amdgcn_readfirstlane(part);
    return t;
  };

  // ---- global -> LDS loads ----
  // An operand slice is made of 1 KiB blocks of RPI rows; wavefront w fills
  // blocks w, w + NW, ... of both operands.  Lane l writes chunk position
  // l % CPR of block row l / CPR and so reads logical chunk (l % CPR) ^ key(row).
  // The w3 rows of a dual tile are reached through a descriptor whose base
  // lies TA / 2 rows before the w3 tile (TA / 2 is a whole number of
  // swizzle periods, so the chunk keys are those of the LDS rows).  Loads j
  // and j + 1 of a wavefront are NW * RPI rows apart, a whole number of
  // swizzle periods, so the lane offsets of load j are those of load 0 plus
  // j times that many rows.
  //
  // Only the first LW wavefronts load (LW <= NW): each then issues NW / LW
  // times as many loads, and the others never stall on a full memory
  // pipeline, so their matrix instructions keep the SIMD's matrix pipe busy
  // while a loading wavefront waits to issue.
  constexpr int JA = G::TA / G::RPI / LW, JB = G::TB / G::RPI / LW, DMA = JA + JB;
  static_assert(JA * G::RPI * LW == G::TA && JB * G::RPI * LW == G::TB, "whole load blocks per loader");
  static_assert(LW <= G::NW && DMA < 64, "loads in flight per wavefront");
  const bool loader = wave < LW;                     // uniform
  const int64_t rowbytes = (int64_t)K * 2;
  static_assert((LW * G::RPI) % 16 == 0, "loads of a wavefront are whole swizzle periods apart");
  auto voff_base = [&]() __attribute__((always_inline)) {
    const int l = lane_now();
    const int r = wave * G::RPI + l / G::CPR;       // row within the operand tile
    return (int)(r * rowbytes) + (((l % G::CPR) ^ G::key(r)) << 4);
  };
  const int vstep = LW * G::RPI * (int)rowbytes;   // uniform
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  // Load cursor: slice lkt (of K) of item li, the item's end and its descriptors.
  i32x4_t d_tok, d_w0, d_w1;
  int li = 0, lkt = 0, lke = 0;
  int tok_off[GATHER ? JB : 1];    // gather: this lane's token-row offsets in x (load q)
  auto load_tile = [&]() __attribute__((always_inline)) {
    if (li < n_items) {
      const Tile t = tile_of(li);
      lkt = t.kb;
      lke = t.ke;
      if constexpr (GATHER) {
        d_tok = make_desc(act, (int64_t)xrows * rowbytes);
        if (loader) {
          const int l = lane_now();
#pragma unroll
          for (int q = 0; q < JB; ++q) {
            const int r = (LW * q + wave) * G::RPI + l / G::CPR;          // row within the token tile
            const int src = gather[t.tok0 + (r < t.tok_rows ? r : 0)];
            const int tok = src < Tk ? src / k : src - Tk;
            tok_off[q] = r < t.tok_rows ? (int)(tok * rowbytes) + (((l % G::CPR) ^ G::key(r)) << 4)
                                        : 0x7ff00000;                        // past x: zeros
          }
        }
      } else {
        d_tok = make_desc(act + (int64_t)t.tok0 * K, t.tok_rows * rowbytes);
      }
      d_w0 = make_desc(wa + ((int64_t)t.e * N + t.ch0) * K, (int64_t)(N - t.ch0) * rowbytes);
      d_w1 = DUAL ? make_desc(wb + ((int64_t)t.e * N + t.ch0 - G::TA / 2) * K,
                              (int64_t)(N - t.ch0 + G::TA / 2) * rowbytes)
                  : d_w0;
    }
  };
  load_tile();
  // Load j (0 .. DMA - 1) of the cursor's slice into stage ls % NS: the first
  // JA weight blocks, then JB token blocks.  Past the last tile the offset
  // lies beyond every buffer's range: such loads write zeros without touching
  // memory, into a stage that is never read again, so every iteration
  // issues the same loads.
  auto dma = [&](int ls, int j, int vb) __attribute__((always_inline)) {
    const int soff = li < n_items ? lkt * BK * 2 : 0x7ff00000;
    const uint32_t sb = lds_base + (uint32_t)((ls % NS) * G::STAGE_BYTES);
    if (j >= JA) {
      const int q = j - JA;
      dma_to_lds(d_tok, GATHER ? tok_off[GATHER ? q : 0] : vb + q * vstep, soff,
                 __builtin_amdgcn_readfirstlane(sb + G::OPA_BYTES + (LW * q + wave) * 1024));
    } else {
      const int blk = LW * j + wave;                    // uniform
      const bool w3 = DUAL && blk * G::RPI >= G::TA / 2;
      dma_to_lds(w3 ? d_w1 : d_w0, vb + j * vstep, soff, __builtin_amdgcn_readfirstlane(sb + blk * 1024));
    }
  };
  auto advance_load = [&]() __attribute__((always_inline)) {
    if (++lkt == lke) {
      ++li;
      load_tile();
    }
  };

  // ---- fragment addressing (v_mfma_f32_32x32x16_bf16: lane (fi, fg) holds
  //      row fi, k = 8 fg .. 8 fg + 7 of the 16-wide substep) ----
  auto frag_offset = [&](int s) __attribute__((always_inline)) {
    const int l = lane_now(), fi = l & 31, fg = l >> 5;
    return fi * G::ROW_B + (((2 * s + fg) ^ G::key(fi)) << 4);
  };
  int arow[WA], bfrow[WB];
#pragma unroll
  for (int a = 0; a < WA; ++a) {
    if constexpr (DUAL) arow[a] = (a / HA) * (G::TA / 2) + wr * (HA * 32) + (a % HA) * 32;
    else arow[a] = wr * (WA * 32) + a * 32;
  }
#pragma unroll
  for (int b = 0; b < WB; ++b) bfrow[b] = wc * (WB * 32) + b * 32;

  f32x16_t acc[WA][WB];

  // fragment f of a substep (lane offset fo) of slice g: 0 .. WA - 1 weight
  // blocks, then WB token blocks
  auto read_frag = [&](int g, int fo, int f) __attribute__((always_inline)) -> bf16x8_t {
    const int off = (g % NS) * G::STAGE_BYTES +
                    (f < WA ? arow[f] * G::ROW_B : G::OPA_BYTES + bfrow[f - WA] * G::ROW_B) + fo;
    return as_bf16x8(*reinterpret_cast<const uint4*>(&smem[off]));
  };

  // One substep: WA * WB matrix instructions, weight block a = i / WB against
  // token block b = i % WB.  Weight fragments are single-buffered: fa[a] is
  // reloaded with the next substep's fragment right after its last use
  // (b == WB - 1).  Token fragments are double-buffered, the next substep's
  // read after the first WB instructions, when the accumulators leave room
  // for it; otherwise fb[b] is reloaded after its last use (a == WA - 1)
  // and the other wavefront on the SIMD covers the wait.  With `loads`, the
  // remaining slots carry the loads of the load cursor's slice `ls`, PER to
  // a slot (slot numbering starts at slot0).  With `reads`, (gn, sn) is the
  // substep whose fragments are read.
  constexpr bool FB2 = WA * WB * 16 + 4 * (WA + 2 * WB) <= 2048 / G::NW - 32;
  bf16x8_t fa[WA], fb[FB2 ? 2 : 1][WB];
  constexpr int NI = WA * WB;
  constexpr int FREE = (WA - 1) * (WB - 1);               // load slots per substep
  auto substep = [&](int cur, int gn, int sn, int slot0, bool loads, int ls, bool reads)
                     __attribute__((always_inline)) {
    const int fo = reads ? frag_offset(sn) : 0;
    const int vb = loads ? voff_base() : 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int a = i / WB, b = i % WB;
      acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[FB2 ? cur : 0][b], acc[a][b], 0, 0, 0);
      if constexpr (FB2) {
        if (reads && i < WB) fb[cur ^ 1][i] = read_frag(gn, fo, WA + i);
      } else {
        if (reads && a == WA - 1) fb[0][b] = read_frag(gn, fo, WA + b);
      }
      if (b == WB - 1) {
        if (reads) fa[a] = read_frag(gn, fo, a);
      } else if (a >= 1 && loads) {
        constexpr int SLOTS = FREE, PER = (DMA + SLOTS - 1) / SLOTS;
        const int sl = slot0 + (a - 1) * (WB - 1) + b;
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if (sl * PER + q < DMA && loader) dma(ls, sl * PER + q, vb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Results of the compute cursor's tile: lane = token (fi), registers = channels.
  // Stores go through a buffer descriptor bounded to the tile's valid rows;
  // columns past N get an offset beyond it.  Either way the store is dropped
  // without a branch.
  auto epilogue = [&](const Tile& t) __attribute__((always_inline)) {
    // Lane coordinates made opaque here, so that the store offsets are formed
    // per tile instead of being hoisted out of the tile loop (where they would
    // occupy registers through the whole K loop).
    int fi = lane & 31, fg = lane >> 5;
    asm volatile("" : "+v"(fi), "+v"(fg));
    constexpr int OB = DUAL ? 2 : 4;            // output element bytes (bf16 h, fp32 y)
    const i32x4_t ro = make_desc(static_cast<uint8_t*>(out) + (int64_t)t.tok0 * N * OB,
                                 (int64_t)t.tok_rows * N * OB);
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      const int tl = wc * (WB * 32) + b * 32 + fi;      // token row within the tile
      const int row_off = tl * N * OB;
      if constexpr (DUAL) {
#pragma unroll
        for (int a = 0; a < HA; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = t.ch0 + wr * (HA * 32) + a * 32 + q * 8 + fg * 4;
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              hv[r] = swiglu_fast(acc[a][b][q * 4 + r], acc[a + HA][b][q * 4 + r]);
            store_b64(ro, c < N ? row_off + c * OB : 0x7fffffff, pack_bf16x2(hv[0], hv[1]),
                      pack_bf16x2(hv[2], hv[3]));
            __builtin_amdgcn_sched_barrier(0);   // one block at a time: few live registers
            if (q == 3) acc[a][b] = acc[a + HA][b] = f32x16_t{};   // the next tile starts from zero
          }
      } else {
        // a K-run of a split tile goes whole to its partial slot ([token][channel], 256 x TA)
        const bool part = SPLIT && t.part >= 0;
        const i32x4_t dst = part ? make_desc(partials + (int64_t)t.part * (TR * G::TA),
                                             TR * G::TA * 4)
                                 : ro;
#pragma unroll
        for (int a = 0; a < WA; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cl = wr * (WA * 32) + a * 32 + q * 8 + fg * 4;   // channel within the tile
            const int c = t.ch0 + cl;
            const u32x4_t v = {__float_as_uint(acc[a][b][q * 4 + 0]), __float_as_uint(acc[a][b][q * 4 + 1]),
                               __float_as_uint(acc[a][b][q * 4 + 2]), __float_as_uint(acc[a][b][q * 4 + 3])};
            store_b128(dst, part ? (tl * G::TA + cl) * 4 : (c < N ? row_off + c * OB : 0x7fffffff), v);
            __builtin_amdgcn_sched_barrier(0);
            if (q == 3) acc[a][b] = f32x16_t{};   // the next tile starts from zero
          }
      }
    }
  };

  // Pipeline.  Slice g of the stream lives in stage g % NS.  Iteration g runs
  // SUB substeps.  The first carries all the loads of slice g + NS - 1
  // (PER per free slot: the earliest issue leaves the longest time before
  // their wait, which the 2-stage ring needs), and they go to the stage that
  // slice g - 1 used (every wavefront finished reading it before the
  // previous barrier).  Before the last substep: wait
  // for this wavefront's loads of slice g + 1 (the loads of later slices
  // stay in flight), finish its LDS reads, barrier -- slice g + 1 is
  // complete in LDS and slice g is no longer read; the last substep then
  // reads substep 0 of slice g + 1, except in a tile's last iteration: the
  // results are stored first and the next tile's fragments read after.
  // Pending stores share the vector-memory counter with the loads; loads
  // complete in order among themselves, so they only make the wait stricter.
  // Instruction order is fixed with scheduling barriers.
  auto iteration = [&](int g, bool last) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < G::SUB - 1; ++s)
      substep(s & 1, g, s + 1, 0, s == 0, g + NS - 1, true);
    advance_load();
    wait_vmcnt<DMA * (NS - 2)>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    substep(1, g + 1, 0, 0, false, 0, !last);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    const int vb = voff_base();
#pragma unroll
    for (int j = 0; j < DMA; ++j)
      if (loader) dma(s, j, vb);
    advance_load();
  }
  wait_vmcnt<DMA * (NS - 2)>();
  __builtin_amdgcn_s_barrier();

#pragma unroll
  for (int a = 0; a < WA; ++a)
#pragma unroll
    for (int b = 0; b < WB; ++b) acc[a][b] = f32x16_t{};
  int g = 0;                      // stream index of the slice being multiplied
  for (int ci = 0; ci < n_items; ++ci) {
    const Tile t = tile_of(ci);
    const int nk = t.ke - t.kb;                  // >= 1
    const int fo = frag_offset(0);
#pragma unroll
    for (int f = 0; f < WA; ++f) fa[f] = read_frag(g, fo, f);
#pragma unroll
    for (int f = 0; f < WB; ++f) fb[0][f] = read_frag(g, fo, WA + f);
    for (int kt = 0; kt < nk - 1; ++kt) iteration(g++, false);
    iteration(g++, true);
    epilogue(t);                  // stores the tile and zeroes the accumulators
  }
  wait_vmcnt<0>();   // the zero loads past the end land before the workgroup's LDS is released
}

// Sum of the K-runs of each split tail tile, in K order, into y_perm.  One
// workgroup per (XCD, tail tile, group of 16 rows of the TR-row token tile):
// lane l covers row 16 g + l / 16 and channels 4 (l % 16) + 64 c, c < CH / 64,
// so every lane has CH / 64 independent 16-byte sums in flight.
template <int CH, int TR>
__global__ __launch_bounds__(256) void split_fixup_kernel(const int32_t* __restrict__ offsets, int E,
                                                          int N, int K, int BK, int n_tiles, int slots,
                                                          const float* __restrict__ partials,
                                                          float* __restrict__ y) {
  constexpr int CPL = CH / 64;
  __shared__ int32_t offs[kMaxExpertGroups + 1];
  __shared__ int32_t tpre[kMaxExpertGroups + 1];
  for (int i = threadIdx.x; i <= E; i += 256) offs[i] = offsets[i];
  __syncthreads();
  if (threadIdx.x < 64) build_tile_prefix(offs, E, TR, tpre, threadIdx.x);
  __syncthreads();
  constexpr int kRowGroups = TR / 16;
  const int rg = blockIdx.x % kRowGroups;
  const int xcd = (blockIdx.x / kRowGroups) & 7, j = blockIdx.x / kRowGroups >> 3;
  const int KT = K / BK;
  const TileSplit sp = TileSplit::of(__builtin_amdgcn_readfirstlane(tpre[E]) * n_tiles, xcd, slots, KT);
  if (sp.whole_tail || j >= sp.tail) return;   // no runs: the tail tiles were stored whole
  int e, r0, r1, mt, nt;
  find_tile(offs, tpre, E, n_tiles, sp.share_begin + sp.R * slots + j, e, r0, r1, mt, nt);
  const int tok0 = r0 + mt * TR, tok_rows = min(TR, r1 - tok0), ch0 = nt * CH;
  const int r = rg * 16 + (threadIdx.x >> 4);
  if (r >= tok_rows) return;
  const int s_lo = (j * KT) / sp.P, s_hi = min(((j + 1) * KT - 1) / sp.P, slots - 1);
  float4 acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = s_lo; s <= s_hi; ++s) {
    const int part = (s * 8 + xcd) * 2 + (j - (s * sp.P) / KT);
    const float* src = partials + (int64_t)part * (TR * CH) + r * CH + (threadIdx.x & 15) * 4;
    float4 p[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) p[c] = *reinterpret_cast<const float4*>(src + 64 * c);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      acc[c].x += p[c].x; acc[c].y += p[c].y; acc[c].z += p[c].z; acc[c].w += p[c].w;
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = ch0 + (threadIdx.x & 15) * 4 + 64 * c;
    if (col < N) *reinterpret_cast<float4*>(y + (int64_t)(tok0 + r) * N + col) = acc[c];
  }
}

// Shapes of the prefill kernels: K slice, LDS ring depth, wavefront grid,
// blocks per wavefront and loading wavefronts.  All run 8 wavefronts (two per
// SIMD).  The kWide gate/up kernel loads from 4 of them (one per SIMD): 3.19
// -> 3.07 ms at the Mixtral prefill shape, 1.58 -> 1.54 ms skewed with the
// fallback (A/B on one MI355X); its down projection gained nothing from it.
//  * kWide (at most kWideMaxGroups expert groups): a 384 x 256 tile (weights x
//    tokens; 192 accumulators per lane), gate/up as 2 x 4 wavefronts of 3 + 3
//    (w1, w3) blocks x 2 token blocks, down as 4 x 2 wavefronts of 3 x 4.  A K
//    slice is 64 wide (128-byte row segments: half as many L2 requests per
//    byte as 64-byte ones) in a ring of 2 stages of 80 KiB, which fills LDS:
//    the group offsets are read with scalar loads.
//  * kNarrow (more groups): the same tile with 32-wide slices in 3 stages of
//    40 KiB, leaving LDS for the group tables.
//  * kTall (experts of at most 320 rows on average, e.g. many small experts):
//    a 256 x 320 tile, 4 x 2 wavefronts of 2 (gate/up: 1 + 1) weight blocks x
//    5 token blocks (160 accumulators).  An expert of up to 320 rows is one
//    token tile, where 256-row tiles cut an expert of 257..320 rows into a
//    full tile and a nearly empty one.  64-wide slices in 2 stages of 72 KiB
//    leave LDS for the group tables, so any number of groups takes 128-byte
//    row segments.
constexpr int kWideMaxGroups = 16;
constexpr int kTallMaxMeanRows = 320;
enum PrefillKind { kNarrow = 0, kWide = 1, kTall = 2 };
template <bool DUAL, int KIND> struct PrefillCfg;
template <> struct PrefillCfg<true, kNarrow> { static constexpr int BK = 32, NS = 3, WR = 2, WC = 4, WA = 6, WB = 2, LW = 8; };
template <> struct PrefillCfg<false, kNarrow> { static constexpr int BK = 32, NS = 3, WR = 4, WC = 2, WA = 3, WB = 4, LW = 8; };
template <> struct PrefillCfg<true, kWide> { static constexpr int BK = 64, NS = 2, WR = 2, WC = 4, WA = 6, WB = 2, LW = 4; };
template <> struct PrefillCfg<false, kWide> { static constexpr int BK = 64, NS = 2, WR = 4, WC = 2, WA = 3, WB = 4, LW = 8; };
template <> struct PrefillCfg<true, kTall> { static constexpr int BK = 64, NS = 2, WR = 4, WC = 2, WA = 2, WB = 5, LW = 8; };
template <> struct PrefillCfg<false, kTall> { static constexpr int BK = 64, NS = 2, WR = 4, WC = 2, WA = 2, WB = 5, LW = 8; };
template <bool DUAL, int KIND>
using PrefillGeom = TileGeom<PrefillCfg<DUAL, KIND>::BK, PrefillCfg<DUAL, KIND>::WR, PrefillCfg<DUAL, KIND>::WC,
                             PrefillCfg<DUAL, KIND>::WA, PrefillCfg<DUAL, KIND>::WB>;
// fp32 partial tile of a split K-run ([token][channel]), the largest of the down shapes
constexpr int64_t kPartialTileBytes =
    std::max((int64_t)PrefillGeom<false, kWide>::TB * PrefillGeom<false, kWide>::TA,
             (int64_t)PrefillGeom<false, kTall>::TB * PrefillGeom<false, kTall>::TA) * 4;
static_assert(PrefillGeom<false, kWide>::TA == PrefillGeom<false, kNarrow>::TA &&
              PrefillGeom<false, kWide>::TB == PrefillGeom<false, kNarrow>::TB, "one partial tile shape per TA");

template <bool DUAL, int KIND, bool GATHER = false>
hipError_t launch_prefill_cfg(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                          float* partials, hipStream_t st, const int32_t* gather = nullptr) {
  using C = PrefillCfg<DUAL, KIND>;
  using G = PrefillGeom<DUAL, KIND>;
  constexpr int CH_TILE = DUAL ? G::TA / 2 : G::TA;
  const int n_tiles = (N + CH_TILE - 1) / CH_TILE;
  const int64_t max_tiles = max_token_tiles(s, G::TB) * n_tiles;
  if (max_tiles <= 0) return hipSuccess;
  const int64_t grid = persistent_grid(max_tiles);
  if constexpr (!DUAL) {
    if (partials != nullptr) {   // split tail: K-runs into partial tiles, then their sum
      hipLaunchKernelGGL((grouped_gemm_bf16_prefill<false, C::BK, C::NS, C::WR, C::WC, C::WA, C::WB, C::LW, true, false>),
                         dim3((unsigned)grid), dim3(G::THREADS), 0, st, act, offsets, expert_groups(s), wa,
                         wb, N, K, out, partials, n_tiles, nullptr, 1, 0, 0);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((split_fixup_kernel<G::TA, G::TB>), dim3((unsigned)(grid * (G::TB / 16))), dim3(256),
                         0, st, offsets, expert_groups(s), N, K, C::BK, n_tiles, (int)(grid / 8), partials,
                         static_cast<float*>(out));
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((grouped_gemm_bf16_prefill<DUAL, C::BK, C::NS, C::WR, C::WC, C::WA, C::WB, C::LW, false, GATHER>),
                     dim3((unsigned)grid), dim3(G::THREADS), 0, st, act, offsets, expert_groups(s), wa,
                     wb, N, K, out, nullptr, n_tiles, gather, s.top_k, s.T * s.top_k, s.T);
  return hipGetLastError();
}

// Mean rows per routed expert (the token tile shape follows it; the shared
// expert's rows do not count).
int64_t mean_routed_rows(const moe_shape_t& s) {
  const int64_t r = (int64_t)s.T * s.top_k / s.n_experts;
  return s.capacity >= 0 ? std::min<int64_t>(r, s.capacity) : r;
}

template <bool DUAL>
hipError_t launch_prefill(const moe_shape_t& s, const uint16_t* act, const int32_t* offsets,
                          const uint16_t* wa, const uint16_t* wb, int N, int K, void* out,
                          float* partials, hipStream_t st) {
  if (mean_routed_rows(s) <= kTallMaxMeanRows)
    return launch_prefill_cfg<DUAL, kTall>(s, act, offsets, wa, wb, N, K, out, partials, st);
  if (expert_groups(s) <= kWideMaxGroups)
    return launch_prefill_cfg<DUAL, kWide>(s, act, offsets, wa, wb, N, K, out, partials, st);
  return launch_prefill_cfg<DUAL, kNarrow>(s, act, offsets, wa, wb, N, K, out, partials, st);
}

// Weight streaming (decode kernels) while no expert can hold more than this many rows.
constexpr int kDecodeMaxRows = 64;

}  // namespace

hipError_t launch_gate_up_bf16(const moe_shape_t& s, const uint16_t* x_perm,
                               const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                               uint16_t* h, hipStream_t st) {
  if (max_rows_per_expert(s) <= kDecodeMaxRows)
    return launch_decode_bf16(s, true, x_perm, offsets, w1, w3, s.d_ff, s.d_model, h, st);
  return launch_prefill<true>(s, x_perm, offsets, w1, w3, s.d_ff, s.d_model, h, nullptr, st);
}

hipError_t launch_down_bf16(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                            const uint16_t* w2, float* y_perm, void* workspace, hipStream_t st) {
  if (max_rows_per_expert(s) <= kDecodeMaxRows)
    return launch_decode_bf16(s, false, h, offsets, w2, nullptr, s.d_model, s.d_ff, y_perm, st);
  return launch_prefill<false>(s, h, offsets, w2, nullptr, s.d_model, s.d_ff, y_perm,
                               static_cast<float*>(workspace), st);
}

bool gate_up_decode_gathers(const moe_shape_t& s) {
  return s.act_dtype == MOE_BF16 && (s.w_dtype == MOE_BF16 || s.w_dtype == MOE_MXFP4) &&
         max_rows_per_expert(s) <= kDecodeMaxRows;
}

bool gate_up_bf16_gathers(const moe_shape_t& s) {
  return s.act_dtype == MOE_BF16 && s.w_dtype == MOE_BF16 && max_rows_per_expert(s) > kDecodeMaxRows &&
         mean_routed_rows(s) <= kTallMaxMeanRows;
}

hipError_t launch_gate_up_bf16_prefill_gather(const moe_shape_t& s, const uint16_t* x, const int32_t* perm_src,
                                              const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                                              uint16_t* h, hipStream_t st) {
  if (!gate_up_bf16_gathers(s)) return hipErrorInvalidValue;
  return launch_prefill_cfg<true, kTall, true>(s, x, offsets, w1, w3, s.d_ff, s.d_model, h, nullptr, st,
                                               perm_src);
}

size_t down_workspace_bytes_bf16(const moe_shape_t& s) {
  if (max_rows_per_expert(s) <= kDecodeMaxRows) return 0;
  return (size_t)kMaxPersistentGroups * 2 * kPartialTileBytes;
}

}  // namespace moe

// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Low / high bf16 of a packed 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  __bf16 b = (__bf16)v;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// E8M0 exponent of an fp8 activation block (x rows in the permute, h in the
// gate/up epilogue: one rule for both): ceil(log2(fp32(amax / 448))) clamped
// to [-127, 127]; 0 for an all-zero block.  amax / 448 is one fp32 division;
// the exponent is read from its bits (a subnormal quotient included).
__device__ __forceinline__ int block_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const uint32_t bits = __float_as_uint(amax / 448.0f);
  const int ex = (int)((bits >> 23) & 255u);
  const uint32_t man = bits & 0x7fffffu;
  if (ex == 0) return man > (1u << 22) ? -126 : -127;  // subnormal quotient
  return man == 0 ? ex - 127 : ex - 126;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// XOR key of the 16-byte-chunk swizzle of 128-byte LDS rows.  A 16-byte LDS
// read is served 16 lanes per cycle across 64 four-byte banks: with one row
// per lane, rows of equal parity share a 32-bank half, so rows i and i + 8
// must get different chunks as well as rows 0..7 among themselves.
// (row & 7) ^ (bit 3 of row) gives distinct chunks to any 8 consecutive rows
// and to each parity class of any 16 consecutive rows.
__device__ __forceinline__ int lds_swizzle_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// 16-byte load marked non-temporal (streamed data that is read exactly once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Grouped-GEMM tile lookup: the linear tile index `t` of a grid that covers,
// expert by expert, ceil(count_e / rows_per_tile) token tiles times
// `n_tiles` channel tiles.  Token tiles vary fastest inside an expert so
// that concurrently running workgroups share the same weight tile.
// Returns false when `t` lies beyond the last real tile.
__device__ __forceinline__ bool locate_tile(const int32_t* __restrict__ offsets, int n_experts,
                                            int rows_per_tile, int n_tiles, int t, int& expert,
                                            int& row_begin, int& row_end, int& m_tile,
                                            int& n_tile) {
  for (int e = 0; e < n_experts; ++e) {
    // the offsets are the same for every lane (also when staged in LDS)
    const int r0 = __builtin_amdgcn_readfirstlane(offsets[e]);
    const int r1 = __builtin_amdgcn_readfirstlane(offsets[e + 1]);
    const int mt = (r1 - r0 + rows_per_tile - 1) / rows_per_tile;
    const int tiles = mt * n_tiles;
    if (t < tiles) {
      expert = e;
      row_begin = r0;
      row_end = r1;
      m_tile = t % mt;
      n_tile = t / mt;
      return true;
    }
    t -= tiles;
  }
  return false;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap so that consecutive logical tiles run on the same XCD:
// logical = (id % 8) * (grid / 8) + id / 8 (grid padded to a multiple of 8).
__device__ __forceinline__ int xcd_remap(int id, int grid_padded) {
  return (id & 7) * (grid_padded >> 3) + (id >> 3);
}

}  // namespace moe

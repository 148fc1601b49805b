// Building blocks of the streaming GEMM kernels: buffer descriptors held in
// scalar registers, buffer loads that write LDS directly, buffer stores, and
// explicit waits on the vector-memory counter.
#pragma once
#include "device_common.hpp"

namespace moe {

constexpr int kRawBufferFlags = 0x00020000;   // raw buffer, 32-bit data format

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor in scalar registers covering [base, base + bytes)
// (clamped to 2^31 - 1 bytes).  Accesses at offsets past the range read
// zeros or are dropped.
__device__ __forceinline__ i32x4_t make_desc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int n = bytes <= 0 ? 0 : bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;   // empty when negative
  i32x4_t d;
  d.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  d.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));   // stride 0
  d.z = __builtin_amdgcn_readfirstlane(n);
  d.w = kRawBufferFlags;
  return d;
}

// Wavefront-wide load of 16 (4) bytes per lane from a buffer straight into
// LDS: lane l's bytes land at lds_addr + 16 l (4 l), so one instruction
// fills 1 KiB (256 bytes).  The load is counted by vmcnt like any vector
// memory read.  It is written as assembly because the compiler, unable to
// tell which LDS bytes such a load writes, would wait for it to finish
// before every LDS read, including reads of other stages.  M0 (the LDS
// address) is declared clobbered; the kernels using these helpers use M0
// for nothing else.
//
// Every vector-memory instruction written in assembly here is preceded by
// `s_nop 4`: a vector-ALU write of a scalar register (v_readfirstlane, or
// v_readlane restoring a spilled descriptor) needs 5 wait states before a
// vector-memory instruction reads that register, and the compiler's hazard
// pass does not look inside assembly.  The wait also covers M0 written just
// before an LDS-DMA load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_to_lds(i32x4_t desc, int voff, int soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(desc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4_to_lds(i32x4_t desc, int voff, int soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(desc), "s"(soff) : "memory", "m0");
}
// The same with the LDS address given as a scalar base plus `off`, which
// must fold to a constant after inlining (it becomes an instruction
// immediate), so that a run of loads into one stage needs one scalar register.
// The scalar add also writes SCC, which is declared clobbered.
__device__ __forceinline__ void dma_to_lds_at(i32x4_t desc, int voff, int soff, uint32_t lds_base,
                                              int off) {
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(desc), "s"(soff), "i"(off) : "memory", "m0", "scc");
}
__device__ __forceinline__ void dma4_to_lds_at(i32x4_t desc, int voff, int soff, uint32_t lds_base,
                                               int off) {
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 4\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(desc), "s"(soff), "i"(off) : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// Buffer stores through a descriptor held in scalar registers (assembly, so
// that the descriptor cannot end up in vector registers and force a per-lane
// loop).  Offsets past the descriptor's range drop the store.  The trailing
// wait states cover a vector-ALU write of the data registers right after a
// store of more than 8 bytes.
// (The leading `s_nop 4` is the scalar-register wait described above.)
__device__ __forceinline__ void store_b8(i32x4_t desc, int voff, uint32_t v) {
  asm volatile("s_nop 4\n\tbuffer_store_byte %0, %1, %2, 0 offen"
               :: "v"(v), "v"(voff), "s"(desc) : "memory");
}
__device__ __forceinline__ void store_b32(i32x4_t desc, int voff, uint32_t v) {
  asm volatile("s_nop 4\n\tbuffer_store_dword %0, %1, %2, 0 offen"
               :: "v"(v), "v"(voff), "s"(desc) : "memory");
}
__device__ __forceinline__ void store_b64(i32x4_t desc, int voff, uint32_t lo, uint32_t hi) {
  asm volatile("s_nop 4\n\tbuffer_store_dwordx2 %0, %1, %2, 0 offen\n\ts_nop 0"
               :: "v"(u32x2_t{lo, hi}), "v"(voff), "s"(desc) : "memory");
}
__device__ __forceinline__ void store_b128(i32x4_t desc, int voff, u32x4_t v) {
  asm volatile("s_nop 4\n\tbuffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 1"
               :: "v"(v), "v"(voff), "s"(desc) : "memory");
}

// Wait until at most n vector-memory operations of this wavefront are pending.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((n >> 4) << 14) | 0x0f70 | (n & 15));
}
// Wait until this wavefront's LDS and scalar-memory operations are done.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// silu(g) * u with hardware exp2 and reciprocal (about 1 ulp in fp32, far
// below the bf16 or fp8 rounding that follows).
__device__ __forceinline__ float swiglu_fast(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

}  // namespace moe

// Host-side launchers of the MoE kernels (internal to libmoe).  Each takes a
// validated shape; the C ABI in api.cpp does the validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moe.h"

namespace moe {

// Router GEMV + top-k + softmax of the kept logits (+ the experts ranked k+1, k+2
// when next_ids != NULL).
// bf16 with more than 64 experts: logits to an fp32 [T, E] buffer (`logits`
// when given, else `workspace` of route_workspace_bytes(s)), then selection.
hipError_t launch_route_topk(const moe_shape_t& s, const void* x, const void* w_gate,
                             const float* bias, int32_t* ids, float* weights, float* logits,
                             int32_t* next_ids, void* workspace, hipStream_t st);
size_t route_workspace_bytes(const moe_shape_t& s);

// Decode steps of moe_forward (bf16, T <= 16, E <= 16, top-2, dropless, no
// shared expert): the router's partial sums over eight workgroups, then one
// workgroup that adds them, selects and groups (route_index_fused; `part` is
// route_index_part_bytes() of workspace), and the gate/up weight streamer
// reading token rows of x through perm_src instead of a permuted copy.
bool route_index_fused(const moe_shape_t& s);
size_t route_index_part_bytes();
hipError_t launch_route_index(const moe_shape_t& s, const void* x, const void* w_gate,
                              const float* bias, int32_t* ids, float* weights, float* logits,
                              int32_t* counts, int32_t* offsets, int32_t* perm_src,
                              int32_t* slot_to_row, void* part, hipStream_t st);
hipError_t launch_gate_up_bf16_gather(const moe_shape_t& s, const uint16_t* x, const int32_t* perm_src,
                                      const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                                      uint16_t* h, hipStream_t st);
hipError_t launch_gate_up_mxfp4_gather(const moe_shape_t& s, const uint16_t* x, const int32_t* perm_src,
                                       const int32_t* offsets, const uint8_t* w1, const uint8_t* w1_scale,
                                       const uint8_t* w3, const uint8_t* w3_scale, uint16_t* h,
                                       hipStream_t st);

// Capacity selection: writes drop_mask[T*k] (0 kept, 1 dropped); with
// MOE_OVERFLOW_NEXT_BEST a second round re-offers the dropped assignments to
// next_ids and marks the ones taken with 2.
hipError_t launch_capacity_select(const moe_shape_t& s, const int32_t* ids, const float* weights,
                                  const int32_t* next_ids, uint8_t* drop_mask, hipStream_t st);

// Counts, offsets, perm_src, slot_to_row (drop_mask may be NULL: nothing
// dropped; next_ids is read for slots marked 2).
hipError_t launch_permute_index(const moe_shape_t& s, const int32_t* ids, const uint8_t* drop_mask,
                                const int32_t* next_ids, int32_t* counts, int32_t* offsets,
                                int32_t* perm_src, int32_t* slot_to_row, hipStream_t st);

// x_perm[row] = x[token of perm_src[row]] (fp8: block-quantised codes + E8M0 scales).
hipError_t launch_permute_scatter(const moe_shape_t& s, const void* x, const int32_t* offsets,
                                  const int32_t* perm_src, void* x_perm, uint8_t* x_perm_scale,
                                  hipStream_t st);

// Grouped gate/up (dual weight, SwiGLU epilogue) and down GEMMs.
// Weight scales: fp32 per output channel (fp8) or E8M0 bytes per 32-element block (MXFP4).
hipError_t launch_gate_up(const moe_shape_t& s, const void* x_perm, const uint8_t* x_scale,
                          const int32_t* offsets, const void* w1, const void* w3,
                          const void* w1_scale, const void* w3_scale, void* h, uint8_t* h_scale,
                          hipStream_t st);
hipError_t launch_down(const moe_shape_t& s, const void* h, const uint8_t* h_scale,
                       const int32_t* offsets, const void* w2, const void* w2_scale,
                       float* y_perm, void* workspace, hipStream_t st);

// Fill n bytes with v (a kernel, so that the call can sit inside a captured graph).
hipError_t launch_fill_u8(uint8_t* p, int64_t n, uint8_t v, hipStream_t st);

hipError_t launch_combine(const moe_shape_t& s, const float* y_perm, const int32_t* slot_to_row,
                          const float* weights, void* y, hipStream_t st);

// fp32 generic GEMM path (act F32 + w F32).
hipError_t launch_gate_up_f32(const moe_shape_t& s, const float* x_perm, const int32_t* offsets,
                              const float* w1, const float* w3, float* h, hipStream_t st);
hipError_t launch_down_f32(const moe_shape_t& s, const float* h, const int32_t* offsets,
                           const float* w2, float* y_perm, hipStream_t st);

// bf16 paths.
hipError_t launch_gate_up_bf16(const moe_shape_t& s, const uint16_t* x_perm,
                               const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                               uint16_t* h, hipStream_t st);
// workspace: down_workspace_bytes_bf16(s) bytes (partial tiles of the split
// tail work), or NULL for the data-parallel schedule only.
hipError_t launch_down_bf16(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                            const uint16_t* w2, float* y_perm, void* workspace, hipStream_t st);
size_t down_workspace_bytes_bf16(const moe_shape_t& s);
// Down projection + combine in one launch for a decode batch (bf16, T <= 16,
// top-2, dropless, no shared expert, E <= 16): y from h, offsets, slot_to_row
// and the gate weights, bit for bit what launch_down_bf16 + launch_combine give.
bool down_combine_fused(const moe_shape_t& s);
// Tiled gate/up reading the token rows of x through perm_src (no x_perm): bf16,
// prefill batches whose routed experts average at most 320 rows (the 256 x 320
// tile); the result equals launch_gate_up_bf16 on the permuted copy bit for bit.
bool gate_up_bf16_gathers(const moe_shape_t& s);
// Weight-streaming (decode) gate/up that can read token rows through perm_src
// (launch_gate_up_bf16_gather / launch_gate_up_mxfp4_gather): bf16 activations,
// bf16 or MXFP4 experts, at most 64 rows per expert.
bool gate_up_decode_gathers(const moe_shape_t& s);
hipError_t launch_gate_up_bf16_prefill_gather(const moe_shape_t& s, const uint16_t* x, const int32_t* perm_src,
                                              const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                                              uint16_t* h, hipStream_t st);
hipError_t launch_down_combine_bf16(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                                    const uint16_t* w2, const int32_t* slot_to_row, const float* gw,
                                    uint16_t* y, hipStream_t st);

// Whether the fp8 matrix-core path is built in.
constexpr bool kFp8Available = true;

// Largest n_experts the library accepts (routed), the largest top_k, and the
// largest n_experts of the fp32-activation router.
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;
constexpr int kMaxExpertsF32 = 64;
// Expert groups of the permuted rows: routed experts, then the shared one.
constexpr int kMaxExpertGroups = kMaxExperts + 1;
inline int expert_groups(const moe_shape_t& s) { return s.n_experts + s.n_shared; }
// Slots (assignments) per token, the shared expert's included.
inline int64_t total_slots(const moe_shape_t& s) { return (int64_t)s.T * (s.top_k + s.n_shared); }
// The router runs as logits + selection (two kernels) rather than one fused kernel.
inline bool route_two_pass(const moe_shape_t& s) { return s.act_dtype == MOE_BF16 && s.n_experts > 64; }

// Compute units of the current device (queried once per device).
int device_cu_count();

// fp8 paths (e4m3 weights with per-channel fp32 scales, block-scaled e4m3 activations).
hipError_t launch_gate_up_fp8(const moe_shape_t& s, const uint8_t* x_perm, const uint8_t* x_scale,
                              const int32_t* offsets, const uint8_t* w1, const uint8_t* w3,
                              const float* w1_scale, const float* w3_scale, uint8_t* h,
                              uint8_t* h_scale, hipStream_t st);
hipError_t launch_down_fp8(const moe_shape_t& s, const uint8_t* h, const uint8_t* h_scale,
                           const int32_t* offsets, const uint8_t* w2, const float* w2_scale,
                           float* y_perm, hipStream_t st);

// MXFP4 expert weights (E2M1 codes + E8M0 block scales) with bf16 activations:
// weight streaming for few rows per expert.
constexpr int kMxfp4MaxRows = 64;
hipError_t launch_gate_up_mxfp4(const moe_shape_t& s, const uint16_t* x_perm,
                                const int32_t* offsets, const uint8_t* w1, const uint8_t* w1_scale,
                                const uint8_t* w3, const uint8_t* w3_scale, uint16_t* h,
                                hipStream_t st);
hipError_t launch_down_mxfp4(const moe_shape_t& s, const uint16_t* h, const int32_t* offsets,
                             const uint8_t* w2, const uint8_t* w2_scale, float* y_perm,
                             hipStream_t st);

// Largest number of rows any routed expert can receive: each token picks an expert at most once.
inline int64_t max_rows_per_routed_expert(const moe_shape_t& s) {
  int64_t m = s.T;
  if (s.capacity >= 0 && s.capacity < m) m = s.capacity;
  return m;
}

// Largest number of rows of any expert group (the shared expert takes all T tokens).
inline int64_t max_rows_per_expert(const moe_shape_t& s) {
  return s.n_shared > 0 ? (int64_t)s.T : max_rows_per_routed_expert(s);
}

// Upper bound of sum_g ceil(count_g / rows_per_tile) over the expert groups given
// sum_e count_e <= T*k over the routed experts (and <= capacity*E), plus the
// shared expert's T rows.
inline int64_t max_token_tiles(const moe_shape_t& s, int rows_per_tile) {
  int64_t total = (int64_t)s.T * s.top_k;
  if (s.capacity >= 0) total = std::min<int64_t>(total, (int64_t)s.capacity * s.n_experts);
  int64_t t = (total + rows_per_tile - 1) / rows_per_tile + s.n_experts;
  int64_t per_expert = (max_rows_per_routed_expert(s) + rows_per_tile - 1) / rows_per_tile;
  t = std::min<int64_t>(t, per_expert * s.n_experts);
  return t + (int64_t)s.n_shared * ((s.T + rows_per_tile - 1) / rows_per_tile);
}

}  // namespace moe

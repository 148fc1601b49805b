// C ABI of the MoE layer: argument validation, workspace layout, dispatch.
// Every public function validates on the host before enqueueing anything.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "launch.hpp"

namespace moe {

// Compute units of the current device, asked of the runtime at every launch
// (the library keeps no state between calls).
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

hipError_t launch_gate_up(const moe_shape_t& s, const void* x_perm, const uint8_t* x_scale,
                          const int32_t* offsets, const void* w1, const void* w3,
                          const void* w1_scale, const void* w3_scale, void* h, uint8_t* h_scale,
                          hipStream_t st) {
  if (s.w_dtype == MOE_F32)
    return launch_gate_up_f32(s, static_cast<const float*>(x_perm), offsets,
                              static_cast<const float*>(w1), static_cast<const float*>(w3),
                              static_cast<float*>(h), st);
  if (s.w_dtype == MOE_BF16)
    return launch_gate_up_bf16(s, static_cast<const uint16_t*>(x_perm), offsets,
                               static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3),
                               static_cast<uint16_t*>(h), st);
  if (s.w_dtype == MOE_MXFP4)
    return launch_gate_up_mxfp4(s, static_cast<const uint16_t*>(x_perm), offsets,
                                static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w1_scale),
                                static_cast<const uint8_t*>(w3), static_cast<const uint8_t*>(w3_scale),
                                static_cast<uint16_t*>(h), st);
  return launch_gate_up_fp8(s, static_cast<const uint8_t*>(x_perm), x_scale, offsets,
                            static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w3),
                            static_cast<const float*>(w1_scale), static_cast<const float*>(w3_scale),
                            static_cast<uint8_t*>(h), h_scale, st);
}

hipError_t launch_down(const moe_shape_t& s, const void* h, const uint8_t* h_scale,
                       const int32_t* offsets, const void* w2, const void* w2_scale,
                       float* y_perm, void* workspace, hipStream_t st) {
  if (s.w_dtype == MOE_F32)
    return launch_down_f32(s, static_cast<const float*>(h), offsets,
                           static_cast<const float*>(w2), y_perm, st);
  if (s.w_dtype == MOE_BF16)
    return launch_down_bf16(s, static_cast<const uint16_t*>(h), offsets,
                            static_cast<const uint16_t*>(w2), y_perm, workspace, st);
  if (s.w_dtype == MOE_MXFP4)
    return launch_down_mxfp4(s, static_cast<const uint16_t*>(h), offsets,
                             static_cast<const uint8_t*>(w2), static_cast<const uint8_t*>(w2_scale),
                             y_perm, st);
  return launch_down_fp8(s, static_cast<const uint8_t*>(h), h_scale, offsets,
                         static_cast<const uint8_t*>(w2), static_cast<const float*>(w2_scale), y_perm,
                         st);
}

}  // namespace moe

namespace {

using moe::launch_fill_u8;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_bytes(int32_t dt) { return dt == MOE_F32 ? 4 : 2; }

// Storage bytes of one element of x_perm / h.
size_t perm_elem_bytes(const moe_shape_t& s) {
  if (s.w_dtype == MOE_FP8_E4M3) return 1;
  return act_bytes(s.act_dtype);
}

moe_status_t validate_shape(const moe_shape_t* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->T > (1 << 24)) return MOE_ERR_INVALID_ARG;
  if (s->top_k < 1 || s->n_experts < 2 || s->top_k > s->n_experts) return MOE_ERR_INVALID_ARG;
  if (s->n_shared < 0) return MOE_ERR_INVALID_ARG;
  if (s->d_model <= 0 || s->d_ff <= 0) return MOE_ERR_INVALID_ARG;
  if (s->capacity < MOE_DROPLESS) return MOE_ERR_INVALID_ARG;
  if (s->overflow != MOE_OVERFLOW_DROP && s->overflow != MOE_OVERFLOW_NEXT_BEST)
    return MOE_ERR_INVALID_ARG;
  const bool known = (s->act_dtype == MOE_F32 || s->act_dtype == MOE_BF16) &&
                     (s->w_dtype == MOE_F32 || s->w_dtype == MOE_BF16 || s->w_dtype == MOE_FP8_E4M3 ||
                      s->w_dtype == MOE_MXFP4);
  if (!known) return MOE_ERR_INVALID_ARG;
  if (s->top_k > moe::kMaxTopK || s->n_experts > moe::kMaxExperts || s->n_shared > 1)
    return MOE_ERR_UNSUPPORTED;
  if (s->act_dtype == MOE_F32 && s->n_experts > moe::kMaxExpertsF32) return MOE_ERR_UNSUPPORTED;
  // the fallback round offers a dropped slot of a top-2 token to its 3rd/4th expert
  if (s->capacity >= 0 && s->overflow == MOE_OVERFLOW_NEXT_BEST && s->top_k != 2)
    return MOE_ERR_UNSUPPORTED;
  if (s->d_model % 64 != 0 || s->d_ff % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (s->d_model > (1 << 16) || s->d_ff > (1 << 18)) return MOE_ERR_UNSUPPORTED;
  const bool combo = (s->act_dtype == MOE_F32 && s->w_dtype == MOE_F32) ||
                     (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_BF16) ||
                     (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_FP8_E4M3) ||
                     (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_MXFP4);
  if (!combo) return MOE_ERR_UNSUPPORTED;
  // MXFP4: weight streaming in stages of 256 elements, for few rows per expert
  if (s->w_dtype == MOE_MXFP4 &&
      (s->d_model % 256 != 0 || s->d_ff % 256 != 0 ||
       moe::max_rows_per_expert(*s) > moe::kMxfp4MaxRows))
    return MOE_ERR_UNSUPPORTED;
  if (s->w_dtype == MOE_FP8_E4M3 && !moe::kFp8Available) return MOE_ERR_UNSUPPORTED;
  // fp8: one K slice of the matrix-core tile is 128 elements
  if (s->w_dtype == MOE_FP8_E4M3 && (s->d_model % 128 != 0 || s->d_ff % 128 != 0))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_ptrs(std::initializer_list<const void*> required,
                        std::initializer_list<const void*> optional) {
  for (const void* p : required) {
    if (p == nullptr) return MOE_ERR_INVALID_ARG;
    if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  }
  for (const void* p : optional)
    if (p != nullptr && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Workspace layout of moe_forward (each region 256-byte aligned).
struct ForwardLayout {
  size_t route_logits, route_part, ids, weights, next_ids, counts, offsets, perm_src, slot_to_row, drop, x_perm,
      x_scale, h, h_scale, y_perm, down_ws, total;
};

// The overflow fallback round runs (and needs the 3rd/4th-ranked experts).
bool fallback_on(const moe_shape_t& s) {
  return s.capacity >= 0 && s.overflow == MOE_OVERFLOW_NEXT_BEST;
}

// Workspace of moe_expert_gemm_down: partial tiles of the split tail work
// (bf16 many-rows path only).
size_t down_workspace_bytes(const moe_shape_t& s) {
  return s.w_dtype == MOE_BF16 ? moe::down_workspace_bytes_bf16(s) : 0;
}

ForwardLayout forward_layout(const moe_shape_t& s) {
  ForwardLayout L{};
  const size_t A = (size_t)s.T * s.top_k;                 // routed assignments
  const size_t R = (size_t)moe::total_slots(s);           // slots incl. the shared expert = max rows
  const size_t G = (size_t)moe::expert_groups(s);
  const size_t eb = perm_elem_bytes(s);
  const bool fp8 = s.w_dtype == MOE_FP8_E4M3;
  size_t o = 0;
  L.route_logits = o; o += align_up(moe::route_workspace_bytes(s));
  L.route_part = o;  o += moe::route_index_fused(s) ? align_up(moe::route_index_part_bytes()) : 0;
  L.ids = o;         o += align_up(A * 4);
  L.weights = o;     o += align_up(A * 4);
  L.next_ids = o;    o += fallback_on(s) ? align_up((size_t)s.T * 2 * 4) : 0;
  L.counts = o;      o += align_up(G * 4);
  L.offsets = o;     o += align_up((G + 1) * 4);
  L.perm_src = o;    o += align_up(R * 4);
  L.slot_to_row = o; o += align_up(R * 4);
  L.drop = o;        o += align_up(A);
  L.x_perm = o;      o += align_up(R * s.d_model * eb);
  L.x_scale = o;     o += fp8 ? align_up(R * (s.d_model / 32)) : 0;
  L.h = o;           o += align_up(R * s.d_ff * eb);
  L.h_scale = o;     o += fp8 ? align_up(R * (s.d_ff / 32)) : 0;
  L.y_perm = o;      o += align_up(R * s.d_model * 4);
  L.down_ws = o;     o += align_up(down_workspace_bytes(s));
  L.total = o;
  return L;
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off); }

moe_status_t forward_impl(const moe_shape_t* s, const void* x, const void* w_gate,
                          const float* router_bias, const void* w1, const void* w3, const void* w2,
                          const void* w1_scale, const void* w3_scale, const void* w2_scale,
                          void* y, int32_t* topk_ids_out, float* topk_weights_out,
                          int32_t* expert_counts_out, uint8_t* drop_mask_out, float* logits_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  if (s->T == 0) return MOE_OK;
  if ((v = check_ptrs({x, w_gate, w1, w3, w2, y},
                      {router_bias, topk_ids_out, topk_weights_out, expert_counts_out,
                       drop_mask_out, logits_out, w1_scale, w3_scale, w2_scale})) != MOE_OK)
    return v;
  const bool fp8 = s->w_dtype == MOE_FP8_E4M3;
  const bool scaled = fp8 || s->w_dtype == MOE_MXFP4;
  if (scaled && (w1_scale == nullptr || w3_scale == nullptr || w2_scale == nullptr))
    return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(*s);
  if (workspace == nullptr || workspace_bytes < L.total || !aligned16(workspace))
    return MOE_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(workspace, L.ids);
  float* gw = topk_weights_out ? topk_weights_out : at<float>(workspace, L.weights);
  int32_t* counts = expert_counts_out ? expert_counts_out : at<int32_t>(workspace, L.counts);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* perm_src = at<int32_t>(workspace, L.perm_src);
  int32_t* slot_to_row = at<int32_t>(workspace, L.slot_to_row);
  uint8_t* drop = drop_mask_out ? drop_mask_out : at<uint8_t>(workspace, L.drop);
  void* x_perm = at<void>(workspace, L.x_perm);
  uint8_t* x_scale = fp8 ? at<uint8_t>(workspace, L.x_scale) : nullptr;
  void* h = at<void>(workspace, L.h);
  uint8_t* h_scale = fp8 ? at<uint8_t>(workspace, L.h_scale) : nullptr;
  float* y_perm = at<float>(workspace, L.y_perm);
  int32_t* next = fallback_on(*s) ? at<int32_t>(workspace, L.next_ids) : nullptr;

  hipError_t e = hipSuccess;
  if (moe::route_index_fused(*s) && (s->w_dtype == MOE_BF16 || s->w_dtype == MOE_MXFP4)) {
    // decode: router partial sums over eight workgroups, then selection + grouping in
    // one; gate/up reads x through perm_src
    e = moe::launch_route_index(*s, x, w_gate, router_bias, ids, gw, logits_out, counts, offsets, perm_src,
                                slot_to_row, at<void>(workspace, L.route_part), st);
    if (e == hipSuccess && drop_mask_out != nullptr)
      e = launch_fill_u8(drop_mask_out, (int64_t)s->T * s->top_k, 0, st);
    if (e == hipSuccess && s->w_dtype == MOE_BF16)
      e = moe::launch_gate_up_bf16_gather(*s, static_cast<const uint16_t*>(x), perm_src, offsets,
                                          static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3),
                                          static_cast<uint16_t*>(h), st);
    if (e == hipSuccess && s->w_dtype == MOE_MXFP4)
      e = moe::launch_gate_up_mxfp4_gather(*s, static_cast<const uint16_t*>(x), perm_src, offsets,
                                           static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w1_scale),
                                           static_cast<const uint8_t*>(w3), static_cast<const uint8_t*>(w3_scale),
                                           static_cast<uint16_t*>(h), st);
  } else {
    e = moe::launch_route_topk(*s, x, w_gate, router_bias, ids, gw, logits_out, next,
                               at<void>(workspace, L.route_logits), st);
    const uint8_t* drop_in = nullptr;
    if (e == hipSuccess) {
      if (s->capacity >= 0) {
        e = moe::launch_capacity_select(*s, ids, gw, next, drop, st);
        drop_in = drop;
      } else if (drop_mask_out != nullptr) {
        e = launch_fill_u8(drop_mask_out, (int64_t)s->T * s->top_k, 0, st);
      }
    }
    if (e == hipSuccess)
      e = moe::launch_permute_index(*s, ids, drop_in, next, counts, offsets, perm_src, slot_to_row, st);
    if (moe::gate_up_bf16_gathers(*s)) {
      // many small experts: gate/up reads the token rows of x through perm_src (no x_perm)
      if (e == hipSuccess)
        e = moe::launch_gate_up_bf16_prefill_gather(*s, static_cast<const uint16_t*>(x), perm_src, offsets,
                                                    static_cast<const uint16_t*>(w1),
                                                    static_cast<const uint16_t*>(w3), static_cast<uint16_t*>(h), st);
    } else if (moe::gate_up_decode_gathers(*s)) {
      // weight streaming (e.g. many experts, a shared expert, a capacity): the same, no x_perm
      if (e == hipSuccess && s->w_dtype == MOE_BF16)
        e = moe::launch_gate_up_bf16_gather(*s, static_cast<const uint16_t*>(x), perm_src, offsets,
                                            static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3),
                                            static_cast<uint16_t*>(h), st);
      if (e == hipSuccess && s->w_dtype == MOE_MXFP4)
        e = moe::launch_gate_up_mxfp4_gather(*s, static_cast<const uint16_t*>(x), perm_src, offsets,
                                             static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w1_scale),
                                             static_cast<const uint8_t*>(w3), static_cast<const uint8_t*>(w3_scale),
                                             static_cast<uint16_t*>(h), st);
    } else {
      if (e == hipSuccess) e = moe::launch_permute_scatter(*s, x, offsets, perm_src, x_perm, x_scale, st);
      if (e == hipSuccess)
        e = moe::launch_gate_up(*s, x_perm, x_scale, offsets, w1, w3, w1_scale, w3_scale, h, h_scale, st);
    }
  }
  if (moe::route_index_fused(*s) && moe::down_combine_fused(*s)) {
    // decode, bf16 experts: down + combine in one launch (no y_perm)
    if (e == hipSuccess)
      e = moe::launch_down_combine_bf16(*s, static_cast<const uint16_t*>(h), offsets,
                                        static_cast<const uint16_t*>(w2), slot_to_row, gw,
                                        static_cast<uint16_t*>(y), st);
    return from_hip(e);
  }
  void* down_ws = down_workspace_bytes(*s) > 0 ? at<void>(workspace, L.down_ws) : nullptr;
  if (e == hipSuccess)
    e = moe::launch_down(*s, h, h_scale, offsets, w2, w2_scale, y_perm, down_ws, st);
  if (e == hipSuccess) e = moe::launch_combine(*s, y_perm, slot_to_row, gw, y, st);
  return from_hip(e);
}


// Device scratch of moe_forward_noalloc: the intermediates of one layer call
// live here instead of in a caller workspace.  Every GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` is only
// a host-side stand-in: kernels get the per-device address that
// hipGetSymbolAddress returns (scratch_address below), never the name.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

// Address of device `dev`'s copy of `scratch` (dev must be the current
// device); looked up once per device, on the first call there.
hipError_t scratch_address(int dev, void** out) {
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p == nullptr) e = hipErrorInvalidSymbol;
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_version(void) { return "moe-mi355x 0.1 gfx950"; }

moe_status_t moe_workspace_bytes(const moe_shape_t* s, moe_call_t call, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  switch (call) {
    case MOE_CALL_PERMUTE: *bytes = 0; return MOE_OK;
    case MOE_CALL_GATE_UP: *bytes = 0; return MOE_OK;
    case MOE_CALL_DOWN: *bytes = down_workspace_bytes(*s); return MOE_OK;
    case MOE_CALL_FORWARD: *bytes = forward_layout(*s).total; return MOE_OK;
    case MOE_CALL_ROUTE: *bytes = moe::route_workspace_bytes(*s); return MOE_OK;
  }
  return MOE_ERR_INVALID_ARG;
}

moe_status_t moe_route_topk(const moe_shape_t* s, const void* x, const void* w_gate,
                            const float* router_bias, int32_t* topk_ids, float* topk_weights,
                            float* logits, int32_t* next_ids, void* workspace,
                            size_t workspace_bytes, void* stream) {
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  if (s->T == 0) return MOE_OK;
  if ((v = check_ptrs({x, w_gate, topk_ids, topk_weights}, {router_bias, logits, next_ids})) != MOE_OK)
    return v;
  const size_t need = moe::route_workspace_bytes(*s);
  if (need > 0 && logits == nullptr &&
      (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_route_topk(*s, x, w_gate, router_bias, topk_ids, topk_weights, logits,
                                         next_ids, need > 0 ? workspace : nullptr,
                                         static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute(const moe_shape_t* s, const int32_t* topk_ids, const float* topk_weights,
                         const int32_t* next_ids, const void* x, int32_t* expert_counts,
                         int32_t* expert_offsets,
                         int32_t* perm_src, int32_t* slot_to_row, uint8_t* drop_mask,
                         void* x_perm, uint8_t* x_perm_scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  if (s->T == 0) return MOE_OK;
  if ((v = check_ptrs({topk_ids, topk_weights, x, expert_counts, expert_offsets, perm_src,
                       slot_to_row, x_perm},
                      {drop_mask, next_ids})) != MOE_OK)
    return v;
  const bool fp8 = s->w_dtype == MOE_FP8_E4M3;
  if (fp8 && x_perm_scale == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->capacity >= 0 && drop_mask == nullptr) return MOE_ERR_INVALID_ARG;
  if (fallback_on(*s) && next_ids == nullptr) return MOE_ERR_INVALID_ARG;
  const int32_t* next = fallback_on(*s) ? next_ids : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  const uint8_t* drop_in = nullptr;
  if (s->capacity >= 0) {
    e = moe::launch_capacity_select(*s, topk_ids, topk_weights, next, drop_mask, st);
    drop_in = drop_mask;
  } else if (drop_mask != nullptr) {
    e = launch_fill_u8(drop_mask, (int64_t)s->T * s->top_k, 0, st);
  }
  if (e == hipSuccess)
    e = moe::launch_permute_index(*s, topk_ids, drop_in, next, expert_counts, expert_offsets,
                                  perm_src, slot_to_row, st);
  if (e == hipSuccess)
    e = moe::launch_permute_scatter(*s, x, expert_offsets, perm_src, x_perm, x_perm_scale, st);
  return from_hip(e);
}

moe_status_t moe_expert_gemm_gate_up(const moe_shape_t* s, const void* x_perm,
                                     const uint8_t* x_perm_scale, const int32_t* expert_offsets,
                                     const void* w1, const void* w3, const void* w1_scale,
                                     const void* w3_scale, void* h, uint8_t* h_scale,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  if (s->T == 0) return MOE_OK;
  if ((v = check_ptrs({x_perm, expert_offsets, w1, w3, h}, {w1_scale, w3_scale})) != MOE_OK) return v;
  if (s->w_dtype == MOE_FP8_E4M3 &&
      (x_perm_scale == nullptr || w1_scale == nullptr || w3_scale == nullptr || h_scale == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (s->w_dtype == MOE_MXFP4 && (w1_scale == nullptr || w3_scale == nullptr))
    return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_gate_up(*s, x_perm, x_perm_scale, expert_offsets, w1, w3, w1_scale,
                                      w3_scale, h, h_scale, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_gemm_down(const moe_shape_t* s, const void* h, const uint8_t* h_scale,
                                  const int32_t* expert_offsets, const void* w2,
                                  const void* w2_scale, float* y_perm, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  if (s->T == 0) return MOE_OK;
  if ((v = check_ptrs({h, expert_offsets, w2, y_perm}, {w2_scale})) != MOE_OK) return v;
  if (s->w_dtype == MOE_FP8_E4M3 && (h_scale == nullptr || w2_scale == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (s->w_dtype == MOE_MXFP4 && w2_scale == nullptr) return MOE_ERR_INVALID_ARG;
  const size_t need = down_workspace_bytes(*s);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_down(*s, h, h_scale, expert_offsets, w2, w2_scale, y_perm,
                                   need > 0 ? workspace : nullptr, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const moe_shape_t* s, const float* y_perm, const int32_t* slot_to_row,
                         const float* topk_weights, void* y, void* stream) {
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  if (s->T == 0) return MOE_OK;
  if ((v = check_ptrs({y_perm, slot_to_row, topk_weights, y}, {})) != MOE_OK) return v;
  return from_hip(moe::launch_combine(*s, y_perm, slot_to_row, topk_weights, y,
                                      static_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward(const moe_shape_t* s, const void* x, const void* w_gate,
                         const float* router_bias, const void* w1, const void* w3, const void* w2,
                         const void* w1_scale, const void* w3_scale, const void* w2_scale,
                         void* y, int32_t* topk_ids_out, float* topk_weights_out,
                         int32_t* expert_counts_out, uint8_t* drop_mask_out, float* logits_out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(s, x, w_gate, router_bias, w1, w3, w2, w1_scale, w3_scale, w2_scale, y,
                      topk_ids_out, topk_weights_out, expert_counts_out, drop_mask_out, logits_out,
                      workspace, workspace_bytes, stream);
}

moe_status_t moe_forward_noalloc(const moe_shape_t* s, const void* x, const void* w_gate,
                                 const float* router_bias, const void* w1, const void* w3,
                                 const void* w2, const void* w1_scale, const void* w3_scale,
                                 const void* w2_scale, void* y, int32_t* topk_ids_out,
                                 float* topk_weights_out, int32_t* expert_counts_out,
                                 uint8_t* drop_mask_out, float* logits_out, void* stream) {
  moe_status_t v = validate_shape(s);
  if (v != MOE_OK) return v;
  if (s->T == 0) return MOE_OK;
  // the shape's intermediates must fit the library's scratch array
  if (forward_layout(*s).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (st != nullptr) {
    int stream_dev = -1;
    if (hipStreamGetDevice(st, &stream_dev) != hipSuccess || stream_dev != dev)
      return MOE_ERR_INVALID_ARG;   // the scratch address belongs to the current device
  }
  void* ws = nullptr;
  if (scratch_address(dev, &ws) != hipSuccess) return MOE_ERR_HIP;
  return forward_impl(s, x, w_gate, router_bias, w1, w3, w2, w1_scale, w3_scale, w2_scale, y,
                      topk_ids_out, topk_weights_out, expert_counts_out, drop_mask_out, logits_out,
                      ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

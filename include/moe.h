/*
 * moe.h -- C ABI of a sparse top-k Mixture-of-Experts feed-forward layer
 * (Mixtral 8x7B style top-2, and the fine-grained many-expert form with a
 * shared expert) implemented with hand-written HIP kernels for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (pages: "Mixtral and Mixture-of-Experts, Explained", section
 * "How it works"; "Mixtral" study notes, section "MoE Layer"):
 *   logits  = x . W_g^T (+ b)                 router, one logit per expert
 *   G(x)    = Softmax(TopK(logits)), k = 2     non-selected logits at -inf
 *   y       = sum_i G(x)_i * Expert_i(x)
 *   Expert  = w2( silu(x w1^T) * (x w3^T) )    SwiGLU, no biases
 * General form ("Mixtral 8x7B" interview page, section on how MoE design
 * changed since Mixtral: DeepSeek-V3 routes each token to 8 of 256 experts
 * and sends every token through one shared expert as well):
 *   top_k = k in 1..8 of up to 256 routed experts, G = softmax over the k
 *   kept logits, and with n_shared = 1
 *   y      += Expert_E(x)                      shared expert, weight 1
 *   (weights of the shared expert are stored as expert index E, after the
 *   routed ones; it takes every token and no capacity limit applies to it).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are DEVICE pointers to row-major arrays owned by
 *   the caller, each 16-byte aligned (as allocator-returned memory is; a
 *   misaligned one returns MOE_ERR_INVALID_ARG): the kernels' vector loads
 *   and stores stay aligned from there under the shape limits below.  The
 *   library allocates no memory, keeps no mutable global state and is
 *   re-entrant; calls on different streams may overlap.  The one
 *   exception is moe_forward_noalloc (below), which uses a device array of the
 *   library's own and remembers its address per device.
 * - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *   stream).  Every call only enqueues work on it and returns without
 *   waiting for the device; no call reads device memory on the host.
 * - Host-side validation happens before anything is enqueued.  On any
 *   error nothing is enqueued and a status other than MOE_OK is returned;
 *   MOE_ERR_HIP means a launch failed (its HIP error is consumed).
 * - Device contents are not validated.  Preconditions: x, W_g, weights and
 *   scales finite; ids written by moe_route_topk (or equivalent) in [0, E).
 * - T = 0 is legal: every call returns MOE_OK and enqueues nothing.
 * - Expert ids count from 0.  A token's slots follow its logits in
 *   descending order (slot 0 the largest); equal logits go to the lower
 *   expert index.
 * - Assignment ("slot") (t, s) of token t has index t*k + s, s < k.  With a
 *   shared expert the T extra assignments (t, shared) have indices
 *   T*k + t.  S = n_shared, R = T*(k + S) is the number of slots.
 * - Rows of the permuted buffers are grouped by expert (routed experts
 *   0..E-1, then the shared expert E); inside an expert they follow
 *   ascending token index (a token has at most one row per expert).
 *   Buffers indexed by row are sized for R rows, the most any call can
 *   produce, so one set of buffers serves dropless and capacity modes.
 *
 * dtypes (moe_shape_t.act_dtype / w_dtype):
 *   act F32  + w F32       : x, W_g, y fp32; x_perm fp32; h fp32.
 *   act BF16 + w BF16      : x, W_g, y bf16; x_perm bf16; h bf16; fp32 accumulate.
 *   act BF16 + w FP8_E4M3  : x, W_g, y bf16; expert weights are OCP e4m3 codes
 *                            with one fp32 scale per output channel (row of the
 *                            [out, in] weight).  Activations are quantised for
 *                            the fp8 matrix cores: x_perm and h are e4m3 codes
 *                            with one power-of-two scale per row and per block
 *                            of 32 consecutive elements, stored as an E8M0
 *                            byte (scale = 2^(byte - 127)); the block exponent
 *                            is ceil(log2(fp32(amax / 448))), 127 for a zero
 *                            block.  fp32 accumulate.
 *   act BF16 + w MXFP4     : x, W_g, y bf16; x_perm bf16; h bf16.  Expert weights
 *                            are OCP Microscaling FP4: E2M1 codes, two per byte
 *                            (even element in the low nibble), [E+S, F, d/2] /
 *                            [E+S, d, F/2] bytes, with one E8M0 scale byte
 *                            (2^(byte - 127)) per row and block of 32
 *                            consecutive input elements, [E+S, F, d/32] /
 *                            [E+S, d, F/32] bytes.  The matrix cores see the
 *                            exact dequantised weights in bf16; fp32
 *                            accumulate.  A weight-streaming (decode) format:
 *                            at most 64 rows per expert (T <= 64, or capacity
 *                            <= 64 without a shared expert), d_model and d_ff
 *                            multiples of 256.
 *   Other combinations return MOE_ERR_UNSUPPORTED.
 *
 * Shape limits: 1 <= top_k <= 8 (top_k <= n_experts); 2 <= n_experts <= 256
 * (fp32 activations: <= 64); n_shared 0 or 1; d_model and d_ff multiples
 * of 64; 1 <= T <= 2^24 (or 0); capacity == MOE_DROPLESS or >= 0;
 * MOE_OVERFLOW_NEXT_BEST with a capacity needs top_k == 2.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* NULL required pointer, pointer not 16-byte aligned, bad shape value */
  MOE_ERR_UNSUPPORTED = 2,   /* legal but not implemented: shape limit, dtype combo */
  MOE_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4            /* a kernel launch failed */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3 } moe_dtype_t;

#define MOE_DROPLESS (-1)

/* What happens to an assignment the capacity limit drops (moe_shape_t.overflow).
 * Pages: "How Mixtral 8x7B uses mixture of experts", section "Routing without
 * auxiliary loss": tokens over an expert's capacity are dropped there and
 * handed to a fallback, most often the token's next-best expert.
 *   MOE_OVERFLOW_DROP       it contributes nothing.
 *   MOE_OVERFLOW_NEXT_BEST  one fallback round: a dropped slot is offered to the
 *     token's best expert outside its top-2 (3rd-ranked by logit; when both
 *     slots of the token were dropped, slot 0 to the 3rd- and slot 1 to the
 *     4th-ranked), keeping its gate weight.  Each expert takes the offers into
 *     the slots the capacity round left free (capacity minus what it kept),
 *     ranked like the capacity round (gate weight descending, then token
 *     ascending); the other offers stay dropped.  The ranking ties to the
 *     lower expert index, like the top-2.  Defined for top_k == 2 only. */
#define MOE_OVERFLOW_DROP 0
#define MOE_OVERFLOW_NEXT_BEST 1

typedef struct {
  int32_t T;          /* tokens (batch * seq_len, flattened) */
  int32_t d_model;    /* hidden size d */
  int32_t d_ff;       /* expert FFN width F */
  int32_t n_experts;  /* E routed experts */
  int32_t top_k;      /* k, 1..8 */
  int32_t capacity;   /* MOE_DROPLESS, or slots per expert (0 drops every assignment) */
  int32_t act_dtype;  /* moe_dtype_t of x, W_g, y */
  int32_t w_dtype;    /* moe_dtype_t of w1, w3, w2 */
  int32_t overflow;   /* MOE_OVERFLOW_DROP or MOE_OVERFLOW_NEXT_BEST (ignored when dropless) */
  int32_t n_shared;   /* S: 0, or 1 shared expert (weights at expert index E) */
} moe_shape_t;

/* Which call a workspace is sized for. */
typedef enum { MOE_CALL_PERMUTE = 0, MOE_CALL_GATE_UP = 1, MOE_CALL_DOWN = 2,
               MOE_CALL_FORWARD = 3, MOE_CALL_ROUTE = 4 } moe_call_t;

/* Human-readable name of a status.  Never NULL. */
const char* moe_status_string(moe_status_t status);

/* Library version string, e.g. "moe-mi355x 0.1 gfx950". */
const char* moe_version(void);

/* Bytes of device workspace `call` needs for `shape` (0 is possible; a
 * NULL workspace is accepted then).  Host-only.  Workspace contents need
 * not be initialised and are garbage after the call.  Errors: NULL
 * argument or invalid shape. */
moe_status_t moe_workspace_bytes(const moe_shape_t* shape, moe_call_t call, size_t* bytes);

/* Router + top-k + gate weights.
 * Pages: "Mixtral" study notes, MixtralMoE.forward (gate, topk, softmax over
 * the kept logits); "Mixtral and Mixture-of-Experts, Explained", gate
 * equation G(x) = Softmax(TopK(x . W_g)).
 *   x            [T, d]   act dtype
 *   w_gate       [E, d]   act dtype (nn.Linear [out, in] layout)
 *   router_bias  [E] fp32 or NULL, added to the fp32 logits after the dot product
 *   topk_ids     [T, k] int32 out: the k largest logits in descending order,
 *                ties -> lower index
 *   topk_weights [T, k] fp32 out.  k == 2: w0 = 1/(1+exp(l1-l0)), w1 = 1-w0
 *                (w0+w1 == 1 exactly).  Otherwise w_j = exp(l_j - l_0) / sum_i
 *                exp(l_i - l_0) over the kept logits (k == 1: w0 = 1).
 *   logits       [T, E] fp32 out, or NULL
 *   next_ids     [T, 2] int32 out, or NULL: the experts ranked k+1 and k+2 of
 *                each token (same order: logit descending, ties -> lower index),
 *                -1 where n_experts is too small.  moe_permute needs them for
 *                MOE_OVERFLOW_NEXT_BEST.
 * Logits accumulate in fp32.
 * Workspace: moe_workspace_bytes(MOE_CALL_ROUTE) bytes, 16-byte aligned: T*E*4
 * (an fp32 logit buffer) for bf16 shapes with more than 64 experts, whose
 * router runs as a logits kernel over a token x expert grid followed by a
 * selection kernel; 0 otherwise.  When `logits` is given it serves as that
 * buffer and the workspace may be NULL.  Too small or NULL when needed ->
 * MOE_ERR_WORKSPACE. */
moe_status_t moe_route_topk(const moe_shape_t* shape, const void* x, const void* w_gate,
                            const float* router_bias, int32_t* topk_ids, float* topk_weights,
                            float* logits, int32_t* next_ids, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Capacity selection (when shape->capacity >= 0) and grouping of tokens by expert.
 * Pages: "How Mixtral 8x7B uses mixture of experts", sections "Routing without
 * auxiliary loss" (capacity-limited dispatch, excess dropped) and the
 * bincount of the top-2 ids (expert activation listing); the simplified
 * forward pass, which batches each expert's tokens and writes results back in
 * token order.
 *   topk_ids, topk_weights [T, k] from moe_route_topk
 *   next_ids       [T, 2] from moe_route_topk; required with a capacity and
 *                  MOE_OVERFLOW_NEXT_BEST, else ignored (may be NULL)
 *   x              [T, d] act dtype
 *   expert_counts  [E+S] int32 out: kept assignments per expert (shared: T)
 *   expert_offsets [E+S+1] int32 out: exclusive prefix sum of counts
 *   perm_src       [R] int32 out: rows 0..offsets[E+S]-1 hold the slot index
 *                  (t*k+s, or T*k+t for the shared expert) of each row
 *   slot_to_row    [R] int32 out: row of each slot, -1 if dropped
 *   drop_mask      [T*k] uint8 out or NULL: 0 = kept by its top-k expert,
 *                  1 = dropped, 2 = kept by its fallback expert (NEXT_BEST)
 *   x_perm         [R, d] out: x_perm[row] = x[token of perm_src[row]]; fp8 configs:
 *                  e4m3 codes [R, d] plus x_perm_scale [R, d/32] E8M0 bytes
 *   x_perm_scale   fp8 configs only (else ignored; may be NULL)
 * Capacity rule: per expert, assignments ranked by gate weight (descending,
 * compared as fp32), ties to the lower token index; the first `capacity`
 * are kept.  A dropped assignment contributes nothing and the token's other
 * slots are not renormalised; with MOE_OVERFLOW_NEXT_BEST the fallback round
 * above runs next and the rows of each expert include the slots it took
 * (still one row per token and expert, in ascending token order).
 * Workspace: moe_workspace_bytes(MOE_CALL_PERMUTE). */
moe_status_t moe_permute(const moe_shape_t* shape, const int32_t* topk_ids,
                         const float* topk_weights, const int32_t* next_ids, const void* x,
                         int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* perm_src, int32_t* slot_to_row,
                         uint8_t* drop_mask, void* x_perm, uint8_t* x_perm_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Grouped expert gate/up projection with the SwiGLU product fused in:
 * h[row] = silu(x_perm[row] . w1[e]^T) * (x_perm[row] . w3[e]^T) for every row of
 * expert e (rows offsets[e] .. offsets[e+1]-1).
 * Pages: "Mixtral" study notes, MixtralExpert.forward and "SwiGLU Experts".
 *   x_perm, x_perm_scale as written by moe_permute
 *   expert_offsets [E+S+1] int32 (device)
 *   w1, w3         [E+S, F, d] weight dtype (MXFP4: [E+S, F, d/2] bytes); w1_scale,
 *                  w3_scale: fp8 [E+S, F] fp32, MXFP4 [E+S, F, d/32] E8M0 bytes, else unused
 *   h              [R, F] out (bf16 / fp32 / e4m3 codes); h_scale [R, F/32] E8M0 (fp8 only)
 * Workspace: moe_workspace_bytes(MOE_CALL_GATE_UP). */
moe_status_t moe_expert_gemm_gate_up(const moe_shape_t* shape, const void* x_perm,
                                     const uint8_t* x_perm_scale, const int32_t* expert_offsets,
                                     const void* w1, const void* w3, const void* w1_scale,
                                     const void* w3_scale, void* h, uint8_t* h_scale,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Grouped expert down projection: y_perm[row] = h[row] . w2[e]^T (fp32 out).
 * Pages: "Mixtral" study notes, MixtralExpert.forward (self.w2).
 *   h, h_scale     as written by moe_expert_gemm_gate_up
 *   expert_offsets [E+S+1] int32
 *   w2             [E+S, d, F] weight dtype (MXFP4: [E+S, d, F/2] bytes); w2_scale: fp8
 *                  [E+S, d] fp32, MXFP4 [E+S, d, F/32] E8M0 bytes, else unused
 *   y_perm         [R, d] fp32 out
 * Workspace: moe_workspace_bytes(MOE_CALL_DOWN) bytes, 16-byte aligned, device
 * memory owned by the caller (0 for shapes that need none; then it may be
 * NULL).  bf16 shapes with more than 64 rows per expert use it for fp32
 * partial tiles: the tiles left over after the last full round of the
 * persistent launch are split along K across workgroups and summed by a
 * second kernel in K order, so results do not depend on timing.  Its
 * contents need no initialisation and are garbage afterwards.  Too small or
 * NULL when needed -> MOE_ERR_WORKSPACE.  Two calls that share a workspace
 * must not run concurrently. */
moe_status_t moe_expert_gemm_down(const moe_shape_t* shape, const void* h, const uint8_t* h_scale,
                                  const int32_t* expert_offsets, const void* w2,
                                  const void* w2_scale, float* y_perm, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Gate-weighted combine back to token order:
 * y[t] = sum over kept slots s of topk_weights[t, s] * y_perm[slot_to_row[t*k+s]]
 *        (+ y_perm[slot_to_row[T*k+t]] with a shared expert),
 * 0 when every slot is dropped and there is no shared expert; accumulated in
 * fp32 in slot order (shared last), cast to the act dtype (round to nearest even).
 * Pages: "Mixtral and Mixture-of-Experts, Explained", y = sum_i G(x)_i Expert_i(x);
 * study notes, an all-zero output of x's shape, then weighted accumulation.
 *   y_perm [R, d] fp32; slot_to_row [R] int32; topk_weights [T, k] fp32
 *   y      [T, d] act dtype out.  No workspace. */
moe_status_t moe_combine(const moe_shape_t* shape, const float* y_perm, const int32_t* slot_to_row,
                         const float* topk_weights, void* y, void* stream);

/* The whole layer on one stream, with no host synchronisation:
 * route -> (capacity) -> permute -> gate/up -> down -> combine.
 *   x [T, d], w_gate [E, d] act dtype; router_bias [E] fp32 or NULL
 *   w1, w3 [E+S, F, d], w2 [E+S, d, F] weight dtype; w*_scale as for the two GEMM calls
 *   (fp8: fp32 per output channel; MXFP4: E8M0 bytes per 32-element block)
 *   y [T, d] act dtype out
 *   optional outputs (NULL to skip): topk_ids_out [T, k] int32, topk_weights_out [T, k]
 *   fp32, expert_counts_out [E+S] int32, drop_mask_out [T*k] uint8 (0 / 1 / 2 as in
 *   moe_permute), logits_out [T, E] fp32
 * topk_ids_out are the router's choices; with MOE_OVERFLOW_NEXT_BEST a slot
 * whose drop mask is 2 was processed by its fallback expert instead.
 * Results equal the five calls above made in order, bit for bit.  Fewer
 * kernels run where they can: with bf16 activations and bf16 or MXFP4 experts,
 * gate/up reads the token rows of x through perm_src instead of a permuted
 * copy when at most 64 rows reach any expert, and (bf16 experts) when the
 * routed experts average at most 320 rows; for decode batches (T <= 16,
 * E <= 16, top-2, dropless, no shared expert) the router's product runs on
 * eight workgroups and a ninth selects and also groups the tokens, and with
 * bf16 experts the down projection and the combine are one kernel (no
 * y_perm).
 * Workspace: moe_workspace_bytes(MOE_CALL_FORWARD) holds every intermediate. */
moe_status_t moe_forward(const moe_shape_t* shape, const void* x, const void* w_gate,
                         const float* router_bias, const void* w1, const void* w3, const void* w2,
                         const void* w1_scale, const void* w3_scale, const void* w2_scale,
                         void* y, int32_t* topk_ids_out, float* topk_weights_out,
                         int32_t* expert_counts_out, uint8_t* drop_mask_out, float* logits_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device scratch array behind moe_forward_noalloc (64 MiB per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results (bit for bit) and errors as moe_forward, without the
 * workspace: the intermediates live in a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends.  This call allocates nothing and calls no
 * allocating routine.
 *   Limit: a shape whose moe_workspace_bytes(shape, MOE_CALL_FORWARD) exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE with nothing enqueued.
 *   That admits the weight-streaming (decode) shapes: at d_model 4096, d_ff
 *   14336, top-2 bf16 a token needs about 106 KiB (T <= 64 there: larger
 *   batches take the tiled path, whose split-tail buffer alone is larger).
 *   Device: `stream` must belong to the current device (else
 *   MOE_ERR_INVALID_ARG); the first call on a device looks up that device's
 *   address of the array (MOE_ERR_HIP if that fails; at most 64 devices).
 *   Concurrency: all calls on one GPU share its array, which keeps the last
 *   call's contents; calls that overlap on one GPU (other streams or threads)
 *   race on it and must be serialised by the caller.  No kernel of the layer
 *   reads scratch it has not written in the same call, so nothing needs
 *   clearing between calls. */
moe_status_t moe_forward_noalloc(const moe_shape_t* shape, const void* x, const void* w_gate,
                                 const float* router_bias, const void* w1, const void* w3,
                                 const void* w2, const void* w1_scale, const void* w3_scale,
                                 const void* w2_scale, void* y, int32_t* topk_ids_out,
                                 float* topk_weights_out, int32_t* expert_counts_out,
                                 uint8_t* drop_mask_out, float* logits_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

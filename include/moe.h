/*
 * moe.h — C ABI of the routed mixture-of-experts expert computation on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (kernelindex.com operation pages):
 *   "Sparse expert dispatch and combine" (description): tokens routed to an
 *     expert are extracted, pass through a gate_up projection, a gated GLU
 *     with clamping and a down projection, and are accumulated back into the
 *     output rows of their tokens.
 *   "MoE training token repeat and expert computation" (description): every
 *     token is repeated once per chosen expert, each expert selects its rows,
 *     runs a SwiGLU FFN, and the routing weights scale the expert outputs
 *     before the sum over the chosen experts.
 *   "MoE expert parallel execution backward" (description): gradients with
 *     respect to hidden_states, topk_weights and the gate, up and down weights.
 *
 * Notation: T tokens, H hidden size, I intermediate size, E experts, K experts
 * per token (the workload lines' hidden_size, intermediate_size,
 * num_local_experts / num_experts / n_routed_experts, num_experts_per_tok).
 * S = T*K slots; slot s = t*K + k is the k-th copy of token t.
 *
 *   out[t] = sum_k w[t,k] * Wd[e] . phi(Wgu[e] . x_t),   e = ids[t,k]
 *
 * phi splits the 2I gate_up outputs into gate g and up u (layout flag) and is
 *   MOE_SWIGLU:      g * sigmoid(g) * u
 *   MOE_CLAMPED_GLU: gc = min(g, L), uc = clamp(u, -L, L),
 *                    (uc + 1) * gc * sigmoid(alpha * gc)     (L = clamp_limit)
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, row-major, contiguous, 16-byte
 *     aligned.  hidden/out/d_out/d_hidden [T,H]; w_gate_up/d_w_gate_up
 *     [E,2I,H]; w_gate/w_up/d_w_gate/d_w_up [E,I,H]; w_down/d_w_down
 *     [E,H,I]; topk_ids int32 [T,K]; topk_weights/d_topk_weights fp32 [T,K];
 *     router logits/d_logits fp32 [T,E].  Activations, weights and
 *     d_hidden have the descriptor's dtype (bf16 or fp32); the weight
 *     gradients have its grad_dtype.
 *   - The caller owns every buffer.  The library never allocates device
 *     memory, never frees, and keeps no pointer after a call returns.
 *   - Outputs are fully overwritten (never accumulated).
 *   - Calls are asynchronous on `stream` and never synchronise the host,
 *     except moe_check_device_status.  Calls are re-entrant given distinct
 *     workspaces; two calls sharing one workspace must be stream-ordered.
 *   - Host-checkable errors are reported before any launch, with nothing
 *     written: MOE_ERR_INVALID_ARG (null pointer where one is required,
 *     T<0, K<1, E<1, H<1, I<1, bad enum, misaligned pointer),
 *     MOE_ERR_UNSUPPORTED (H or I not a multiple of 8, E > 1024, K > 64,
 *     S >= 2^31), MOE_ERR_WORKSPACE (ws_bytes below the required size).
 *     A failed kernel launch returns MOE_ERR_HIP.
 *   - An expert id outside [0,E) is found on the device and its slot is
 *     dropped: out, d_hidden and the weight gradients are those of the same
 *     call with that slot's routing weight set to zero, its d_topk_weights
 *     entry is 0, and routing places it after every valid slot (inv_pos -1).
 *     A count is kept in the workspace and moe_check_device_status reports
 *     MOE_ERR_BAD_EXPERT_ID.  No memory outside the caller's buffers is
 *     touched for such an id.
 *   - T = 0 is valid: nothing is launched for the activations; the forward
 *     and backward entry points and moe_router clear the workspace status
 *     word (so moe_check_device_status reports MOE_OK for the call), and the
 *     backward entry points write zero weight gradients.
 *   - Entry points that take router logits or separate gate/up tensors
 *     (moe_router, moe_fwd_logits, moe_router_bwd, moe_fwd_sep, moe_bwd_sep)
 *     follow the same conventions; their own comments give the shapes.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4,
  MOE_ERR_BAD_EXPERT_ID = 5
} moe_status_t;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype_t;
typedef enum { MOE_SWIGLU = 0, MOE_CLAMPED_GLU = 1 } moe_act_t;
/* CONCAT: rows [0,I) of w_gate_up[e] are the gate, rows [I,2I) the up
 * projection.  INTERLEAVED: row 2j is gate column j, row 2j+1 up column j. */
typedef enum { MOE_GU_CONCAT = 0, MOE_GU_INTERLEAVED = 1 } moe_gu_layout_t;

typedef struct {
  int64_t T, H, I, E, K;
  int32_t dtype;      /* moe_dtype_t */
  int32_t act;        /* moe_act_t */
  int32_t gu_layout;  /* moe_gu_layout_t */
  float clamp_limit;  /* L of the clamped GLU (7.0 for the gpt-oss shapes) */
  float glu_alpha;    /* alpha of the clamped GLU (1.702) */
  int32_t grad_dtype; /* moe_dtype_t of d_w_gate_up / d_w_down (accumulation is
                         always fp32; MOE_F32 stores the fp32 sums) */
} moe_desc_t;

/* Sizes in bytes of the workspaces moe_fwd and moe_bwd need, and of the
 * optional `saved` buffer (the gate_up projection outputs Z, fp32 [S,2I] in
 * expert-sorted slot order) that moe_fwd can fill for moe_bwd.  Any output
 * pointer may be NULL.
 * The routing part of both workspaces is moe_route_workspace_size(). */
moe_status_t moe_workspace_size(const moe_desc_t* desc, size_t* fwd_ws,
                                size_t* bwd_ws, size_t* saved_bytes);
moe_status_t moe_route_workspace_size(const moe_desc_t* desc, size_t* route_ws);

/* Expert histogram and stable grouping of the slots by expert — the "masked
 * indexing" / "sparse token extraction" step of the pages' descriptions.
 * Outputs (device, int32):
 *   counts[E]       slots routed to each expert
 *   offsets[E+1]    exclusive prefix sum of counts
 *   sorted_slot[S]  slots in expert order; ascending slot id inside an expert;
 *                   slots with an id outside [0,E) last, in ascending order
 *   inv_pos[S]      position of slot s in sorted_slot (-1 for a bad id)
 * Bit-exact and deterministic.  Any of the four outputs may be NULL (then not
 * written).  ws: at least moe_route_workspace_size() bytes. */
moe_status_t moe_route(const moe_desc_t* desc, const int32_t* topk_ids,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                       int32_t* inv_pos, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Router + routing in one pipeline.  The pages take the top-k expert ids and
 * weights as inputs of the layer ("MoE expert parallel execution backward"
 * lists topk_weights among the tensors it differentiates); this produces
 * them from router logits the way the workloads define routing: the softmax
 * over a token's E logits, its K largest entries, renormalised to sum to one
 * (equal, up to rounding, to the softmax of the K largest logits).
 *   logits        fp32 [T,E] (read only; finite values expected: an infinite
 *                 logit can give NaN weights, and a token whose remaining
 *                 logits are all NaN gets id -1 in the slots left, reported
 *                 as MOE_ERR_BAD_EXPERT_ID by moe_check_device_status)
 *   topk_ids      int32 [T,K] out: ids by descending logit; equal logits in
 *                 ascending id (bit-exact: ids are decided by comparisons of
 *                 the fp32 logits only)
 *   topk_weights  fp32 [T,K] out: exp(l_k - l_0) / sum_j exp(l_j - l_0) in
 *                 fp32, summed in k order (a few ulp from the exact value)
 *   counts, offsets, sorted_slot, inv_pos: as moe_route for these ids (each
 *                 may be NULL).
 * Requires K <= E (else MOE_ERR_INVALID_ARG).  ws: at least
 * moe_route_workspace_size() bytes; the routing it leaves there is the one
 * moe_fwd would compute from topk_ids. */
moe_status_t moe_router(const moe_desc_t* desc, const float* logits,
                        int32_t* topk_ids, float* topk_weights, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_slot, int32_t* inv_pos,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* Forward: out [T,H] = sum_k w[t,k] * FFN_{ids[t,k]}(hidden[t]).
 * Routing, gate_up projection with the gated activation, down projection with
 * the routing weight, and a deterministic per-token sum over the K slots
 * (fp32, k order, one rounding).  `saved` may be NULL; if given, it receives
 * Z for moe_bwd and `saved_bytes` (its size) must be at least the
 * saved_bytes of moe_workspace_size, else MOE_ERR_WORKSPACE (nothing
 * launched). */
moe_status_t moe_fwd(const moe_desc_t* desc, const void* hidden,
                     const int32_t* topk_ids, const float* topk_weights,
                     const void* w_gate_up, const void* w_down, void* out,
                     void* saved, size_t saved_bytes, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* Backward of moe_fwd given d_out = dL/dout [T,H]:
 *   d_hidden [T,H], d_topk_weights fp32 [T,K] (<d_out[t], expert output of
 *   slot s>), d_w_gate_up [E,2I,H] (gate rows = dW_gate, up rows = dW_up, in
 *   w_gate_up's layout), d_w_down [E,H,I].  Weight gradients are accumulated
 *   in fp32 over the tokens and stored in grad_dtype; an expert with no slots
 *   gets exact zeros.  `saved` is the buffer moe_fwd filled for the same
 *   inputs, or NULL (then Z is recomputed); when given, `saved_bytes` (its
 *   size) must be at least moe_workspace_size's saved_bytes, else
 *   MOE_ERR_WORKSPACE (nothing launched). */
moe_status_t moe_bwd(const moe_desc_t* desc, const void* hidden,
                     const int32_t* topk_ids, const float* topk_weights,
                     const void* w_gate_up, const void* w_down,
                     const void* d_out, const void* saved, size_t saved_bytes,
                     void* d_hidden, float* d_topk_weights, void* d_w_gate_up,
                     void* d_w_down, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Forward from router logits [T,E] (fp32): moe_router's top-k and weights
 * (written to topk_ids [T,K] and topk_weights [T,K] for the backward), then
 * moe_fwd on them in the same call.  Same outputs, workspace, `saved` /
 * `saved_bytes` and errors as moe_fwd (plus K <= E). */
moe_status_t moe_fwd_logits(const moe_desc_t* desc, const void* hidden,
                            const float* logits, const void* w_gate_up,
                            const void* w_down, void* out, int32_t* topk_ids,
                            float* topk_weights, void* saved,
                            size_t saved_bytes, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Gradient of the router's weights with respect to its logits, given
 * d_topk_weights fp32 [T,K] (from moe_bwd): d_logits fp32 [T,E] with
 *   d_logits[t, ids[t,k]] = w[t,k] * (g[t,k] - sum_j w[t,j] g[t,j])
 * and zero for experts not chosen (the choice is piecewise constant in the
 * logits).  Ids outside [0,E) contribute nothing; a repeated id of one token
 * receives the sum of its terms.  fp32, one writer per element. */
moe_status_t moe_router_bwd(const moe_desc_t* desc, const int32_t* topk_ids,
                            const float* topk_weights,
                            const float* d_topk_weights, float* d_logits,
                            hipStream_t stream);

/* Separate gate and up weights ("MoE expert parallel execution backward",
 * description, differentiates gate, up and down weights as three tensors):
 * w_gate, w_up [E,I,H] in place of w_gate_up, and in moe_bwd_sep d_w_gate,
 * d_w_up [E,I,H] (grad_dtype) in place of d_w_gate_up; gate and up rows are
 * then g = w_gate[e].x and u = w_up[e].x, and desc->gu_layout is ignored.
 * Everything else (outputs, workspace sizes, `saved`, errors) is as for
 * moe_fwd / moe_bwd; a `saved` buffer filled by moe_fwd_sep is meant for
 * moe_bwd_sep (its Z columns are the I gate columns, then the I up columns).
 * w_up and d_w_up must not be NULL. */
moe_status_t moe_fwd_sep(const moe_desc_t* desc, const void* hidden,
                         const int32_t* topk_ids, const float* topk_weights,
                         const void* w_gate, const void* w_up,
                         const void* w_down, void* out, void* saved,
                         size_t saved_bytes, void* ws, size_t ws_bytes,
                         hipStream_t stream);
moe_status_t moe_bwd_sep(const moe_desc_t* desc, const void* hidden,
                         const int32_t* topk_ids, const float* topk_weights,
                         const void* w_gate, const void* w_up,
                         const void* w_down, const void* d_out,
                         const void* saved, size_t saved_bytes,
                         void* d_hidden, float* d_topk_weights, void* d_w_gate,
                         void* d_w_up, void* d_w_down, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * computation, outputs, `saved` / `saved_bytes` and errors as moe_fwd, with
 * the workspace taken from an array of MOE_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on (part of its code object, kept until
 * the process ends); the call allocates nothing.
 *   - Shapes whose moe_fwd workspace (moe_workspace_size's fwd_ws) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE before any device
 *     call (for H = I = 2880, E = 128, K = 4: up to about 3800 slots).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on
 *     a GPU (other streams, other threads) race and must be ordered by the
 *     caller.  Nothing in the array needs to start at zero.
 *   - bad_ids (device int32, nullable) receives the number of slots with an
 *     id outside [0,E) (the status moe_check_device_status reports for
 *     moe_fwd's workspace). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_fwd_noalloc(const moe_desc_t* desc, const void* hidden,
                             const int32_t* topk_ids,
                             const float* topk_weights, const void* w_gate_up,
                             const void* w_down, void* out, void* saved,
                             size_t saved_bytes, int32_t* bad_ids,
                             hipStream_t stream);

/* Synchronises `stream` and reports MOE_ERR_BAD_EXPERT_ID if the last
 * routing done in `ws` met an id outside [0,E), else MOE_OK. */
moe_status_t moe_check_device_status(const void* ws, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* moe_status_str(moe_status_t status);

/* Kernel timing (instrumentation for benchmarks).  While enabled, every
 * kernel the library launches is bracketed by two HIP events recorded on the
 * launch stream (events come from a library-owned pool of `max_launches`
 * pairs, created on enable; later launches are not timed).  moe_timing_read
 * synchronises those events and returns, per kernel name, the number of
 * timed launches and their summed duration; it resets the pool.
 * Not thread-safe; meant for one benchmarking thread. */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
} moe_kernel_time_t;
moe_status_t moe_timing_enable(int32_t max_launches);
moe_status_t moe_timing_disable(void);
moe_status_t moe_timing_read(moe_kernel_time_t* out, int32_t max_entries,
                             int32_t* n_entries);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */

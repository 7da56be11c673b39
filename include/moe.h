/*
 * moe.h -- C ABI of one GPU's Mixture-of-Experts layer, forward and backward, on
 * AMD Instinct MI355X (gfx950).
 *
 * The path follows "MoE Parallel Folding: Heterogeneous Parallelism Mappings for
 * Efficient Large-Scale MoE Model Training with Megatron Core" (arXiv 2504.14960),
 * knowledge-base notes page, method paragraph: the router assigns every token to
 * its Top-K experts, a permutation makes the tokens of one expert contiguous, the
 * experts' FFNs run, and an un-permutation restores token order; the backward pass
 * runs the same steps' duals.  Section 3.3 (Token Dispatcher) makes sub-sequence
 * dropping the default token-drop strategy.  The cross-GPU exchanges of that
 * pipeline (All-to-All-V, AllGather-V, ReduceScatter-V) are not part of this
 * library: every call works on one GPU's share.
 *
 * Readings of points the pages leave open (each stated where it is used):
 *   - gating: softmax over all E experts in fp32, the K most probable experts
 *     (ties to the lower expert index), gates renormalised over those K;
 *   - capacity per (sub-sequence, expert) = ceil(cf * S * K / E); within each
 *     group the assignments kept are the `capacity` best under (probability desc,
 *     token asc); a dropped assignment contributes nothing and its gate is not
 *     renormalised away;
 *   - permuted rows are expert-major, tokens ascending inside an expert;
 *   - expert FFN = SwiGLU: (silu(x W_g) * (x W_u)) W_d, no biases;
 *   - an optional always-on shared expert is scaled by sigmoid(x . w_sg).
 *
 * Conventions for every call:
 *   - All tensor pointers are device pointers, caller-allocated, row-major and
 *     densely packed.  The library allocates nothing, frees nothing, keeps no
 *     pointer after returning, never synchronises the stream and never reads a
 *     device value on the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work
 *     is enqueued asynchronously; errors of the kernels themselves show up on the
 *     stream like any HIP error.
 *   - Arguments are validated on the host before any HIP call; on failure the call
 *     returns a negative status, launches nothing and sets moe_last_error().
 *   - dtype MOE_F32: every tensor is float.  MOE_BF16: activations, weights and
 *     their gradients are bfloat16 (round-to-nearest-even from fp32 accumulators);
 *     logits, probabilities, gates and their gradients are always float.
 *   - R = moe_max_rows(desc) bounds the rows of every permuted buffer ([R, *]);
 *     only the first n_kept rows are written, the rest are left as they were.
 *   - Weight layouts (y = x . W): w_router [d, E]; w_gate, w_up [E, d, f];
 *     w_down [E, f, d]; w_sg [d].  Weight gradients have the weights' layouts and
 *     are overwritten, not accumulated.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, bad size, K > E, T % S != 0, ... */
#define MOE_ERR_UNSUPPORTED (-2) /* a dtype or shape the library does not handle */
#define MOE_ERR_WORKSPACE (-3)   /* workspace smaller than moe_workspace_size() */
#define MOE_ERR_HIP (-4)         /* a HIP launch failed; see moe_last_error() */

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Shape of one layer call.  T tokens, hidden size d, E experts, top-K, expert ffn
 * size f, sub-sequence length S (T % S == 0; drops are decided inside each block
 * of S consecutive tokens), capacity per (sub-sequence, expert) or -1 for
 * dropless.  Limits: 1 <= K <= min(E, 8), E <= 64, d % 8 == 0, f % 8 == 0.
 * The grouped GEMMs run on the bf16 matrix cores when dtype is MOE_BF16 and
 * d % 256 == 0 and f % 256 == 0, on the vector ALUs otherwise (or when flags has
 * MOE_FLAG_VALU_GEMM). */
typedef struct moe_desc {
    int32_t T;
    int32_t d;
    int32_t E;
    int32_t K;
    int32_t f;
    int32_t sub_seq;
    int32_t capacity;
    int32_t dtype; /* moe_dtype */
    int32_t flags; /* MOE_FLAG_* */
} moe_desc;

#define MOE_FLAG_VALU_GEMM 1 /* force the vector-ALU grouped GEMMs */
/* Expert-tensor-parallel shard (knowledge-base notes page, method paragraph: the
 * ETP group shares the dispatched rows by AllGather-V and the expert outputs are
 * summed by ReduceScatter-V).  On one ETP rank the call gets an f-slice of every
 * expert's weights (desc f = f / ETP), so the down GEMM's o and the gate/up dgrad's
 * dxp are partial sums over that slice: with this flag moe_expert_ffn_fwd writes
 * o_out and moe_expert_ffn_bwd writes dxp_out as float [R, d] (one rounding after
 * the cross-shard sum instead of one per shard).  Every other output keeps the
 * layer dtype.  moe_unpermute, moe_unpermute_bwd and moe_permute_bwd reject the
 * flag with MOE_ERR_INVALID_ARG: they take rows already summed over the shards. */
#define MOE_FLAG_F32_PARTIAL 2

/* Routing results, all device pointers written by moe_route / moe_route_from_logits:
 *   topk_idx      int32 [T, K]  expert of slot k, slot 0 the most probable
 *   topk_prob     float [T, K]  softmax probability (over all E) of that expert
 *   topk_gate     float [T, K]  gate: probability / sum of the K chosen probabilities
 *   keep          uint8 [T, K]  1 if the assignment survived the capacity drop
 *   row_of        int32 [T, K]  its row in the permuted buffer, -1 if dropped
 *   src_of        int32 [R]     t*K + k of each permuted row (first n_kept valid)
 *   routed_counts int32 [T/S, E] assignments per (sub-sequence, expert) before drops
 *   kept_counts   int32 [E]     kept assignments per expert
 *   offsets       int32 [E+1]   exclusive scan of kept_counts; offsets[E] = n_kept
 *   n_kept        int32 [1]                                                       */
typedef struct moe_routing {
    int32_t* topk_idx;
    float* topk_prob;
    float* topk_gate;
    uint8_t* keep;
    int32_t* row_of;
    int32_t* src_of;
    int32_t* routed_counts;
    int32_t* kept_counts;
    int32_t* offsets;
    int32_t* n_kept;
} moe_routing;

/* Workspace kinds for moe_workspace_size(). */
#define MOE_WS_ROUTE 0     /* moe_route, moe_route_from_logits */
#define MOE_WS_FFN_FWD 1   /* moe_expert_ffn_fwd */
#define MOE_WS_FFN_BWD 2   /* moe_expert_ffn_bwd */
#define MOE_WS_ROUTE_BWD 3 /* moe_route_bwd */
#define MOE_WS_PERMUTE_BWD 4 /* moe_permute_bwd */

/* ---- host helpers: synchronous, launch nothing --------------------------------- */

int32_t moe_abi_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Capacity per (sub-sequence, expert): ceil(cf * S * K / E) computed in double;
 * a negative cf means dropless and returns -1.  cf = 0 gives 0 (drop everything).
 * (capacity factor: knowledge-base notes page, prerequisites and setup.) */
int32_t moe_capacity(int32_t S, int32_t K, int32_t E, double cf);

/* Upper bound R on permuted rows: T*K when dropless, else
 * min(T*K, (T/S) * E * capacity).  Returns -1 for an invalid desc. */
int64_t moe_max_rows(const moe_desc* desc);

/* Bytes of device workspace a call of kind `which` needs (0 is possible).
 * Returns (size_t)-1 for an invalid desc. */
size_t moe_workspace_size(const moe_desc* desc, int32_t which);

/* ---- forward --------------------------------------------------------------------- */

/* Router (method paragraph: the router picks each token's K experts; capacity
 * drop per sub-sequence, Section 3.3).  logits = x . w_router (+ bias), fp32 accumulation,
 * written to logits_out [T, E]; then softmax, top-K, gates, per-(sub-sequence,
 * expert) capacity drop and the permutation maps into *r.
 *   x [T, d] dtype; w_router [d, E] dtype; bias [E] float or NULL (added before the
 *   softmax, a constant); w_sg [d] dtype or NULL: the shared expert's gate vector,
 *   then sg_logit_out [T] float receives z = x . w_sg (else it may be NULL).
 *   ws: workspace of moe_workspace_size(desc, MOE_WS_ROUTE) bytes. */
moe_status moe_route(const moe_desc* desc, const void* x, const void* w_router,
                     const float* bias, const void* w_sg, float* logits_out,
                     float* sg_logit_out, const moe_routing* r, void* ws, size_t ws_bytes,
                     void* stream);

/* moe_route for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * and results as moe_route without the workspace.  Its scratch (what moe_route keeps
 * in `ws`) is a fixed array of MOE_ROUTE_SCRATCH_BYTES in the library's device memory,
 * one copy per GPU, reserved for the life of the process; the call itself allocates
 * nothing.  A shape whose moe_workspace_size(desc, MOE_WS_ROUTE) exceeds it is
 * rejected with MOE_ERR_UNSUPPORTED before any launch.  Every call on one GPU uses
 * that GPU's copy, so calls that overlap in time on one GPU (different streams, or
 * different host threads) race and must be serialised by the caller; calls on one
 * stream are ordered and safe.  Nothing of the scratch needs clearing between calls.
 * The first call on each GPU looks the array's address up on that GPU. */
#define MOE_ROUTE_SCRATCH_BYTES (16u << 20)
moe_status moe_route_noalloc(const moe_desc* desc, const void* x, const void* w_router,
                             const float* bias, const void* w_sg, float* logits_out,
                             float* sg_logit_out, const moe_routing* r, void* stream);

/* The routing steps of moe_route from given fp32 logits [T, E] (no GEMM).  The
 * decisions are bit-exact functions of the logits: softmax with this library's
 * own exp (Cody-Waite reduction, degree-7 Taylor polynomial), pairwise sums, IEEE
 * division, no fused multiply-add. */
moe_status moe_route_from_logits(const moe_desc* desc, const float* logits,
                                 const moe_routing* r, void* ws, size_t ws_bytes,
                                 void* stream);

/* Permutation (method paragraph: each expert's tokens are gathered into one
 * contiguous block): xp[row] = x[src_of[row] / K] for row < n_kept.
 *   x [T, d]; xp_out [R, d]. */
moe_status moe_permute(const moe_desc* desc, const void* x, const moe_routing* r,
                       void* xp_out, void* stream);

/* Grouped SwiGLU expert FFN (method paragraph: the experts' feed-forward step) on the
 * segments [offsets[e], offsets[e+1]) of xp:
 *   a = xp W_g,e ; b = xp W_u,e ; h = silu(a) * b (from the fp32 accumulators);
 *   o = h W_d,e.
 *   xp [R, d]; w_gate, w_up [E, d, f]; w_down [E, f, d]; offsets [E+1] (device);
 *   a_out, b_out, h_out [R, f] (a and b are kept for the backward pass); o_out [R, d]
 *   (float with MOE_FLAG_F32_PARTIAL).
 * R = moe_max_rows(desc); rows from offsets[E] to R are not touched.  On the side of
 * the expert-parallel exchange the rows come from several source GPUs: pass
 * T = rows received, K = 1, capacity = -1 (then R = T) and the local experts'
 * offsets.  The shared expert is this call with E = 1, K = 1, f = its ffn size and
 * offsets = {0, T} on x itself. */
moe_status moe_expert_ffn_fwd(const moe_desc* desc, const void* xp, const void* w_gate,
                              const void* w_up, const void* w_down, const int32_t* offsets,
                              void* a_out, void* b_out, void* h_out, void* o_out, void* ws,
                              size_t ws_bytes, void* stream);

/* Un-permutation (method paragraph: rows go back to token order), gate
 * weighted: y_t = sum over kept slots k, ascending, of g_tk * o[row_of[t,k]], in
 * fp32; plus sigmoid(z_t) * shared_t when shared_out is not NULL.
 *   o [R, d]; shared_out [T, d] or NULL; sg_logit [T] float (with shared_out);
 *   y_out [T, d].  A token whose every slot was dropped gets 0 (+ the shared term). */
moe_status moe_unpermute(const moe_desc* desc, const void* o, const moe_routing* r,
                         const void* shared_out, const float* sg_logit, void* y_out,
                         void* stream);

/* ---- backward (loss L with dL/dy = dy) ------------------------------------------- */

/* Dual of moe_unpermute (method paragraph: the backward pass runs the forward steps'
 * duals; this is the un-permutation's): d_o[row_of[t,k]] = g_tk * dy_t and
 * dgate[t,k] = <dy_t, o[row_of[t,k]]> (0 for a dropped slot).  With a shared
 * expert: dshared_t = sigmoid(z_t) * dy_t and dsg_logit_t = <dy_t, shared_t> *
 * s_t (1 - s_t).  dy [T, d]; d_o_out [R, d]; dgate_out [T, K] float;
 * dshared_out [T, d] and dsg_logit_out [T] float, or NULL without a shared expert. */
moe_status moe_unpermute_bwd(const moe_desc* desc, const void* dy, const void* o,
                             const moe_routing* r, const void* shared_out,
                             const float* sg_logit, void* d_o_out, float* dgate_out,
                             void* dshared_out, float* dsg_logit_out, void* stream);

/* Dual of moe_expert_ffn_fwd (method paragraph: the backward pass runs the duals; this
 * is the expert FFN's), per segment e:
 *   dh = d_o W_d,e^T ; da = dh * b * sig(a) (1 + a (1 - sig(a))) ; db = dh * silu(a)
 *   dW_d,e = h^T d_o ; dW_g,e = xp^T da ; dW_u,e = xp^T db ;
 *   dxp = da W_g,e^T + db W_u,e^T.
 * An expert with no rows gets zero weight gradients.
 *   a, b, h: the buffers moe_expert_ffn_fwd wrote; d_o [R, d]; dxp_out [R, d]
 *   (float with MOE_FLAG_F32_PARTIAL);
 *   dw_gate_out, dw_up_out [E, d, f]; dw_down_out [E, f, d]; ws of
 *   moe_workspace_size(desc, MOE_WS_FFN_BWD) bytes (holds da, db). */
moe_status moe_expert_ffn_bwd(const moe_desc* desc, const void* xp, const void* a,
                              const void* b, const void* h, const void* w_gate,
                              const void* w_up, const void* w_down, const int32_t* offsets,
                              const void* d_o, void* dxp_out, void* dw_gate_out,
                              void* dw_up_out, void* dw_down_out, void* ws, size_t ws_bytes,
                              void* stream);

/* Router backward (method paragraph: the backward pass runs the duals; this is the
 * router's, with the Top-K selection and the Section 3.3 drops held fixed).  Gates are
 * the softmax of the K chosen logits, so for the
 * chosen experts dl_{e_j} = g_j (dgate_j - sum_k g_k dgate_k) and every other
 * logit gets 0 (the selection and the drops are piecewise constant).  Writes
 * dlogits_out [T, E] float and dw_router_out = x^T dl [d, E]; with dsg_logit
 * (shared gate, [T] float) also dw_sg_out = x^T dsg_logit [d].  The reduction over
 * T is two-stage and has a fixed order (deterministic).  x [T, d]; dgate [T, K];
 * ws of moe_workspace_size(desc, MOE_WS_ROUTE_BWD) bytes. */
moe_status moe_route_bwd(const moe_desc* desc, const void* x, const moe_routing* r,
                         const float* dgate, const float* dsg_logit, float* dlogits_out,
                         void* dw_router_out, void* dw_sg_out, void* ws, size_t ws_bytes,
                         void* stream);

/* Dual of moe_permute plus the router's input gradient (method paragraph: the backward
 * pass runs the duals; this is the permutation's):
 *   dx_t = sum over kept k (ascending) of dxp[row_of[t,k]]
 *          + sum_k dlogits[t, e_tk] * w_router[:, e_tk]     (if dlogits != NULL)
 *          + dsg_logit_t * w_sg                              (if dsg_logit != NULL)
 *          + dx_add_t                                        (if dx_add != NULL)
 * accumulated in fp32 and stored once.  dxp [R, d]; dlogits [T, E]; w_router [d, E];
 * dsg_logit [T]; w_sg [d]; dx_add [T, d] (e.g. the shared expert's dx); dx_out [T, d].
 * ws of moe_workspace_size(desc, MOE_WS_PERMUTE_BWD) bytes: 0 for E <= 15 (each block
 * then keeps its slice of the router weight in LDS; ws may be NULL), else a transposed
 * copy of the router weight, (E + 1) * d elements. */
moe_status moe_permute_bwd(const moe_desc* desc, const void* dxp, const moe_routing* r,
                           const float* dlogits, const void* w_router, const float* dsg_logit,
                           const void* w_sg, const void* dx_add, void* dx_out, void* ws,
                           size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

/*
 * moe_ffn.h -- C ABI of the routed-expert FFN layer for MI355X (gfx950).
 *
 * The layer (per token x, per layer):
 *   router logits  l = W_r x, one score per expert;
 *   top-k          the k largest logits, in descending order (ties to the lower id),
 *                  re-chosen in every layer;
 *   weights        w = softmax over the k selected logits;
 *   experts        channel j of expert e owns row j of G_e, row j of V_e and column j of
 *                  D_e (stored as row j of D_e^T); a_j = silu(g_j . x) * (v_j . x);
 *   output         y = sum_e w_e sum_j a_j d_j  +  sum_s sum_j a_j d_j  (shared experts,
 *                  weight 1, read by every token).
 * Sources: the jaehun.me review of arXiv:2610.37386, section "Background: channels and
 * keep rules" (channel anatomy, Fig. 2(a)) and "The weights-only reader" stage 2 (D
 * transposed once at load so d_j is contiguous; ||d_j|| precomputed at load);
 * "Mixture of Experts Changes the Arithmetic", section "Two Numbers Instead of One"
 * (k of E experts per token, +1/+2 shared experts read by every token).
 *
 * Conventions for every call:
 *  - Tensors are device memory owned by the caller and borrowed by the library; weights
 *    must outlive the layer handle.  The handle owns host metadata only; all derived
 *    data (down-norm table, routing scratch, partial sums, flags) lives in the caller's
 *    workspace.  The library never allocates device memory.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null stream).
 *    There are no implicit device synchronisations, except in moe_layer_check.
 *  - Arguments are validated on the host before any HIP call; a failing call returns a
 *    status, enqueues nothing and leaves the outputs untouched.  HIP launch failures
 *    return MOE_ERR_DEVICE.  moe_last_error() holds a thread-local message.
 *  - Activations (x, y, logits, router weights w) are fp32 row-major; ids are int32.
 *  - Same inputs give bit-identical outputs (no floating-point atomics).
 *  - A layer handle (and its workspace) serves one stream at a time.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_layer_s* moe_layer;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null pointer, size out of range, bad enum */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not built: dtype combination, shape limit */
  MOE_ERR_WORKSPACE = 3,    /* workspace too small or misaligned */
  MOE_ERR_DEVICE = 4        /* a HIP call failed, or a kernel reported an error */
} moe_status;

typedef enum { MOE_DTYPE_NONE = -1, MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2 } moe_dtype;

typedef enum {
  MOE_EXPERT_SWIGLU = 0,   /* G, V, D^T per expert, each [inter][hidden] */
  MOE_EXPERT_LINEAR = 1    /* one matrix M_e [inter][hidden] per expert: y = sum w_e M_e x */
} moe_kind;

typedef enum {
  MOE_SCORE_GATE_DNORM = 0,      /* s_j = |silu(g_j . x)| * ||d_j||_2               */
  MOE_SCORE_ROUTER_WEIGHTED = 1  /* s_j = w_e * |silu(g_j . x)| * ||d_j||_2 (eq. 1  */
                                 /* output units with the exact gate)                */
} moe_score;

typedef struct {
  int32_t hidden;        /* H: multiple of 32 */
  int32_t n_experts;     /* E: 1..4096 */
  int32_t top_k;         /* k: 1..min(E, 32), or up to E when E <= 64 */
  int32_t inter;         /* I: channels per expert (LINEAR: output width), multiple of 8 */
  int32_t n_shared;      /* 0..4 shared experts (SWIGLU only) */
  int32_t shared_inter;  /* I_s (multiple of 8) */
  int32_t kind;          /* moe_kind */
  int32_t router_dtype;  /* MOE_F32, MOE_BF16, or MOE_DTYPE_NONE (route from given logits) */
  int32_t expert_dtype;  /* MOE_F32, MOE_BF16, MOE_MXFP4 (MXFP4: SWIGLU only) */
  int32_t shared_dtype;  /* MOE_F32 or MOE_BF16 */
  int32_t max_batch;     /* largest B any call will pass: 1..4096; sizes the workspace */
} moe_layer_desc;

/* Device pointers.  Expert tensors are stacked [E][inter][hidden], row-major.
 * MXFP4 rows: codes [E][inter][hidden/2] bytes (even element in the low nibble) and
 * e8m0 scales [E][inter][hidden/32] bytes, one per 32 consecutive elements of a row
 * (OCP Microscaling Formats v1.0).  Shared experts are [n_shared][shared_inter][hidden].
 * Every pointer is 16-byte aligned. */
typedef struct {
  const void* router;           /* [E][H] router_dtype; NULL iff router_dtype is NONE */
  const void* gate;             /* G  (SWIGLU) */
  const void* up;               /* V  (SWIGLU) */
  const void* down_t;           /* D^T: row j is d_j (SWIGLU) */
  const uint8_t* gate_scale;    /* MXFP4 scales of G, V, D^T; NULL otherwise */
  const uint8_t* up_scale;
  const uint8_t* down_scale;
  const void* linear;           /* M (LINEAR) */
  const void* sh_gate;          /* shared experts (n_shared > 0) */
  const void* sh_up;
  const void* sh_down_t;
} moe_weights;

/* Bytes of workspace a layer with this descriptor needs (0 on an invalid descriptor).
 * Host only; makes no HIP call. */
size_t moe_layer_workspace_bytes(const moe_layer_desc* desc);

/* Validate desc and weights, bind the caller's workspace (256-byte aligned, at least
 * moe_layer_workspace_bytes), and enqueue the load-time preparation: clear the control
 * block and compute ||d_j||_2 for every routed channel (the table the channel selector
 * reads).  *out receives the handle. */
moe_status moe_layer_create(const moe_layer_desc* desc, const moe_weights* weights,
                            void* workspace, size_t workspace_bytes, void* stream,
                            moe_layer* out);
moe_status moe_layer_destroy(moe_layer layer);

/* Routing only.  Exactly one of x [B][H] / logits_in [B][E] is non-NULL (x needs a
 * router).  Writes ids [B][k] (routing order: descending logit, ties to the lower id),
 * w [B][k] (softmax over the selected logits) and, if non-NULL, logits_out [B][E]. */
moe_status moe_route(moe_layer layer, const float* x, const float* logits_in, int32_t B,
                     int32_t* ids, float* w, float* logits_out, void* stream);

/* The layer.  x [B][H]; y [B][H] (LINEAR: [B][inter]) is overwritten.
 * ids/w: both NULL to route inside the call (needs a router), or both given [B][k].
 * B = 1 runs as one persistent launch (router, top-k, shared and routed experts, and
 * the deterministic cross-workgroup reduction); B > 1 reads each touched expert once
 * for all the tokens routed to it. */
moe_status moe_ffn_forward(moe_layer layer, const float* x, int32_t B, const int32_t* ids,
                           const float* w, float* y, void* stream);

/* Channel-sparse layer for one token (B = 1, SWIGLU; the fixed-count top-K keep rule of
 * the review's section "Background: channels and keep rules" with the output-unit score
 * of "The weights-only reader" stage 2).  Candidates are the k*I channels of the routed
 * experts (shared experts are always read in full and never candidates).  Every gate row
 * is read to score; only the kept channels' up rows and down rows are read.
 * ids/w: both NULL to route inside the call, or both given [k].  keep: 0..k*I.
 * kept [keep] receives the kept candidates as ascending flat ids slot*I + j (slot in
 * routing order); ties in the score go to the lower flat id.  y [H] (may be NULL). */
moe_status moe_channel_select(moe_layer layer, const float* x, const int32_t* ids,
                              const float* w, int32_t keep, int32_t mode, int32_t* kept,
                              float* y, void* stream);

/* Touched-expert union of a batch (the "experts touched by a batch" count of the
 * 501B/23B post, section 2).  ids [B][k] with distinct experts per token, 0 <= id < E.
 * Writes n_touched [1], touched [E] (ascending; first n_touched valid), offsets [E+1]
 * (prefix sum of per-expert counts) and slots [B*k] (flat b*k+i grouped by expert,
 * ascending within an expert).  One workgroup; needs E*(ceil(B/32) | 1)*8 + 8*E bytes of
 * LDS, at most 144 KiB (else MOE_ERR_UNSUPPORTED). */
moe_status moe_union_experts(const int32_t* ids, int32_t B, int32_t k, int32_t E,
                             int32_t* n_touched, int32_t* touched, int32_t* offsets,
                             int32_t* slots, void* stream);

/* Synchronise `stream` and read the layer's device error word (0 = none; nonzero means a
 * bounded in-kernel wait expired, or a given id was outside [0, E) or repeated within a
 * token -- such ids are skipped); clears it. */
moe_status moe_layer_check(moe_layer layer, void* stream, int32_t* device_error);

/* Launch geometry of the persistent kernels (workgroups, threads per workgroup). */
moe_status moe_layer_geometry(moe_layer layer, int32_t* workgroups, int32_t* threads);

const char* moe_status_string(moe_status status);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */

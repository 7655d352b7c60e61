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
 * the deterministic cross-workgroup reduction); B = 2 (SWIGLU, hidden <= 8192) as two such
 * launches, one per token; larger B reads each touched expert once for all the tokens
 * routed to it (BF16 or MXFP4 experts with BF16 shared experts: otherwise
 * MOE_ERR_UNSUPPORTED). */
moe_status moe_ffn_forward(moe_layer layer, const float* x, int32_t B, const int32_t* ids,
                           const float* w, float* y, void* stream);

/* moe_ffn_forward without a layer handle or a caller workspace, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops, harnesses that
 * forbid it).  It validates desc and weights as moe_layer_create does and runs the same
 * kernels as moe_ffn_forward, with the layer's workspace (less the down-norm table, which
 * only moe_channel_select reads) in a static scratch array of the library: 32 MiB per GPU,
 * held from the first call on that GPU until the process ends.  A descriptor whose
 * workspace exceeds it returns MOE_ERR_UNSUPPORTED (moe_layer_workspace_bytes gives an upper
 * bound).  Calls no allocator.  Every call on a GPU shares that GPU's scratch: each call first
 * clears what must start at zero (a fill kernel on `stream`), and calls that overlap on one
 * GPU (concurrent streams or threads) race and give undefined results.  The device error
 * word (bad ids, expired waits) is not reported: it lives in the scratch and the next call
 * clears it. */
moe_status moe_ffn_forward_noalloc(const moe_layer_desc* desc, const moe_weights* weights,
                                   const float* x, int32_t B, const int32_t* ids,
                                   const float* w, float* y, void* stream);

/* Channel-sparse layer for one token (B = 1, SWIGLU; the fixed-count top-K keep rule of
 * the review's section "Background: channels and keep rules" with the output-unit score
 * of "The weights-only reader" stage 2).  Candidates are the k*I channels of the routed
 * experts (shared experts are always read in full and never candidates).  Every gate row
 * is read to score; only the kept channels' up rows and down rows are read.
 * ids/w: both NULL to route inside the call, or both given [k].  keep: 0..k*I.
 * kept [keep] receives the kept channels as ascending ids e*I + j (channel j of expert e;
 * -1 for a channel of a skipped given id); ties in the score go to the lower e*I + j.  The
 * kept rows are split evenly over the workgroups.  y [H] (may be NULL). */
moe_status moe_channel_select(moe_layer layer, const float* x, const int32_t* ids,
                              const float* w, int32_t keep, int32_t mode, int32_t* kept,
                              float* y, void* stream);

/* The channel-sparse layer under the threshold keep rule (the review's section "Background:
 * channels and keep rules", the rule of its first row, and the calibration discussion that
 * follows it): every candidate whose score (the same exact output-unit score as
 * moe_channel_select, mode as there) is at least `tau` is kept, so the number kept -- and the
 * bytes read -- vary per token.  A tau at or below 0 keeps every candidate; NaN is rejected.
 * kept [k*I] receives the kept ids ascending (e*I + j), kept_count [1] (device int32) their
 * number; both must be given.  y [H] (may be NULL).  ids/w as for moe_channel_select.  Each
 * workgroup streams its own kept channels as soon as its own scores are known (no global
 * selection). */
moe_status moe_channel_select_threshold(moe_layer layer, const float* x, const int32_t* ids,
                                        const float* w, float tau, int32_t mode, int32_t* kept,
                                        int32_t* kept_count, float* y, void* stream);

/* The k*I channel scores of the layer's last moe_channel_select(_threshold, _sketch) call,
 * read back (for calibrating tau): enqueues on `stream` a copy into scores [k*I] (fp32,
 * device) in candidate order, slot-major: slot s (the routing order of moe_layer_routing)
 * times I plus channel j.  The lowest mantissa bit of each score is cleared (inside the call it
 * carries the launch parity). */
moe_status moe_layer_scores(moe_layer layer, float* scores, void* stream);

/* The ternary-sketch channel screen (the review of arXiv:2610.37386, "The weights-only
 * reader", stages 1 and 2).  Load time, once: every routed channel's gate row and up row is
 * rotated in blocks of 128 coordinates by a randomized Hadamard transform (unnormalized:
 * u = H_128 (s * w) per block, s the layer's random signs, H_128 the Sylvester-ordered
 * Walsh-Hadamard matrix; g.x = sum over blocks of u.z / 128 with z = H_128 (s * x)), and each
 * rotated block is stored as ternary codes {-1, 0, 1} (threshold 0.7 mean|u|, the codes' sign),
 * an FP16 scale (the mean |u| over the nonzero codes) and rho, the block's mean squared
 * quantization error (FP16).  Per token: x is rotated once, only the 80 coordinates of largest
 * |z| of each block are scanned (ties to the lower coordinate), the estimates g^, v^ give the
 * eq.-1 score w_e ||d_j|| |silu(g^) v^| (mode MOE_SCORE_GATE_DNORM drops w_e), the `keep` best
 * of the k*I candidates (ties to the lower e*I + j) are computed exactly from their full gate,
 * up and down rows, and the rest are not read.
 *
 * moe_sketch_bytes: bytes of the sketch of a layer with this descriptor (0 if it has none:
 * SWIGLU experts in BF16 or F32, hidden a multiple of 128 and at most 4096).  Host only.
 * Layout of the buffer: 2-bit codes of G then V [E*I][H/16] uint32 (coordinate c of a row at
 * bits 2 (c % 16) of word c / 16: 0 -> 00, +1 -> 01, -1 -> 11), then FP16 scales of G, of V,
 * rho of G, of V [E*I][nbp] with nbp = H/128 rounded up to a multiple of 8 (each row 16-byte
 * aligned; the padding holds zeros), each region 256-byte aligned. */
size_t moe_sketch_bytes(const moe_layer_desc* desc);

/* Build the sketch of the layer's routed gate and up rows into the caller's device buffer
 * `sketch` (256-byte aligned, at least moe_sketch_bytes) from the rotation signs `signs` [H]
 * (int8 device memory, +1 or -1, 4-byte aligned), and bind both to the layer (they must
 * outlive it).
 * Enqueues on `stream`. */
moe_status moe_layer_build_sketch(moe_layer layer, const int8_t* signs, void* sketch,
                                  size_t sketch_bytes, void* stream);

/* moe_channel_select with the sketch screen in place of the exact gate pass: the same
 * arguments and outputs (kept [keep]: ascending ids e*I + j); needs moe_layer_build_sketch. */
moe_status moe_channel_select_sketch(moe_layer layer, const float* x, const int32_t* ids,
                                     const float* w, int32_t keep, int32_t mode, int32_t* kept,
                                     float* y, void* stream);

/* The reader's stage 3 (the review's "The weights-only reader", stage 3, eq. 2): the
 * dropped channels S are added back through a rank-32 map, y^ = sum_K w_j d_j a_j +
 * U sum_S w_j b_j p_j, with U [H][32] the top-32 left singular vectors of the layer's stacked
 * down columns d_j, b_j = U^T d_j per routed channel, and p_j = silu(g^_j) v^_j the screen's
 * own activation estimates (no further reads of gate or up rows).
 *
 * moe_recovery_bytes: bytes of a layer's recovery buffer (0 if it has no sketch form). Host
 * only.  Layout: U [H][32] fp32, then b [E*I][32] FP16, each 256-byte aligned.
 *
 * moe_layer_build_recovery: U [H][rank] (fp32 device memory, 4-byte aligned, computed by the
 * caller; rank must be 32) is copied into the caller's buffer `rec` (256-byte aligned, at
 * least moe_recovery_bytes), b_j = U^T d_j is computed there (fp32 sums, stored FP16), and the
 * buffer is bound to the layer (it must outlive it).  Enqueues on `stream`.
 *
 * moe_channel_select_reader: moe_channel_select_sketch (the same arguments and kept list)
 * with the dropped channels recovered into y [H] (NULL: the workspace's output row); needs
 * moe_layer_build_sketch and moe_layer_build_recovery.  Two launches on `stream`: the
 * screen, which also leaves each workgroup's sum over its dropped candidates of w_e b_j p_j
 * in the workspace, then y += U times their total. */
size_t moe_recovery_bytes(const moe_layer_desc* desc);
moe_status moe_layer_build_recovery(moe_layer layer, const float* U, int32_t rank, void* rec,
                                    size_t rec_bytes, void* stream);
moe_status moe_channel_select_reader(moe_layer layer, const float* x, const int32_t* ids,
                                     const float* w, int32_t keep, int32_t mode, int32_t* kept,
                                     float* y, void* stream);

/* Batch-wide channel selection for B tokens (the review of arXiv:2610.37386, "Limits":
 * choosing the channels for a whole batch at once is left by the authors as future work; its
 * Table 7 runs the per-token reader at B = 4 and 8).  Reading taken: the candidates are the
 * channels (e, j) of every expert that some token of the batch routes to (candidate order:
 * ascending e*I + j); a channel's batch score is ||d_j|| times the sum, over the tokens b
 * routed to e, of w_{b,e} |silu(g_j . x_b)| (the router-weighted output-unit score, summed);
 * the `keep` best batch scores are kept (ties to the lower e*I + j); each kept channel is
 * computed exactly for every token routed to its expert, its three rows read once for the
 * batch; dropped channels add nothing; shared experts are computed in full for every token.
 *
 * x [B][H] fp32, 1 <= B <= min(max_batch, 16); ids/w [B][k] as for moe_ffn_forward (NULL:
 * routed inside the call; given ids must be distinct per token and in [0, E)).  0 <= keep <=
 * min(E, B*k)*I (kept are min(keep, n_touched*I)).  kept [keep] (device int32, may be NULL when
 * keep is 0) receives the kept ids ascending, -1 past the kept count; kept_count [1] (device
 * int32, may be NULL) their number.  y [B][H] fp32 (must be given).  BF16 or F32 experts
 * (MOE_ERR_UNSUPPORTED for MXFP4, or for min(E, B*k)*I above 98304).  Enqueues on `stream`
 * the routing (when ids is NULL), the touched-expert union and five launches: batch scores
 * (one wave per candidate), the selection (one workgroup), the kept and shared channels'
 * activations (one wave per channel), the down products in 32 channel chunks, their sum. */
moe_status moe_channel_select_batch(moe_layer layer, const float* x, int32_t B,
                                    const int32_t* ids, const float* w, int32_t keep,
                                    int32_t* kept, int32_t* kept_count, float* y, void* stream);

/* Touched-expert union of a batch (the "experts touched by a batch" count of the
 * 501B/23B post, section 2).  ids [B][k] with distinct experts per token, 0 <= id < E.
 * Writes n_touched [1], touched [E] (ascending; first n_touched valid), offsets [E+1]
 * (prefix sum of per-expert counts) and slots [B*k] (flat b*k+i grouped by expert,
 * ascending within an expert).  One workgroup; needs E*(ceil(B/32) | 1)*8 + 8*E bytes of
 * LDS, at most 144 KiB (else MOE_ERR_UNSUPPORTED). */
moe_status moe_union_experts(const int32_t* ids, int32_t B, int32_t k, int32_t E,
                             int32_t* n_touched, int32_t* touched, int32_t* offsets,
                             int32_t* slots, void* stream);

/* The routing a layer call last used, read back for checking: enqueues on `stream` a copy
 * of B rows of ids [B][k] (int32, routing order) and w [B][k] (fp32) from the workspace
 * into the caller's device buffers.  Valid after a moe_ffn_forward or moe_channel_select
 * call that routed inside the call (ids == NULL): at B <= 2 the top-k chosen inside each
 * token's single launch, for larger B that of the routing step in front of the batched
 * kernels.  At B <= 2 with given ids it holds the ids the launches used (-1 for a skipped
 * id).  Other
 * rows, and rows past the last call's B, are unspecified.  Routing k of E experts per
 * token, re-chosen in every layer: "Mixture of Experts Changes the Arithmetic", section
 * "Two Numbers Instead of One".  1 <= B <= max_batch; ids and w must be given. */
moe_status moe_layer_routing(moe_layer layer, int32_t B, int32_t* ids, float* w, void* stream);

/* Synchronise `stream` and read the layer's device error word (0 = none; nonzero means a
 * bounded in-kernel wait expired, or a given id was outside [0, E) or repeated within a
 * token -- such ids are skipped); clears it. */
moe_status moe_layer_check(moe_layer layer, void* stream, int32_t* device_error);

/* Launch geometry of the persistent kernels (workgroups, threads per workgroup). */
moe_status moe_layer_geometry(moe_layer layer, int32_t* workgroups, int32_t* threads);

/* Text of a status code: `status` is a moe_status value passed as its integer (any other
 * value gives "unknown status"; taking an int keeps out-of-range codes well defined in C++). */
const char* moe_status_string(int32_t status);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */

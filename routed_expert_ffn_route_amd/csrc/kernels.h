// kernels.h -- launch interfaces between the host library and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

// Arguments of the single-launch batch-1 layer kernel.
struct B1Args {
  const float* x;                       // [H]
  const void* router;                   // [E][H]
  const void* gate;                     // [E][I][H]
  const void* up;
  const void* down_t;
  const uint8_t* gate_s;                // MXFP4 scales or null
  const uint8_t* up_s;
  const uint8_t* down_s;
  const void* sh_gate;                  // [NS][IS][H]
  const void* sh_up;
  const void* sh_down_t;
  const int32_t* ids_in;                // given routing [k] or null
  const float* w_in;
  uint64_t* rlog;                       // [E] router logits with their launch tag
  const uint8_t* zrow;                  // zeroed bytes, at least H * 4: read by empty slots
  int32_t* ids_ws;                      // [k]
  float* w_ws;                          // [k]
  float* partials;                      // [P][H]
  float* y;                             // [H]
  Ctrl* ctrl;
  int H, E, k, I, NS, IS;
  int route_inside;
  uint64_t* stamps;                     // [P][kStamps] phase clock (timeline build) or null
};

// occupancy != null: launch nothing; *occupancy = workgroups of this kernel and LDS size that
// fit on one CU at once (the persistent kernels need at least 1)
hipError_t launch_b1(const B1Args& a, DT et, DT st, DT rt, int workgroups, int threads,
                     hipStream_t s, int* occupancy = nullptr);
int b1_lds_bytes(int H, int threads, int E, int k, bool two_layouts);
int team_size(int H);

// Channel-sparse batch-1 layer (fixed-count top-K keep rule over the k*I candidates).
// kept [K] receives the kept channels as ascending ids e*I + j (-1 for a channel of a
// skipped given id); g_ws [k*I] (32-bit words) holds the gate values with the launch parity.
// sketch != null: the candidates are scored from the ternary sketch of their gate and up
// rows (eq. 1 with the estimates) instead of their exact gate values, and kept channels
// read their gate row too.
struct CsSketch {
  const uint32_t *g, *v;    // 2-bit codes [E*I][H/16]
  const uint16_t *ag, *av;  // FP16 scales [E*I][nbp]
  const int8_t* signs;      // rotation signs [H]
  uint64_t* mask;           // workspace: launch-tagged scan masks, kPollCopies x kSkMaskWords
  // the reader's recovery (null: none): b_j FP16 [E*I][kRecRank]; per-workgroup sums r
  // [workgroups][kRecRank] (workspace)
  const uint16_t* rec_b;
  float* rec_r;
};
constexpr int kSkMaskWords = 128;  // words per copy: 4 per 128-block, H <= 4096
constexpr int kRecRank = 32;       // rank of the reader's recovery map
// b_j = U^T d_j (FP16 [nrows][kRecRank]) from D^T [nrows][H] and U [H][kRecRank] (fp32)
hipError_t launch_rec_build(const void* down_t, DT dt, size_t nrows, int H, const float* U,
                            uint16_t* b, hipStream_t s);
// y [H] += U R, R = the sum over P workgroups of r [P][kRecRank]
hipError_t launch_rec_apply(float* y, const float* U, const float* r, int P, int H,
                            hipStream_t s);
// The threshold keep rule: every candidate whose score pattern is at least tau_bits is kept;
// their number goes to count (device).
struct CsThreshold {
  uint32_t tau_bits;
  int32_t* count;
};
hipError_t launch_cs(const B1Args& a, const float* dnorm, uint64_t* g_ws, int32_t* kept,
                     int K, int mode, DT et, DT st, DT rt, int workgroups, int threads,
                     hipStream_t s, int* occupancy = nullptr, const CsSketch* sketch = nullptr,
                     const CsThreshold* thr = nullptr);
// Ternary sketch of nrows rows of H (H % 128 == 0, BF16 or F32): codes [nrows][H/16],
// alpha and rho [nrows][H/128] (FP16 bits), with the rotation signs [H].
hipError_t launch_sketch_build(const void* rows, DT dt, size_t nrows, int H,
                               const int8_t* signs, uint32_t* codes, uint16_t* alpha,
                               uint16_t* rho, hipStream_t s);
int cs_lds_bytes(int H, int threads, int E, int k, int I, int workgroups, int K, bool sketch);
constexpr int kCsMaxPerThread = 8;  // k*I <= 8 * threads
constexpr int kCsOwnMax = 64;       // ceil(k*I / workgroups) <= 64 (own candidates)

// Batch-wide channel selection for B <= kBselMaxBatch tokens, after the routing and the
// union: batch scores S [min(E, B*k)*I], gate values G [same][B], descriptors desc (4 ints
// per kept channel) [min(E, B*k)*I], kept ids
// kept_out [keep] (-1 past the kept count, which goes to nkept), activations A [(kept + NS*IS)
// * B], partial outputs part [kBselPartChunks][B][H], y [B][H].  keep <= min(E, B*k)*I and
// min(E, B*k)*I <= kBselMaxCandidates.  sel: the threshold's words (4 ints) and the kept
// counts of every chunk of kBselChunkCand candidates (2 ints each).
struct BselLaunch {
  const float* x;
  const int32_t* ids;
  const float* w;
  const int32_t *n_touched, *touched, *offsets, *slots;
  const void *gate, *up, *down_t, *sh_gate, *sh_up, *sh_down_t;
  const float* dnorm;
  float* S;
  float* G;
  int32_t* desc;
  int32_t* kept_out;
  int32_t* nkept;
  int32_t* sel;
  float* A;
  float* part;
  float* y;
  int H, I, E, k, B, NS, IS, keep;
};
constexpr int kBselMaxBatch = 16;
constexpr int kBselMaxExperts = 4096;  // (the descriptor's E bound)
constexpr int kBselPartChunks = 32;  // channel chunks of the down products
constexpr int kBselMaxCandidates = 96 * 1024;  // held in the selection's registers
constexpr int kBselChunkCand = 1024;  // candidates per workgroup of the kept-list kernels
inline size_t bsel_sel_bytes(size_t cand) {
  return cand ? 16 + ((cand + kBselChunkCand - 1) / kBselChunkCand) * 8 : 0;
}
hipError_t launch_bsel(const BselLaunch& L, DT et, DT st, hipStream_t s);

// Routing: router GEMV for B tokens, then one workgroup per token for top-k + softmax.
struct RouteArgs {
  const float* x;          // [B][H] or null
  const float* logits_in;  // [B][E] or null
  const void* router;      // [E][H]
  float* logits;           // [B][E] (workspace or caller's logits_out)
  int32_t* ids;            // [B][k]
  float* w;                // [B][k]
  int H, E, k, B;
};
hipError_t launch_route(const RouteArgs& a, DT rt, hipStream_t s);

// Touched-expert union: one workgroup (with x: more workgroups split x [nx] into xh, xl as
// launch_split_x does, in the same launch).
hipError_t launch_union(const int32_t* ids, int B, int k, int E, int32_t* n_touched,
                        int32_t* touched, int32_t* offsets, int32_t* slots, Ctrl* ctrl,
                        hipStream_t s, const float* x = nullptr, size_t nx = 0,
                        uint16_t* xh = nullptr, uint16_t* xl = nullptr);
int union_lds_bytes(int B, int E);
constexpr int kUnionMaxLds = 144 * 1024;  // dynamic LDS the union kernel may use

// Linear experts (one [I][H] bf16 matrix each) for a batch: x is split into bf16 hi/lo
// (xh, xl workspace [B][H]) and the touched experts are applied with MFMA; y [B][I].
hipError_t launch_linear(const void* M, const float* x, const float* w, const int32_t* n_touched,
                         const int32_t* touched, const int32_t* offsets, const int32_t* slots,
                         uint16_t* xh, uint16_t* xl, float* y, int H, int I, int E, int k,
                         int B, hipStream_t s);

// Linear experts at batches of up to kGemvMaxBatch tokens on VALU (whole-line weight
// loads; workgroup r owns RW output rows of every touched expert): y [B][I], from the
// routing ids [B][k] and weights directly (no union launch; an id outside [0, E) or
// repeated within a token sets kErrBadId in *err and is skipped).  `zrow` is zeroed memory
// of at least H * 2 bytes (empty slots read it).  `workgroups` bounds the grid.  Returns
// hipErrorInvalidValue outside linear_gemv_fits, for E > 4096 or B * k > 256.
constexpr int kGemvMaxBatch = 4;
bool linear_gemv_fits(int H, int I, int B);
hipError_t launch_linear_gemv(const void* M, const float* x, const int32_t* ids, const float* w,
                              uint32_t* err, const uint8_t* zrow, float* y, int H, int I, int E,
                              int k, int B, int workgroups, hipStream_t s);

// Linear experts at batches of up to 256 / k tokens on VALU, each touched expert against
// its own tokens only (passes of up to four tokens): partial rows per (token, choice)
// [B*k][I] in `part`, then launch_part_combine into y [B][I].  `zrow` is zeroed memory of
// at least H * 4 bytes.  Returns hipErrorInvalidValue outside linear_pass_fits.
bool linear_pass_fits(int H, int I, int B, int k);
hipError_t launch_linear_pass(const void* M, const float* x, const float* w,
                              const int32_t* ids, const int32_t* n_touched,
                              const int32_t* touched, const int32_t* offsets,
                              const int32_t* slots, const uint8_t* zrow, float* part, float* y,
                              int H, int I, int E, int k, int B, int workgroups,
                              hipStream_t s);

// y[b] = sum over i < k, in order, of part[b*k + i] (rows of I floats; I % 4 == 0), over
// the choices of ids [B][k] that were used (choice_used).
hipError_t launch_part_combine(const float* part, const int32_t* ids, float* y, int B, int k,
                               int I, int E, hipStream_t s);

// Linear experts for larger batches: x in both MFMA operand forms (bf16 hi/lo in xh, xl;
// scaled f16 in x16 with per-token scales xsc, workspace [B][H] each and [B]), then one
// register-blocked MFMA tile per (touched expert, 256 output rows) with the tokens' x staged in LDS, partial rows per (token, choice)
// [B*k][I] in `part`, then a combine in routing order into y [B][I].
hipError_t launch_linear_tiled(const void* M, const float* x, const float* w,
                               const int32_t* ids, const int32_t* n_touched,
                               const int32_t* touched,
                               const int32_t* offsets, const int32_t* slots, uint16_t* xh,
                               uint16_t* xl, uint16_t* x16, float* xsc, float* part, float* y,
                               int H, int I, int E, int k, int B, hipStream_t s);

// x [n] fp32 -> bf16 hi, lo with hi + lo ~= x (the MFMA paths' activation operand).
hipError_t launch_split_x(const float* x, size_t n, uint16_t* xh, uint16_t* xl, hipStream_t s);

// SwiGLU experts for a batch (B > 1): after routing and the touched-expert union, gate/up
// on MFMA into act, down into per-(token, choice) partials, and the per-token combine.
struct BsArgs {
  const void* gate;                     // [E][I][H] (bf16 or MXFP4 codes)
  const void* up;
  const void* down_t;
  const uint8_t* gate_s;                // MXFP4 scales [E][I][H/32] or null
  const uint8_t* up_s;
  const uint8_t* down_s;
  const void* sh_gate;                  // [NS][IS][H] bf16
  const void* sh_up;
  const void* sh_down_t;
  const uint16_t* xh;                   // [B][H] bf16 hi of x
  const uint16_t* xl;                   // [B][H] bf16 lo of x
  const float* w;                       // [B][k] router weights
  const int32_t* ids;                   // [B][k] routing ids (the combine skips unused ones)
  const int32_t* n_touched;             // union: [1], [E], [E+1], [B*k]
  const int32_t* touched;
  const int32_t* offsets;
  const int32_t* slots;
  float* act;                           // [B*k + NS*B][IA] activations
  float* part;                          // [kDownRowSlices][pairs][H] partial outputs
  float* y;                             // [B][H]
  int H, I, IS, IA, E, k, B, NS;
  int pairs;                            // B*k + NS*B
  int slots_max;                        // min(E, B*k): routed expert slots launched
};
// The down products of an expert are split in this many channel slices, each with its own
// partial rows (more, shorter workgroups); the combine adds them in slice order.
constexpr int kDownRowSlices = 2;
hipError_t launch_batched_swiglu(const BsArgs& a, DT et, DT st, hipStream_t s);

// Load-time preparation: ||d_j||_2 of every row of a stacked [rows][H] tensor.
hipError_t launch_row_norms(const void* rows_base, const uint8_t* scales, DT dt, size_t rows,
                            int H, float* out, hipStream_t s);

}  // namespace moe

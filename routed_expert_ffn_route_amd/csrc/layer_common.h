// layer_common.h -- phases shared by the single-launch layer kernels (dense and
// channel-sparse): the x vector in registers, router rows with the exact top-k, streamed
// SwiGLU channels, and the deterministic cross-workgroup reduction of the output.
//
// Thread layout: a workgroup is `nteams` teams of tsz threads (whole waves); a team covers
// one weight row (lane i takes the E-element chunks i, i+tsz, ...), so a wave's loads of a
// row are contiguous 16-byte (bf16, E = 8), 32-byte (fp32, E = 8), 4-byte (MXFP4, E = 8)
// or 8-byte (wide MXFP4, E = 16) pieces.  Each thread keeps the x values and the partial
// output of its chunks in registers (CPT chunks; the team width is chosen so that CPT is
// 1).  A kernel may use two layouts (two Ctx): the routed experts in wide MXFP4 chunks,
// the router and shared experts in 8-element ones.
#pragma once
#include "kernels.h"

namespace moe {
namespace lc {


template <int N> struct NextPow2 {
  static constexpr int value = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16;
};

template <DT dt>
__device__ __forceinline__ typename Fmt<dt>::Raw zero_raw() {
  typename Fmt<dt>::Raw r;
  __builtin_memset(&r, 0, sizeof(r));
  return r;
}

template <DT dt> constexpr int kE = Fmt<dt>::kE;

template <DT dt, int CPT>
__device__ __forceinline__ float chunk_dot(const typename Fmt<dt>::Raw (&r)[CPT],
                                           const float (&xv)[CPT * kE<dt>]) {
  constexpr int E = kE<dt>;
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    float v[E];
    Fmt<dt>::decode(r[m], v);
#pragma unroll
    for (int i = 0; i < E; ++i) s = fmaf(v[i], xv[m * E + i], s);
  }
  return s;
}

// Per-thread view of the workgroup.
struct Ctx {
  int tid, nthreads, nteams, team, t, lane, wit, P, wg, H, nch;
  int tsz, wpt;   // threads and waves per team (a team covers one weight row)
  float* red;     // [2][nteams][4][NP] team-reduction buffers (double buffered)
  int red_stride; // floats per buffer
  int parity;
  uint32_t epoch; // launches completed on this workspace before this one
  const uint8_t* zrow;  // zeroed global memory of at least one weight row and scale row
  uint64_t* stamps = nullptr;  // phase timeline (MOE_STAMP) or null
  __device__ float* next_red() {
    float* r = red + parity * red_stride;
    parity ^= 1;
    return r;
  }
};

// Team layout of a context: teams of tsz threads (whole waves).  The team and the wave
// within it are wave-uniform, so they live in scalar registers: item indices and weight-row
// addresses derived from them are then scalar arithmetic.
__device__ __forceinline__ void set_teams(Ctx& c, int tsz) {
  c.tsz = tsz;
  c.wpt = tsz / kWave;
  c.nteams = c.nthreads / tsz;
  c.team = __builtin_amdgcn_readfirstlane(c.tid / tsz);
  c.t = c.tid % tsz;
  c.wit = __builtin_amdgcn_readfirstlane(c.t / kWave);
}

// x values of this thread's chunks (E elements each; zero past the row end).
template <int E, int CPT>
__device__ __forceinline__ void load_x(const float* x, const Ctx& c, float (&xv)[CPT * E]) {
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int ch = c.t + m * c.tsz;
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      f32x4 v = {0, 0, 0, 0};
      if (ch < c.nch) v = reinterpret_cast<const f32x4*>(x)[(E / 4) * ch + q];
      xv[m * E + 4 * q + 0] = v.x; xv[m * E + 4 * q + 1] = v.y;
      xv[m * E + 4 * q + 2] = v.z; xv[m * E + 4 * q + 3] = v.w;
    }
  }
}

// x of a thread's 16-element chunks as f16 pairs for the MXFP4 dot products: per chunk,
// x * 2^-e with e chosen from the chunk's largest |x| so that the values sit well inside
// the f16 range (largest magnitude in [2^14, 2^15)), and 2^e to scale the dot back.
template <int CPT>
struct XHalf {
  f16x2 p[CPT][8];
  float sc[CPT];
};

template <int CPT>
__device__ __forceinline__ void load_x_half(const float* x, const Ctx& c, XHalf<CPT>& xh) {
  float v[CPT * 16];
  load_x<16, CPT>(x, c, v);
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[16 * m + i]));
    // binary exponent of mx (subnormal or zero: -127; the scale then stays finite)
    const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFF) - 127;
    const int e = ex - 14;
    xh.sc[m] = ldexpf(1.0f, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xh.p[m][j].x = (_Float16)ldexpf(v[16 * m + 2 * j], -e);
      xh.p[m][j].y = (_Float16)ldexpf(v[16 * m + 2 * j + 1], -e);
    }
  }
}

// This thread's share of the dot product of a weight row with x (before the sum over the
// team): fp32 fused multiply-adds for float x, or, for MXFP4 chunks with x as f16 pairs,
// the hardware fp4 -> f16 conversion and two-element f16 dot products accumulated in fp32,
// scaled by the block scale and 2^e afterwards.
template <DT dt, int CPT, int N>
__device__ __forceinline__ float xdot(const typename Fmt<dt>::Raw (&r)[CPT],
                                      const float (&xv)[N]) {
  return chunk_dot<dt, CPT>(r, xv);
}
template <DT dt, int CPT>
__device__ __forceinline__ float xdot(const typename Fmt<dt>::Raw (&r)[CPT],
                                      const XHalf<CPT>& xh) {
  static_assert(dt == DT::MXFP4W, "f16 x pairs serve the 16-element MXFP4 chunks");
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const uint32_t w[2] = {r[m].q.x, r[m].q.y};
    float d = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const f16x2* xp = &xh.p[m][4 * k];
      d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 0),
                                 xp[0], d, false);
      d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 1),
                                 xp[1], d, false);
      d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 2),
                                 xp[2], d, false);
      d = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 3),
                                 xp[3], d, false);
    }
    // e8m0 scale 2^(s-127) (a zero byte gives 0, as in the fp32 decode)
    s = fmaf(d * __uint_as_float((uint32_t)r[m].s << 23), xh.sc[m], s);
  }
  return s;
}

// Where the chunks of one slot (weight row `row`, row < 0 for an empty slot) are loaded
// from.  Every slot is loaded unconditionally: a load under a branch makes the compiler wait
// for all loads in flight before the next use of any of them.
//   BUF: buffer resources over the row and its scale row.  An empty slot gets resources of
//     0 bytes, whose loads return zeros without a memory access, and the lanes past the row
//     end read zeros: for streams with many empty slots.
//   otherwise: global loads from wave-uniform pointers, slightly cheaper per load.  An empty
//     slot reads the zeroed row; lanes past the row end re-read its last chunk (their x
//     values are zero and their outputs are never stored).
template <DT dt, bool BUF> struct RowSrc;
template <DT dt> struct RowSrc<dt, true> {
  rsrc_t w, s;
  __device__ __forceinline__ void set(const void* base, const uint8_t* scales, size_t r,
                                      bool ok, const Ctx& c) {
    w = make_rsrc(row_ptr<dt>(base, r, c.H), ok ? (uint32_t)Fmt<dt>::row_bytes(c.H) : 0u);
    s = make_rsrc(scales ? scale_row_ptr(scales, r, c.H) : base,
                  ok && scales ? (uint32_t)(c.H / 32) : 0u);
  }
  __device__ __forceinline__ typename Fmt<dt>::Raw load(int ch, const Ctx&) const {
    return Fmt<dt>::load_b(w, s, ch);
  }
};
template <DT dt> struct RowSrc<dt, false> {
  const gbl_u8 *w, *s;
  __device__ __forceinline__ void set(const void* base, const uint8_t* scales, size_t r,
                                      bool ok, const Ctx& c) {
    w = uniform_ptr(ok ? reinterpret_cast<const uint8_t*>(row_ptr<dt>(base, r, c.H)) : c.zrow);
    s = uniform_ptr(ok && scales ? scale_row_ptr(scales, r, c.H) : c.zrow);
  }
  __device__ __forceinline__ typename Fmt<dt>::Raw load(int ch, const Ctx& c) const {
    return Fmt<dt>::load_g(w, s, ch < c.nch ? ch : c.nch - 1);
  }
};

template <DT dt, bool BUF>
__device__ __forceinline__ RowSrc<dt, BUF> slot_rows(const void* base, const uint8_t* scales,
                                                     long long row, const Ctx& c) {
  // the row index is wave-uniform: in scalar registers, the address arithmetic is scalar too
  const uint64_t ru = (uint64_t)row;
  const long long rs = (long long)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ru >> 32))
                                    << 32) |
                                   __builtin_amdgcn_readfirstlane((uint32_t)ru));
  RowSrc<dt, BUF> src;
  src.set(base, scales, rs >= 0 ? (size_t)rs : 0, rs >= 0, c);
  return src;
}

// After the barrier that follows the waves' writes of their NP partial totals to
// red[(team * wpt + wave) * NP + p]: the team totals, lane l holding total l % NP.  Lane l
// sums the partials l, l + 64, ... of the team's wpt * NP, then lanes of equal l % NP are
// summed by exchanges across the higher lane bits.  Total p is then readlane(v, p).
template <int NP>
__device__ __forceinline__ float team_totals(const float* red, const Ctx& c) {
  const float* tr = red + c.team * c.wpt * NP;
  const int n = c.wpt * NP;
  float v = c.lane < n ? tr[c.lane] : 0.0f;
  for (int o = c.lane + kWave; o < n; o += kWave) v += tr[o];
  return sum_lanes_above<NP>(v);
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Team dot products of C rows with x, in two halves so that the loads can be issued early
// and other loads queued behind them: team_dots_load issues the loads of rows[] (rows[c] < 0
// marks an empty slot), team_dots_compute returns, in every thread of the team, the C totals
// (out[c]) -- one barrier; all threads must call.  team_dots does both.
template <DT dt, int C, int CPT>
struct TeamRows {
  typename Fmt<dt>::Raw r[C][CPT];
};
template <DT dt, int C, int CPT>
__device__ __forceinline__ void team_dots_load(const void* base, const uint8_t* scales,
                                               const long long (&rows)[C], const Ctx& c,
                                               TeamRows<dt, C, CPT>& tr) {
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const RowSrc<dt, true> src = slot_rows<dt, true>(base, scales, rows[q], c);
#pragma unroll
    for (int m = 0; m < CPT; ++m) tr.r[q][m] = src.load(c.t + m * c.tsz, c);
  }
}
template <DT dt, int C, int CPT>
__device__ __forceinline__ void team_dots_compute(const TeamRows<dt, C, CPT>& tr,
                                                  const float (&xv)[CPT * kE<dt>], Ctx& c,
                                                  float (&out)[C]) {
  constexpr int NP = NextPow2<C>::value;
  float acc[NP];
#pragma unroll
  for (int q = 0; q < C; ++q) acc[q] = chunk_dot<dt, CPT>(tr.r[q], xv);
#pragma unroll
  for (int q = C; q < NP; ++q) acc[q] = 0.0f;
  const float tot = wave_multi_sum<NP>(acc, c.lane);
  float* red = c.next_red();
  if (c.lane < NP) red[(c.team * c.wpt + c.wit) * NP + c.lane] = tot;
  __syncthreads();
  const float v = team_totals<NP>(red, c);
#pragma unroll
  for (int q = 0; q < C; ++q) out[q] = lane_value(v, q);
}
template <DT dt, int C, int CPT>
__device__ __forceinline__ void team_dots(const void* base, const uint8_t* scales,
                                          const long long (&rows)[C],
                                          const float (&xv)[CPT * kE<dt>], Ctx& c,
                                          float (&out)[C]) {
  TeamRows<dt, C, CPT> tr;
  team_dots_load<dt, C, CPT>(base, scales, rows, c, tr);
  team_dots_compute<dt, C, CPT>(tr, xv, c, out);
}

// Raw weight chunks of one batch of C SwiGLU channels per team (one pipeline stage).
template <DT dt, int C, int CPT>
struct Stage {
  typename Fmt<dt>::Raw g[C][CPT], v[C][CPT], d[C][CPT];
  float wt[C], gv[C];
  bool live;
};

// Issue the loads of one batch (rows row[q] < 0 are empty slots; G == nullptr: no gate
// rows, the gate values come in gv[]).
template <DT dt, int C, int CPT, bool HAS_G, bool BUF>
__device__ __forceinline__ void stage_load(Stage<dt, C, CPT>& st, const void* G, const void* V,
                                           const void* D, const uint8_t* Gs, const uint8_t* Vs,
                                           const uint8_t* Ds, const long long (&row)[C],
                                           const Ctx& c) {
#pragma unroll
  for (int q = 0; q < C; ++q) {
    // the row is the same for every lane of the wave (one team = whole waves)
    RowSrc<dt, BUF> gs;
    if constexpr (HAS_G) gs = slot_rows<dt, BUF>(G, Gs, row[q], c);
    const RowSrc<dt, BUF> vs = slot_rows<dt, BUF>(V, Vs, row[q], c);
    const RowSrc<dt, BUF> ds = slot_rows<dt, BUF>(D, Ds, row[q], c);
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int ch = c.t + m * c.tsz;
      if constexpr (HAS_G) st.g[q][m] = gs.load(ch, c);
      st.v[q][m] = vs.load(ch, c);
      st.d[q][m] = ds.load(ch, c);
    }
  }
}

// Gate and up dots of a loaded batch, team reduction through LDS (one barrier),
// silu(g)*u*wt, and the accumulation of that activation times the down row into yv.
// All threads of the workgroup must call.
template <DT dt, int C, int CPT, bool HAS_G, typename X>
__device__ __forceinline__ void stage_compute(const Stage<dt, C, CPT>& st, const X& xv,
                                              float (&yv)[CPT * kE<dt>], Ctx& c) {
  constexpr int E = kE<dt>;
  constexpr int NP = NextPow2<2 * C>::value;
  float acc[NP];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    acc[q] = HAS_G ? xdot<dt, CPT>(st.g[q], xv) : 0.0f;
    acc[C + q] = xdot<dt, CPT>(st.v[q], xv);
  }
#pragma unroll
  for (int i = 2 * C; i < NP; ++i) acc[i] = 0.0f;
  const float tot = wave_multi_sum<NP>(acc, c.lane);
  float* red = c.next_red();
  if (c.lane < NP) red[(c.team * c.wpt + c.wit) * NP + c.lane] = tot;
  __syncthreads();
  const float v = team_totals<NP>(red, c);
#pragma unroll
  for (int q = 0; q < C; ++q) {
    float g = lane_value(v, q);
    const float u = lane_value(v, C + q);
    if (!HAS_G) g = st.gv[q];
    const float act = silu(g) * u * st.wt[q];
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      float d[E];
      Fmt<dt>::decode(st.d[q][m], d);
#pragma unroll
      for (int i = 0; i < E; ++i) yv[m * E + i] = fmaf(act, d[i], yv[m * E + i]);
    }
  }
}

// Stream items [i0, i1) in batches of C per team, two batches in flight: the loads of
// batch b+1 are issued before batch b is reduced.  map(i, row, wt, gv) gives the weight
// row of item i (row < 0: skip), its weight and (HAS_G false: no gate rows are read) its
// gate value  BUF: the load path (RowSrc).
template <DT dt, int C, int CPT, bool HAS_G, bool BUF, typename Map, typename X,
          typename Between>
__device__ inline void stream_channels(const void* G, const void* V, const void* D,
                                       const uint8_t* Gs, const uint8_t* Vs, const uint8_t* Ds,
                                       int i0, int i1, Map map, const X& xv,
                                       float (&yv)[CPT * kE<dt>], Ctx& c, Between between) {
  const int per = c.nteams * C;
  const int nb = i1 > i0 ? (i1 - i0 + per - 1) / per : 0;
  auto fill = [&](Stage<dt, C, CPT>& st, int b) {
    long long row[C];
#pragma unroll
    for (int q = 0; q < C; ++q) {
      const int i = i0 + b * per + c.team * C + q;
      row[q] = -1;
      st.wt[q] = 0.0f;
      st.gv[q] = 0.0f;
      if (i < i1) map(i, row[q], st.wt[q], st.gv[q]);
    }
    stage_load<dt, C, CPT, HAS_G, BUF>(st, G, V, D, Gs, Vs, Ds, row, c);
  };
  // Pairs of batches, then an odd last one.  The loads of every stage are issued without
  // a condition (a batch past the end reads the zero row), so that the compiler's wait
  // before each compute covers exactly that stage's loads: after a conditional load it
  // would also wait for the other stage.
  Stage<dt, C, CPT> A, B;
  fill(A, 0);
  between();  // work that waits on loads issued before this stream's first ones
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    fill(B, b + 1);
    stage_compute<dt, C, CPT, HAS_G>(A, xv, yv, c);
    fill(A, b + 2);
    stage_compute<dt, C, CPT, HAS_G>(B, xv, yv, c);
  }
  if (b < nb) stage_compute<dt, C, CPT, HAS_G>(A, xv, yv, c);
}
template <DT dt, int C, int CPT, bool HAS_G, bool BUF, typename Map, typename X>
__device__ inline void stream_channels(const void* G, const void* V, const void* D,
                                       const uint8_t* Gs, const uint8_t* Vs, const uint8_t* Ds,
                                       int i0, int i1, Map map, const X& xv,
                                       float (&yv)[CPT * kE<dt>], Ctx& c) {
  stream_channels<dt, C, CPT, HAS_G, BUF>(G, V, D, Gs, Vs, Ds, i0, i1, map, xv, yv, c, [] {});
}

// Expert rows of a slot stream: NS shared slots first (slot s < NS: the I_s rows of shared
// expert s, weight 1), then the k routed slots (slot NS + r: the I rows of expert s_ids[r],
// weight s_w[r]; an id < 0 is an empty slot).  All slots share one row format.
struct SlotSet {
  const uint8_t *G, *V, *D;        // routed [E][I][H]
  const uint8_t *Gs, *Vs, *Ds;     // routed MXFP4 scales or null
  const uint8_t *SG, *SV, *SD;     // shared [NS][IS][H] (NS > 0)
  int I, IS, NS, k;
  const int* s_ids;
  const float* s_w;
};

// A workgroup's share of the slot stream: shared channels [s0, s1) (flat shared channel f is
// row f % IS of shared expert f / IS) followed by routed channels [r0, r1) (flat routed
// channel f is row f % I of routed slot f / I), walked as one sequence of items.  Giving
// every workgroup a slice of both keeps the shared rows spread over the whole chip.
struct SlotShare {
  int s0, s1, r0, r1;
};
// Reducer workgroups have the reduction to do after their stream, so they take a smaller
// share of it: kReducerShare / kShareUnit of a plain workgroup's.  share_prefix(w) is the
// stream position (in units) where workgroup w's share starts.
constexpr int kShareUnit = 16, kReducerShare = 16;
__host__ __device__ __forceinline__ long long share_prefix(int w, int P, int R) {
  // reducers below w: the odd w' < w with (w' >> 1) < R (all w' < w when P < 2)
  const int red = P < 2 ? (w < R ? w : R) : (w / 2 < R ? w / 2 : R);
  return (long long)w * kShareUnit - (long long)red * (kShareUnit - kReducerShare);
}
__device__ __forceinline__ SlotShare slot_share(const SlotSet& ss, const Ctx& c, int R) {
  const long long nsh = (long long)ss.NS * ss.IS, nrt = (long long)ss.k * ss.I;
  const long long tot = share_prefix(c.P, c.P, R);
  const long long a = share_prefix(c.wg, c.P, R), b = share_prefix(c.wg + 1, c.P, R);
  SlotShare sh;
  sh.s0 = (int)(nsh * a / tot);
  sh.s1 = (int)(nsh * b / tot);
  sh.r0 = (int)(nrt * a / tot);
  sh.r1 = (int)(nrt * b / tot);
  return sh;
}

// The share's items, in batches of C per team, two batches in flight, as stream_channels.
// The team's items are walked incrementally: (slot, j) of its next first item advances by a
// batch per fill, and the current and next slot's row bases stay in scalar registers, so an
// item's three row addresses are a 32-bit multiply and pointer adds (a row offset within one
// expert, I * row bytes, stays below 2^32).  Every wave of the compute unit issues this
// scalar code, and scalar instructions issue at the rate of vector ones, so per-item
// divisions and 64-bit multiplications made the stream scalar-bound.  Only the step from the
// shared items to the routed ones (once per team) divides again.
template <DT dt, int C, int CPT, typename X>
__device__ inline void stream_routed(const SlotSet& ss, const SlotShare& sh, const X& xv,
                                     float (&yv)[CPT * kE<dt>], Ctx& c) {
  using F = Fmt<dt>;
  const int per = c.nteams * C;
  const int ns = sh.s1 - sh.s0, n = ns + (sh.r1 - sh.r0);
  const int nb = (n + per - 1) / per;
  const uint32_t rb = (uint32_t)F::row_bytes(c.H);
  const uint32_t sb = (uint32_t)(c.H / 32);
  const int nsl = ss.NS + ss.k;
  struct SlotState {
    const uint8_t *g, *v, *d;     // first row of the slot's expert
    const uint8_t *gs, *vs, *ds;  // its scale rows (or null)
    float wt;
    int width;                    // channels of the slot
    bool ok;
  };
  auto slot_state = [&](int sl) {
    SlotState st;
    st.gs = st.vs = st.ds = nullptr;
    if (sl < ss.NS) {
      const uint64_t o = (uint64_t)(uint32_t)sl * (uint32_t)ss.IS * rb;
      st.g = ss.SG + o;
      st.v = ss.SV + o;
      st.d = ss.SD + o;
      st.wt = 1.0f;
      st.width = ss.IS;
      st.ok = true;
    } else {
      const int r = sl - ss.NS;
      const int rc = r < ss.k ? r : 0;
      const int e = __builtin_amdgcn_readfirstlane(ss.s_ids[rc]);
      st.ok = r < ss.k && e >= 0;
      const uint64_t row = (uint64_t)(st.ok ? e : 0) * (uint64_t)ss.I;
      st.g = ss.G + row * rb;
      st.v = ss.V + row * rb;
      st.d = ss.D + row * rb;
      if (ss.Gs) {
        st.gs = ss.Gs + row * sb;
        st.vs = ss.Vs + row * sb;
        st.ds = ss.Ds + row * sb;
      }
      st.wt = ss.s_w[rc];
      st.width = ss.I;
    }
    return st;
  };
  // (slot, j) of the share's item v (divisions)
  auto pos_of = [&](int v, int& slot, int& j) {
    if (v < ns) {
      const int f = sh.s0 + v;
      slot = f / ss.IS;
      j = f - slot * ss.IS;
    } else {
      const int f = sh.r0 + (v - ns);
      slot = ss.NS + f / ss.I;
      j = f - (slot - ss.NS) * ss.I;
    }
    if (slot > nsl) slot = nsl;
  };
  int v = c.team * C;  // the team's first item of the next batch
  int slot, j;
  pos_of(v, slot, j);
  SlotState cur = slot_state(slot), nxt = slot_state(slot + 1 < nsl ? slot + 1 : nsl);
  const int ch0 = c.t;
  auto fill = [&](Stage<dt, C, CPT>& st) {
    const bool straddle = v < ns && v + C > ns;  // the batch holds both kinds of items
#pragma unroll
    for (int q = 0; q < C; ++q) {
      int jq;
      SlotState sq;
      if (C > 1 && straddle) {
        int sl;
        pos_of(v + q, sl, jq);
        sq = slot_state(sl);
      } else {
        const bool wrap = j + q >= cur.width;
        jq = wrap ? j + q - cur.width : j + q;
        sq = wrap ? nxt : cur;
      }
      const bool live = v + q < n && sq.ok;
      const uint32_t od = (uint32_t)jq * rb;
      const uint32_t os = (uint32_t)jq * sb;
      RowSrc<dt, false> gsrc, vsrc, dsrc;
      gsrc.w = uniform_ptr(live ? sq.g + od : c.zrow);
      vsrc.w = uniform_ptr(live ? sq.v + od : c.zrow);
      dsrc.w = uniform_ptr(live ? sq.d + od : c.zrow);
      gsrc.s = uniform_ptr(live && sq.gs ? sq.gs + os : c.zrow);
      vsrc.s = uniform_ptr(live && sq.vs ? sq.vs + os : c.zrow);
      dsrc.s = uniform_ptr(live && sq.ds ? sq.ds + os : c.zrow);
      st.wt[q] = live ? sq.wt : 0.0f;
      st.gv[q] = 0.0f;
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const int ch = ch0 + m * c.tsz;
        st.g[q][m] = gsrc.load(ch, c);
        st.v[q][m] = vsrc.load(ch, c);
        st.d[q][m] = dsrc.load(ch, c);
      }
    }
    const int v0 = v;
    v += per;
    if (v0 < ns && v >= ns) {  // from the shared items to the routed ones
      pos_of(v, slot, j);
      cur = slot_state(slot);
      nxt = slot_state(slot + 1 < nsl ? slot + 1 : nsl);
    } else {
      j += per;
      while (j >= cur.width && slot < nsl) {
        j -= cur.width;
        ++slot;
        cur = nxt;
        nxt = slot_state(slot + 1 < nsl ? slot + 1 : nsl);
      }
    }
  };
  Stage<dt, C, CPT> A, B;
  fill(A);
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    fill(B);
    stage_compute<dt, C, CPT, true>(A, xv, yv, c);
    fill(A);
    stage_compute<dt, C, CPT, true>(B, xv, yv, c);
  }
  if (b < nb) stage_compute<dt, C, CPT, true>(A, xv, yv, c);
}

// The routed experts only (no shared slots; the MXFP4 layer), channels [i0, i1): flat
// channel f = slot * I + j is row j of expert
// s_ids[slot] (negative: an empty slot), weighted by s_w[slot].  The same two-stage stream
// as stream_channels, but the team's items are walked incrementally: (slot, j) of its next
// first item advances by a batch per fill, and the current and next slot's expert offsets
// stay in scalar registers, so an item's three row addresses are a 32-bit multiply and
// 64-bit adds (the host admits E * I < 2^31; a row offset within one expert, I * row bytes,
// stays below 2^32).  Every wave of the compute unit issues this scalar code, and scalar
// instructions issue at the rate of vector ones, so the per-item divisions and 64-bit
// multiplications of the generic map made the stream scalar-bound.
template <DT dt, int C, int CPT, typename X>
__device__ inline void stream_routed_flat(const void* G, const void* V, const void* D,
                                     const uint8_t* Gs, const uint8_t* Vs, const uint8_t* Ds,
                                     int i0, int i1, int I, int k, const int* s_ids,
                                     const float* s_w, const X& xv,
                                     float (&yv)[CPT * kE<dt>], Ctx& c) {
  using F = Fmt<dt>;
  const int per = c.nteams * C;
  const int nb = i1 > i0 ? (i1 - i0 + per - 1) / per : 0;
  const uint32_t rb = (uint32_t)F::row_bytes(c.H);
  const uint32_t sb = (uint32_t)(c.H / 32);
  const uint8_t* const gb = reinterpret_cast<const uint8_t*>(G);
  const uint8_t* const vb = reinterpret_cast<const uint8_t*>(V);
  const uint8_t* const db = reinterpret_cast<const uint8_t*>(D);
  struct SlotState {
    uint64_t od, os;  // byte offsets of the expert's rows and scale rows
    float wt;
    bool ok;
  };
  auto slot_state = [&](int sl) {
    SlotState st;
    const int sc = sl < k ? sl : 0;
    const int e = __builtin_amdgcn_readfirstlane(s_ids[sc]);
    st.ok = sl < k && e >= 0;
    const uint64_t r = (uint64_t)(st.ok ? e : 0) * (uint64_t)I;
    st.od = r * rb;
    st.os = r * sb;
    st.wt = s_w[sc];
    return st;
  };
  int f = i0 + c.team * C;  // the team's first item of the next batch
  int slot = f / I, j = f - slot * I;
  SlotState cur = slot_state(slot), nxt = slot_state(slot + 1);
  const int ch0 = c.t;
  auto fill = [&](Stage<dt, C, CPT>& st) {
#pragma unroll
    for (int q = 0; q < C; ++q) {
      const bool wrap = j + q >= I;
      const int jq = wrap ? j + q - I : j + q;
      const SlotState& ss = wrap ? nxt : cur;
      const bool live = f + q < i1 && ss.ok;
      const uint64_t od = ss.od + (uint64_t)((uint32_t)jq * rb);
      const uint64_t os = ss.os + (uint64_t)((uint32_t)jq * sb);
      RowSrc<dt, false> gs, vs, ds;
      gs.w = uniform_ptr(live ? gb + od : c.zrow);
      vs.w = uniform_ptr(live ? vb + od : c.zrow);
      ds.w = uniform_ptr(live ? db + od : c.zrow);
      gs.s = uniform_ptr(live && Gs ? Gs + os : c.zrow);
      vs.s = uniform_ptr(live && Vs ? Vs + os : c.zrow);
      ds.s = uniform_ptr(live && Ds ? Ds + os : c.zrow);
      st.wt[q] = live ? ss.wt : 0.0f;
      st.gv[q] = 0.0f;
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const int ch = ch0 + m * c.tsz;
        st.g[q][m] = gs.load(ch, c);
        st.v[q][m] = vs.load(ch, c);
        st.d[q][m] = ds.load(ch, c);
      }
    }
    f += per;
    j += per;
    while (j >= I) {
      j -= I;
      ++slot;
      cur = nxt;
      nxt = slot_state(slot + 1);
    }
  };
  Stage<dt, C, CPT> A, B;
  fill(A);
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    fill(B);
    stage_compute<dt, C, CPT, true>(A, xv, yv, c);
    fill(A);
    stage_compute<dt, C, CPT, true>(B, xv, yv, c);
  }
  if (b < nb) stage_compute<dt, C, CPT, true>(A, xv, yv, c);
}

// Warm L2 with rows [s0, s1) of three stacked [rows][H] tensors (a share's shared-expert
// rows, which do not depend on routing), using the threads from `first` on (whose waves have
// nothing else in flight): one 4-byte load per 128-byte line, plain loads so that the lines
// are allocated in L2 and the stream's later reads of them hit there, at most kWarmLoads per
// thread.  The values go to w[], which the caller keeps alive to the end of the kernel, so
// the loads are neither removed nor waited for before then.
constexpr int kWarmLoads = 2;
__device__ inline void warm_rows(const uint8_t* G, const uint8_t* V, const uint8_t* D, int s0,
                                 int s1, uint32_t rb, int first, const Ctx& c,
                                 uint32_t (&w)[kWarmLoads]) {
  const uint32_t lines = s1 > s0 ? (uint32_t)(s1 - s0) * (rb / 128) : 0u;  // per tensor
  const uint32_t nthr = c.nthreads > first ? (uint32_t)(c.nthreads - first) : 1u;
  const uint32_t me = c.tid >= first ? (uint32_t)(c.tid - first) : 3u * lines;
#pragma unroll
  for (int u = 0; u < kWarmLoads; ++u) {
    const uint32_t i = me + (uint32_t)u * nthr;
    w[u] = 0;
    if (i < 3 * lines) {
      const uint32_t t = i / lines, r = i - t * lines;
      const uint8_t* base = t == 0 ? G : t == 1 ? V : D;
      w[u] = *reinterpret_cast<const uint32_t*>(base + (size_t)s0 * rb + 128ull * r);
    }
  }
}

// Router logits, spread over all workgroups: workgroup wg computes rows wg, wg + P, ...
// (one team per row), so every router row is done at about the same time and no workgroup
// carries more than ceil(E / P) rows.  In two halves: router_issue issues the loads of the
// first round of rows (one row per team) so that the shared experts' first loads can be
// queued right behind them; router_finish computes those dots (then any further rounds),
// and publishes each logit as one 64-bit word: the launch tag (epoch + 1) in the upper half
// and the fp32 bits in the lower half, so readers wait on the data itself.  Every workgroup
// also learns the launch epoch here (thread 0 loaded it at the start).  `buf` is LDS of at
// least ceil(E / P) floats; s_ep one LDS word.
template <DT RT, int CPT>
struct RouterRound {
  int nrows;  // this workgroup's rows (wave-uniform)
  TeamRows<RT, 1, CPT> tr;
};
template <DT RT, int CPT>
__device__ inline void router_issue(bool compute, const void* router, int E, const Ctx& c,
                                    RouterRound<RT, CPT>& rr) {
  rr.nrows = compute && c.wg < E ? (E - 1 - c.wg) / c.P + 1 : 0;
  // issued by every team (a row of -1 loads nothing): not under a branch, so that waits for
  // loads issued before it need not wait for it
  const long long rows[1] = {c.team < rr.nrows ? (long long)c.wg + (long long)c.P * c.team
                                               : -1ll};
  team_dots_load<RT, 1, CPT>(router, nullptr, rows, c, rr.tr);
}
template <DT RT, int CPT>
__device__ inline void router_finish(const RouterRound<RT, CPT>& rr, const void* router, int E,
                                     const float (&xv)[CPT * kE<RT>], uint64_t* rlog,
                                     float* buf, uint32_t* s_ep, Ctx& c) {
  const int nrows = rr.nrows;
  if (nrows > 0) {
    float l[1];
    team_dots_compute<RT, 1, CPT>(rr.tr, xv, c, l);
    if (c.t == 0 && c.team < nrows) buf[c.team] = l[0];
    for (int m0 = c.nteams; m0 < nrows; m0 += c.nteams) {
      const int m = m0 + c.team;
      const long long rows[1] = {m < nrows ? (long long)c.wg + (long long)c.P * m : -1ll};
      team_dots<RT, 1, CPT>(router, nullptr, rows, xv, c, l);
      if (c.t == 0 && m < nrows) buf[m] = l[0];
    }
    MOE_STAMP(c.stamps, kStampRouterDots);
  }
  if (c.tid == 0) *s_ep = c.epoch;
  __syncthreads();
  c.epoch = *s_ep;
  const uint64_t tag = (uint64_t)(c.epoch + 1u) << 32;
  // one copy per XCD (E rounded up to whole 128-byte lines per copy)
  const int Ep = (E + 15) & ~15;
  for (int i = c.tid; i < nrows * kPollCopies; i += c.nthreads) {
    const int m = i % nrows, x = i / nrows;
    st_dev64(rlog + (size_t)x * Ep + c.wg + (size_t)c.P * m, tag | __float_as_uint(buf[m]));
  }
}

// Exact top-k of the E logits and the softmax over the k selected, computed by the whole
// workgroup into LDS (s_ids, s_w): the waves poll the tagged logits themselves and select in
// registers (wg_topk_bitonic); wave 0 then forms the weights.  `keys` is LDS scratch of
// topk_lds_bytes(E, k) bytes.
template <int KP, typename AfterKeys>
__device__ inline void topk_local_kp(const uint64_t* rlog, int E, int k, uint64_t* keys,
                                     int* s_ids, float* s_w, uint32_t* err, const Ctx& c,
                                     AfterKeys after_keys) {
  const uint32_t tag = c.epoch + 1u;
  const uint64_t* copy = rlog + (size_t)(c.wg % kPollCopies) * ((E + 15) & ~15);
  const uint64_t top = wg_topk_bitonic<KP>(
      E,
      [&](int e) {
        const uint64_t v = wait_tagged(copy + e, tag, err, kErrRouteWait);
        return make_key(__uint_as_float((uint32_t)v), (uint32_t)e);
      },
      keys, c.stamps, after_keys);
  MOE_STAMP_AFTER(c.stamps, kStampRanked, top);
  if (c.tid < kWave) {
    // the largest selected logit (lane 0's key) for a max-subtracted softmax
    const float l0 = from_ordered_bits(__builtin_amdgcn_readfirstlane((uint32_t)(top >> 32)));
    const float ex = c.tid < k ? expf(key_value(top) - l0) : 0.0f;
    const float sum = wave_sum(ex);
    if (c.tid < k) {
      s_ids[c.tid] = (int)key_index(top);
      s_w[c.tid] = ex / sum;
    }
  }
  __syncthreads();
}
template <typename AfterKeys>
__device__ inline void topk_local(const uint64_t* rlog, int E, int k, uint64_t* keys,
                                  int* s_ids, float* s_w, uint32_t* err, const Ctx& c,
                                  AfterKeys after_keys) {
  if (k <= 1) topk_local_kp<1>(rlog, E, k, keys, s_ids, s_w, err, c, after_keys);
  else if (k <= 2) topk_local_kp<2>(rlog, E, k, keys, s_ids, s_w, err, c, after_keys);
  else if (k <= 4) topk_local_kp<4>(rlog, E, k, keys, s_ids, s_w, err, c, after_keys);
  else if (k <= 8) topk_local_kp<8>(rlog, E, k, keys, s_ids, s_w, err, c, after_keys);
  else if (k <= 16) topk_local_kp<16>(rlog, E, k, keys, s_ids, s_w, err, c, after_keys);
  else if (k <= 32) topk_local_kp<32>(rlog, E, k, keys, s_ids, s_w, err, c, after_keys);
  else topk_local_kp<64>(rlog, E, k, keys, s_ids, s_w, err, c, after_keys);
}

// The routing of this token in LDS (s_ids, s_w).  Inside the launch: wait until every
// router workgroup has published its logits, then select the top-k in this workgroup (each
// workgroup sorts the E logits itself, which costs less than one more cross-workgroup
// hand-off).  Given routing: copy ids/w; an id outside [0, E), or equal to an earlier id of
// the token, is reported and skipped (-1), so a repeated expert counts once (its first
// choice).  Workgroup 0 also stores the routing it used into ids_ws / w_ws [k], where the
// host can read back what the launch chose.
template <typename AfterKeys = NoHook>
__device__ inline void fetch_routing(bool inside, const uint64_t* rlog, const int32_t* ids_in,
                                     const float* w_in, int E, int k, Ctrl* ctrl,
                                     uint64_t* keys, int* s_ids, float* s_w, int32_t* ids_ws,
                                     float* w_ws, const Ctx& c,
                                     AfterKeys after_keys = AfterKeys()) {
  if (inside) {
    topk_local(rlog, E, k, keys, s_ids, s_w, &ctrl->err, c, after_keys);
  } else {
    if (c.tid < k) {
      int e = ids_in[c.tid];
      bool bad = e < 0 || e >= E;
      for (int j = 0; j < c.tid && !bad; ++j) bad = ids_in[j] == e;
      if (bad) {
        if (c.wg == 0)
          __hip_atomic_fetch_or(&ctrl->err, kErrBadId, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        e = -1;
      }
      s_ids[c.tid] = e;
      s_w[c.tid] = w_in[c.tid];
    }
    __syncthreads();
  }
  if (c.wg == 0 && c.tid < k) {
    ids_ws[c.tid] = s_ids[c.tid];
    w_ws[c.tid] = s_w[c.tid];
  }
}

// This workgroup's output partial in LDS big[0 .. H): the teams' register vectors summed
// in team order (big needs nteams * H floats).  E-element chunks.
template <int E, int CPT>
__device__ inline void teams_to_lds(const float (&yv)[CPT * E], float* big, const Ctx& c) {
  const int H = c.H;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int ch = c.t + m * c.tsz;
    if (ch < c.nch) {
#pragma unroll
      for (int q = 0; q < E / 4; ++q)
        reinterpret_cast<f32x4*>(big + c.team * H)[(E / 4) * ch + q] =
            f32x4{yv[m * E + 4 * q], yv[m * E + 4 * q + 1], yv[m * E + 4 * q + 2],
                  yv[m * E + 4 * q + 3]};
    }
  }
  __syncthreads();
  if (c.nteams > 1) {
    for (int h = c.tid; h < H; h += c.nthreads) {
      float s = big[h];
      for (int tm = 1; tm < c.nteams; ++tm) s += big[tm * H + h];
      big[h] = s;
    }
    __syncthreads();
  }
}

// Each team's register vector to its own H-vector of LDS, buf[team * H .. + H) (16-byte
// stores, no read-modify-write: a team's lanes hold E consecutive values each, so E-float
// read-modify-writes at that stride serialised on a few LDS banks, ~3 us per team at
// H = 7168).  The sum over teams is taken by the reader, in team order.
template <int E, int CPT>
__device__ inline void teams_to_lds_split(const float (&yv)[CPT * E], float* buf, const Ctx& c) {
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int ch = c.t + m * c.tsz;
    if (ch < c.nch) {
#pragma unroll
      for (int q = 0; q < E / 4; ++q)
        reinterpret_cast<f32x4*>(buf + c.team * c.H)[(E / 4) * ch + q] =
            f32x4{yv[m * E + 4 * q], yv[m * E + 4 * q + 1], yv[m * E + 4 * q + 2],
                  yv[m * E + 4 * q + 3]};
    }
  }
  __syncthreads();
}

// Publish src[0 .. H) (default: big), plus nadds more H-vectors at adds, as this workgroup's
// partial output row, then (R fixed
// workgroups, every (P/R)-th) sum an SW-column slice of y over all P partial rows in a
// fixed order.  Deterministic: no float atomics, the same order in every launch.
//
// Hand-off without counters or fences: every value of a partial row carries the launch's
// parity ((epoch + 1) & 1) in its lowest mantissa bit, and is written with device-scope
// 64-bit stores; the reducer clears that bit again before adding, so the sum sees the value
// with its last mantissa bit cleared in every launch (a change of at most one unit in the
// last place, the same in every launch: results stay bit-identical).  Every launch writes every
// partial row in full, so before this launch's store a word holds the previous launch's
// value, whose parity differs (or the zeros of layer creation, parity 0, before the first
// launch, whose parity is 1).  A reducer therefore polls the partial values themselves:
// it is done with a word once both of its floats show this launch's parity, so the sum
// starts as the partials arrive and ends one round trip after the last one lands.  The
// first reducer, once it has seen every workgroup's partial (so every workgroup has read the
// epoch), advances the epoch for the next launch.  `big` is LDS of at least
// max(H, nthreads) floats.
// Which workgroups reduce: the odd ones, 1, 3, ..., 2R - 1 (R <= P / 2), so that the reducers
// are spread over the XCDs of odd index (workgroup w runs on XCD w % 8) rather than stacked on
// two of them.  Returns the reducer index, or -1.
__host__ __device__ __forceinline__ int reducer_index(int wg, int P, int R) {
  if (P < 2) return wg < R ? wg : -1;
  return (wg & 1) && (wg >> 1) < R ? wg >> 1 : -1;
}

__device__ __forceinline__ float with_parity(float v, uint32_t par) {
  return __uint_as_float((__float_as_uint(v) & ~1u) | par);
}
__device__ inline bool parity_ok(uint64_t v, uint32_t par) {
  return (((uint32_t)v & 1u) == par) && (((uint32_t)(v >> 32) & 1u) == par);
}
__device__ inline void publish_and_reduce(float* partials, float* y, Ctrl* ctrl, int R, int SW,
                                          float* big, const Ctx& c, const float* src = nullptr,
                                          uint32_t* ctr2 = nullptr, uint32_t ctr2_next = 0,
                                          const float* adds = nullptr, int nadds = 0) {
  const int H = c.H;
  if (!src) src = big;
  const uint32_t par = (c.epoch + 1u) & 1u;
  uint64_t* prow = reinterpret_cast<uint64_t*>(partials + (size_t)c.wg * H);
  for (int h2 = c.tid; h2 < H / 2; h2 += c.nthreads) {
    // src plus the nadds H-vectors at adds (in order)
    float a = src[2 * h2], b = src[2 * h2 + 1];
    for (int t = 0; t < nadds; ++t) {
      a += adds[t * H + 2 * h2];
      b += adds[t * H + 2 * h2 + 1];
    }
    const uint32_t lo = __float_as_uint(with_parity(a, par));
    const uint32_t hi = __float_as_uint(with_parity(b, par));
    st_dev64(prow + h2, ((uint64_t)hi << 32) | lo);
  }
  MOE_STAMP(c.stamps, kStampPublished);
  MOE_CLOCK(c.stamps, kStampClk1);
  const int r = reducer_index(c.wg, c.P, R);
  if (r < 0) return;
  __syncthreads();  // src may alias big, which the reduction below reuses
  // Thread layout of a reducer: word q = tid % NW of the slice (two columns), partial rows
  // p = g, g + G, ... with g = tid / NW; each thread sums its rows in ascending p, then the
  // G groups are summed in a fixed tree (across the lanes of a wave, then across waves).
  const int h0 = r * SW;
  const int wslice = min(SW, H - h0);
  const int NW = SW / 2;                       // words per slice row (SW is a power of two)
  const int G = c.nthreads / NW;               // row groups (NW <= 64 keeps G >= 16)
  const int q = c.tid % NW, g = c.tid / NW;
  const bool live = 2 * q < wslice;
  float s0 = 0.0f, s1 = 0.0f;
  if (live) {
    constexpr int kBatch = 8;  // loads in flight per thread
    for (int p0 = g; p0 < c.P; p0 += kBatch * G) {
      const uint64_t* src[kBatch];
      uint64_t v[kBatch];
      // rows past P are not read: a word that passes the parity check and is not summed
      const uint64_t none = (uint64_t)par | ((uint64_t)par << 32);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = min(p0 + u * G, c.P - 1);
        src[u] = reinterpret_cast<const uint64_t*>(partials + (size_t)p * H + h0) + q;
        v[u] = p0 + u * G < c.P ? ld_dev64(src[u]) : none;
      }
      // the words not yet of this launch are polled again together, so the batch costs one
      // round trip after its last word lands (bounded like wait_tagged)
      uint32_t late = 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) late |= parity_ok(v[u], par) ? 0u : 1u << u;
      if (late) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (late) {
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
            if (late & (1u << u)) v[u] = ld_dev64(src[u]);
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
            if (parity_ok(v[u], par)) late &= ~(1u << u);
          if (late && __builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
            __hip_atomic_fetch_or(&ctrl->err, kErrReduceWait, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (p0 + u * G < c.P) {
          s0 += __uint_as_float((uint32_t)v[u] & ~1u);
          s1 += __uint_as_float((uint32_t)(v[u] >> 32) & ~1u);
        }
      }
    }
  }
  MOE_STAMP(c.stamps, kStampArrived);
  // groups within a wave: lanes that share q (lane % NW), summed over the higher lane bits
  if (NW < kWave) {
    if (NW == 16) { s0 = sum_lanes_above<16>(s0); s1 = sum_lanes_above<16>(s1); }
    else if (NW == 32) { s0 = sum_lanes_above<32>(s0); s1 = sum_lanes_above<32>(s1); }
    else if (NW == 8) { s0 = sum_lanes_above<8>(s0); s1 = sum_lanes_above<8>(s1); }
    else if (NW == 4) { s0 = sum_lanes_above<4>(s0); s1 = sum_lanes_above<4>(s1); }
    else if (NW == 2) { s0 = sum_lanes_above<2>(s0); s1 = sum_lanes_above<2>(s1); }
    else { s0 = sum_lanes_above<1>(s0); s1 = sum_lanes_above<1>(s1); }
  }
  // then the waves (each holds every word of the slice once when NW <= 64), in wave order
  const int wave = c.tid / kWave, nw = c.nthreads / kWave;
  const int lane = c.tid % kWave;
  const int NWw = NW < kWave ? NW : kWave;     // words per wave
  const int wpr = NW / NWw;                    // waves per group row (NW > 64: several)
  if (lane < NWw) {
    big[2 * (wave * NWw + lane)] = s0;
    big[2 * (wave * NWw + lane) + 1] = s1;
  }
  __syncthreads();
  MOE_STAMP(c.stamps, kStampAllPolled);
  if (r == 0 && c.tid == 0) {
    store_relaxed_dev(&ctrl->epoch, c.epoch + 1u);
    if (ctr2) store_relaxed_dev(ctr2, ctr2_next);
  }
  for (int col = c.tid; col < wslice; col += c.nthreads) {
    const int qq = col / 2, par2 = col % 2;
    const int wq = qq / NWw, lq = qq % NWw;    // wave within a group row, lane
    // the (at most 16) values are read together, then added in wave order
    constexpr int kMaxWaves = 1024 / kWave;
    float v[kMaxWaves];
#pragma unroll
    for (int u = 0; u < kMaxWaves; ++u) {
      const int w0 = wq + u * wpr;
      v[u] = w0 < nw ? big[2 * (w0 * NWw + lq) + par2] : 0.0f;
    }
    float t = 0.0f;
#pragma unroll
    for (int u = 0; u < kMaxWaves; ++u) t += v[u];
    y[h0 + col] = t;
  }
  MOE_STAMP(c.stamps, kStampReduced);
}

// The whole output step for one register layout.
template <int CPT, int E = 8>
__device__ inline void reduce_output(const float (&yv)[CPT * E], float* partials, float* y,
                                     Ctrl* ctrl, int R, int SW, float* big, const Ctx& c,
                                     uint32_t* ctr2 = nullptr, uint32_t ctr2_next = 0) {
  teams_to_lds<E, CPT>(yv, big, c);
  publish_and_reduce(partials, y, ctrl, R, SW, big, c, nullptr, ctr2, ctr2_next);
}

// Read the epoch (launches completed on this workspace) at the start of a launch.  Only
// thread 0 waits on counters, so only it needs the value; no barrier, so the load's
// latency overlaps the first weight loads.
// (every thread loads it: a load under a branch makes the compiler's waits for the loads
// before it wait for everything in flight)
__device__ inline void read_epoch(Ctrl* ctrl, Ctx& c) { c.epoch = load_relaxed_dev(&ctrl->epoch); }

// Reducer count and slice width for H columns over P workgroups: power-of-two slices of at
// least 32 columns, at most P/2 reducers.
inline void reducer_split(int H, int P, int* R, int* SW) {
  const int rmax = P / 2 > 0 ? P / 2 : 1;
  int sw = 32;
  while ((long long)sw * rmax < H) sw <<= 1;
  *SW = sw;
  *R = (H + sw - 1) / sw;
}

}  // namespace lc
}  // namespace moe

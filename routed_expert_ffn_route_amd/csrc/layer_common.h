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

// Team dot products of C rows with x: returns, in every thread of the team, the C totals
// (out[c]).  rows[c] < 0 marks an empty slot.  One barrier.  All threads must call.
template <DT dt, int C, int CPT>
__device__ __forceinline__ void team_dots(const void* base, const uint8_t* scales,
                                          const long long (&rows)[C],
                                          const float (&xv)[CPT * kE<dt>], Ctx& c,
                                          float (&out)[C]) {
  using F = Fmt<dt>;
  typename F::Raw r[C][CPT];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const RowSrc<dt, true> src = slot_rows<dt, true>(base, scales, rows[q], c);
#pragma unroll
    for (int m = 0; m < CPT; ++m) r[q][m] = src.load(c.t + m * c.tsz, c);
  }
  constexpr int NP = NextPow2<C>::value;
  float acc[NP];
#pragma unroll
  for (int q = 0; q < C; ++q) acc[q] = chunk_dot<dt, CPT>(r[q], xv);
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
template <DT dt, int C, int CPT, bool HAS_G, bool BUF, typename Map, typename X>
__device__ inline void stream_channels(const void* G, const void* V, const void* D,
                                       const uint8_t* Gs, const uint8_t* Vs, const uint8_t* Ds,
                                       int i0, int i1, Map map, const X& xv,
                                       float (&yv)[CPT * kE<dt>], Ctx& c) {
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
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    fill(B, b + 1);
    stage_compute<dt, C, CPT, HAS_G>(A, xv, yv, c);
    fill(A, b + 2);
    stage_compute<dt, C, CPT, HAS_G>(B, xv, yv, c);
  }
  if (b < nb) stage_compute<dt, C, CPT, HAS_G>(A, xv, yv, c);
}

// The routed experts' channels [i0, i1): flat channel f = slot * I + j is row j of expert
// s_ids[slot] (negative: an empty slot), weighted by s_w[slot].  The same two-stage stream
// as stream_channels, but the team's items are walked incrementally: (slot, j) of its next
// first item advances by a batch per fill, and the current and next slot's expert offsets
// stay in scalar registers, so an item's three row addresses are a 32-bit multiply and
// 64-bit adds (the host admits E * I < 2^31; a row offset within one expert, I * row bytes,
// stays below 2^32).  Every wave of the compute unit issues this scalar code, and scalar
// instructions issue at the rate of vector ones, so the per-item divisions and 64-bit
// multiplications of the generic map made the stream scalar-bound.
template <DT dt, int C, int CPT, typename X>
__device__ inline void stream_routed(const void* G, const void* V, const void* D,
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

// Router logits, spread over the first workgroups (one team per row).  Each logit is
// published as one 64-bit word: the launch tag (epoch + 1) in the upper half and the fp32
// bits in the lower half, so readers wait on the data itself.  Every workgroup also learns
// the launch epoch here (thread 0 loaded it at the start; the router rows hide the wait).
// `buf` is LDS of at least ceil(E / P) + nteams floats; s_ep one LDS word.
template <DT RT, int CPT>
__device__ inline void router_rows(bool compute, const void* router, int E,
                                   const float (&xv)[CPT * kE<RT>], uint64_t* rlog, float* buf,
                                   uint32_t* s_ep, Ctx& c) {
  const int n_router_wgs = min(c.P, (E + c.nteams - 1) / c.nteams);
  const bool mine = compute && c.wg < n_router_wgs;
  int nloc = 0;
  if (mine) {
    for (int base = c.wg * c.nteams; base < E; base += c.P * c.nteams, nloc += c.nteams) {
      const int e = base + c.team;
      const long long rows[1] = {e < E ? (long long)e : -1};
      float l[1];
      team_dots<RT, 1, CPT>(router, nullptr, rows, xv, c, l);
      if (c.t == 0) buf[nloc + c.team] = l[0];
    }
  }
  if (c.tid == 0) *s_ep = c.epoch;
  __syncthreads();
  c.epoch = *s_ep;
  if (mine) {
    const uint64_t tag = (uint64_t)(c.epoch + 1u) << 32;
    for (int i = c.tid; i < nloc; i += c.nthreads) {
      const int e = c.wg * c.nteams + (i / c.nteams) * c.P * c.nteams + i % c.nteams;
      if (e < E) st_dev64(rlog + e, tag | __float_as_uint(buf[i]));
    }
  }
}

// Exact top-k of the E logits and the softmax over the k selected, computed by the whole
// workgroup into LDS (s_ids, s_w).  `keys` is LDS scratch of topk_lds_bytes(E) bytes.
__device__ inline void topk_local(const uint64_t* rlog, int E, int k, uint64_t* keys,
                                  int* s_ids, float* s_w, uint32_t* err, const Ctx& c) {
  const int E64 = (E + 63) & ~63;
  uint64_t* sel = keys + E64;
  const uint32_t tag = c.epoch + 1u;
  for (int e = c.tid; e < E64; e += c.nthreads) {
    uint64_t key = 0ull;  // padding: below every real key
    if (e < E) {
      const uint64_t v = wait_tagged(rlog + e, tag, err, kErrRouteWait);
      key = make_key(__uint_as_float((uint32_t)v), (uint32_t)e);
    }
    keys[e] = key;
  }
  __syncthreads();
  wg_topk_rank(keys, sel + 64, E, k, sel);
  if (c.tid < kWave) {
    const float l0 = key_value(sel[0]);
    const float ex = c.tid < k ? expf(key_value(sel[c.tid]) - l0) : 0.0f;
    const float sum = wave_sum(ex);
    if (c.tid < k) {
      s_ids[c.tid] = (int)key_index(sel[c.tid]);
      s_w[c.tid] = ex / sum;
    }
  }
  __syncthreads();
}

// The routing of this token in LDS (s_ids, s_w).  Inside the launch: wait until every
// router workgroup has published its logits, then select the top-k in this workgroup (each
// workgroup sorts the E logits itself, which costs less than one more cross-workgroup
// hand-off).  Given routing: copy ids/w; an id outside [0, E), or equal to an earlier id of
// the token, is reported and skipped (-1), so a repeated expert counts once (its first
// choice).  Workgroup 0 also stores the routing it used into ids_ws / w_ws [k], where the
// host can read back what the launch chose.
__device__ inline void fetch_routing(bool inside, const uint64_t* rlog, const int32_t* ids_in,
                                     const float* w_in, int E, int k, Ctrl* ctrl,
                                     uint64_t* keys, int* s_ids, float* s_w, int32_t* ids_ws,
                                     float* w_ws, const Ctx& c) {
  if (inside) {
    topk_local(rlog, E, k, keys, s_ids, s_w, &ctrl->err, c);
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

// Add a second layout's register vectors to big[0 .. H), one team after the other (a fixed
// order).
template <int E, int CPT>
__device__ inline void add_teams_to_lds(const float (&yv)[CPT * E], float* big, const Ctx& c) {
  for (int tm = 0; tm < c.nteams; ++tm) {
    if (c.team == tm) {
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const int ch = c.t + m * c.tsz;
        if (ch < c.nch) {
#pragma unroll
          for (int i = 0; i < E; ++i) big[E * ch + i] += yv[m * E + i];
        }
      }
    }
    __syncthreads();
  }
}

// Publish src[0 .. H) (default: big) as this workgroup's partial output and arrive on the
// done counters;
// R fixed workgroups (every (P/R)-th) then each sum an SW-column slice over all P
// partials in a fixed order (p ascending in strided groups, then a fixed tree).  The first
// reducer, once every workgroup has arrived, advances the epoch for the next launch.
// `big` is LDS of at least max(H, nthreads) floats.
__device__ inline void publish_and_reduce(float* partials, float* y, Ctrl* ctrl, int R, int SW,
                                          float* big, const Ctx& c, const float* src = nullptr) {
  const int H = c.H;
  if (!src) src = big;
  for (int h = c.tid; h < H; h += c.nthreads) st_dev(partials + (size_t)c.wg * H + h, src[h]);
  stores_complete();
  __syncthreads();
  MOE_STAMP(c.stamps, kStampPublished);
  if (c.tid == 0) arrive(ctrl->done, c.wg);
  const int stride = c.P / R;
  if (c.wg % stride != 0 || c.wg / stride >= R) return;
  const int r = c.wg / stride;
  if (c.tid == 0) {
    wait_family(ctrl->done, c.P, c.epoch, &ctrl->err, kErrReduceWait);
    if (r == 0) store_relaxed_dev(&ctrl->epoch, c.epoch + 1u);
  }
  __syncthreads();
  MOE_STAMP(c.stamps, kStampArrived);
  const int h0 = r * SW;
  const int wslice = min(SW, H - h0);
  const int SWB = SW < c.nthreads ? SW : c.nthreads;  // columns per pass (power of two)
  const int G = c.nthreads / SWB;
  const int g = c.tid / SWB, col0 = c.tid % SWB;
  for (int cb = 0; cb < wslice; cb += SWB) {
    const int col = cb + col0;
    float s = 0.0f;
    if (col < wslice) {
      // eight loads in flight, summed in ascending p (a fixed order)
      for (int p0 = g; p0 < c.P; p0 += 8 * G) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int p = p0 + u * G;
          v[u] = p < c.P ? ld_dev(partials + (size_t)p * H + h0 + col) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
    }
    big[g * SWB + col0] = s;
    __syncthreads();
    for (int st = G >> 1; st >= 1; st >>= 1) {
      if (g < st) big[g * SWB + col0] += big[(g + st) * SWB + col0];
      __syncthreads();
    }
    if (g == 0 && col < wslice) y[h0 + col] = big[col0];
    __syncthreads();
  }
  MOE_STAMP(c.stamps, kStampReduced);
}

// The whole output step for one register layout.
template <int CPT, int E = 8>
__device__ inline void reduce_output(const float (&yv)[CPT * E], float* partials, float* y,
                                     Ctrl* ctrl, int R, int SW, float* big, const Ctx& c) {
  teams_to_lds<E, CPT>(yv, big, c);
  publish_and_reduce(partials, y, ctrl, R, SW, big, c);
}

// Read the epoch (launches completed on this workspace) at the start of a launch.  Only
// thread 0 waits on counters, so only it needs the value; no barrier, so the load's
// latency overlaps the first weight loads.
__device__ inline void read_epoch(Ctrl* ctrl, Ctx& c) {
  c.epoch = c.tid == 0 ? load_relaxed_dev(&ctrl->epoch) : 0u;
}

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

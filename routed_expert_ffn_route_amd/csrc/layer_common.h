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
  __device__ float* next_red() {
    float* r = red + parity * red_stride;
    parity ^= 1;
    return r;
  }
};

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
    const bool ok = rows[q] >= 0;
    const size_t rr = ok ? (size_t)rows[q] : 0;
    const void* p = row_ptr<dt>(base, rr, c.H);
    const uint8_t* sp = scales ? scale_row_ptr(scales, rr, c.H) : nullptr;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int ch = c.t + m * c.tsz;
      r[q][m] = (ok && ch < c.nch) ? F::load(p, sp, ch) : zero_raw<dt>();
    }
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
#pragma unroll
  for (int q = 0; q < C; ++q) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < c.wpt; ++w) s += red[(c.team * c.wpt + w) * NP + q];
    out[q] = s;
  }
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
template <DT dt, int C, int CPT, bool HAS_G>
__device__ __forceinline__ void stage_load(Stage<dt, C, CPT>& st, const void* G, const void* V,
                                           const void* D, const uint8_t* Gs, const uint8_t* Vs,
                                           const uint8_t* Ds, const long long (&row)[C],
                                           const Ctx& c) {
  using F = Fmt<dt>;
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const bool ok = row[q] >= 0;
    const size_t r = ok ? (size_t)row[q] : 0;
    // the row is the same for every lane of the wave (one team = whole waves)
    const void* vp = row_ptr<dt>(V, r, c.H);
    const void* dp = row_ptr<dt>(D, r, c.H);
    const uint8_t* vsp = Vs ? scale_row_ptr(Vs, r, c.H) : nullptr;
    const uint8_t* dsp = Ds ? scale_row_ptr(Ds, r, c.H) : nullptr;
    const void* gp = HAS_G ? row_ptr<dt>(G, r, c.H) : nullptr;
    const uint8_t* gsp = (HAS_G && Gs) ? scale_row_ptr(Gs, r, c.H) : nullptr;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int ch = c.t + m * c.tsz;
      const bool live = ok && ch < c.nch;
      if constexpr (HAS_G)
        st.g[q][m] = live ? F::load(gp, gsp, ch) : zero_raw<dt>();
      st.v[q][m] = live ? F::load(vp, vsp, ch) : zero_raw<dt>();
      st.d[q][m] = live ? F::load(dp, dsp, ch) : zero_raw<dt>();
    }
  }
}

// Gate and up dots of a loaded batch, team reduction through LDS (one barrier),
// silu(g)*u*wt, and the accumulation of that activation times the down row into yv.
// All threads of the workgroup must call.
template <DT dt, int C, int CPT, bool HAS_G>
__device__ __forceinline__ void stage_compute(const Stage<dt, C, CPT>& st,
                                              const float (&xv)[CPT * kE<dt>],
                                              float (&yv)[CPT * kE<dt>], Ctx& c) {
  constexpr int E = kE<dt>;
  constexpr int NP = NextPow2<2 * C>::value;
  float acc[NP];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    acc[q] = HAS_G ? chunk_dot<dt, CPT>(st.g[q], xv) : 0.0f;
    acc[C + q] = chunk_dot<dt, CPT>(st.v[q], xv);
  }
#pragma unroll
  for (int i = 2 * C; i < NP; ++i) acc[i] = 0.0f;
  const float tot = wave_multi_sum<NP>(acc, c.lane);
  float* red = c.next_red();
  if (c.lane < NP) red[(c.team * c.wpt + c.wit) * NP + c.lane] = tot;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < C; ++q) {
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int w = 0; w < c.wpt; ++w) {
      g += red[(c.team * c.wpt + w) * NP + q];
      u += red[(c.team * c.wpt + w) * NP + C + q];
    }
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
// gate value.
template <DT dt, int C, int CPT, bool HAS_G, typename Map>
__device__ inline void stream_channels(const void* G, const void* V, const void* D,
                                       const uint8_t* Gs, const uint8_t* Vs, const uint8_t* Ds,
                                       long long i0, long long i1, Map map,
                                       const float (&xv)[CPT * kE<dt>],
                                       float (&yv)[CPT * kE<dt>], Ctx& c) {
  const long long per = (long long)c.nteams * C;
  const long long nb = i1 > i0 ? (i1 - i0 + per - 1) / per : 0;
  auto fill = [&](Stage<dt, C, CPT>& st, long long b) {
    long long row[C];
#pragma unroll
    for (int q = 0; q < C; ++q) {
      const long long i = i0 + b * per + c.team * C + q;
      row[q] = -1;
      st.wt[q] = 0.0f;
      st.gv[q] = 0.0f;
      if (i < i1) map(i, row[q], st.wt[q], st.gv[q]);
    }
    stage_load<dt, C, CPT, HAS_G>(st, G, V, D, Gs, Vs, Ds, row, c);
  };
  Stage<dt, C, CPT> A, B;
  if (nb > 0) fill(A, 0);
  for (long long b = 0; b < nb; b += 2) {
    if (b + 1 < nb) fill(B, b + 1);
    stage_compute<dt, C, CPT, HAS_G>(A, xv, yv, c);
    if (b + 1 < nb) {
      if (b + 2 < nb) fill(A, b + 2);
      stage_compute<dt, C, CPT, HAS_G>(B, xv, yv, c);
    }
  }
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
// hand-off).  Given routing: copy ids/w.  Out-of-range ids are reported and skipped (-1).
__device__ inline void fetch_routing(bool inside, const uint64_t* rlog, const int32_t* ids_in,
                                     const float* w_in, int E, int k, Ctrl* ctrl,
                                     uint64_t* keys, int* s_ids, float* s_w, const Ctx& c) {
  if (inside) {
    topk_local(rlog, E, k, keys, s_ids, s_w, &ctrl->err, c);
    return;
  }
  if (c.tid < k) {
    int e = ids_in[c.tid];
    if (e < 0 || e >= E) {
      __hip_atomic_fetch_or(&ctrl->err, kErrBadId, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      e = -1;
    }
    s_ids[c.tid] = e;
    s_w[c.tid] = w_in[c.tid];
  }
  __syncthreads();
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
  if (c.tid == 0) arrive(ctrl->done, c.wg);
  const int stride = c.P / R;
  if (c.wg % stride != 0 || c.wg / stride >= R) return;
  const int r = c.wg / stride;
  if (c.tid == 0) {
    wait_family(ctrl->done, c.P, c.epoch, &ctrl->err, kErrReduceWait);
    if (r == 0) store_relaxed_dev(&ctrl->epoch, c.epoch + 1u);
  }
  __syncthreads();
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

// expert_b1.hip -- the batch-1 layer in one persistent launch.
//
// Per token and layer the layer reads the router, the k routed experts and the shared
// experts once each, so its time is the weight bytes over the bandwidth; launching one
// small kernel per expert instead makes per-launch overhead the floor ("Mixture of
// Experts Changes the Arithmetic", section "What the Runtime Does With the Promise").
// This kernel therefore does the whole layer in one launch of one workgroup per CU:
//
//  1. router rows are spread over the first workgroups (one team of 256 threads per
//     row); the last router workgroup to finish sorts the logits (exact top-k on
//     ordered 64-bit keys) and publishes ids and softmax weights;
//  2. meanwhile every workgroup streams its share of the shared experts' channels,
//     which do not depend on routing;
//  3. every workgroup waits for the routing, then streams its contiguous share of the
//     k*I routed channels.  For a channel j it reads row j of G_e and V_e and row j of
//     D_e^T (the review of arXiv:2610.37386, "Background: channels and keep rules":
//     channel j owns those rows/columns; D is stored transposed so d_j is contiguous),
//     forms a_j = silu(g_j.x)(v_j.x) w_e and accumulates a_j d_j into registers;
//  4. each workgroup writes one partial H-vector; the last R workgroups to finish each
//     sum an H/R slice over all partials in a fixed order (deterministic, no float
//     atomics); the last reducer resets the control block for the next launch.
//
// All cross-workgroup waits are on work of workgroups that never wait before producing
// it, and every wait is bounded in time (an expired wait sets an error bit).
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWavesPerTeam = kTeam / kWave;

template <int N> struct NextPow2 {
  static constexpr int value = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16;
};

template <DT dt, int CPT>
__device__ __forceinline__ float chunk_dot(const typename Fmt<dt>::Raw (&r)[CPT],
                                           const float (&xv)[CPT * 8]) {
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    float v[8];
    Fmt<dt>::decode(r[m], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(v[i], xv[m * 8 + i], s);
  }
  return s;
}

template <DT dt>
__device__ __forceinline__ typename Fmt<dt>::Raw zero_raw() {
  typename Fmt<dt>::Raw r;
  __builtin_memset(&r, 0, sizeof(r));
  return r;
}

// One batch of C channels per team: gate/up dot products, team reduction through LDS
// (one barrier), SwiGLU, and the weighted down-row accumulation into yv.
// row[c] < 0 marks an empty slot (tail).  Every thread of the workgroup must call.
template <DT dt, int C, int CPT>
__device__ __forceinline__ void channel_batch(
    const void* G, const void* V, const void* D, const uint8_t* Gs, const uint8_t* Vs,
    const uint8_t* Ds, const long long (&row)[C], const float (&wt)[C],
    const float (&xv)[CPT * 8], float (&yv)[CPT * 8], int t, int nch, int H, float* red,
    int team, int wit, int lane) {
  using F = Fmt<dt>;
  typename F::Raw rg[C][CPT], rv[C][CPT], rd[C][CPT];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool ok = row[c] >= 0;
    const size_t r = ok ? (size_t)row[c] : 0;
    const void* gp = row_ptr<dt>(G, r, H);
    const void* vp = row_ptr<dt>(V, r, H);
    const void* dp = row_ptr<dt>(D, r, H);
    const uint8_t* gsp = scale_row_ptr(Gs, r, H);
    const uint8_t* vsp = scale_row_ptr(Vs, r, H);
    const uint8_t* dsp = scale_row_ptr(Ds, r, H);
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int ch = t + m * kTeam;
      if (ok && ch < nch) {
        rg[c][m] = F::load(gp, gsp, ch);
        rv[c][m] = F::load(vp, vsp, ch);
        rd[c][m] = F::load(dp, dsp, ch);
      } else {
        rg[c][m] = zero_raw<dt>();
        rv[c][m] = zero_raw<dt>();
        rd[c][m] = zero_raw<dt>();
      }
    }
  }
  constexpr int NP = NextPow2<2 * C>::value;
  float acc[NP];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    acc[c] = chunk_dot<dt, CPT>(rg[c], xv);
    acc[C + c] = chunk_dot<dt, CPT>(rv[c], xv);
  }
#pragma unroll
  for (int i = 2 * C; i < NP; ++i) acc[i] = 0.0f;
  const float tot = wave_multi_sum<NP>(acc, lane);
  if (lane < NP) red[(team * kWavesPerTeam + wit) * NP + lane] = tot;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < C; ++c) {
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerTeam; ++w) {
      g += red[(team * kWavesPerTeam + w) * NP + c];
      u += red[(team * kWavesPerTeam + w) * NP + C + c];
    }
    const float act = silu(g) * u * wt[c];
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      float d[8];
      F::decode(rd[c][m], d);
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[m * 8 + i] = fmaf(act, d[i], yv[m * 8 + i]);
    }
  }
}

__device__ __forceinline__ void acquire_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

struct B1Launch {
  B1Args a;
  int R;   // reducers
  int SW;  // slice width of each reducer (columns of y)
};

template <DT ET, DT ST, DT RT, int C, int CPT>
__global__ __launch_bounds__(1024) void b1_kernel(B1Launch L) {
  const B1Args& a = L.a;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, nthreads = blockDim.x;
  const int nteams = nthreads / kTeam;
  const int team = tid / kTeam, t = tid % kTeam, lane = tid & (kWave - 1);
  const int wit = t / kWave;
  const int P = gridDim.x, wg = blockIdx.x;
  const int H = a.H, nch = H / 8;
  Ctrl* ctrl = a.ctrl;
  constexpr int NP = NextPow2<2 * C>::value;

  float* red = reinterpret_cast<float*>(smem);            // [2][nteams][4][NP]
  int* s_int = reinterpret_cast<int*>(red + 2 * nteams * kWavesPerTeam * NP);  // [16]
  int* s_ids = s_int + 16;                                 // [64]
  float* s_w = reinterpret_cast<float*>(s_ids + 64);       // [64]
  unsigned char* big = reinterpret_cast<unsigned char*>(s_w + 64);
  int parity = 0;

  float xv[CPT * 8], yv[CPT * 8];
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int ch = t + m * kTeam;
    f32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (ch < nch) {
      lo = reinterpret_cast<const f32x4*>(a.x)[2 * ch];
      hi = reinterpret_cast<const f32x4*>(a.x)[2 * ch + 1];
    }
    xv[m * 8 + 0] = lo.x; xv[m * 8 + 1] = lo.y; xv[m * 8 + 2] = lo.z; xv[m * 8 + 3] = lo.w;
    xv[m * 8 + 4] = hi.x; xv[m * 8 + 5] = hi.y; xv[m * 8 + 6] = hi.z; xv[m * 8 + 7] = hi.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) yv[m * 8 + i] = 0.0f;
  }

  // ---- 1. router rows and the top-k --------------------------------------------------
  if (a.route_inside) {
    const int n_router_wgs = min(P, (a.E + nteams - 1) / nteams);
    if (wg < n_router_wgs) {
      for (int base = wg * nteams; base < a.E; base += P * nteams) {
        const int e = base + team;
        float part = 0.0f;
        if (e < a.E) {
          const void* rp = row_ptr<RT>(a.router, (size_t)e, H);
#pragma unroll
          for (int m = 0; m < CPT; ++m) {
            const int ch = t + m * kTeam;
            if (ch < nch) {
              typename Fmt<RT>::Raw r[1] = {Fmt<RT>::load(rp, nullptr, ch)};
              float v[8];
              Fmt<RT>::decode(r[0], v);
#pragma unroll
              for (int i = 0; i < 8; ++i) part = fmaf(v[i], xv[m * 8 + i], part);
            }
          }
        }
        part = wave_sum(part);
        float* rb = red + parity * nteams * kWavesPerTeam * NP;
        parity ^= 1;
        if (lane == 0) rb[(team * kWavesPerTeam + wit) * NP] = part;
        __syncthreads();
        if (t == 0 && e < a.E) {
          float l = 0.0f;
#pragma unroll
          for (int w = 0; w < kWavesPerTeam; ++w) l += rb[(team * kWavesPerTeam + w) * NP];
          a.logits_ws[e] = l;
        }
      }
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = atomic_add_dev(&ctrl->router_done, 1u);
        s_int[0] = (old == (uint32_t)(n_router_wgs - 1));
      }
      __syncthreads();
      if (s_int[0]) {
        acquire_fence();
        uint64_t* keys = reinterpret_cast<uint64_t*>(big);
        uint64_t* tmp = keys + ((a.E + 63) & ~63);
        for (int e = tid; e < a.E; e += nthreads)
          keys[e] = make_key(__builtin_nontemporal_load(a.logits_ws + e), (uint32_t)e);
        __syncthreads();
        wg_topk_keys(keys, tmp, a.E, a.k);
        if (tid < kWave) {
          const float l0 = key_value(keys[0]);
          float ex = 0.0f;
          if (tid < a.k) ex = expf(key_value(keys[tid]) - l0);
          const float sum = wave_sum(ex);
          if (tid < a.k) {
            a.ids_ws[tid] = (int32_t)key_index(keys[tid]);
            a.w_ws[tid] = ex / sum;
          }
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) atomic_store_dev(&ctrl->route_ready, 1u);
      }
    }
  }

  // ---- 2. shared experts (independent of routing) -------------------------------------
  if (a.NS > 0) {
    const long long nsc = (long long)a.NS * a.IS;
    const long long s0 = nsc * wg / P, s1 = nsc * (wg + 1) / P;
    for (long long base = s0; base < s1; base += (long long)nteams * C) {
      long long row[C];
      float wt[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const long long f = base + team * C + c;
        row[c] = f < s1 ? f : -1;
        wt[c] = 1.0f;
      }
      float* rb = red + parity * nteams * kWavesPerTeam * NP;
      parity ^= 1;
      channel_batch<ST, C, CPT>(a.sh_gate, a.sh_up, a.sh_down_t, nullptr, nullptr, nullptr,
                                row, wt, xv, yv, t, nch, H, rb, team, wit, lane);
    }
  }

  // ---- 3. routed experts --------------------------------------------------------------
  const int32_t* src_ids = a.ids_in;
  const float* src_w = a.w_in;
  if (a.route_inside) {
    if (tid == 0) wait_geq(&ctrl->route_ready, 1u, &ctrl->err, kErrRouteWait);
    __syncthreads();
    acquire_fence();
    src_ids = a.ids_ws;
    src_w = a.w_ws;
  }
  if (tid < a.k) {
    int e = __builtin_nontemporal_load(src_ids + tid);
    if (e < 0 || e >= a.E) {
      __hip_atomic_fetch_or(&ctrl->err, kErrBadId, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      e = -1;
    }
    s_ids[tid] = e;
    s_w[tid] = __builtin_nontemporal_load(src_w + tid);
  }
  __syncthreads();
  {
    const long long nrc = (long long)a.k * a.I;
    const long long r0 = nrc * wg / P, r1 = nrc * (wg + 1) / P;
    for (long long base = r0; base < r1; base += (long long)nteams * C) {
      long long row[C];
      float wt[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const long long f = base + team * C + c;
        row[c] = -1;
        wt[c] = 0.0f;
        if (f < r1) {
          const int slot = (int)(f / a.I), j = (int)(f - (long long)slot * a.I);
          const int e = s_ids[slot];
          if (e >= 0) {
            row[c] = (long long)e * a.I + j;
            wt[c] = s_w[slot];
          }
        }
      }
      float* rb = red + parity * nteams * kWavesPerTeam * NP;
      parity ^= 1;
      channel_batch<ET, C, CPT>(a.gate, a.up, a.down_t, a.gate_s, a.up_s, a.down_s, row, wt,
                                xv, yv, t, nch, H, rb, team, wit, lane);
    }
  }

  // ---- 4. partial of this workgroup, then the deterministic cross-workgroup sum --------
  float* ybuf = reinterpret_cast<float*>(big);  // [nteams][H]
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int ch = t + m * kTeam;
    if (ch < nch) {
      f32x4 lo = {yv[m * 8 + 0], yv[m * 8 + 1], yv[m * 8 + 2], yv[m * 8 + 3]};
      f32x4 hi = {yv[m * 8 + 4], yv[m * 8 + 5], yv[m * 8 + 6], yv[m * 8 + 7]};
      reinterpret_cast<f32x4*>(ybuf + team * H)[2 * ch] = lo;
      reinterpret_cast<f32x4*>(ybuf + team * H)[2 * ch + 1] = hi;
    }
  }
  __syncthreads();
  for (int h = tid; h < H; h += nthreads) {
    float s = ybuf[h];
    for (int tm = 1; tm < nteams; ++tm) s += ybuf[tm * H + h];
    a.partials[(size_t)wg * H + h] = s;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_int[1] = (int)atomic_add_dev(&ctrl->done, 1u);
  __syncthreads();
  const int ticket = s_int[1];
  const int R = L.R, SW = L.SW;
  if (ticket >= P - R) {
    const int r = ticket - (P - R);
    if (tid == 0) wait_geq(&ctrl->done, (uint32_t)P, &ctrl->err, kErrReduceWait);
    __syncthreads();
    acquire_fence();
    const int h0 = r * SW;
    const int wslice = min(SW, H - h0);
    const int SWB = SW < nthreads ? SW : nthreads;  // columns per pass (power of two)
    const int G = nthreads / SWB;
    const int g = tid / SWB, c = tid % SWB;
    float* tmp = reinterpret_cast<float*>(big);
    for (int cb = 0; cb < wslice; cb += SWB) {
      const int col = cb + c;
      float s = 0.0f;
      if (col < wslice)
        for (int p = g; p < P; p += G)
          s += __builtin_nontemporal_load(a.partials + (size_t)p * H + h0 + col);
      tmp[g * SWB + c] = s;
      __syncthreads();
      for (int stride = G >> 1; stride >= 1; stride >>= 1) {
        if (g < stride) tmp[g * SWB + c] += tmp[(g + stride) * SWB + c];
        __syncthreads();
      }
      if (g == 0 && col < wslice) a.y[h0 + col] = tmp[c];
      __syncthreads();
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = atomic_add_dev(&ctrl->exit, 1u);
      if (old == (uint32_t)(R - 1)) {
        atomic_store_dev(&ctrl->router_done, 0u);
        atomic_store_dev(&ctrl->route_ready, 0u);
        atomic_store_dev(&ctrl->done, 0u);
        atomic_store_dev(&ctrl->exit, 0u);
      }
    }
  }
}

template <DT ET, DT ST, DT RT, int C, int CPT>
hipError_t launch_t(const B1Launch& L, int wgs, int threads, int lds, hipStream_t s) {
  auto fn = b1_kernel<ET, ST, RT, C, CPT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(wgs), dim3(threads), lds, s, L);
  return hipGetLastError();
}

template <DT ET, DT ST, DT RT>
hipError_t launch_cpt(const B1Launch& L, int wgs, int threads, int lds, hipStream_t s) {
  const int nch = L.a.H / 8;
  const int cpt = (nch + kTeam - 1) / kTeam;
  if (cpt <= 1) return launch_t<ET, ST, RT, 2, 1>(L, wgs, threads, lds, s);
  if (cpt <= 2) return launch_t<ET, ST, RT, 2, 2>(L, wgs, threads, lds, s);
  if (cpt <= 4) return launch_t<ET, ST, RT, 2, 4>(L, wgs, threads, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace

int b1_lds_bytes(int H, int threads, int E, int k) {
  const int nteams = threads / kTeam;
  const int red = 2 * nteams * kWavesPerTeam * 8 * 4;
  const int small = (16 + 64 + 64) * 4;
  const int ybuf = nteams * H * 4;
  const int ek = (E + 63) & ~63;
  const int topk = (ek + ((E + 63) / 64) * k + 64) * 8;
  const int reduce = 1024 * 4;
  int big = ybuf > topk ? ybuf : topk;
  big = big > reduce ? big : reduce;
  return red + small + big;
}

hipError_t launch_b1(const B1Args& a, DT et, DT st, DT rt, int wgs, int threads,
                     hipStream_t s) {
  B1Launch L;
  L.a = a;
  // Reducer slices: power-of-two widths of at least 32 columns, at most half the grid.
  const int rmax = wgs / 2 > 0 ? wgs / 2 : 1;
  int sw = 32;
  while ((long long)sw * rmax < a.H) sw <<= 1;
  L.SW = sw;
  L.R = (a.H + sw - 1) / sw;
  const int lds = b1_lds_bytes(a.H, threads, a.E, a.k);
  if (et == DT::F32 && st == DT::F32 && rt == DT::F32)
    return launch_cpt<DT::F32, DT::F32, DT::F32>(L, wgs, threads, lds, s);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::BF16)
    return launch_cpt<DT::BF16, DT::BF16, DT::BF16>(L, wgs, threads, lds, s);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::F32)
    return launch_cpt<DT::BF16, DT::BF16, DT::F32>(L, wgs, threads, lds, s);
  if (et == DT::MXFP4 && st == DT::BF16 && rt == DT::BF16)
    return launch_cpt<DT::MXFP4, DT::BF16, DT::BF16>(L, wgs, threads, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace moe

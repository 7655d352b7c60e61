// channel_sparse.hip -- the channel-sparse batch-1 layer in one persistent launch.
//
// The fixed-count keep rule of the review of arXiv:2610.37386 ("Background: channels and
// keep rules"): of the k*I candidate channels of a token's routed experts, keep a fixed
// number K, compute those exactly from their full rows, and never read the dropped
// channels' up rows and down rows.  Channels are ranked by an output-unit score so that
// channels of different experts compare directly ("The weights-only reader", stage 2,
// eq. 1): here s_j = |silu(g_j.x)| * ||d_j||_2, optionally times the router weight, with
// the exact gate value (every gate row is read to score) and ||d_j|| precomputed at load.
//
// Phases inside the launch (one workgroup per CU):
//  1. router rows, then the exact top-k in every workgroup (as in the dense kernel);
//     shared experts stream meanwhile;
//  2. gate pass: each workgroup scores its contiguous share of the k*I candidates and
//     stores g and s (device-coherent);
//  3. grid barrier (every workgroup waits for all scores);
//  4. every workgroup selects the same K kept channels from the k*I scores: a 4-pass
//     radix select on the score bits finds the K-th largest score T, the candidates above
//     T and the lowest-indexed ones equal to T are kept (ties to the lower flat id), and a
//     block scan compacts them in ascending flat-id order;
//  5. each workgroup streams its share of the kept channels: the up row and the down row
//     only, with the stored gate value;
//  6. the deterministic cross-workgroup sum of the partial outputs.
#include "layer_common.h"

namespace moe {
namespace {

using namespace lc;

constexpr int kMaxNP = 16;
constexpr int kGateBatch = 4;

struct CSLaunch {
  B1Args a;
  const float* dnorm;  // [E*I]
  float* g_ws;         // [k*I]
  float* s_ws;         // [k*I]
  int32_t* kept_out;   // [K]
  int K, mode, R, SW, tsz;
};

// Exclusive prefix sum over the workgroup (sh: LDS of nwaves+1 ints).  *total = sum.
__device__ inline int block_excl_scan(int v, int* sh, const Ctx& c, int* total) {
  const int lane = c.lane, wave = c.tid >> 6, nw = c.nthreads >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int wv = lane < nw ? sh[lane] : 0;
    int s = wv;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(s, d, kWave);
      if (lane >= d) s += y;
    }
    if (lane < nw) sh[lane] = s - wv;
    if (lane == nw - 1) sh[nw] = s;
  }
  __syncthreads();
  const int res = sh[wave] + x - v;
  *total = sh[nw];
  __syncthreads();
  return res;
}

// Select the K largest of n non-negative scores (as uint32 bit patterns in `u`, which
// order like the floats), ties to the lower index; write the kept indices ascending to
// `kept`.  Returns the kept count.  `hist` is LDS of 256 ints, `sh` of 32 ints.
__device__ inline int select_topk_ascending(const uint32_t* u, int n, int K, int* kept,
                                            int* hist, int* sh, const Ctx& c) {
  if (K <= 0) return 0;
  const int seg = (n + c.nthreads - 1) / c.nthreads;
  const int f0 = min(n, c.tid * seg), f1 = min(n, f0 + seg);
  if (K >= n) {
    for (int f = c.tid; f < n; f += c.nthreads) kept[f] = f;
    __syncthreads();
    return n;
  }
  uint32_t prefix = 0, mask = 0;
  int need = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = c.tid; i < 256; i += c.nthreads) hist[i] = 0;
    __syncthreads();
    for (int f = c.tid; f < n; f += c.nthreads) {
      const uint32_t v = u[f];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & 255], 1);
    }
    __syncthreads();
    if (c.tid < kWave) {
      // lane l holds digits 255-4l .. 252-4l (descending); find where `need` falls
      int cnt[4], s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { cnt[q] = hist[255 - 4 * c.lane - q]; s += cnt[q]; }
      int incl = s;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(incl, d, kWave);
        if (c.lane >= d) incl += y;
      }
      int before = incl - s;  // count of larger digits
      if (before < need && need <= incl) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (before < need && need <= before + cnt[q]) {
            sh[0] = 255 - 4 * c.lane - q;
            sh[1] = need - before;
          }
          before += cnt[q];
        }
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)sh[0];
    need = sh[1];
    prefix |= digit << shift;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the K-th largest score; take `need` of the ties, lowest first
  int eq = 0;
  for (int f = f0; f < f1; ++f) eq += u[f] == T;
  int tot;
  int eq_base = block_excl_scan(eq, sh + 2, c, &tot);
  int mine = 0;
  for (int f = f0, r = eq_base; f < f1; ++f) {
    const uint32_t v = u[f];
    const bool take = v > T || (v == T && r < need);
    r += v == T;
    mine += take;
  }
  int kept_total;
  int base = block_excl_scan(mine, sh + 2, c, &kept_total);
  for (int f = f0, r = eq_base; f < f1; ++f) {
    const uint32_t v = u[f];
    const bool take = v > T || (v == T && r < need);
    r += v == T;
    if (take) kept[base++] = f;
  }
  __syncthreads();
  return kept_total;
}

template <DT ET, DT ST, DT RT, int C, int CPT>
__global__ __launch_bounds__(1024) void cs_kernel(CSLaunch L) {
  const B1Args& a = L.a;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = blockDim.x;
  c.tsz = L.tsz;
  c.wpt = c.tsz / kWave;
  c.nteams = c.nthreads / c.tsz;
  c.team = c.tid / c.tsz;
  c.t = c.tid % c.tsz;
  c.lane = c.tid & (kWave - 1);
  c.wit = c.t / kWave;
  c.P = gridDim.x;
  c.wg = blockIdx.x;
  c.H = a.H;
  c.nch = a.H / 8;
  c.red = reinterpret_cast<float*>(smem);
  c.red_stride = (c.nthreads / kWave) * kMaxNP;
  c.parity = 0;
  int* s_int = reinterpret_cast<int*>(c.red + 2 * c.red_stride);  // [16]
  int* s_ids = s_int + 16;                                          // [64]
  float* s_w = reinterpret_cast<float*>(s_ids + 64);                // [64]
  int* hist = reinterpret_cast<int*>(s_w + 64);                     // [256]
  int* sh = hist + 256;                                             // [48]
  float* big = reinterpret_cast<float*>(sh + 48);
  Ctrl* ctrl = a.ctrl;
  const int I = a.I;
  const int n = a.k * I;

  float xv[CPT * 8], yv[CPT * 8];
  load_x<CPT>(a.x, c, xv);
#pragma unroll
  for (int i = 0; i < CPT * 8; ++i) yv[i] = 0.0f;

  // 1. routing, and the shared experts while it is in flight
  read_epoch(ctrl, c);
  router_rows<RT, CPT>(a.route_inside, a.router, a.E, xv, a.rlog, reinterpret_cast<float*>(big),
                       reinterpret_cast<uint32_t*>(s_int), c);
  if (a.NS > 0) {
    const long long nsc = (long long)a.NS * a.IS;
    stream_channels<ST, C, CPT, true>(
        a.sh_gate, a.sh_up, a.sh_down_t, nullptr, nullptr, nullptr, nsc * c.wg / c.P,
        nsc * (c.wg + 1) / c.P,
        [](long long f, long long& row, float& wt, float&) { row = f; wt = 1.0f; }, xv, yv, c);
  }
  fetch_routing(a.route_inside, a.rlog, a.ids_in, a.w_in, a.E, a.k, ctrl,
                reinterpret_cast<uint64_t*>(big), s_ids, s_w, c);

  // 2. gate pass over this workgroup's share of the candidates
  {
    const int f0 = (int)((long long)n * c.wg / c.P), f1 = (int)((long long)n * (c.wg + 1) / c.P);
    for (int base = f0; base < f1; base += c.nteams * kGateBatch) {
      long long rows[kGateBatch];
#pragma unroll
      for (int q = 0; q < kGateBatch; ++q) {
        const int f = base + c.team * kGateBatch + q;
        rows[q] = -1;
        if (f < f1) {
          const int e = s_ids[f / I];
          if (e >= 0) rows[q] = (long long)e * I + (f % I);
        }
      }
      float g[kGateBatch];
      team_dots<ET, kGateBatch, CPT>(a.gate, a.gate_s, rows, xv, c, g);
      if (c.t < kGateBatch) {
        float gq = 0.0f;
#pragma unroll
        for (int q = 0; q < kGateBatch; ++q) gq = (q == c.t) ? g[q] : gq;
        const int f = base + c.team * kGateBatch + c.t;
        if (f < f1) {
          const int slot = f / I;
          const long long row = rows[c.t];
          float s = 0.0f;
          if (row >= 0) {
            s = fabsf(silu(gq)) * L.dnorm[row];
            if (L.mode == 1) s *= s_w[slot];
          }
          st_dev(L.g_ws + f, gq);
          st_dev(L.s_ws + f, s);
        }
      }
    }
  }

  // 3. grid barrier: all scores written
  stores_complete();
  __syncthreads();
  if (c.tid == 0) {
    arrive(ctrl->phase2, c.wg);
    wait_family(ctrl->phase2, c.P, c.epoch, &ctrl->err, kErrPhaseWait);
  }
  __syncthreads();

  // 4. the same selection in every workgroup
  uint32_t* sbits = reinterpret_cast<uint32_t*>(big);
  int* kept = reinterpret_cast<int*>(sbits + n);
  for (int f = c.tid; f < n; f += c.nthreads) sbits[f] = __float_as_uint(ld_dev(L.s_ws + f));
  __syncthreads();
  const int K = select_topk_ascending(sbits, n, L.K, kept, hist, sh, c);
  if (c.wg == 0)
    for (int i = c.tid; i < K; i += c.nthreads) L.kept_out[i] = kept[i];

  // 5. the kept channels: up row and down row only, gate value from the gate pass
  {
    const float* g_ws = L.g_ws;
    stream_channels<ET, C, CPT, false>(
        nullptr, a.up, a.down_t, nullptr, a.up_s, a.down_s, (long long)K * c.wg / c.P,
        (long long)K * (c.wg + 1) / c.P,
        [=](long long i, long long& row, float& wt, float& gv) {
          const int f = kept[i];
          const int slot = f / I;
          const int e = s_ids[slot];
          if (e >= 0) {
            row = (long long)e * I + (f % I);
            wt = s_w[slot];
            gv = ld_dev(g_ws + f);
          }
        },
        xv, yv, c);
  }
  __syncthreads();  // `big` is reused by the reduction below

  // 6. deterministic cross-workgroup sum
  reduce_output<CPT>(yv, a.partials, a.y, ctrl, L.R, L.SW, big, c);
}

template <DT ET, DT ST, DT RT, int C, int CPT>
hipError_t launch_t(const CSLaunch& L, int wgs, int threads, int lds, hipStream_t s) {
  auto fn = cs_kernel<ET, ST, RT, C, CPT>;
  static bool lds_set = false;
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    lds_set = true;
  }
  hipLaunchKernelGGL(fn, dim3(wgs), dim3(threads), lds, s, L);
  return hipGetLastError();
}

template <DT ET, DT ST, DT RT>
hipError_t launch_cpt(const CSLaunch& L, int wgs, int threads, int lds, hipStream_t s) {
  const int cpt = (L.a.H / 8 + L.tsz - 1) / L.tsz;
  if (cpt <= 1 && ET != DT::F32) return launch_t<ET, ST, RT, 2, 1>(L, wgs, threads, lds, s);
  if (cpt <= 1) return launch_t<ET, ST, RT, 1, 1>(L, wgs, threads, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace

int cs_lds_bytes(int H, int threads, int E, int k, int I) {
  const int nteams = threads / team_size(H);
  const int fixed = 2 * (threads / kWave) * kMaxNP * 4 + (16 + 64 + 64 + 256 + 48) * 4;
  const int n = k * I;
  const int sel = 2 * n * 4;
  const int ybuf = nteams * H * 4;
  const int topk = topk_lds_bytes(E, k);
  int big = sel > ybuf ? sel : ybuf;
  big = big > topk ? big : topk;
  big = big > threads * 4 ? big : threads * 4;
  return fixed + big;
}

hipError_t launch_cs(const B1Args& a, const float* dnorm, float* g_ws, float* s_ws,
                     int32_t* kept, int K, int mode, DT et, DT st, DT rt, int wgs, int threads,
                     hipStream_t s) {
  CSLaunch L;
  L.a = a;
  L.dnorm = dnorm;
  L.g_ws = g_ws;
  L.s_ws = s_ws;
  L.kept_out = kept;
  L.K = K;
  L.mode = mode;
  L.tsz = team_size(a.H);
  lc::reducer_split(a.H, wgs, &L.R, &L.SW);
  const int lds = cs_lds_bytes(a.H, threads, a.E, a.k, a.I);
  if (et == DT::F32 && st == DT::F32 && rt == DT::F32)
    return launch_cpt<DT::F32, DT::F32, DT::F32>(L, wgs, threads, lds, s);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::BF16)
    return launch_cpt<DT::BF16, DT::BF16, DT::BF16>(L, wgs, threads, lds, s);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::F32)
    return launch_cpt<DT::BF16, DT::BF16, DT::F32>(L, wgs, threads, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace moe

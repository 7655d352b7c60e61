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
constexpr int kGateBatch = 8;  // gate rows per team per batch (one batch covers a share)
constexpr int kPrefetch = 4;   // likeliest kept channels per share warmed in L2

struct CSLaunch {
  B1Args a;
  const float* dnorm;  // [E*I]
  uint64_t* s_ws;      // [k*I] launch-tagged scores
  int32_t* kept_out;   // [K]
  int K, mode, R, SW, tsz;
};

// Exclusive prefix sum over the workgroup (sh: LDS of nwaves+1 ints).  *total = sum.
__device__ inline int block_excl_scan(int v, int* sh, const Ctx& c, int* total) {
  const int lane = c.lane, wave = c.tid >> 6, nw = c.nthreads >> 6;
  const int x = wave_incl_scan(v);
  if (lane == kWave - 1) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int wv = lane < nw ? sh[lane] : 0;
    const int s = wave_incl_scan(wv);
    if (lane < nw) sh[lane] = s - wv;
    if (lane == nw - 1) sh[nw] = s;
  }
  __syncthreads();
  const int res = sh[wave] + x - v;
  *total = sh[nw];
  __syncthreads();
  return res;
}

// The K-th largest of n non-negative scores (as uint32 bit patterns in `u`, which order
// like the floats), ties to the lower index: returns T (the K-th largest pattern) and, in
// *need, how many of the values equal to T are kept (the lowest-indexed ones).  T is found
// digit by digit, most significant first (11, 11 and 10 bits): a histogram of the digit
// over the values that match the digits found so far, and the digit where the running
// count from the top reaches the remaining need.  Requires 0 < K < n.  `hist` is LDS of
// kSelBins ints, `sh` of 48 ints.
constexpr int kSelBins = 2048;
// LDS of the histogram: the binned selection keeps one padding int after every 32 bins
// (bin b at b + b / 32), so that a wave reading 32 consecutive bins per lane spreads over
// the banks
constexpr int kSelHist = kSelBins + kSelBins / 32;
__device__ __forceinline__ int sel_slot(int b) { return b + (b >> 5); }
__device__ inline uint32_t select_threshold(const uint32_t* u, int n, int K, int* need_out,
                                            int* hist, int* sh, const Ctx& c) {
  uint32_t prefix = 0, mask = 0;
  int need = K;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    const int nb = 1 << widths[pass];
    for (int i = c.tid; i < nb; i += c.nthreads) hist[i] = 0;
    __syncthreads();
    for (int f = c.tid; f < n; f += c.nthreads) {
      const uint32_t v = u[f];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & dmask], 1);
    }
    __syncthreads();
    // thread t owns the bins nb-1-b for b in [t*per, (t+1)*per): counts from the top
    const int per = (nb + c.nthreads - 1) / c.nthreads;
    int local = 0;
    for (int b = c.tid * per; b < (c.tid + 1) * per && b < nb; ++b) local += hist[nb - 1 - b];
    int total;
    const int before0 = block_excl_scan(local, sh + 2, c, &total);
    if (before0 < need && need <= before0 + local) {
      int before = before0;
      for (int b = c.tid * per; b < (c.tid + 1) * per && b < nb; ++b) {
        const int cnt = hist[nb - 1 - b];
        if (before < need && need <= before + cnt) {
          sh[0] = nb - 1 - b;
          sh[1] = need - before;
        }
        before += cnt;
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)sh[0];
    need = sh[1];
    prefix |= digit << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  *need_out = need;
  return prefix;
}

// The same threshold in one histogram pass where it can be done (returns false otherwise,
// and the caller runs select_threshold).  The radix digits above pile most scores into a
// few bins (the leading bits are sign and exponent), and LDS atomics on one bin serialize.
// Here the bins split [lo, hi] of the patterns evenly instead: bin(v) =
// floor((v - lo) * 2048 / (hi - lo + 1)) in float, which is monotone in v, so the K-th
// largest lies in the bin where the count from the top reaches K.  The values of that bin
// (at most kSelCand) are then ranked by brute force: T is the one with fewer than `need`
// values above it and at least `need` at or above it.  Returns false when all values are
// equal or that bin holds more than kSelCand values.  lo and hi come in per wave in
// sh[4 + w] and sh[20 + w], and `hist` (kSelHist ints) comes in cleared (both done while
// the scores arrive); wave 0 alone finds the bin, so the whole selection takes four
// barriers.
constexpr int kSelCand = 256;
__device__ inline bool select_threshold_binned(const uint32_t* u, int n, int K, uint32_t* T_out,
                                               int* need_out, int* hist, int* sh,
                                               const Ctx& c) {
  const int lane = c.lane, wave = c.tid >> 6, nw = c.nthreads >> 6;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int w = 0; w < nw; ++w) {
    const uint32_t ol = (uint32_t)sh[4 + w], oh = (uint32_t)sh[20 + w];
    lo = ol < lo ? ol : lo;
    hi = oh > hi ? oh : hi;
  }
  if (hi == lo) return false;  // uniform: every thread read the same words
  const float inv = (float)kSelBins / ((float)(hi - lo) + 1.0f);
  auto bin = [&](uint32_t v) {
    const int b = (int)((float)(v - lo) * inv);
    return b < kSelBins - 1 ? b : kSelBins - 1;
  };
  for (int f = c.tid; f < n; f += c.nthreads) atomicAdd(&hist[sel_slot(bin(u[f]))], 1);
  __syncthreads();
  if (wave == 0) {
    // lane l counts bins kSelBins - 1 - PB l - i, i < PB, from the top
    // (the counts stay in registers: all reads are issued at once, none waits on another)
    // Those PB bins share (b >> 5) = kWave - 1 - lane, so their padded slots are the PB
    // consecutive words from 33 * (kWave - 1 - lane): one base address and constant offsets.
    constexpr int PB = kSelBins / kWave;
    static_assert(PB == 32, "the padded histogram layout puts 32 bins per 33 words");
    const lds_i32* hb = (const lds_i32*)hist + 33 * (kWave - 1 - lane);
    int cnt[PB];
    int local = 0;
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      cnt[i] = hb[PB - 1 - i];
      local += cnt[i];
    }
    const int incl = wave_incl_scan(local);
    int before = incl - local;
    if (before < K && K <= incl) {
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        if (before < K && K <= before + cnt[i]) {
          sh[40] = kSelBins - 1 - PB * lane - i;
          sh[41] = K - before;  // the rank wanted within the bin
          sh[42] = cnt[i];
        }
        before += cnt[i];
      }
    }
    if (lane == 0) sh[44] = 0;
  }
  __syncthreads();
  const int bstar = sh[40], needb = sh[41], m = sh[42];
  if (m > kSelCand) return false;
  // the bin's values (hist is free now; its counts were read before the barrier), then
  // their ranks
  for (int f = c.tid; f < n; f += c.nthreads) {
    const uint32_t v = u[f];
    if (bin(v) == bstar) hist[atomicAdd(&sh[44], 1)] = (int)v;
  }
  __syncthreads();
  if (c.tid < m) {
    const uint32_t key = (uint32_t)hist[c.tid];
    int gt = 0, ge = 0;
    for (int j = 0; j < m; ++j) {
      const uint32_t o = (uint32_t)hist[j];
      gt += o > key ? 1 : 0;
      ge += o >= key ? 1 : 0;
    }
    if (gt < needb && needb <= ge) {  // the needb-th largest of the bin (equal keys agree)
      sh[45] = (int)key;
      sh[46] = needb - gt;
    }
  }
  __syncthreads();
  *T_out = (uint32_t)sh[45];
  *need_out = sh[46];
  return true;
}

// Counts, over u[0 .. m), of the values above T and of those equal to T (whole workgroup;
// sh: LDS of 48 ints).
__device__ inline void count_before(const uint32_t* u, int m, uint32_t T, int* gt, int* eq,
                                    int* sh, const Ctx& c) {
  int a = 0, b = 0;
  for (int f = c.tid; f < m; f += c.nthreads) {
    const uint32_t v = u[f];
    a += v > T ? 1 : 0;
    b += v == T ? 1 : 0;
  }
  if (m < 32768) {  // both counts in one scan: a in the upper, b in the lower 16 bits
    int t;
    block_excl_scan(a * 65536 + b, sh + 2, c, &t);
    *gt = t >> 16;
    *eq = t & 0xFFFF;
    return;
  }
  int ta, tb;
  block_excl_scan(a, sh + 2, c, &ta);
  block_excl_scan(b, sh + 2, c, &tb);
  *gt = ta;
  *eq = tb;
}

template <DT ET, DT ST, DT RT, int C, int CPT>
__global__ __launch_bounds__(1024) void cs_kernel(CSLaunch L) {
  const B1Args& a = L.a;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = blockDim.x;
  set_teams(c, L.tsz);
  c.lane = c.tid & (kWave - 1);
  c.P = gridDim.x;
  c.wg = blockIdx.x;
  c.H = a.H;
  c.nch = a.H / 8;
  c.red = reinterpret_cast<float*>(smem);
  c.red_stride = (c.nthreads / kWave) * kMaxNP;
  c.parity = 0;
  c.zrow = a.zrow;
  c.stamps = a.stamps;
  MOE_STAMP(c.stamps, kStampStart);
  int* s_int = reinterpret_cast<int*>(c.red + 2 * c.red_stride);  // [16]
  int* s_ids = s_int + 16;                                          // [64]
  float* s_w = reinterpret_cast<float*>(s_ids + 64);                // [64]
  int* hist = reinterpret_cast<int*>(s_w + 64);                     // [kSelHist]
  int* sh = hist + kSelHist;                                        // [48]
  float* big = reinterpret_cast<float*>(sh + 48);
  Ctrl* ctrl = a.ctrl;
  const int I = a.I;
  const int n = a.k * I;

  float xv[CPT * 8], yv[CPT * 8];
  load_x<8, CPT>(a.x, c, xv);
#pragma unroll
  for (int i = 0; i < CPT * 8; ++i) yv[i] = 0.0f;

  // 1. routing, and the shared experts while it is in flight
  read_epoch(ctrl, c);
  RouterRound<RT, CPT> rr;
  router_issue<RT, CPT>(a.route_inside, a.router, a.E, c, rr);
  auto finish_router = [&] {
    router_finish<RT, CPT>(rr, a.router, a.E, xv, a.rlog, reinterpret_cast<float*>(big),
                           reinterpret_cast<uint32_t*>(s_int), c);
  };
  if (a.NS > 0) {
    const long long nsc = (long long)a.NS * a.IS;
    stream_channels<ST, C, CPT, true, true>(
        a.sh_gate, a.sh_up, a.sh_down_t, nullptr, nullptr, nullptr, (int)(nsc * c.wg / c.P),
        (int)(nsc * (c.wg + 1) / c.P),
        [](int f, long long& row, float& wt, float&) { row = f; wt = 1.0f; }, xv, yv, c,
        finish_router);
  } else {
    finish_router();
  }
  fetch_routing(a.route_inside, a.rlog, a.ids_in, a.w_in, a.E, a.k, ctrl,
                reinterpret_cast<uint64_t*>(big), s_ids, s_w, a.ids_ws, a.w_ws, c);

  // 2. gate pass over this workgroup's share [g0, g1) of the candidates; g stays in LDS
  const int g0 = (int)((long long)n * c.wg / c.P), g1 = (int)((long long)n * (c.wg + 1) / c.P);
  uint32_t* sbits = reinterpret_cast<uint32_t*>(big);  // [n] all scores
  float* s_g = reinterpret_cast<float*>(sbits + n);     // [g1 - g0] this share's gate values
  int* loc = reinterpret_cast<int*>(s_g + (g1 - g0));   // [g1 - g0] this share's kept channels
  float* s_loc = reinterpret_cast<float*>(loc + (g1 - g0));  // [g1 - g0] this share's scores
  {
    for (int base = g0; base < g1; base += c.nteams * kGateBatch) {
      long long rows[kGateBatch];
#pragma unroll
      for (int q = 0; q < kGateBatch; ++q) {
        const int f = base + c.team * kGateBatch + q;
        rows[q] = -1;
        if (f < g1) {
          const int e = s_ids[f / I];
          if (e >= 0) rows[q] = (long long)e * I + (f % I);
        }
      }
      // the down-row norm of this thread's candidate is loaded with the gate rows
      long long myrow = -1;
#pragma unroll
      for (int q = 0; q < kGateBatch; ++q) myrow = (q == c.t) ? rows[q] : myrow;
      const float dn = (c.t < kGateBatch && myrow >= 0) ? L.dnorm[myrow] : 0.0f;
      float g[kGateBatch];
      team_dots<ET, kGateBatch, CPT>(a.gate, a.gate_s, rows, xv, c, g);
      if (c.t < kGateBatch) {
        float gq = 0.0f;
#pragma unroll
        for (int q = 0; q < kGateBatch; ++q) gq = (q == c.t) ? g[q] : gq;
        const int f = base + c.team * kGateBatch + c.t;
        if (f < g1) {
          const int slot = f / I;
          const long long row = myrow;
          float s = 0.0f;
          if (row >= 0) {
            s = fabsf(silu(gq)) * dn;
            if (L.mode == 1) s *= s_w[slot];
          }
          s_g[f - g0] = gq;
          s_loc[f - g0] = s;
          st_dev64(L.s_ws + f, ((uint64_t)(c.epoch + 1u) << 32) | __float_as_uint(s));
        }
      }
    }
  }

  // 2b. warm L2 with the up and down rows of this share's likeliest kept channels (the
  // kPrefetch highest local scores, one wave each, a load per 128-byte line): the kept
  // stream reads them right after the selection, and these loads overlap the gathering of
  // the other workgroups' scores.  Which rows are warmed affects only timing.
  uint32_t warm[4] = {0, 0, 0, 0};
  __syncthreads();
  {
    const int share = g1 - g0;
    const int wave = c.tid >> 6;
    if (wave < kPrefetch && wave < share) {
      const int i = c.lane;
      const float me = i < share ? s_loc[i] : -1.0f;
      int rank = 0;
      for (int j = 0; j < min(share, kWave); ++j) {
        const float o = s_loc[j];
        rank += (o > me || (o == me && j < i)) ? 1 : 0;
      }
      const unsigned long long hit = __ballot(i < share && rank == wave);
      if (hit) {
        const int src = __ffsll(hit) - 1;
        const int f = g0 + src;
        const int e = s_ids[f / I];
        if (e >= 0 && s_loc[src] > 0.0f) {
          const size_t row = (size_t)e * I + (f % I);
          const size_t rb = Fmt<ET>::row_bytes(a.H);
          const uint8_t* p = reinterpret_cast<const uint8_t*>(c.lane < 32 ? a.up : a.down_t) +
                             row * rb;
          // up to 4 lines per lane (rows of at most 16 KB); each value stays in its own
          // register until the end of the kernel, so nothing waits for these loads
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const size_t off = (size_t)(c.lane & 31) * 128 + (size_t)q * 32 * 128;
            warm[q] = *reinterpret_cast<const uint32_t*>(p + (off < rb ? off : rb - 4));
          }
        }
      }
    }
  }

  // 3. every workgroup gathers all k*I scores (each published with its launch tag, so
  // waiting on the scores themselves is the grid-wide hand-off)
  // (meanwhile the range of the scores per wave and a cleared histogram for the selection)
  {
    // eight scores per thread in flight at once (the loads are unconditional, so none
    // waits for another); only a score not yet tagged with this launch is polled again
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    const uint32_t tag = c.epoch + 1u;
    constexpr int kG = 8;
    for (int f0 = c.tid; f0 < n; f0 += kG * c.nthreads) {
      uint64_t w[kG];
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int f = f0 + u * c.nthreads;
        w[u] = ld_dev64(L.s_ws + (f < n ? f : n - 1));
      }
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int f = f0 + u * c.nthreads;
        if (f < n) {
          if ((uint32_t)(w[u] >> 32) != tag)
            w[u] = wait_tagged(L.s_ws + f, tag, &ctrl->err, kErrPhaseWait);
          const uint32_t v = (uint32_t)w[u];
          sbits[f] = v;
          lo = v < lo ? v : lo;
          hi = v > hi ? v : hi;
        }
      }
    }
    for (int i = c.tid; i < kSelHist; i += c.nthreads) hist[i] = 0;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const uint32_t ol = (uint32_t)__shfl_xor((int)lo, m);
      const uint32_t oh = (uint32_t)__shfl_xor((int)hi, m);
      lo = ol < lo ? ol : lo;
      hi = oh > hi ? oh : hi;
    }
    if (c.lane == 0) {
      sh[4 + (c.tid >> 6)] = (int)lo;
      sh[20 + (c.tid >> 6)] = (int)hi;
    }
  }
  __syncthreads();

  // 4. the same threshold in every workgroup; each keeps the channels of its own share:
  // above T, or equal to T and among the first `need` ties in flat-id order
  int nk = 0, kept_before = 0;
  if (L.K >= n) {
    for (int f = g0 + c.tid; f < g1; f += c.nthreads) loc[f - g0] = f;
    nk = g1 - g0;
    kept_before = g0;
  } else if (L.K > 0) {
    int need;
    uint32_t T;
    if (!select_threshold_binned(sbits, n, L.K, &T, &need, hist, sh, c))
      T = select_threshold(sbits, n, L.K, &need, hist, sh, c);
    int gt, eq;
    count_before(sbits, g0, T, &gt, &eq, sh, c);
    kept_before = gt + min(eq, need);
    if ((c.tid >> 6) == 0) {  // wave 0: 64 candidates of the share at a time
      const uint64_t below = (1ull << c.lane) - 1ull;
      int r = eq, pos = 0;  // T-valued candidates before, kept so far
      for (int base = g0; base < g1; base += kWave) {
        const int f = base + c.lane;
        const bool in = f < g1;
        const uint32_t v = in ? sbits[f] : 0u;
        const bool isT = in && v == T;
        const uint64_t mT = __ballot(isT);
        const bool take = in && (v > T || (isT && r + __popcll(mT & below) < need));
        const uint64_t mk = __ballot(take);
        if (take) loc[pos + __popcll(mk & below)] = f;
        pos += __popcll(mk);
        r += __popcll(mT);
      }
      if (c.lane == 0) sh[0] = pos;
    }
    __syncthreads();
    nk = sh[0];
  }
  __syncthreads();
  for (int i = c.tid; i < nk; i += c.nthreads) L.kept_out[kept_before + i] = loc[i];

  // 5. the kept channels of this share: up row and down row only, gate value from LDS
  stream_channels<ET, C, CPT, false, false>(
      nullptr, a.up, a.down_t, nullptr, a.up_s, a.down_s, 0, nk,
      [=](int i, long long& row, float& wt, float& gv) {
        // i is wave-uniform, so are f and e: scalar, and so is the row arithmetic
        const int f = __builtin_amdgcn_readfirstlane(loc[i]);
        const int slot = f / I;
        const int e = __builtin_amdgcn_readfirstlane(s_ids[slot]);
        if (e >= 0) {
          row = (long long)e * I + (f % I);
          wt = s_w[slot];
          gv = s_g[f - g0];
        }
      },
      xv, yv, c);
  __syncthreads();  // `big` is reused by the reduction below

  // 6. deterministic cross-workgroup sum
  reduce_output<CPT>(yv, a.partials, a.y, ctrl, L.R, L.SW, big, c);
  s_int[15] = warm[0] ^ warm[1] ^ warm[2] ^ warm[3];  // keeps the warming loads
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

int cs_lds_bytes(int H, int threads, int E, int k, int I, int wgs) {
  const int nteams = threads / team_size(H);
  const int fixed = 2 * (threads / kWave) * kMaxNP * 4 + (16 + 64 + 64 + kSelHist + 48) * 4;
  const int n = k * I;
  const int share = (n + wgs - 1) / wgs;
  const int sel = (n + 3 * share) * 4;  // all scores; this share's gate values, kept ids, scores
  const int ybuf = nteams * H * 4;
  const int topk = topk_lds_bytes(E, k);
  int big = sel > ybuf ? sel : ybuf;
  big = big > topk ? big : topk;
  big = big > threads * 8 ? big : threads * 8;
  return fixed + big;
}

hipError_t launch_cs(const B1Args& a, const float* dnorm, uint64_t* s_ws,
                     int32_t* kept, int K, int mode, DT et, DT st, DT rt, int wgs, int threads,
                     hipStream_t s) {
  CSLaunch L;
  L.a = a;
  L.dnorm = dnorm;
  L.s_ws = s_ws;
  L.kept_out = kept;
  L.K = K;
  L.mode = mode;
  L.tsz = team_size(a.H);
  lc::reducer_split(a.H, wgs, &L.R, &L.SW);
  const int lds = cs_lds_bytes(a.H, threads, a.E, a.k, a.I, wgs);
  if (et == DT::F32 && st == DT::F32 && rt == DT::F32)
    return launch_cpt<DT::F32, DT::F32, DT::F32>(L, wgs, threads, lds, s);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::BF16)
    return launch_cpt<DT::BF16, DT::BF16, DT::BF16>(L, wgs, threads, lds, s);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::F32)
    return launch_cpt<DT::BF16, DT::BF16, DT::F32>(L, wgs, threads, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace moe

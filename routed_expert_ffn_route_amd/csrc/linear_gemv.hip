// linear_gemv.hip -- experts that are one matrix each, at batches of up to four tokens, on
// VALU with whole-line loads.
//
// The batch-sweep workload of the "501B of which 23B are switched on" post (section 3):
// each expert is one H_out x H bf16 matrix M_e, a token picks k experts, and
// y_b = sum_i w_{b,i} M_{e_{b,i}} x_b.  At one to four tokens every touched matrix is
// read once and the arithmetic is a handful of multiply-adds per weight, so the layer is a
// pure weight stream.  The MFMA kernel's operand layout (16 rows x 64 bytes per load
// instruction) streams at about 5 TB/s at best; here a team of threads covers one weight
// row with one 16-byte chunk per thread, so each wave's load is 1 KB of one row (whole
// 128-byte lines), as in the batch-1 SwiGLU layer.
//
// Work layout: workgroup r owns output rows [r*RW, (r+1)*RW) of every touched expert
// (RW >= rows per batch of the whole workgroup), so it accumulates y[b][its rows] alone,
// in touched-expert order: no cross-workgroup reduction and a fixed summation order.
// Items are (touched expert, row) pairs, expert-major; a team takes C items per batch and
// two batches are in flight (the loads of batch b+1 go out before batch b is reduced).
// Per batch: the team's dot products of C rows with the NB tokens' x, one wave reduction
// (DPP) and one LDS round, then thread q*NB+t adds w_{t,e} * dot into LDS.  Since RW is at
// least a batch's item count, one batch never holds two items of the same row.
#include "layer_common.h"

namespace moe {
namespace {

using namespace lc;

constexpr int kMaxNP = 16;      // values per wave reduction (C * NB)
// rows per team and batch: as many as the registers of two stages allow
template <int NB> constexpr int gemv_rows() { return NB >= 2 ? 4 : 6; }
constexpr int kGemvMaxT = 256;  // touched experts (B * k <= 4 * 64)

struct GemvArgs {
  const void* M;             // [E][I][H] bf16
  const float* x;            // [B][H]
  const int32_t* ids;        // [B][k]
  const float* w;            // [B][k]
  uint32_t* err;             // sticky error bits (bad or repeated ids)
  const uint8_t* zrow;       // zeroed bytes, at least H * 2
  float* y;                  // [B][I]
  int H, I, E, k, B;
  int tsz;                   // threads per team
  int rw;                    // output rows per workgroup
};

template <int NB>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvArgs a) {
  using F = Fmt<DT::BF16>;
  constexpr int C = gemv_rows<NB>();
  constexpr int NP = NextPow2<C * NB>::value;
  static_assert(NP <= kMaxNP, "reduction width");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = blockDim.x;
  set_teams(c, a.tsz);
  c.lane = c.tid & (kWave - 1);
  c.P = gridDim.x;
  c.wg = blockIdx.x;
  c.H = a.H;
  c.nch = a.H / 8;
  c.red = reinterpret_cast<float*>(smem);
  c.red_stride = (c.nthreads / kWave) * kMaxNP;
  c.parity = 0;
  c.epoch = 0;
  c.zrow = a.zrow;
  const int rw = a.rw;
  float* ys = c.red + 2 * c.red_stride;               // [rw][NB] this workgroup's rows of y
  int* s_t = reinterpret_cast<int*>(ys + rw * NB);    // [kGemvMaxT] touched experts
  float* s_w = reinterpret_cast<float*>(s_t + kGemvMaxT);  // [kGemvMaxT][NB] token weights
  uint32_t* bm = reinterpret_cast<uint32_t*>(s_w + kGemvMaxT * NB);  // [EW] experts routed to
  int* s_nt = reinterpret_cast<int*>(bm + (a.E + 31) / 32);          // [1] touched count

  // The touched experts in ascending order and, per expert, each token's routing weight (0
  // if not routed to it), from the ids directly (B * k <= 256 entries; every workgroup
  // builds the same table): a bitmap of the routed experts, then an expert's place is the
  // number of set bits below it.
  const int EW = (a.E + 31) / 32, nf = a.B * a.k;
  for (int i = c.tid; i < EW; i += c.nthreads) bm[i] = 0u;
  for (int i = c.tid; i < kGemvMaxT * NB; i += c.nthreads) s_w[i] = 0.0f;
  for (int i = c.tid; i < kGemvMaxT; i += c.nthreads) s_t[i] = 0;  // (no ids valid: expert 0)
  __syncthreads();
  for (int f = c.tid; f < nf; f += c.nthreads) {
    const int e = a.ids[f];
    bool bad = e < 0 || e >= a.E;
    for (int j = f - f % a.k; j < f && !bad; ++j) bad = a.ids[j] == e;  // repeated in a token
    if (bad) {
      if (c.wg == 0) __hip_atomic_fetch_or(a.err, kErrBadId, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    atomicOr(&bm[e / 32], 1u << (e % 32));
  }
  __syncthreads();
  for (int f = c.tid; f < nf; f += c.nthreads) {
    const int e = a.ids[f];
    if (e < 0 || e >= a.E) continue;
    bool dup = false;
    for (int j = f - f % a.k; j < f && !dup; ++j) dup = a.ids[j] == e;
    if (dup) continue;
    int r = __popc(bm[e / 32] & ((1u << (e % 32)) - 1u));
    for (int q = 0; q < e / 32; ++q) r += __popc(bm[q]);
    s_t[r] = e;
    s_w[r * NB + f / a.k] = a.w[f];
  }
  if (c.tid == 0) {
    int n = 0;
    for (int q = 0; q < EW; ++q) n += __popc(bm[q]);
    *s_nt = n;
  }
  for (int i = c.tid; i < rw * NB; i += c.nthreads) ys[i] = 0.0f;
  // x of the tokens (zero for the padding tokens past B)
  float xv[NB][8];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if (t < a.B) {
      load_x<8, 1>(a.x + (size_t)t * a.H, c, xv[t]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[t][i] = 0.0f;
    }
  }
  __syncthreads();
  const int nt = *s_nt;

  const int r0 = c.wg * rw;
  const int nitems = nt * rw;
  const int per = c.nteams * C;
  const int nb = (nitems + per - 1) / per;
  // Item i = ti * rw + j is row r0 + j of touched expert ti (wave-uniform).  The batches
  // are filled in order, so the team's first item of a batch is tracked as (ti, j) and
  // advanced by `per` (<= rw) per batch: no division per item.  Every wave runs this scalar
  // code, and the scalar unit issues for all waves of the compute unit, so it is kept short.
  // rw is a multiple of `per`, so a batch never spans two experts: its C rows per team are
  // consecutive rows of one matrix, each one 64-bit add from the previous (the host admits
  // I * H * 2 < 2^32 for the 32-bit row offset).
  const uint32_t row_bytes = (uint32_t)a.H * 2u;
  auto expert_base = [&](int ti) -> const uint8_t* {
    const int e = __builtin_amdgcn_readfirstlane(s_t[ti < nt ? ti : 0]);
    return reinterpret_cast<const uint8_t*>(a.M) + (size_t)e * a.I * row_bytes;
  };
  int f_ti = 0, f_j = c.team * C;  // next batch's first item of this team
  const uint8_t* base = expert_base(0);
  const int ch = c.t < c.nch ? c.t : c.nch - 1;
  auto fill = [&](F::Raw (&st)[C]) {
    const uint8_t* rp = base + (uint32_t)(r0 + f_j) * row_bytes;
    const int live = f_ti < nt ? a.I - r0 - f_j : 0;  // rows of this batch inside the matrix
#pragma unroll
    for (int q = 0; q < C; ++q) {
      st[q] = F::load_g(uniform_ptr(q < live ? rp : c.zrow), nullptr, ch);
      rp += row_bytes;
    }
    f_j += per;
    if (f_j >= rw) {
      f_j -= rw;
      ++f_ti;
      base = expert_base(f_ti);
    }
  };
  auto compute = [&](const F::Raw (&st)[C], int b) {
    float acc[NP];
#pragma unroll
    for (int q = 0; q < C; ++q) {
      float v[8];
      F::decode(st[q], v);
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(v[i], xv[t][i], s);
        acc[q * NB + t] = s;
      }
    }
#pragma unroll
    for (int i = C * NB; i < NP; ++i) acc[i] = 0.0f;
    const float tot = wave_multi_sum<NP>(acc, c.lane);
    float* red = c.next_red();
    if (c.lane < NP) red[(c.team * c.wpt + c.wit) * NP + c.lane] = tot;
    __syncthreads();
    // lane l of the team holds the team total of value l % NP: thread q*NB + t finishes
    // (item q, token t)
    const float v = team_totals<NP>(red, c);
    if (c.t < C * NB) {
      const int q = c.t / NB, t = c.t - q * NB;
      const int i = b * per + c.team * C + q;
      const int ti = i / rw, j = i - ti * rw;
      if (i < nitems && r0 + j < a.I) ys[j * NB + t] = fmaf(s_w[ti * NB + t], v, ys[j * NB + t]);
    }
  };
  F::Raw A[C], B[C];
  fill(A);
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    fill(B);
    compute(A, b);
    fill(A);
    compute(B, b + 1);
  }
  if (b < nb) compute(A, b);
  __syncthreads();
  for (int i = c.tid; i < rw * NB; i += c.nthreads) {
    const int j = i / NB, t = i - j * NB;
    if (t < a.B && r0 + j < a.I) a.y[(size_t)t * a.I + r0 + j] = ys[i];
  }
}

// Batches of five to 31 tokens.  Computing every token against every touched row (as above)
// would cost B multiply-adds per weight for about B * k / n_touched tokens that use it, so
// here each touched expert is paired with its own tokens only: a *pass* is (expert, up to
// four of its tokens), and an expert with more tokens takes several passes (rare at these
// batches: 1.4 tokens per touched expert at B = 16, k = 3, E = 64).  The (pass, row) items
// are laid out pass-major and cut into contiguous ranges, one per workgroup, so a team
// changes pass once or twice per launch and keeps its passes' x in registers in between.
// A workgroup no longer owns whole output rows, so each item writes w * dot into the partial
// row of its (token, choice) -- each written exactly once -- and a second kernel adds a
// token's k partials in routing order.
constexpr int kPassTok = 4;     // tokens per pass
constexpr int kMaxPass = 256;   // passes per launch (B * k <= 256)
constexpr int kPassRows = 4;    // rows per team and batch (I % kPassRows == 0)

struct PassArgs {
  const void* M;             // [E][I][H] bf16
  const float* x;            // [B][H]
  const float* w;            // [B][k]
  const int32_t* n_touched;  // [1]
  const int32_t* touched;    // [E]
  const int32_t* offsets;    // [E+1]
  const int32_t* slots;      // [B*k]
  const uint8_t* zrow;       // zeroed bytes, at least H * 4
  float* part;               // [B*k][I]
  int H, I, k, B;
  int tsz;                   // threads per team
};

__global__ __launch_bounds__(1024) void gemv_pass_kernel(PassArgs a) {
  using F = Fmt<DT::BF16>;
  constexpr int C = kPassRows;
  constexpr int NT = kPassTok;
  constexpr int NP = C * NT;
  static_assert(NP <= kMaxNP, "reduction width");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = blockDim.x;
  set_teams(c, a.tsz);
  c.lane = c.tid & (kWave - 1);
  c.P = gridDim.x;
  c.wg = blockIdx.x;
  c.H = a.H;
  c.nch = a.H / 8;
  c.red = reinterpret_cast<float*>(smem);
  c.red_stride = (c.nthreads / kWave) * kMaxNP;
  c.parity = 0;
  c.epoch = 0;
  c.zrow = a.zrow;
  int* s_pe = reinterpret_cast<int*>(c.red + 2 * c.red_stride);  // [kMaxPass] expert of pass
  int* s_ps = s_pe + kMaxPass;                                   // [kMaxPass][NT] slot or -1
  int* s_np = s_ps + kMaxPass * NT;                              // [1] pass count

  // The passes, in touched-expert order: wave 0 scans the per-expert pass counts
  // (ceil(tokens / NT)) 64 experts at a time.
  if (c.tid < kWave) {
    const int nt = *a.n_touched;
    int carry = 0;
    for (int i0 = 0; i0 < nt; i0 += kWave) {
      const int i = i0 + c.lane;
      int e = 0, o = 0, n = 0;
      if (i < nt) {
        e = a.touched[i];
        o = a.offsets[e];
        n = a.offsets[e + 1] - o;
      }
      const int np = (n + NT - 1) / NT;
      int inc = np;
      for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(inc, d, kWave);
        if (c.lane >= d) inc += t;
      }
      const int p0 = carry + inc - np;
      for (int q = 0; q < np; ++q) {
        const int p = p0 + q;
        if (p < kMaxPass) {
          s_pe[p] = e;
#pragma unroll
          for (int u = 0; u < NT; ++u) s_ps[p * NT + u] = q * NT + u < n ? a.slots[o + q * NT + u] : -1;
        }
      }
      carry += __shfl(inc, kWave - 1, kWave);
    }
    if (c.lane == 0) *s_np = min(carry, kMaxPass);
  }
  __syncthreads();
  const int npass = *s_np;

  // Items are chunks of C consecutive rows of one pass: chunk q = pass * IC + row / C.
  // Workgroup r takes chunks [q0, q1); in batch b, team t takes chunk q0 + b * nteams + t.
  const int IC = a.I / C;
  const long long nchunks = (long long)npass * IC;
  const int q0 = (int)(nchunks * c.wg / c.P), q1 = (int)(nchunks * (c.wg + 1) / c.P);
  const int nb = (q1 - q0 + c.nteams - 1) / c.nteams;
  const uint32_t row_bytes = (uint32_t)a.H * 2u;
  const int ch = c.t < c.nch ? c.t : c.nch - 1;
  // walk state of this team's next chunk (incremental: no division per batch)
  int f_q = q0 + c.team;
  int f_p = f_q / IC, f_j = f_q - f_p * IC;
  auto pass_base = [&](int p) -> const uint8_t* {
    const int e = __builtin_amdgcn_readfirstlane(s_pe[p < npass ? p : 0]);
    return reinterpret_cast<const uint8_t*>(a.M) + (size_t)e * a.I * row_bytes;
  };
  const uint8_t* base = pass_base(f_p);
  struct Stage {
    F::Raw r[C];
    int p;    // pass, -1 past the range
    int row;  // first row
  };
  auto fill = [&](Stage& st) {
    const bool live = f_q < q1;
    const uint8_t* rp = base + (uint32_t)(f_j * C) * row_bytes;
#pragma unroll
    for (int q = 0; q < C; ++q) {
      st.r[q] = F::load_g(uniform_ptr(live ? rp : c.zrow), nullptr, ch);
      rp += row_bytes;
    }
    st.p = live ? f_p : -1;
    st.row = f_j * C;
    f_q += c.nteams;
    f_j += c.nteams;
    bool moved = false;
    while (f_j >= IC) {
      f_j -= IC;
      ++f_p;
      moved = true;
    }
    if (moved) base = pass_base(f_p);
  };
  // x of the pass in registers (zero for the empty token places)
  float xv[NT][8];
  int x_pass = -1;
  auto compute = [&](const Stage& st) {
    if (st.p >= 0 && st.p != x_pass) {
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int slot = s_ps[st.p * NT + u];
        const float* xp = slot >= 0 ? a.x + (size_t)(slot / a.k) * a.H
                                    : reinterpret_cast<const float*>(c.zrow);
        load_x<8, 1>(xp, c, xv[u]);
      }
      x_pass = st.p;
    }
    float acc[NP];
#pragma unroll
    for (int q = 0; q < C; ++q) {
      float v[8];
      F::decode(st.r[q], v);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(v[i], xv[u][i], s);
        acc[q * NT + u] = s;
      }
    }
    const float tot = wave_multi_sum<NP>(acc, c.lane);
    float* red = c.next_red();
    if (c.lane < NP) red[(c.team * c.wpt + c.wit) * NP + c.lane] = tot;
    __syncthreads();
    // lane l of the team holds the team total of value l: thread q*NT + u finishes
    // (row q, token place u)
    const float v = team_totals<NP>(red, c);
    if (c.t < NP && st.p >= 0) {
      const int q = c.t / NT, u = c.t - q * NT;
      const int slot = s_ps[st.p * NT + u];
      if (slot >= 0) a.part[(size_t)slot * a.I + st.row + q] = a.w[slot] * v;
    }
  };
  Stage A, B;
  fill(A);
  int b = 0;
  for (; b + 1 < nb; b += 2) {
    fill(B);
    compute(A);
    fill(A);
    compute(B);
  }
  if (b < nb) compute(A);
}

int gemv_team(int H) {
  const int nch = H / 8;
  int t = 64;
  while (t < nch && t < 1024) t <<= 1;
  return t;
}

}  // namespace

bool linear_gemv_fits(int H, int I, int B) {
  return B >= 1 && B <= kGemvMaxBatch && H % 8 == 0 && H / 8 <= 1024 &&
         (unsigned long long)I * H * 2 < (1ull << 32);
}

bool linear_pass_fits(int H, int I, int B, int k) {
  return B >= 1 && (long long)B * k <= kMaxPass && H % 8 == 0 && H / 8 <= 1024 &&
         I % kPassRows == 0 && (unsigned long long)I * H * 2 < (1ull << 32);
}

hipError_t launch_linear_pass(const void* M, const float* x, const float* w,
                              const int32_t* ids, const int32_t* n_touched, const int32_t* touched,
                              const int32_t* offsets, const int32_t* slots,
                              const uint8_t* zrow, float* part, float* y, int H, int I, int E,
                              int k, int B, int workgroups, hipStream_t s) {
  if (!linear_pass_fits(H, I, B, k) || workgroups < 1) return hipErrorInvalidValue;
  PassArgs a{M, x, w, n_touched, touched, offsets, slots, zrow, part, H, I, k, B, 0};
  a.tsz = gemv_team(H);
  const int threads = 1024;
  const int lds = 2 * (threads / kWave) * kMaxNP * 4 + kMaxPass * 4 + kMaxPass * kPassTok * 4 + 16;
  hipLaunchKernelGGL(gemv_pass_kernel, dim3(workgroups), dim3(threads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_part_combine(part, ids, y, B, k, I, E, s);
}

hipError_t launch_linear_gemv(const void* M, const float* x, const int32_t* ids, const float* w,
                              uint32_t* err, const uint8_t* zrow, float* y, int H, int I, int E,
                              int k, int B, int workgroups, hipStream_t s) {
  if (!linear_gemv_fits(H, I, B) || workgroups < 1 || E < 1 || E > 4096 ||
      B * k > kGemvMaxT)
    return hipErrorInvalidValue;
  GemvArgs a{M, x, ids, w, err, zrow, y, H, I, E, k, B, 0, 0};
  a.tsz = gemv_team(H);
  const int threads = 1024;
  const int nb = B <= 1 ? 1 : B <= 2 ? 2 : 4;
  const int rows = nb == 1 ? gemv_rows<1>() : nb == 2 ? gemv_rows<2>() : gemv_rows<4>();
  const int per = (threads / a.tsz) * rows;  // items per batch of the workgroup
  int rw = (I + workgroups - 1) / workgroups;
  rw = (rw + per - 1) / per * per;  // a multiple of the batch's item count
  a.rw = rw;
  const int wgs = (I + rw - 1) / rw;
  const int lds = 2 * (threads / kWave) * kMaxNP * 4 + rw * nb * 4 + kGemvMaxT * 4 +
                  kGemvMaxT * nb * 4 + ((E + 31) / 32) * 4 + 16;
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (nb == 1)
    hipLaunchKernelGGL(gemv_kernel<1>, dim3(wgs), dim3(threads), lds, s, a);
  else if (nb == 2)
    hipLaunchKernelGGL(gemv_kernel<2>, dim3(wgs), dim3(threads), lds, s, a);
  else
    hipLaunchKernelGGL(gemv_kernel<4>, dim3(wgs), dim3(threads), lds, s, a);
  return hipGetLastError();
}

}  // namespace moe

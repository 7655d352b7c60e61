// route.hip -- batched routing (router logits, exact top-k, softmax over the selected
// logits), the touched-expert union of a batch, and the load-time row-norm table.
//
// Routing: every token scores all E experts with the router, keeps the k largest logits
// and weights them with a softmax over those k ("Mixture of Experts Changes the
// Arithmetic", section "Two Numbers Instead of One": k of E experts per token, re-chosen
// in every layer).  The order of the ids is the routing order: descending logit, ties to
// the lower id.
//
// Union: the distinct experts a batch touches, E[1-(1-k/E)^B] on average for uniform
// routing ("501B of which 23B are switched on", section 2), with each expert's token
// list, so that a batched layer reads every touched expert once.
#include "bf16_split.h"
#include "kernels.h"

namespace moe {
namespace {

// Router GEMV for B tokens: one team (256 threads) per R router rows, held in registers;
// each x chunk load serves the R rows (x is read from L2 once per R rows, not per row), and
// R rows x TB tokens are reduced per LDS round.
template <DT RT, int CPT, int R, int TB>
__global__ __launch_bounds__(256) void router_gemv_kernel(RouteArgs a) {
  constexpr int NP = R * TB;
  static_assert(NP <= 16, "wave_multi_sum reduces at most 16 values");
  __shared__ float red[2][4][NP];
  const int t = threadIdx.x, lane = t & 63, wit = t >> 6;
  const int nch = a.H / 8;
  for (int e0 = blockIdx.x * R; e0 < a.E; e0 += gridDim.x * R) {
    typename Fmt<RT>::Raw r[R][CPT];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int e = e0 + rr < a.E ? e0 + rr : a.E - 1;  // rows past E: computed, dropped
      const void* rp = row_ptr<RT>(a.router, (size_t)e, a.H);
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const int ch = t + m * kTeam;
        if (ch < nch) r[rr][m] = Fmt<RT>::load(rp, nullptr, ch);
        else __builtin_memset(&r[rr][m], 0, sizeof(r[rr][m]));
      }
    }
    int parity = 0;
    for (int b0 = 0; b0 < a.B; b0 += TB) {
      float acc[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
      // x loads without conditions (tokens past B re-read token B-1 and are dropped;
      // chunks past the row end re-read the last chunk against zero weights), so that all
      // of a chunk's token loads are in flight together
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const int ch = min(t + m * kTeam, nch - 1);
        f32x4 lo[TB], hi[TB];
#pragma unroll
        for (int q = 0; q < TB; ++q) {
          const float* xb = a.x + (size_t)min(b0 + q, a.B - 1) * a.H;
          lo[q] = reinterpret_cast<const f32x4*>(xb)[2 * ch];
          hi[q] = reinterpret_cast<const f32x4*>(xb)[2 * ch + 1];
        }
#pragma unroll
        for (int q = 0; q < TB; ++q) {
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
            float w[8];
            Fmt<RT>::decode(r[rr][m], w);
            float s = acc[rr * TB + q];
            s = fmaf(w[0], lo[q].x, s); s = fmaf(w[1], lo[q].y, s);
            s = fmaf(w[2], lo[q].z, s); s = fmaf(w[3], lo[q].w, s);
            s = fmaf(w[4], hi[q].x, s); s = fmaf(w[5], hi[q].y, s);
            s = fmaf(w[6], hi[q].z, s); s = fmaf(w[7], hi[q].w, s);
            acc[rr * TB + q] = s;
          }
        }
      }
      const float tot = wave_multi_sum<NP>(acc, lane);
      if (lane < NP) red[parity][wit][lane] = tot;
      __syncthreads();
      if (t < NP) {
        const int rr = t / TB, q = t % TB, b = b0 + q, e = e0 + rr;
        if (b < a.B && e < a.E)
          a.logits[(size_t)b * a.E + e] =
              red[parity][0][t] + red[parity][1][t] + red[parity][2][t] + red[parity][3][t];
      }
      parity ^= 1;
    }
  }
}

// Top-k + softmax: one workgroup per token (wg_topk_bitonic: the waves read the logits and
// select in registers; wave 0 forms the weights).
template <int KP>
__global__ __launch_bounds__(1024) void topk_kernel(const float* logits, float* logits_copy,
                                                   int E, int k, int B, int32_t* ids,
                                                   float* w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const float* lb = logits + (size_t)b * E;
    if (logits_copy)
      for (int e = threadIdx.x; e < E; e += blockDim.x) logits_copy[(size_t)b * E + e] = lb[e];
    const uint64_t top = wg_topk_bitonic<KP>(
        E, [&](int e) { return make_key(lb[e], (uint32_t)e); }, cand);
    if (threadIdx.x < kWave) {
      const int i = threadIdx.x;
      const float l0 = from_ordered_bits(__builtin_amdgcn_readfirstlane((uint32_t)(top >> 32)));
      const float ex = i < k ? expf(key_value(top) - l0) : 0.0f;
      const float sum = wave_sum(ex);
      if (i < k) {
        ids[(size_t)b * k + i] = (int32_t)key_index(top);
        w[(size_t)b * k + i] = ex / sum;
      }
    }
    __syncthreads();  // cand is reused by the next token
  }
}

// Union of the batch's experts in one workgroup: a bitmap of tokens per expert in LDS
// (LDS atomics give a schedule-independent result), per-expert counts, a prefix sum, and
// each (token, slot) placed by the rank of its token among the expert's tokens.  The
// bitmap rows are padded to an odd word count, so that threads reading the same word of
// different experts hit different banks, and the count pass also keeps each row's running
// popcount per word, so a rank is two reads however large the batch.
// With x given, workgroups 1.. meanwhile split x [nx] into bf16 hi, lo (the batched MFMA
// paths' operand), which saves that step a launch of its own.
__global__ __launch_bounds__(1024) void union_kernel(const int32_t* ids, int B, int k, int E,
                                                     int32_t* n_touched, int32_t* touched,
                                                     int32_t* offsets, int32_t* slots,
                                                     Ctrl* ctrl, const float* x, size_t nx,
                                                     uint16_t* xh, uint16_t* xl) {
  if (blockIdx.x > 0) {
    split_x_range(x, nx, xh, xl, (blockIdx.x - 1) * (size_t)blockDim.x + threadIdx.x,
                  (size_t)(gridDim.x - 1) * blockDim.x);
    return;
  }
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int W = (B + 31) / 32, Wp = W | 1;
  uint32_t* bits = reinterpret_cast<uint32_t*>(smem);                // [E][Wp]
  int32_t* pre = reinterpret_cast<int32_t*>(bits + (size_t)E * Wp);  // [E][Wp] set bits before word q
  int32_t* cnt = pre + (size_t)E * Wp;                               // [E]
  int32_t* off = cnt + E;                                      // [E+1]
  __shared__ int32_t part[1024 / kWave];
  __shared__ int32_t tpart[1024 / kWave];
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < E * Wp; i += nt) bits[i] = 0u;
  __syncthreads();
  for (int f = tid; f < B * k; f += nt) {
    const int e = ids[f], b = f / k;
    if (e < 0 || e >= E) {
      if (ctrl)
        __hip_atomic_fetch_or(&ctrl->err, kErrBadId, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    const uint32_t old = atomicOr(&bits[e * Wp + b / 32], 1u << (b % 32));
    if ((old >> (b % 32)) & 1u) {
      if (ctrl)
        __hip_atomic_fetch_or(&ctrl->err, kErrBadId, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int c = 0;
    for (int q = 0; q < W; ++q) {
      pre[e * Wp + q] = c;
      c += __popc(bits[e * Wp + q]);
    }
    cnt[e] = c;
  }
  __syncthreads();
  // Exclusive scan of counts (and of touched flags): contiguous segments per thread, an
  // inclusive scan of the segment sums within each wave (shuffles), then the wave totals
  // in order.
  const int seg = (E + nt - 1) / nt;
  const int e0 = tid * seg, e1 = min(E, e0 + seg);
  int s = 0, ts = 0;
  for (int e = e0; e < e1; ++e) { s += cnt[e]; ts += cnt[e] > 0; }
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  int is = s, its = ts;
  for (int d = 1; d < kWave; d <<= 1) {
    const int a = __shfl_up(is, d, kWave), b = __shfl_up(its, d, kWave);
    if (lane >= d) { is += a; its += b; }
  }
  if (lane == kWave - 1) { part[wave] = is; tpart[wave] = its; }
  __syncthreads();
  if (tid == 0) {
    int run = 0, trun = 0;
    for (int i = 0; i < nt / kWave; ++i) {
      const int v = part[i], tv = tpart[i];
      part[i] = run; tpart[i] = trun;
      run += v; trun += tv;
    }
    off[E] = run;
    offsets[E] = run;
    *n_touched = trun;
  }
  __syncthreads();
  s = part[wave] + is - s;
  ts = tpart[wave] + its - ts;
  for (int e = e0; e < e1; ++e) {
    off[e] = s;
    offsets[e] = s;
    if (cnt[e] > 0) touched[ts++] = e;
    s += cnt[e];
  }
  __syncthreads();
  for (int f = tid; f < B * k; f += nt) {
    const int e = ids[f], b = f / k;
    if (e < 0 || e >= E) continue;
    // a repeated expert within a token keeps its first choice only (the token is counted
    // once above); the later choice gets no slot
    bool dup = false;
    for (int j = b * k; j < f && !dup; ++j) dup = ids[j] == e;
    if (dup) continue;
    const int q = e * Wp + b / 32;
    const int rank = pre[q] + __popc(bits[q] & ((1u << (b % 32)) - 1u));
    slots[off[e] + rank] = f;
  }
}

// ||row||_2 of every row, fp32 sum of squares; one team per row, grid-stride.
template <DT dt, int CPT>
__global__ __launch_bounds__(256) void row_norms_kernel(const void* base, const uint8_t* sc,
                                                        size_t rows, int H, float* out) {
  __shared__ float red[4];
  const int t = threadIdx.x, nch = H / 8;
  for (size_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const void* rp = row_ptr<dt>(base, r, H);
    const uint8_t* sp = scale_row_ptr(sc, r, H);
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int ch = t + m * kTeam;
      if (ch < nch) {
        float v[8];
        Fmt<dt>::decode(Fmt<dt>::load(rp, sp, ch), v);
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(v[i], v[i], s);
      }
    }
    s = wave_sum(s);
    if ((t & 63) == 0) red[t >> 6] = s;
    __syncthreads();
    if (t == 0) out[r] = sqrtf(red[0] + red[1] + red[2] + red[3]);
    __syncthreads();
  }
}

int cpt_for(int H) {
  const int nch = H / 8;
  const int c = (nch + kTeam - 1) / kTeam;
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 0;
}

template <DT RT, int R>
hipError_t launch_gemv_r(const RouteArgs& a, hipStream_t s) {
  const int rows = (a.E + R - 1) / R;  // R router rows per workgroup pass
  const int grid = rows < 2048 ? rows : 2048;
  // tokens per round: 4 for B <= 4, else 16 / max(R, CPT) (at least 4), so that a round's
  // x loads (2 TB CPT 16-byte loads per thread) and R TB sums stay within 16 of each; 16
  // tokens at H = 2048 and one row per workgroup are then one round (one x round trip and
  // one LDS reduction instead of four)
  const bool wide = a.B > 4;
#define MOE_GEMV_CASE(C)                                                                   \
  case C: {                                                                                \
    constexpr int tbw = 16 / (R > C ? R : C) > 4 ? 16 / (R > C ? R : C) : 4;                \
    if (wide)                                                                              \
      hipLaunchKernelGGL((router_gemv_kernel<RT, C, R, tbw>), dim3(grid), dim3(256), 0, s, a); \
    else                                                                                   \
      hipLaunchKernelGGL((router_gemv_kernel<RT, C, R, 4>), dim3(grid), dim3(256), 0, s, a);   \
    break;                                                                                 \
  }
  switch (cpt_for(a.H)) {
    MOE_GEMV_CASE(1)
    MOE_GEMV_CASE(2)
    MOE_GEMV_CASE(4)
    MOE_GEMV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_GEMV_CASE
  return hipGetLastError();
}
// Rows per workgroup: four where that still gives most CUs a workgroup (each x load then
// serves four rows), fewer for small routers (E = 256 with four rows per workgroup left
// three quarters of the CUs idle).
template <DT RT>
hipError_t launch_gemv(const RouteArgs& a, hipStream_t s) {
  if (a.E >= 768) return launch_gemv_r<RT, 4>(a, s);
  if (a.E >= 384) return launch_gemv_r<RT, 2>(a, s);
  return launch_gemv_r<RT, 1>(a, s);
}

template <DT dt>
hipError_t launch_norms_t(const void* base, const uint8_t* sc, size_t rows, int H, float* out,
                          hipStream_t s) {
  const int grid = rows < 65536 ? (int)rows : 65536;
  switch (cpt_for(H)) {
    case 1: hipLaunchKernelGGL((row_norms_kernel<dt, 1>), dim3(grid), dim3(256), 0, s, base, sc, rows, H, out); break;
    case 2: hipLaunchKernelGGL((row_norms_kernel<dt, 2>), dim3(grid), dim3(256), 0, s, base, sc, rows, H, out); break;
    case 4: hipLaunchKernelGGL((row_norms_kernel<dt, 4>), dim3(grid), dim3(256), 0, s, base, sc, rows, H, out); break;
    case 8: hipLaunchKernelGGL((row_norms_kernel<dt, 8>), dim3(grid), dim3(256), 0, s, base, sc, rows, H, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, DT rt, hipStream_t s) {
  const float* lsrc = a.logits_in;
  if (!lsrc) {
    hipError_t e = rt == DT::F32 ? launch_gemv<DT::F32>(a, s) : launch_gemv<DT::BF16>(a, s);
    if (e != hipSuccess) return e;
    lsrc = a.logits;
  }
  const int lds = 16 * topk_kp(a.k) * 8;
  const int grid = a.B < 4096 ? a.B : 4096;
  float* copy = (a.logits_in && a.logits) ? a.logits : nullptr;
  switch (topk_kp(a.k)) {
#define MOE_TOPK_CASE(KP)                                                                   \
  case KP:                                                                                  \
    hipLaunchKernelGGL(topk_kernel<KP>, dim3(grid), dim3(1024), lds, s, lsrc, copy, a.E, a.k, \
                       a.B, a.ids, a.w);                                                    \
    break;
    MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(4) MOE_TOPK_CASE(8) MOE_TOPK_CASE(16)
    MOE_TOPK_CASE(32) MOE_TOPK_CASE(64)
#undef MOE_TOPK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int union_lds_bytes(int B, int E) {
  return E * (((B + 31) / 32) | 1) * 8 + (2 * E + 1) * 4;
}

hipError_t launch_union(const int32_t* ids, int B, int k, int E, int32_t* n_touched,
                        int32_t* touched, int32_t* offsets, int32_t* slots, Ctrl* ctrl,
                        hipStream_t s, const float* x, size_t nx, uint16_t* xh, uint16_t* xl) {
  const int lds = union_lds_bytes(B, E);
  static int lds_set = 0;
  if (lds > lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(union_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kUnionMaxLds);
    if (e != hipSuccess) return e;
    lds_set = kUnionMaxLds;
  }
  // one split workgroup per 8192 elements (8 per thread), at most 64
  const size_t nsplit = x && nx ? (nx + 8191) / 8192 : 0;
  const unsigned grid = 1u + (unsigned)(nsplit < 64 ? nsplit : 64);
  hipLaunchKernelGGL(union_kernel, dim3(grid), dim3(1024), lds, s, ids, B, k, E, n_touched,
                     touched, offsets, slots, ctrl, x, nx, xh, xl);
  return hipGetLastError();
}

hipError_t launch_row_norms(const void* base, const uint8_t* sc, DT dt, size_t rows, int H,
                            float* out, hipStream_t s) {
  switch (dt) {
    case DT::F32: return launch_norms_t<DT::F32>(base, sc, rows, H, out, s);
    case DT::BF16: return launch_norms_t<DT::BF16>(base, sc, rows, H, out, s);
    case DT::MXFP4: return launch_norms_t<DT::MXFP4>(base, sc, rows, H, out, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace moe

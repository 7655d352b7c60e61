// batched_swiglu.hip -- SwiGLU experts for a batch of B > 1 tokens.
//
// A batch reads each touched expert once for every token routed to it (the union of the
// routings with per-expert token buckets): per-token time falls with the batch because the
// reads are shared, not skipped ("501B of which 23B are switched on", section 3[B]); the
// expert FFN itself is the gated one of the "Routed experts" section of the arXiv
// 2610.37386 review.  After routing and the union, three launches:
//   1. gate/up  (MFMA): for every (touched or shared expert, block of 256 channels), the
//      products g = G x and u = V x for the expert's tokens, then a = w * silu(g) * u with
//      w the router weight of that token's choice (1 for a shared expert);
//   2. down (VALU): for every (expert, block of output columns), one partial output
//      p = sum_j a_j d_j per (token, choice) over all the expert's channels;
//   3. combine: y_b = the token's k partials in routing order, then the shared experts'.
// Every output element has one writer and a fixed summation order, so results do not
// depend on scheduling.
//
// Gate/up on MFMA (v_mfma_f32_16x16x32_bf16; lane l holds A[l%16][8*(l/16)..+8],
// B[8*(l/16)..+8][l%16], D[4*(l/16)..+4][l%16]).  A is 16 channel rows, B is 16 tokens.
// x enters as bf16 hi + lo (two MFMAs per product, ~16 significant bits).  The K order
// inside a step is permuted so each lane loads one contiguous piece of its row: a step
// spans 4*LC elements and lane group g = l/16 owns [kb + LC*g, kb + LC*g + LC); MFMA number
// c of the step takes its 8-element slice c from A and B alike (a permutation of K applied
// to both operands leaves the product unchanged).  bf16 rows: LC = 8 (one 16-byte load);
// MXFP4 rows: LC = 32 (one 16-byte load of codes = exactly one scale block), decoded to
// bf16 in registers (e2m1 times a power of two is exact in bf16).
#include "kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------------------
// Gate/up
// ------------------------------------------------------------------------------------
constexpr int kGuWaves = 4;
constexpr int kGuRowsPerWave = 64;
constexpr int kGuRows = kGuWaves * kGuRowsPerWave;  // channels per workgroup
constexpr int kGuTok = 64;                          // tokens per pass (4 MFMA token tiles)

template <DT dt> struct Gu;

template <> struct Gu<DT::BF16> {
  static constexpr int LC = 8;  // elements per lane per step
  struct Raw { u32x4 q; };
  static __device__ __forceinline__ Raw load(const uint8_t* row, const uint8_t*, int k) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + (size_t)k * 2));
    return r;
  }
  static __device__ __forceinline__ bf16x8 slice(const Raw& r, int) {
    return __builtin_bit_cast(bf16x8, r.q);
  }
  static __device__ __forceinline__ Raw zero_if(Raw r, bool live) {
    const uint32_t m = live ? 0xFFFFFFFFu : 0u;
    r.q &= u32x4{m, m, m, m};
    return r;
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H * 2; }
};

template <> struct Gu<DT::MXFP4> {
  static constexpr int LC = 32;
  struct Raw { u32x4 q; uint32_t s; };
  static __device__ __forceinline__ Raw load(const uint8_t* row, const uint8_t* srow, int k) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + k / 2));
    r.s = __builtin_nontemporal_load(srow + k / 32);
    return r;
  }
  // slice c = elements 8c .. 8c+7 of the lane's 32: code dword c, low nibble first
  static __device__ __forceinline__ bf16x8 slice(const Raw& r, int c) {
    const float sc = __uint_as_float(r.s << 23);
    const uint32_t w = c == 0 ? r.q.x : c == 1 ? r.q.y : c == 2 ? r.q.z : r.q.w;
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  }
  static __device__ __forceinline__ Raw zero_if(Raw r, bool live) {
    const uint32_t m = live ? 0xFFFFFFFFu : 0u;
    r.q &= u32x4{m, m, m, m};
    return r;
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H / 2; }
};

// One pass of the gate/up products of R 16-row tiles of one wave (rows rbase + 16r + l%16)
// for NT 16-token tiles, over all of K.  U steps are loaded before their MFMAs.
template <DT dt, int R, int NT, int U>
__device__ __forceinline__ void gu_tiles(const uint8_t* G, const uint8_t* V, const uint8_t* Gs,
                                         const uint8_t* Vs, int H, int rows, int rbase,
                                         const uint16_t* xh, const uint16_t* xl,
                                         const int* tok_b, int np, f32x4 (&ag)[R][NT],
                                         f32x4 (&au)[R][NT]) {
  using F = Gu<dt>;
  constexpr int LC = F::LC;
  constexpr int SC = LC / 8;      // MFMAs per step and operand
  constexpr int STEP = 4 * LC;    // elements of K per step
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const size_t rb = F::row_bytes(H);
  const uint8_t* gp[R];
  const uint8_t* vp[R];
  const uint8_t* gsp[R];
  const uint8_t* vsp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int row = rbase + 16 * r + l16;
    row = row < rows ? row : rows - 1;  // rows past the end compute values that are dropped
    gp[r] = G + (size_t)row * rb;
    vp[r] = V + (size_t)row * rb;
    gsp[r] = Gs ? Gs + (size_t)row * (H / 32) : nullptr;
    vsp[r] = Vs ? Vs + (size_t)row * (H / 32) : nullptr;
  }
  const uint16_t* xhp[NT];
  const uint16_t* xlp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tc = 16 * t + l16;
    const int b = tok_b[tc < np ? tc : 0];  // padded token columns repeat the first token
    xhp[t] = xh + (size_t)b * H;
    xlp[t] = xl + (size_t)b * H;
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      ag[r][t] = f32x4{0, 0, 0, 0};
      au[r][t] = f32x4{0, 0, 0, 0};
    }
  for (int kb = 0; kb < H; kb += U * STEP) {
    typename F::Raw A[U][2][R];
    u32x4 Bh[U][NT][SC], Bl[U][NT][SC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + u * STEP + LC * g;
      const bool live = k < H;  // H is a multiple of 32: a lane's piece is all in or all out
      const int kc = live ? k : 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        A[u][0][r] = F::zero_if(F::load(gp[r], gsp[r], kc), live);
        A[u][1][r] = F::zero_if(F::load(vp[r], vsp[r], kc), live);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < SC; ++c) {
          Bh[u][t][c] = *reinterpret_cast<const u32x4*>(xhp[t] + kc + 8 * c);
          Bl[u][t][c] = *reinterpret_cast<const u32x4*>(xlp[t] + kc + 8 * c);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < SC; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bf16x8 a0 = F::slice(A[u][0][r], c);
          const bf16x8 a1 = F::slice(A[u][1][r], c);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const bf16x8 bh = __builtin_bit_cast(bf16x8, Bh[u][t][c]);
            const bf16x8 bl = __builtin_bit_cast(bf16x8, Bl[u][t][c]);
            ag[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bh, ag[r][t], 0, 0, 0);
            ag[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl, ag[r][t], 0, 0, 0);
            au[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bh, au[r][t], 0, 0, 0);
            au[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl, au[r][t], 0, 0, 0);
          }
        }
  }
}

// a = w * silu(g) * u for the lane's 4 rows of each tile and its token column.
template <int R, int NT>
__device__ __forceinline__ void gu_store(const f32x4 (&ag)[R][NT], const f32x4 (&au)[R][NT],
                                         int rows, int rbase, const int* tok_slot,
                                         const float* tok_w, int np, float* act, int IA) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tc = 16 * t + l16;
    if (tc >= np) continue;
    const float wt = tok_w[tc];
    float* arow = act + (size_t)tok_slot[tc] * IA;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = rbase + 16 * r + 4 * g;
      f32x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = wt * silu(ag[r][t][i]) * au[r][t][i];
      if (row + 3 < rows) {
        *reinterpret_cast<f32x4*>(arow + row) = a;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (row + i < rows) arow[row + i] = a[i];
      }
    }
  }
}

// The wave's 64 rows for np <= 64 tokens: R*NT <= 4 keeps the accumulators in 32*R*NT
// registers; fewer tiles per sweep when there are more token tiles.
template <DT dt, int U>
__device__ __forceinline__ void gu_wave(const uint8_t* G, const uint8_t* V, const uint8_t* Gs,
                                        const uint8_t* Vs, int H, int rows, int rbase,
                                        const uint16_t* xh, const uint16_t* xl, const int* tok_b,
                                        const int* tok_slot, const float* tok_w, int np,
                                        float* act, int IA) {
  const int nt = (np + 15) / 16;
  if (nt <= 1) {
    f32x4 ag[4][1], au[4][1];
    gu_tiles<dt, 4, 1, U>(G, V, Gs, Vs, H, rows, rbase, xh, xl, tok_b, np, ag, au);
    gu_store<4, 1>(ag, au, rows, rbase, tok_slot, tok_w, np, act, IA);
  } else if (nt <= 2) {
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      f32x4 ag[2][2], au[2][2];
      gu_tiles<dt, 2, 2, U>(G, V, Gs, Vs, H, rows, rbase + 32 * h, xh, xl, tok_b, np, ag, au);
      gu_store<2, 2>(ag, au, rows, rbase + 32 * h, tok_slot, tok_w, np, act, IA);
    }
  } else {
#pragma unroll 1
    for (int h = 0; h < 4; ++h) {
      f32x4 ag[1][4], au[1][4];
      gu_tiles<dt, 1, 4, U>(G, V, Gs, Vs, H, rows, rbase + 16 * h, xh, xl, tok_b, np, ag, au);
      gu_store<1, 4>(ag, au, rows, rbase + 16 * h, tok_slot, tok_w, np, act, IA);
    }
  }
}

// Token bucket of expert slot t: routed (t < slots_max) -> the union's bucket, shared ->
// every token of the batch.
struct Bucket {
  int count;
  bool shared;
  int e;  // routed expert id, or shared index
};

__device__ __forceinline__ Bucket bucket_of(const BsArgs& a, int t) {
  Bucket b;
  if (t < a.slots_max) {
    b.shared = false;
    if (t >= *a.n_touched) {
      b.count = 0;
      b.e = 0;
      return b;
    }
    b.e = a.touched[t];
    b.count = a.offsets[b.e + 1] - a.offsets[b.e];
  } else {
    b.shared = true;
    b.e = t - a.slots_max;
    b.count = a.B;
  }
  return b;
}

// Fill the pass's token list: token index, act/partial row, weight.
__device__ __forceinline__ void fill_tokens(const BsArgs& a, const Bucket& bk, int p0, int np,
                                            int* tok_b, int* tok_slot, float* tok_w) {
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    if (bk.shared) {
      const int b = p0 + i;
      tok_b[i] = b;
      tok_slot[i] = a.B * a.k + bk.e * a.B + b;
      tok_w[i] = 1.0f;
    } else {
      const int slot = a.slots[a.offsets[bk.e] + p0 + i];
      tok_b[i] = slot / a.k;
      tok_slot[i] = slot;
      tok_w[i] = a.w[slot];
    }
  }
}

template <DT et, DT st>
__global__ __launch_bounds__(kGuWaves * 64) void bs_gateup_kernel(BsArgs a) {
  __shared__ int tok_b[kGuTok];
  __shared__ int tok_slot[kGuTok];
  __shared__ float tok_w[kGuTok];
  const Bucket bk = bucket_of(a, blockIdx.y);
  const int rows = bk.shared ? a.IS : a.I;
  const int rbase = blockIdx.x * kGuRows + (threadIdx.x >> 6) * kGuRowsPerWave;
  if (bk.count == 0 || blockIdx.x * kGuRows >= rows) return;  // whole workgroup leaves
  for (int p0 = 0; p0 < bk.count; p0 += kGuTok) {
    const int np = min(kGuTok, bk.count - p0);
    __syncthreads();  // the previous pass is done with the token list
    fill_tokens(a, bk, p0, np, tok_b, tok_slot, tok_w);
    __syncthreads();
    if (rbase >= rows) continue;
    if (bk.shared) {
      const size_t off = (size_t)bk.e * a.IS;
      gu_wave<st, st == DT::MXFP4 ? 1 : 2>(
          reinterpret_cast<const uint8_t*>(a.sh_gate) + off * Gu<st>::row_bytes(a.H),
          reinterpret_cast<const uint8_t*>(a.sh_up) + off * Gu<st>::row_bytes(a.H), nullptr,
          nullptr, a.H, rows, rbase, a.xh, a.xl, tok_b, tok_slot, tok_w, np, a.act, a.IA);
    } else {
      const size_t off = (size_t)bk.e * a.I;
      const uint8_t* gs = a.gate_s ? a.gate_s + off * (a.H / 32) : nullptr;
      const uint8_t* vs = a.up_s ? a.up_s + off * (a.H / 32) : nullptr;
      gu_wave<et, et == DT::MXFP4 ? 1 : 2>(
          reinterpret_cast<const uint8_t*>(a.gate) + off * Gu<et>::row_bytes(a.H),
          reinterpret_cast<const uint8_t*>(a.up) + off * Gu<et>::row_bytes(a.H), gs, vs, a.H,
          rows, rbase, a.xh, a.xl, tok_b, tok_slot, tok_w, np, a.act, a.IA);
    }
  }
}

// ------------------------------------------------------------------------------------
// Down: p[pair][h] = sum_j a[pair][j] * d_j[h]
// ------------------------------------------------------------------------------------
constexpr int kDnWaves = 4;  // the expert's channels are split in 4 contiguous ranges
constexpr int kDnU = 8;      // rows loaded before they are used

template <DT dt> struct Dn;

template <> struct Dn<DT::BF16> {
  static constexpr int EPT = 8;   // output columns per lane
  static constexpr int NTMAX = 8; // token pairs per pass
  struct Raw { u32x4 q; };
  static __device__ __forceinline__ Raw load(const uint8_t* row, const uint8_t*, int h) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + (size_t)h * 2));
    return r;
  }
  static __device__ __forceinline__ void decode(const Raw& r, float (&v)[EPT]) {
    v[0] = __uint_as_float(r.q.x << 16); v[1] = __uint_as_float(r.q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(r.q.y << 16); v[3] = __uint_as_float(r.q.y & 0xFFFF0000u);
    v[4] = __uint_as_float(r.q.z << 16); v[5] = __uint_as_float(r.q.z & 0xFFFF0000u);
    v[6] = __uint_as_float(r.q.w << 16); v[7] = __uint_as_float(r.q.w & 0xFFFF0000u);
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H * 2; }
};

template <> struct Dn<DT::MXFP4> {
  static constexpr int EPT = 32;
  static constexpr int NTMAX = 2;
  struct Raw { u32x4 q; uint32_t s; };
  static __device__ __forceinline__ Raw load(const uint8_t* row, const uint8_t* srow, int h) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + h / 2));
    r.s = __builtin_nontemporal_load(srow + h / 32);
    return r;
  }
  static __device__ __forceinline__ void decode(const Raw& r, float (&v)[EPT]) {
    const float sc = __uint_as_float(r.s << 23);
    const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[c], sc, 0);
      const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[c], sc, 1);
      const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[c], sc, 2);
      const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[c], sc, 3);
      v[8 * c + 0] = p0.x; v[8 * c + 1] = p0.y; v[8 * c + 2] = p1.x; v[8 * c + 3] = p1.y;
      v[8 * c + 4] = p2.x; v[8 * c + 5] = p2.y; v[8 * c + 6] = p3.x; v[8 * c + 7] = p3.y;
    }
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H / 2; }
};

template <DT dt> constexpr int dn_cols() { return 64 * Dn<dt>::EPT; }

// kDnU rows starting at j (TAIL: some of them past j1, which get weight 0).
template <DT dt, int NT, bool TAIL>
__device__ __forceinline__ void dn_rows(const uint8_t* D, const uint8_t* Ds, size_t rb, int H,
                                        int hc, int j, int j1, const float* const (&ap)[NT],
                                        float (&acc)[NT][Dn<dt>::EPT]) {
  using F = Dn<dt>;
  constexpr int EPT = F::EPT;
  typename F::Raw r[kDnU];
  float av[NT][kDnU];
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    const int jj = TAIL ? (j + u < j1 ? j + u : j1 - 1) : j + u;
    r[u] = F::load(D + (size_t)jj * rb, Ds ? Ds + (size_t)jj * (H / 32) : nullptr, hc);
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      const float v = ap[p][jj];
      av[p][u] = (!TAIL || j + u < j1) ? v : 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < kDnU; ++u) {
    float d[EPT];
    F::decode(r[u], d);
#pragma unroll
    for (int p = 0; p < NT; ++p)
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[p][e] = fmaf(av[p][u], d[e], acc[p][e]);
  }
}

// One pass of NT pairs over the wave's channel range [j0, j1) of one expert.
template <DT dt, int NT>
__device__ __forceinline__ void dn_pass(const uint8_t* D, const uint8_t* Ds, int H, int h,
                                        bool live, int j0, int j1, const float* act, int IA,
                                        const int* pslot, float (&acc)[NT][Dn<dt>::EPT]) {
  using F = Dn<dt>;
  constexpr int EPT = F::EPT;
  const size_t rb = F::row_bytes(H);
  const int hc = live ? h : 0;  // dead lanes read column 0 and store nothing
  const float* ap[NT];
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    ap[p] = uniform_ptr(act + (size_t)pslot[p] * IA);
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[p][e] = 0.0f;
  }
  int j = j0;
  for (; j + kDnU <= j1; j += kDnU) dn_rows<dt, NT, false>(D, Ds, rb, H, hc, j, j1, ap, acc);
  if (j < j1) dn_rows<dt, NT, true>(D, Ds, rb, H, hc, j, j1, ap, acc);
}

// Sum the 4 waves' accumulators of pair p in wave order and store the partial row.
template <DT dt, int NT>
__device__ __forceinline__ void dn_reduce_store(float (&acc)[NT][Dn<dt>::EPT], float* red,
                                                const int* pslot, int np, float* part, int H,
                                                int h, bool live) {
  constexpr int EPT = Dn<dt>::EPT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    if (wave > 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4)
        *reinterpret_cast<f32x4*>(red + ((wave - 1) * EPT + e) * 64 + lane * 4) =
            f32x4{acc[p][e], acc[p][e + 1], acc[p][e + 2], acc[p][e + 3]};
    }
    __syncthreads();
    if (wave == 0 && p < np && live) {
      float* out = part + (size_t)pslot[p] * H + h;
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        f32x4 s = {acc[p][e], acc[p][e + 1], acc[p][e + 2], acc[p][e + 3]};
#pragma unroll
        for (int w = 0; w < kDnWaves - 1; ++w)
          s += *reinterpret_cast<const f32x4*>(red + (w * EPT + e) * 64 + lane * 4);
        *reinterpret_cast<f32x4*>(out + e) = s;
      }
    }
    __syncthreads();
  }
}

template <DT dt>
__device__ __forceinline__ void dn_item(const BsArgs& a, const Bucket& bk, const uint8_t* D,
                                        const uint8_t* Ds, int rows, float* red, int* pslot) {
  constexpr int EPT = Dn<dt>::EPT;
  constexpr int NTM = Dn<dt>::NTMAX;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.x * dn_cols<dt>() + EPT * lane;
  const bool live = h < a.H;  // H is a multiple of 32 and EPT divides 32
  const int per = (rows + kDnWaves - 1) / kDnWaves;
  const int j0 = min(rows, wave * per), j1 = min(rows, j0 + per);
  for (int p0 = 0; p0 < bk.count; p0 += NTM) {
    const int np = min(NTM, bk.count - p0);
    __syncthreads();
    if (threadIdx.x < np) {
      const int i = p0 + threadIdx.x;
      pslot[threadIdx.x] =
          bk.shared ? a.B * a.k + bk.e * a.B + i : a.slots[a.offsets[bk.e] + i];
    }
    __syncthreads();
    int ps[NTM];
#pragma unroll
    for (int p = 0; p < NTM; ++p) ps[p] = pslot[p < np ? p : 0];
    if (NTM >= 8 && np > 4) {
      float acc[8][EPT];
      dn_pass<dt, 8>(D, Ds, a.H, h, live, j0, j1, a.act, a.IA, ps, acc);
      dn_reduce_store<dt, 8>(acc, red, ps, np, a.part, a.H, h, live);
    } else if (NTM >= 4 && np > 2) {
      float acc[4][EPT];
      dn_pass<dt, 4>(D, Ds, a.H, h, live, j0, j1, a.act, a.IA, ps, acc);
      dn_reduce_store<dt, 4>(acc, red, ps, np, a.part, a.H, h, live);
    } else if (np > 1) {
      float acc[2][EPT];
      dn_pass<dt, 2>(D, Ds, a.H, h, live, j0, j1, a.act, a.IA, ps, acc);
      dn_reduce_store<dt, 2>(acc, red, ps, np, a.part, a.H, h, live);
    } else {
      float acc[1][EPT];
      dn_pass<dt, 1>(D, Ds, a.H, h, live, j0, j1, a.act, a.IA, ps, acc);
      dn_reduce_store<dt, 1>(acc, red, ps, np, a.part, a.H, h, live);
    }
  }
}

template <DT et, DT st>
__global__ __launch_bounds__(kDnWaves * 64) void bs_down_kernel(BsArgs a) {
  constexpr int EPT_MAX = Dn<et>::EPT > Dn<st>::EPT ? Dn<et>::EPT : Dn<st>::EPT;
  __shared__ __attribute__((aligned(16))) float red[(kDnWaves - 1) * EPT_MAX * 64];
  __shared__ int pslot[8];
  const Bucket bk = bucket_of(a, blockIdx.y);
  if (bk.count == 0) return;
  if (bk.shared) {
    if (blockIdx.x * dn_cols<st>() >= a.H) return;
    const uint8_t* D = reinterpret_cast<const uint8_t*>(a.sh_down_t) +
                       (size_t)bk.e * a.IS * Dn<st>::row_bytes(a.H);
    dn_item<st>(a, bk, D, nullptr, a.IS, red, pslot);
  } else {
    if (blockIdx.x * dn_cols<et>() >= a.H) return;
    const size_t off = (size_t)bk.e * a.I;
    const uint8_t* D =
        reinterpret_cast<const uint8_t*>(a.down_t) + off * Dn<et>::row_bytes(a.H);
    const uint8_t* Ds = a.down_s ? a.down_s + off * (a.H / 32) : nullptr;
    dn_item<et>(a, bk, D, Ds, a.I, red, pslot);
  }
}

// ------------------------------------------------------------------------------------
// Combine: y[b] = sum_i part[b*k + i] (routing order) + sum_s part[B*k + s*B + b]
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bs_combine_kernel(BsArgs a) {
  const int n4 = a.H / 4;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < (size_t)a.B * n4;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int b = (int)(idx / n4), c = (int)(idx % n4);
    const f32x4* P = reinterpret_cast<const f32x4*>(a.part);
    f32x4 s = {0, 0, 0, 0};
    for (int i = 0; i < a.k; ++i) s += P[(size_t)(b * a.k + i) * n4 + c];
    for (int sh = 0; sh < a.NS; ++sh) s += P[(size_t)(a.B * a.k + sh * a.B + b) * n4 + c];
    reinterpret_cast<f32x4*>(a.y)[(size_t)b * n4 + c] = s;
  }
}

template <DT et, DT st>
hipError_t launch_bs_typed(const BsArgs& a, hipStream_t s) {
  const int items = a.slots_max + a.NS;
  const int rows = a.I > a.IS ? a.I : a.IS;
  hipLaunchKernelGGL((bs_gateup_kernel<et, st>), dim3((rows + kGuRows - 1) / kGuRows, items),
                     dim3(kGuWaves * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int cmin = dn_cols<et>() < dn_cols<st>() ? dn_cols<et>() : dn_cols<st>();
  hipLaunchKernelGGL((bs_down_kernel<et, st>), dim3((a.H + cmin - 1) / cmin, items),
                     dim3(kDnWaves * 64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = (size_t)a.B * (a.H / 4);
  int g = (int)((n + 255) / 256);
  g = g > 2048 ? 2048 : g;
  hipLaunchKernelGGL(bs_combine_kernel, dim3(g), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_batched_swiglu(const BsArgs& a, DT et, DT st, hipStream_t s) {
  if (et == DT::BF16 && st == DT::BF16) return launch_bs_typed<DT::BF16, DT::BF16>(a, s);
  if (et == DT::MXFP4 && st == DT::BF16) return launch_bs_typed<DT::MXFP4, DT::BF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe

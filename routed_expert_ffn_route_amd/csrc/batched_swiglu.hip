// batched_swiglu.hip -- SwiGLU experts for a batch of B > 1 tokens.
//
// A batch reads each touched expert once for every token routed to it (the union of the
// routings with per-expert token buckets): per-token time falls with the batch because the
// reads are shared, not skipped ("501B of which 23B are switched on", section 3[B]); the
// expert FFN itself is the gated one of the "Routed experts" section of the arXiv
// 2610.37386 review.  After routing and the union, three launches:
//   1. gate/up  (MFMA): for every (touched or shared expert, block of 128 channels), the
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
// inside a step is permuted (the same permutation for A and B leaves the product
// unchanged) so that each lane's operand pieces are whole 16-byte pieces of its row: bf16
// steps of 64 elements (lane group g: elements 32c + 8g .. +8 of sub-step c), MXFP4 steps of
// 256 elements (lane group g: elements 32g .. +32 and 128 + 32g .. +32, one scale block
// each), decoded to bf16 in registers (e2m1 times a power of two is exact in bf16).
// Buckets of up to 16 tokens stream the weights into LDS with line-complete direct copies
// and read the fragments back from there; larger buckets load them into a register ring.
#include "kernels.h"
#include "lds_copy.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------------------
// Gate/up
// ------------------------------------------------------------------------------------
constexpr int kGuWaves = 4;
constexpr int kGuRowsW = 32;                    // channels per wave (2 MFMA row tiles)
constexpr int kGuRows = kGuWaves * kGuRowsW;    // channels per workgroup
constexpr int kGuTok = 64;                      // tokens per pass (up to 4 token tiles)
constexpr int kGuXElems = 8192;                 // staged x elements per buffer and array
constexpr int kGuPad = 8;                       // bf16 padding per staged x row
constexpr int kGuBuf = kGuXElems + kGuTok * kGuPad;
constexpr int kGuLds = 2 * 2 * kGuBuf * 2;      // dynamic LDS: [2 buffers][hi, lo][kGuBuf] bf16

// K width of one staged x chunk for NT token tiles (fixed LDS budget).
template <int NT> constexpr int gu_kx() { return kGuXElems / (16 * NT); }
template <int NT> constexpr int gu_ldx() { return gu_kx<NT>() + kGuPad; }
constexpr int gu_gcd(int a, int b) { return b == 0 ? a : gu_gcd(b, a % b); }
constexpr int gu_lcm(int a, int b) { return a / gu_gcd(a, b) * b; }

// Weight fragments of one K step for one 16-row tile.  A step is STEP elements; MFMA
// sub-step c of it takes A and B from the same K positions (boff).
template <DT dt> struct Gu;

template <> struct Gu<DT::BF16> {
  static constexpr int STEP = 64, SUB = 2;  // lane: 16 bytes per sub-step
  static constexpr bool kWideScales = false;
  struct Raw { u32x4 f[2]; };
  static __device__ __forceinline__ Raw load(const uint8_t* row, const uint8_t*, int k, int g,
                                             bool) {
    Raw r;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      r.f[c] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(row + (size_t)(k + 32 * c + 8 * g) * 2));
    return r;
  }
  static __device__ __forceinline__ void pass_on(const Raw&, Raw&) {}
  static __device__ __forceinline__ bf16x8 frag(const Raw& r, int c, int) {
    return __builtin_bit_cast(bf16x8, r.f[c]);
  }
  static __device__ __forceinline__ int boff(int c, int g) { return 32 * c + 8 * g; }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H * 2; }
};

// MXFP4 step of 256 elements: lane group g takes elements [32g, 32g + 32) and
// [128 + 32g, 160 + 32g), so each load instruction reads 64 contiguous code bytes of each of
// its 16 rows.  The scales of two steps are 16 bytes of the row (16-aligned when H is a
// multiple of 512), read once with the even step by all four lanes of the row: lane g's
// scale bytes are byte g of each dword (dwords 0, 1 for the even step's two pieces, 2, 3 for
// the odd step's, handed to the odd step's fragments by pass_on).  Loading a scale per
// piece and step instead doubled the cache lines each step touches, and line lookups, not
// bytes, bound this stream.
template <> struct Gu<DT::MXFP4> {
  static constexpr int STEP = 256, SUB = 8;
  static constexpr bool kWideScales = true;
  struct Raw { u32x4 q[2]; u32x4 s; };
  static __device__ __forceinline__ Raw load(const uint8_t* row, const uint8_t* srow, int k,
                                             int g, bool even) {
    Raw r;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      r.q[p] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(row + (k + 32 * g + 128 * p) / 2));
    if (even)  // scale lines are reused by later steps: cached load
      r.s = *(const __attribute__((address_space(1))) u32x4*)(srow + k / 32);
    return r;
  }
  static __device__ __forceinline__ void pass_on(const Raw& even, Raw& odd) {
    odd.s.x = even.s.z;
    odd.s.y = even.s.w;
  }
  // sub-step c = elements 8(c & 3) .. +7 of piece c >> 2: code dword c & 3, low nibble first
  static __device__ __forceinline__ bf16x8 frag(const Raw& r, int c, int g) {
    const uint32_t sb = __builtin_amdgcn_ubfe((c >> 2) ? r.s.y : r.s.x, 8 * g, 8);
    const float sc = __uint_as_float(sb << 23);
    const u32x4& q = r.q[c >> 2];
    const uint32_t w = (c & 3) == 0 ? q.x : (c & 3) == 1 ? q.y : (c & 3) == 2 ? q.z : q.w;
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  }
  static __device__ __forceinline__ int boff(int c, int g) {
    return 32 * g + 128 * (c >> 2) + 8 * (c & 3);
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H / 2; }
};

// Steps the pipelined loops may run with the wide scale loads (all of them for bf16).
template <DT dt>
__device__ __forceinline__ bool gu_wide_ok(int H) {
  return !Gu<dt>::kWideScales || H % 512 == 0;
}

// The staged x of tokens tok_b[0..np) (token columns past np repeat the first token, and
// their results are dropped; unconditional loads keep the load counters exact), K [kc, kc + kx):
// 1024 pieces of 16 bytes per array, 4 per thread; K past H reads the last valid piece
// and is never used.
struct GuX {
  u32x4 h[4], l[4];
};

template <int NT>
__device__ __forceinline__ void gu_x_load(GuX& xr, const uint16_t* xh, const uint16_t* xl,
                                          int H, const lds_i32* tok_b, int np, int kc) {
  constexpr int PR = gu_kx<NT>() / 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = threadIdx.x + i * kGuWaves * 64;
    const int tok = p / PR, q = p % PR;
    const int b = tok_b[tok < np ? tok : 0];
    int k = kc + 8 * q;
    k = k < H ? k : H - 8;
    const size_t off = (size_t)b * H + k;
    xr.h[i] = *reinterpret_cast<const u32x4*>(xh + off);
    xr.l[i] = *reinterpret_cast<const u32x4*>(xl + off);
  }
}

template <int NT>
__device__ __forceinline__ void gu_x_store(const GuX& xr, lds_u16* xs_h, lds_u16* xs_l) {
  constexpr int PR = gu_kx<NT>() / 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = threadIdx.x + i * kGuWaves * 64;
    const int tok = p / PR, q = p % PR;
    lds_st128(xs_h + tok * gu_ldx<NT>() + 8 * q, xr.h[i]);
    lds_st128(xs_l + tok * gu_ldx<NT>() + 8 * q, xr.l[i]);
  }
}

template <DT dt>
struct GuRing {
  typename Gu<dt>::Raw r[2][2];  // [matrix: G, V][row tile]
};

template <DT dt>
__device__ __forceinline__ void gu_a_load(GuRing<dt>& ar, const uint8_t* const (&rp)[2][2],
                                          const uint8_t* const (&sp)[2][2], int k, int g,
                                          bool even) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 2; ++r) ar.r[m][r] = Gu<dt>::load(rp[m][r], sp[m][r], k, g, even);
}

// The odd step's scales come from the even step's fragments (MXFP4).
template <DT dt>
__device__ __forceinline__ void gu_pass_on(const GuRing<dt>& even, GuRing<dt>& odd) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 2; ++r) Gu<dt>::pass_on(even.r[m][r], odd.r[m][r]);
}

// MFMAs of one K step (all its sub-steps) against the staged x: token tile t of the lane
// starts at xo[t], the step at k0.  CLAMP (a K tail): x positions past kmax read the piece
// at kmax, whose finite values meet zeroed weights.
template <DT dt, int NT, bool CLAMP = false>
__device__ __forceinline__ void gu_step(const GuRing<dt>& ar, const lds_u16* xs_h,
                                        const lds_u16* xs_l, const int (&xo)[NT], int k0,
                                        int g, f32x4 (&acc)[2][2][NT],
                                        int kmax = 0) {
  using F = Gu<dt>;
#pragma unroll
  for (int c = 0; c < F::SUB; ++c) {
    bf16x8 af[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 2; ++r) af[m][r] = F::frag(ar.r[m][r], c, g);
    int kk = k0 + F::boff(c, g);
    if (CLAMP) kk = kk < kmax ? kk : kmax;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int o = xo[t] + kk;
      const bf16x8 bh = __builtin_bit_cast(bf16x8, lds_ld128(xs_h + o));
      const bf16x8 bl = __builtin_bit_cast(bf16x8, lds_ld128(xs_l + o));
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 2; ++r)
          acc[m][r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m][r], bh, acc[m][r][t], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 2; ++r)
          acc[m][r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m][r], bl, acc[m][r][t], 0, 0, 0);
    }
  }
}

// Row pointers of the lane's two row tiles in G and V (and their scale rows).
template <DT dt>
struct GuRows {
  const uint8_t* rp[2][2];  // [matrix][tile]
  const uint8_t* sp[2][2];
};

template <DT dt>
__device__ __forceinline__ GuRows<dt> gu_rows(const uint8_t* G, const uint8_t* V,
                                              const uint8_t* Gs, const uint8_t* Vs, int H,
                                              int rows, int rbase, int l16, int g) {
  using F = Gu<dt>;
  GuRows<dt> R;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    int row = rbase + 16 * r + l16;
    row = row < rows ? row : rows - 1;  // rows past the end compute values that are dropped
    R.rp[0][r] = G + (size_t)row * F::row_bytes(H);
    R.rp[1][r] = V + (size_t)row * F::row_bytes(H);
    R.sp[0][r] = Gs ? Gs + (size_t)row * (H / 32) : nullptr;
    R.sp[1][r] = Vs ? Vs + (size_t)row * (H / 32) : nullptr;
  }
  return R;
}

// Weight fragments of a step that may reach past H: pieces that start past H read the
// row's last piece and are zeroed.
template <DT dt>
__device__ __forceinline__ void gu_a_load_masked(GuRing<dt>& ar, const GuRows<dt>& R, int H,
                                                 int k, int g) {
  using F = Gu<dt>;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      typename F::Raw v;
      if constexpr (dt == DT::MXFP4) {
        // any H that is a multiple of 32: the scale byte is read from the aligned dword
        // holding it and placed where frag looks for it (byte g of s.x, s.y)
        uint32_t sw[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int e0 = k + 32 * g + 128 * p;
          const int ec = e0 < H ? e0 : H - 32;
          v.q[p] = *reinterpret_cast<const u32x4*>(R.rp[m][r] + ec / 2);
          const uintptr_t a = reinterpret_cast<uintptr_t>(R.sp[m][r] + ec / 32);
          const uint32_t w = *(const __attribute__((address_space(1))) uint32_t*)(
              a & ~static_cast<uintptr_t>(3));
          sw[p] = __builtin_amdgcn_ubfe(w, 8 * static_cast<uint32_t>(a & 3), 8) << (8 * g);
          if (e0 >= H) v.q[p] = u32x4{0, 0, 0, 0};
        }
        v.s = u32x4{sw[0], sw[1], 0, 0};
      } else {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int e0 = k + 32 * cc + 8 * g;
          const int ec = e0 < H ? e0 : H - 8;
          v.f[cc] = *reinterpret_cast<const u32x4*>(R.rp[m][r] + (size_t)ec * 2);
          if (e0 >= H) v.f[cc] = u32x4{0, 0, 0, 0};
        }
      }
      ar.r[m][r] = v;
    }
}

// a = w * silu(g) * u for the lane's 4 rows of each tile and its token column.
template <int NT>
__device__ __forceinline__ void gu_epilogue(const f32x4 (&acc)[2][2][NT], int rows, int rbase,
                                            int l16, int g, const lds_i32* tok_slot,
                                            const lds_f32* tok_w, int np, float* act, int IA) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tc = 16 * t + l16;
    if (tc >= np) continue;
    const float wt = tok_w[tc];
    float* arow = act + (size_t)tok_slot[tc] * IA;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = rbase + 16 * r + 4 * g;
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = wt * silu(acc[0][r][t][i]) * acc[1][r][t][i];
      if (row + 3 < rows) {
        *reinterpret_cast<f32x4*>(arow + row) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (row + i < rows) arow[row + i] = v[i];
      }
    }
  }
}

template <int NT>
__device__ __forceinline__ void gu_acc_zero(f32x4 (&acc)[2][2][NT]) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][r][t] = f32x4{0, 0, 0, 0};
}

// One pass of one wave's 32 channels (rows rbase ..) for tokens tok_*[0..np), np <= 16 NT,
// with x staged in chunks.  Weight fragments run DA steps ahead in registers; the x chunk
// one chunk ahead.  The full steps run pipelined; a K tail (H not a multiple of the step)
// runs after them with masked fragments.
template <DT dt, int NT, int DA>
__device__ __forceinline__ void gu_pass(const uint8_t* G, const uint8_t* V, const uint8_t* Gs,
                                        const uint8_t* Vs, int H, int rows, int rbase,
                                        const uint16_t* xh, const uint16_t* xl,
                                        const lds_i32* tok_b, const lds_i32* tok_slot,
                                        const lds_f32* tok_w, int np, lds_u16* xs, float* act,
                                        int IA) {
  using F = Gu<dt>;
  constexpr int KX = gu_kx<NT>();
  constexpr int SPC = KX / F::STEP;
  static_assert(SPC >= 1 && KX % F::STEP == 0, "an x chunk holds whole steps");
  constexpr int GRP = gu_lcm(SPC, DA);  // keeps both the ring slot and the chunk phase
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const GuRows<dt> R = gu_rows<dt>(G, V, Gs, Vs, H, rows, rbase, l16, g);
  int xo[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) xo[t] = (16 * t + l16) * gu_ldx<NT>();
  lds_u16* xs_h[2] = {xs, xs + 2 * kGuBuf};
  lds_u16* xs_l[2] = {xs + kGuBuf, xs + 3 * kGuBuf};
  f32x4 acc[2][2][NT];
  gu_acc_zero<NT>(acc);
  // full chunks, in groups of GRP steps
  const int nfull = (H / KX) * SPC;                  // steps in full chunks
  // steps run by the pipelined loop (none without the wide scale loads)
  const int ngrp = gu_wide_ok<dt>(H) ? nfull / GRP * GRP : 0;
  GuRing<dt> ring[DA];
  GuX xr;
  gu_x_load<NT>(xr, xh, xl, H, tok_b, np, 0);
  if (ngrp > 0) {
#pragma unroll
    for (int d = 0; d < DA; ++d)
      gu_a_load<dt>(ring[d], R.rp, R.sp, d * F::STEP, g, d % 2 == 0);
  }
  gu_x_store<NT>(xr, xs_h[0], xs_l[0]);
  __syncthreads();
  for (int base = 0; base < ngrp; base += GRP) {
#pragma unroll
    for (int u = 0; u < GRP; ++u) {
      const int st = base + u;
      const int c = st / SPC;
      const bool first = u % SPC == 0, last = u % SPC == SPC - 1;
      // x of the next chunk, also past the end of K (pieces clamp to H - 8; the buffer is
      // not read again): a load under a run-time branch would leave the load counters
      // unknown after it, and every later wait would drain all loads in flight
      if (first) gu_x_load<NT>(xr, xh, xl, H, tok_b, np, (c + 1) * KX);
      // Issue order is kept as written: the load counter completes in order, so a refill
      // the scheduler sank below the x loads would be waited for at the x store.
      __builtin_amdgcn_sched_barrier(0);
      gu_step<dt, NT>(ring[u % DA], xs_h[c & 1], xs_l[c & 1], xo, (u % SPC) * F::STEP, g,
                      acc);
      if (u % 2 == 0) gu_pass_on<dt>(ring[u % DA], ring[(u + 1) % DA]);
      const int sn = st + DA < ngrp ? st + DA : st;  // spare refills reread this step
      gu_a_load<dt>(ring[u % DA], R.rp, R.sp, sn * F::STEP, g, u % 2 == 0);
      __builtin_amdgcn_sched_barrier(0);
      if (last) {
        gu_x_store<NT>(xr, xs_h[(c + 1) & 1], xs_l[(c + 1) & 1]);
        __syncthreads();
      }
    }
  }
  // the rest of K (ngrp steps are done; x of chunk ngrp/SPC is staged): masked steps,
  // staging further chunks as they are reached
  for (int st = ngrp; st * F::STEP < H; ++st) {
    const int c = st / SPC;
    const int k = st * F::STEP;
    if (st > ngrp && st % SPC == 0) {
      gu_x_load<NT>(xr, xh, xl, H, tok_b, np, c * KX);
      gu_x_store<NT>(xr, xs_h[c & 1], xs_l[c & 1]);
      __syncthreads();
    }
    GuRing<dt> ar;
    gu_a_load_masked<dt>(ar, R, H, k, g);
    gu_step<dt, NT>(ar, xs_h[c & 1], xs_l[c & 1], xo, k - c * KX, g, acc);
  }
  gu_epilogue<NT>(acc, rows, rbase, l16, g, tok_slot, tok_w, np, act, IA);
}

// LDS bytes of x held whole for np tokens (hi and lo rows of H + kGuPad bf16).
__host__ __device__ constexpr int gu_res_bytes(int np, int H) { return np * (H + kGuPad) * 4; }
// ------------------------------------------------------------------------------------
// Gate/up with the weights streamed into LDS (buckets of <= kGuSmall tokens)
//
// Loads in the MFMA operand layout touch 16 rows x 64 B per instruction, and the line
// lookups, not the bytes, then bound the stream (about 5 TB/s on this part).  Here each wave
// copies its 64 rows (32 of G, 32 of V) of a step straight into LDS with line-complete
// 16-byte direct loads (8 rows x 128 B per instruction, about 6.3 TB/s), then reads the
// MFMA fragments back from LDS.  A step is 128 bytes of every row for both formats (64 bf16
// or 256 MXFP4 elements), so the same copy and read-back serve both.  The ring lives in LDS
// (kGlDA steps per wave), not in registers; its waits are explicit load-counter waits whose
// counts follow the issue order, which is pinned.
// ------------------------------------------------------------------------------------
constexpr int kGlDA = 2;                                  // steps in flight per wave
constexpr int kGlSlot = 64 * 128;                         // one step of a wave's 64 rows
constexpr int kGlScale = 64 * 16;                         // scale blocks of a step pair
constexpr int kGlWave = kGlDA * kGlSlot;                  // a wave's weight ring
constexpr int kGlRing = kGuWaves * kGlWave;               // static LDS of the rings
constexpr int kGlScales = kGuWaves * 2 * kGlScale;        // static LDS of the scale slots

// Direct copies of step st into a ring slot: instruction i holds rows 8i .. 8i+7 of the
// wave's 64 (matrix i / 4, tile (i / 2) % 2, half i % 2); lane l takes row l / 8 and the
// 16-byte chunk (l % 8) ^ (l / 8), so that lane l of the instruction lands at 16 l and the
// read-back of 16 rows at a 128-byte pitch spreads over all banks.
__device__ __forceinline__ void gl_issue(lds_u8* slot, const uint8_t* G, const uint8_t* V,
                                         const uint32_t (&off)[2][2], int st) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    gl_copy16(slot + 1024 * i, (i >> 2 ? V : G) + off[(i >> 1) & 1][i & 1] + (size_t)st * 128);
}

// Scale blocks of an even step (MXFP4), copied like the codes: lane l takes row l of the
// wave's 64 (matrix l / 32, tile (l / 16) % 2, row l % 16 of the tile) and its 16 scale
// bytes of the step pair, landing at 16 l of the scale slot.
__device__ __forceinline__ void gl_issue_scales(lds_u8* sslot, const uint8_t* src) {
  gl_copy16(sslot, src);
}

// Fragments of a ring slot: tile (m, r) is rows 16 (2m + r) .. +15 of the slot; piece x of
// lane (l16, g) is chunk 4x + g of row l16 (bf16: sub-step x; MXFP4: piece x), at ro[x].
template <DT dt>
__device__ __forceinline__ void gl_frags(GuRing<dt>& ar, const lds_u8* slot,
                                         const uint32_t (&ro)[2]) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const lds_u8* tp = slot + 2048 * (2 * m + r);
      if constexpr (dt == DT::MXFP4) {
        ar.r[m][r].q[0] = lds_ld128(tp + ro[0]);
        ar.r[m][r].q[1] = lds_ld128(tp + ro[1]);
      } else {
        ar.r[m][r].f[0] = lds_ld128(tp + ro[0]);
        ar.r[m][r].f[1] = lds_ld128(tp + ro[1]);
      }
    }
}

// x chunk c of 16 token rows (hi and lo) copied into LDS buffer (xs_h, xs_l): each token
// row of the chunk is 512 bf16 = one copy instruction; wave w copies tokens 4w .. 4w+3.
// Pieces past H copy the row's last piece (never used); token rows past np copy token 0.
__device__ __forceinline__ void gl_x_chunk(lds_u16* xs_h, lds_u16* xs_l, const uint16_t* const (&xrh)[4],
                                           const uint16_t* const (&xrl)[4], int H, int kc,
                                           int wv, int lane) {
  int k = kc + 8 * lane;
  k = k < H ? k : H - 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int tok = 4 * wv + t;
    gl_copy16((const lds_u8*)(xs_h + tok * gu_ldx<1>()), (const uint8_t*)(xrh[t] + k));
    gl_copy16((const lds_u8*)(xs_l + tok * gu_ldx<1>()), (const uint8_t*)(xrl[t] + k));
  }
}

// One pass of one wave's 32 channels for np <= 16 tokens, weights through LDS.  RES: the
// whole x of the tokens is in LDS (staged once); else x goes in 512-element chunks copied
// into LDS one chunk ahead.  Per step, the wave issues (in this order) the x chunk copies
// (8, first step of a chunk), then after using the step, the step pair's scale copy
// (MXFP4, even steps) and the 8 weight copies of the step DA ahead.
template <DT dt, bool RES>
__device__ __forceinline__ void gu_pass_lds(const uint8_t* G, const uint8_t* V,
                                            const uint8_t* Gs, const uint8_t* Vs, int H,
                                            int rows, int rbase, const uint16_t* xh,
                                            const uint16_t* xl, const lds_i32* tok_b,
                                            const lds_i32* tok_slot, const lds_f32* tok_w,
                                            int np, lds_u16* __restrict__ xs,
                                            lds_u8* __restrict__ ring,
                                            lds_u8* __restrict__ scl, float* act, int IA) {
  using F = Gu<dt>;
  constexpr bool MX = dt == DT::MXFP4;
  constexpr int DA = kGlDA;
  constexpr int KX = gu_kx<1>();
  static_assert(KX == 512, "a chunk row is one 1 KB copy");
  constexpr int SPC = RES ? 1 : KX / F::STEP;            // steps per x chunk
  // steps per unrolled group: whole x chunks and ring turns, and for MXFP4 two step pairs,
  // so that every slot index is a compile-time constant
  constexpr int GRP = gu_lcm(gu_lcm(SPC, DA), MX ? 4 : 1);
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lds_u8* wring = ring + wv * kGlWave;
  const GuRows<dt> R = gu_rows<dt>(G, V, Gs, Vs, H, rows, rbase, l16, g);
  const size_t rb = F::row_bytes(H);
  uint32_t off[2][2];
  {
    const int lr = lane >> 3, lc = (lane & 7) ^ lr;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int row = rbase + 16 * r + 8 * h + lr;
        row = row < rows ? row : rows - 1;  // rows past the end give values that are dropped
        off[r][h] = (uint32_t)(row * rb) + 16 * lc;
      }
  }
  uint32_t ro[2];
  {
    const int r8 = l16 & 7, hi = l16 >> 3;
#pragma unroll
    for (int x = 0; x < 2; ++x) ro[x] = 1024 * hi + 16 * (8 * r8 + ((4 * x + g) ^ r8));
  }
  // scale copy of this lane (MXFP4): row lane % 16 of tile (lane / 16) % 2 of matrix
  // lane / 32; rows clamp like the codes'
  const uint8_t* ssrc = nullptr;
  if constexpr (MX) {
    int row = rbase + 16 * ((lane >> 4) & 1) + (lane & 15);
    row = row < rows ? row : rows - 1;
    ssrc = (lane >> 5 ? Vs : Gs) + (size_t)row * (H / 32);
  }
  lds_u8* sring = scl + wv * 2 * kGlScale;  // two scale slots, by step pair parity
  // x buffers
  int xo[1];
  lds_u16* xs_h[2];
  lds_u16* xs_l[2];
  const uint16_t* xrh[4];  // token rows this wave copies (chunked x)
  const uint16_t* xrl[4];
  if constexpr (RES) {
    const int ldr = H + kGuPad;
    xs_h[0] = xs_h[1] = xs;
    xs_l[0] = xs_l[1] = xs + np * ldr;
    xo[0] = (l16 < np ? l16 : 0) * ldr;
  } else {
    xs_h[0] = xs; xs_h[1] = xs + 2 * kGuBuf;
    xs_l[0] = xs + kGuBuf; xs_l[1] = xs + 3 * kGuBuf;
    xo[0] = l16 * gu_ldx<1>();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = 4 * wv + t;
      const size_t b = (size_t)tok_b[tok < np ? tok : 0] * H;
      xrh[t] = xh + b;
      xrl[t] = xl + b;
    }
  }
  f32x4 acc[2][2][1];
  gu_acc_zero<1>(acc);
  const int nfull = RES ? H / F::STEP : (H / KX) * SPC;
  const int ngrp = gu_wide_ok<dt>(H) ? nfull / GRP * GRP : 0;
  // x: staged whole (RES), or the first chunk copied
  if constexpr (RES) {
    const int pr = H / 8;  // 16-byte pieces per x row
    for (int p = threadIdx.x; p < np * pr; p += kGuWaves * 64) {
      const int tok = p / pr, q = p - tok * pr;
      const size_t o = (size_t)tok_b[tok] * H + 8 * q;
      lds_st128(xs_h[0] + tok * (H + kGuPad) + 8 * q, *reinterpret_cast<const u32x4*>(xh + o));
      lds_st128(xs_l[0] + tok * (H + kGuPad) + 8 * q, *reinterpret_cast<const u32x4*>(xl + o));
    }
  } else {
    gl_x_chunk(xs_h[0], xs_l[0], xrh, xrl, H, 0, wv, lane);
  }
  if (ngrp > 0) {
    if constexpr (MX) gl_issue_scales(sring, ssrc);  // step pair 0
#pragma unroll
    for (int d = 0; d < DA; ++d) gl_issue(wring + d * kGlSlot, G, V, off, d);
  }
  gl_wait_vm<0>();  // x chunk 0 (and the first copies) landed
  __syncthreads();
  for (int base = 0; base < ngrp; base += GRP) {
#pragma unroll
    for (int u = 0; u < GRP; ++u) {
      const int st = base + u;
      const int c = RES ? 0 : st / SPC;
      const bool first = !RES && u % SPC == 0;
      const bool last = !RES && u % SPC == SPC - 1;
      // the next chunk's x (past the end of K: the last pieces again, into the buffer that
      // is not read any more)
      if (first) gl_x_chunk(xs_h[(c + 1) & 1], xs_l[(c + 1) & 1], xrh, xrl, H, (c + 1) * KX, wv, lane);
      __builtin_amdgcn_sched_barrier(0);
      // this step's copies have landed once at most this many later copies are in flight:
      // the next step's weights (and its scales if it is even), and the x chunk copies of
      // the previous step and of this one
      {
        const bool first_prev = !RES && (u + GRP - 1) % GRP % SPC == 0;
        gl_wait_n(8 + (MX && u % 2 == 1 ? 1 : 0) + (first_prev ? 8 : 0) + (first ? 8 : 0));
      }
      GuRing<dt> ar;
      gl_frags<dt>(ar, wring + (u % DA) * kGlSlot, ro);
      if constexpr (MX) {
        // the step pair's scale block of each of the lane's rows; the odd step takes dwords 2, 3
        const lds_u8* sp = sring + ((u >> 1) & 1) * kGlScale + 16 * l16;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const u32x4 b = lds_ld128(sp + 16 * (32 * m + 16 * r));
            ar.r[m][r].s = u % 2 == 0 ? b : u32x4{b.z, b.w, 0, 0};
          }
      }
      gu_step<dt, 1>(ar, xs_h[c & 1], xs_l[c & 1], xo, RES ? st * F::STEP : (u % SPC) * F::STEP,
                     g, acc);
      __builtin_amdgcn_sched_barrier(0);
      const int sn = st + DA < ngrp ? st + DA : st;  // spare refills copy this step again
      gl_wait_lds();  // the slot's reads are done
      if constexpr (MX)  // sn has the parity of st; its pair's slot is not the one in use
        if (u % 2 == 0)
          gl_issue_scales(sring + (((u + DA) >> 1) & 1) * kGlScale, ssrc + sn * F::STEP / 32);
      gl_issue(wring + (u % DA) * kGlSlot, G, V, off, sn);
      __builtin_amdgcn_sched_barrier(0);
      if (last) {
        // the next chunk's copies (issued at this chunk's first step) have landed once at
        // most the copies issued after them are in flight: per step of the chunk, the
        // weights (8) and the scales of its even steps
        int after = 0;
#pragma unroll
        for (int v = u - SPC + 1; v <= u; ++v) after += 8 + (MX && v % 2 == 0 ? 1 : 0);
        gl_wait_n(after);
        __syncthreads();
      }
    }
  }
  gl_wait_vm<0>();  // every copy has landed (none may outlive the workgroup)
  __syncthreads();
  // the rest of K: masked steps with fragments in registers
  for (int st = ngrp; st * F::STEP < H; ++st) {
    const int c = RES ? 0 : st / SPC;
    const int k = st * F::STEP;
    if (!RES && st > ngrp && st % SPC == 0) {
      __syncthreads();
      GuX xr;
      gu_x_load<1>(xr, xh, xl, H, tok_b, np, c * KX);
      gu_x_store<1>(xr, xs_h[c & 1], xs_l[c & 1]);
      __syncthreads();
    }
    GuRing<dt> ar;
    gu_a_load_masked<dt>(ar, R, H, k, g);
    if constexpr (RES)
      gu_step<dt, 1, true>(ar, xs_h[0], xs_l[0], xo, k, g, acc, H - 8);
    else
      gu_step<dt, 1>(ar, xs_h[c & 1], xs_l[c & 1], xo, k - c * KX, g, acc);
  }
  gu_epilogue<1>(acc, rows, rbase, l16, g, tok_slot, tok_w, np, act, IA);
}

// Token bucket of work item t: the shared experts first (t < NS, every token of the batch;
// their workgroups read the most and are dispatched first), then the routed expert slots
// (the union's buckets; slots past n_touched are empty).
struct Bucket {
  int count;
  bool shared;
  int e;  // routed expert id, or shared index
};

__device__ __forceinline__ Bucket bucket_of(const BsArgs& a, int t) {
  Bucket b;
  if (t < a.NS) {
    b.shared = true;
    b.e = t;
    b.count = a.B;
    return b;
  }
  t -= a.NS;
  b.shared = false;
  if (t >= *a.n_touched) {
    b.count = 0;
    b.e = 0;
    return b;
  }
  b.e = a.touched[t];
  b.count = a.offsets[b.e + 1] - a.offsets[b.e];
  return b;
}

// Fill the pass's token list: token index, act/partial row, weight.
__device__ __forceinline__ void fill_tokens(const BsArgs& a, const Bucket& bk, int p0, int np,
                                            lds_i32* tok_b, lds_i32* tok_slot, lds_f32* tok_w) {
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

// Buckets of at most kGuSmall tokens (every bucket at small batches) run in a launch of
// their own with one token tile and the weights streamed through LDS; larger buckets run
// in the other launch with 2 or 4 token tiles and a register ring.
constexpr int kGuSmall = 16;
template <DT dt> constexpr int gu_pass_tokens() {
  return gu_kx<4>() >= Gu<dt>::STEP ? 64 : 32;
}
constexpr int kGuDALarge = 2;
static_assert(kGuDALarge % 2 == 0,
              "MXFP4 rings pair even and odd steps (their scales are read together)");

template <DT et, DT st, bool SMALL>
__device__ __forceinline__ void gateup_body(const BsArgs& a, lds_u16* xs, lds_i32* tok_b,
                                            lds_i32* tok_slot, lds_f32* tok_w,
                                            lds_u8* ring = nullptr, lds_u8* scl = nullptr) {
  const Bucket bk = bucket_of(a, blockIdx.y);
  const int rows = bk.shared ? a.IS : a.I;
  if (bk.count == 0 || (bk.count <= kGuSmall) != SMALL || blockIdx.x * kGuRows >= rows)
    return;  // whole workgroup leaves
  const int rbase = blockIdx.x * kGuRows + (threadIdx.x >> 6) * kGuRowsW;
  const uint8_t *G, *V, *Gs = nullptr, *Vs = nullptr;
  if (bk.shared) {
    const size_t off = (size_t)bk.e * a.IS * Gu<st>::row_bytes(a.H);
    G = reinterpret_cast<const uint8_t*>(a.sh_gate) + off;
    V = reinterpret_cast<const uint8_t*>(a.sh_up) + off;
  } else {
    const size_t off = (size_t)bk.e * a.I;
    G = reinterpret_cast<const uint8_t*>(a.gate) + off * Gu<et>::row_bytes(a.H);
    V = reinterpret_cast<const uint8_t*>(a.up) + off * Gu<et>::row_bytes(a.H);
    if (a.gate_s) Gs = a.gate_s + off * (a.H / 32);
    if (a.up_s) Vs = a.up_s + off * (a.H / 32);
  }
  if constexpr (SMALL) {
    fill_tokens(a, bk, 0, bk.count, tok_b, tok_slot, tok_w);
    __syncthreads();
    if (bk.shared) {
      if (gu_res_bytes(bk.count, a.H) <= kGuLds)
        gu_pass_lds<st, true>(G, V, nullptr, nullptr, a.H, rows, rbase, a.xh, a.xl, tok_b,
                              tok_slot, tok_w, bk.count, xs, ring, scl, a.act, a.IA);
      else
        gu_pass_lds<st, false>(G, V, nullptr, nullptr, a.H, rows, rbase, a.xh, a.xl, tok_b,
                               tok_slot, tok_w, bk.count, xs, ring, scl, a.act, a.IA);
    } else {
      if (gu_res_bytes(bk.count, a.H) <= kGuLds)
        gu_pass_lds<et, true>(G, V, Gs, Vs, a.H, rows, rbase, a.xh, a.xl, tok_b, tok_slot,
                              tok_w, bk.count, xs, ring, scl, a.act, a.IA);
      else
        gu_pass_lds<et, false>(G, V, Gs, Vs, a.H, rows, rbase, a.xh, a.xl, tok_b, tok_slot,
                               tok_w, bk.count, xs, ring, scl, a.act, a.IA);
    }
  } else {
    // tokens per pass: 64 (four token tiles) where a four-tile x chunk holds a weight step,
    // else 32 (the 256-element MXFP4 step)
    const int ptok = bk.shared ? gu_pass_tokens<st>() : gu_pass_tokens<et>();
    for (int p0 = 0; p0 < bk.count; p0 += ptok) {
      const int np = min(ptok, bk.count - p0);
      __syncthreads();  // the previous pass is done with the token list and x buffers
      fill_tokens(a, bk, p0, np, tok_b, tok_slot, tok_w);
      __syncthreads();
      const bool two = np <= 32;
      if (bk.shared) {
        if (two)
          gu_pass<st, 2, kGuDALarge>(G, V, nullptr, nullptr, a.H, rows, rbase, a.xh, a.xl,
                                     tok_b, tok_slot, tok_w, np, xs, a.act, a.IA);
        else if constexpr (gu_pass_tokens<st>() == 64)
          gu_pass<st, 4, kGuDALarge>(G, V, nullptr, nullptr, a.H, rows, rbase, a.xh, a.xl,
                                     tok_b, tok_slot, tok_w, np, xs, a.act, a.IA);
      } else {
        if (two)
          gu_pass<et, 2, kGuDALarge>(G, V, Gs, Vs, a.H, rows, rbase, a.xh, a.xl, tok_b,
                                     tok_slot, tok_w, np, xs, a.act, a.IA);
        else if constexpr (gu_pass_tokens<et>() == 64)
          gu_pass<et, 4, kGuDALarge>(G, V, Gs, Vs, a.H, rows, rbase, a.xh, a.xl, tok_b,
                                     tok_slot, tok_w, np, xs, a.act, a.IA);
      }
    }
  }
}

// Buckets of <= kGuSmall tokens with the weights streamed through LDS (one workgroup per
// CU: the x buffers in dynamic LDS and the weight ring in static LDS).
template <DT et, DT st>
__global__ __launch_bounds__(kGuWaves * 64) void bs_gateup_lds_kernel(BsArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kGlRing];
  __shared__ __attribute__((aligned(1024))) unsigned char scl[kGlScales];
  __shared__ int tok_b[kGuTok];
  __shared__ int tok_slot[kGuTok];
  __shared__ float tok_w[kGuTok];
  gateup_body<et, st, true>(a, (lds_u16*)smem, (lds_i32*)tok_b, (lds_i32*)tok_slot,
                                  (lds_f32*)tok_w, (lds_u8*)ring, (lds_u8*)scl);
}

template <DT et, DT st>
__global__ __launch_bounds__(kGuWaves * 64) void bs_gateup_large_kernel(BsArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int tok_b[kGuTok];
  __shared__ int tok_slot[kGuTok];
  __shared__ float tok_w[kGuTok];
  gateup_body<et, st, false>(a, (lds_u16*)smem, (lds_i32*)tok_b, (lds_i32*)tok_slot,
                             (lds_f32*)tok_w);
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
    const float sc = __uint_as_float((uint32_t)r.s << 23);
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
                                        int hc, int j, int j1, const gbl_f32* const (&ap)[NT],
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
  // dead lanes (past the row's end) read the row's last chunk, which a live lane of the same
  // wave loads too, and store nothing: column 0 would be a line that another XCD's workgroup
  // reads, fetched from memory once more
  const int hc = live ? h : H - F::EPT;
  const gbl_f32* ap[NT];
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

// The down kernel's work: column block x (dn_cols columns), bucket y, and z = row slice +
// kDownRowSlices * pass group.  A bucket's passes (at most B pairs) are spread over up to 8
// pass groups.
__host__ __device__ inline int dn_pass_groups(int B) {
  const int g = (B + 7) / 8;
  return g > 8 ? 8 : g;
}
// Blocks are numbered so that every column block of one (bucket, z) runs on the same XCD
// (block L runs on XCD L % 8): L = 8 (NX (g / 8) + x) + g % 8 with g = y + items z.  The
// column blocks of a row then share its lines in one L2 (an MXFP4 row's 224 scale bytes span
// lines that neighbouring column blocks both read), and consecutive (bucket, z) pairs still
// go round the XCDs.
struct DnPos {
  int x, y, z, nz;
};
__device__ __forceinline__ bool dn_pos(const BsArgs& a, int nx, DnPos& p) {
  const int items = a.slots_max + a.NS;
  p.nz = kDownRowSlices * dn_pass_groups(a.B);
  const int L = blockIdx.x;
  const int g = (L / (8 * nx)) * 8 + L % 8;
  p.x = (L / 8) % nx;
  if (g >= items * p.nz) return false;
  p.y = g % items;
  p.z = g / items;
  return true;
}

template <DT dt>
__device__ __forceinline__ void dn_item(const BsArgs& a, const Bucket& bk, const uint8_t* D,
                                        const uint8_t* Ds, int rows, float* red, int* pslot,
                                        const DnPos& pos) {
  constexpr int EPT = Dn<dt>::EPT;
  constexpr int NTM = Dn<dt>::NTMAX;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = pos.x * dn_cols<dt>() + EPT * lane;
  const bool live = h < a.H;  // H is a multiple of 32 and EPT divides 32
  // z = row slice + kDownRowSlices * pass group: the slice's channels, split in kDnWaves
  // contiguous ranges, and every pass group-th pass of the bucket
  const int rs = pos.z % kDownRowSlices, pg = pos.z / kDownRowSlices;
  const int ngroups = pos.nz / kDownRowSlices;
  const int per_s = (rows + kDownRowSlices - 1) / kDownRowSlices;
  const int s0 = min(rows, rs * per_s), s1 = min(rows, s0 + per_s);
  const int per = (s1 - s0 + kDnWaves - 1) / kDnWaves;
  const int j0 = min(s1, s0 + wave * per), j1 = min(s1, j0 + per);
  float* part = a.part + (size_t)rs * a.pairs * a.H;  // this slice's partial rows
  for (int p0 = pg * NTM; p0 < bk.count; p0 += ngroups * NTM) {
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
      dn_reduce_store<dt, 8>(acc, red, ps, np, part, a.H, h, live);
    } else if (NTM >= 4 && np > 2) {
      float acc[4][EPT];
      dn_pass<dt, 4>(D, Ds, a.H, h, live, j0, j1, a.act, a.IA, ps, acc);
      dn_reduce_store<dt, 4>(acc, red, ps, np, part, a.H, h, live);
    } else if (np > 1) {
      float acc[2][EPT];
      dn_pass<dt, 2>(D, Ds, a.H, h, live, j0, j1, a.act, a.IA, ps, acc);
      dn_reduce_store<dt, 2>(acc, red, ps, np, part, a.H, h, live);
    } else {
      float acc[1][EPT];
      dn_pass<dt, 1>(D, Ds, a.H, h, live, j0, j1, a.act, a.IA, ps, acc);
      dn_reduce_store<dt, 1>(acc, red, ps, np, part, a.H, h, live);
    }
  }
}

template <DT et, DT st>
__global__ __launch_bounds__(kDnWaves * 64) void bs_down_kernel(BsArgs a) {
  constexpr int EPT_MAX = Dn<et>::EPT > Dn<st>::EPT ? Dn<et>::EPT : Dn<st>::EPT;
  __shared__ __attribute__((aligned(16))) float red[(kDnWaves - 1) * EPT_MAX * 64];
  __shared__ int pslot[8];
  constexpr int cmin = dn_cols<et>() < dn_cols<st>() ? dn_cols<et>() : dn_cols<st>();
  DnPos pos;
  if (!dn_pos(a, (a.H + cmin - 1) / cmin, pos)) return;
  const Bucket bk = bucket_of(a, pos.y);
  if (bk.count == 0) return;
  if (bk.shared) {
    if (pos.x * dn_cols<st>() >= a.H) return;
    const uint8_t* D = reinterpret_cast<const uint8_t*>(a.sh_down_t) +
                       (size_t)bk.e * a.IS * Dn<st>::row_bytes(a.H);
    dn_item<st>(a, bk, D, nullptr, a.IS, red, pslot, pos);
  } else {
    if (pos.x * dn_cols<et>() >= a.H) return;
    const size_t off = (size_t)bk.e * a.I;
    const uint8_t* D =
        reinterpret_cast<const uint8_t*>(a.down_t) + off * Dn<et>::row_bytes(a.H);
    const uint8_t* Ds = a.down_s ? a.down_s + off * (a.H / 32) : nullptr;
    dn_item<et>(a, bk, D, Ds, a.I, red, pslot, pos);
  }
}

// ------------------------------------------------------------------------------------
// Combine: y[b] = sum_i part[b*k + i] (routing order, the choices that were used) +
// sum_s part[B*k + s*B + b], each partial row the sum of its row slices in slice order
// ------------------------------------------------------------------------------------
constexpr int kCombineChunk = 8;  // choices whose partial rows are loaded together
__global__ __launch_bounds__(256) void bs_combine_kernel(BsArgs a) {
  // workgroup (x, b): token b, columns 4 * [256 x, 256 (x + 1)); which of the token's choices
  // were used is decided once per workgroup (k <= 64)
  __shared__ int s_used[64];
  const int n4 = a.H / 4;
  const int b = blockIdx.y;
  if (threadIdx.x < a.k) s_used[threadIdx.x] = choice_used(a.ids + (size_t)b * a.k, threadIdx.x, a.E);
  __syncthreads();
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n4) return;
  const size_t slice = (size_t)a.pairs * n4;  // f32x4 per row slice of the partials
  const f32x4* P = reinterpret_cast<const f32x4*>(a.part);
  const f32x4 zero = {0, 0, 0, 0};
  f32x4 s = zero;
  // kCombineChunk choices at a time: every row of the chunk is loaded before any is added,
  // so the loads are in flight together (a load behind the used test would wait for the
  // previous sum).  Rows past k are clamped to row k - 1 and rows of unused choices, which
  // hold an earlier call's data, are read and dropped; every row lies in the partials buffer.
  for (int i0 = 0; i0 < a.k; i0 += kCombineChunk) {
    f32x4 v[kCombineChunk][kDownRowSlices];
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j) {
      const size_t row = (size_t)b * a.k + min(i0 + j, a.k - 1);
#pragma unroll
      for (int r = 0; r < kDownRowSlices; ++r) v[j][r] = P[r * slice + row * n4 + c];
    }
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j) {
      const bool u = i0 + j < a.k && s_used[min(i0 + j, a.k - 1)];
#pragma unroll
      for (int r = 0; r < kDownRowSlices; ++r) s += u ? v[j][r] : zero;
    }
  }
  for (int sh = 0; sh < a.NS; ++sh)
#pragma unroll
    for (int r = 0; r < kDownRowSlices; ++r)
      s += P[r * slice + (size_t)(a.B * a.k + sh * a.B + b) * n4 + c];
  reinterpret_cast<f32x4*>(a.y)[(size_t)b * n4 + c] = s;
}

template <DT et, DT st>
hipError_t launch_bs_typed(const BsArgs& a, hipStream_t s) {
  const int items = a.slots_max + a.NS;
  const int rows = a.I > a.IS ? a.I : a.IS;
  constexpr int gu_lds = kGuLds;
  static bool lds_set = false;
  if (!lds_set) {
    hipError_t e0 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(bs_gateup_lds_kernel<et, st>),
        hipFuncAttributeMaxDynamicSharedMemorySize, gu_lds);
    if (e0 == hipSuccess)
      e0 = hipFuncSetAttribute(reinterpret_cast<const void*>(bs_gateup_large_kernel<et, st>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, gu_lds);
    if (e0 != hipSuccess) return e0;
    lds_set = true;
  }
  const dim3 gu_grid((rows + kGuRows - 1) / kGuRows, items);
  hipLaunchKernelGGL((bs_gateup_lds_kernel<et, st>), gu_grid, dim3(kGuWaves * 64), gu_lds, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.B > kGuSmall) {  // no bucket holds more tokens than the batch
    hipLaunchKernelGGL((bs_gateup_large_kernel<et, st>), gu_grid, dim3(kGuWaves * 64), gu_lds,
                       s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int cmin = dn_cols<et>() < dn_cols<st>() ? dn_cols<et>() : dn_cols<st>();
  // column blocks x (bucket, slice, pass group) pairs, the latter padded to a multiple of 8
  const long long nx = (a.H + cmin - 1) / cmin;
  const long long ng = (long long)items * kDownRowSlices * dn_pass_groups(a.B);
  const long long nblk = nx * ((ng + 7) / 8) * 8;
  if (nblk > 0x7FFFFFFFll) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bs_down_kernel<et, st>), dim3((unsigned)nblk), dim3(kDnWaves * 64), 0,
                     s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bs_combine_kernel, dim3((a.H / 4 + 255) / 256, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_batched_swiglu(const BsArgs& a, DT et, DT st, hipStream_t s) {
  if (et == DT::BF16 && st == DT::BF16) return launch_bs_typed<DT::BF16, DT::BF16>(a, s);
  if (et == DT::MXFP4 && st == DT::BF16) return launch_bs_typed<DT::MXFP4, DT::BF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe

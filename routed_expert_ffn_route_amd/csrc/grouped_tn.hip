// grouped_tn.hip -- linear experts for larger batches: a register-blocked MFMA tile per
// (touched expert, block of 128 output rows) with the bucket's x staged in LDS.
//
// Same product as linear_mfma.hip (y_b = sum_i w_{b,i} M_{e_{b,i}} x_b, each touched expert
// read once for all its tokens; "501B of which 23B are switched on", section 3[B]), laid out
// for many tokens per expert: there, every wave loads its own copy of the tokens' x for its
// 16 rows, so at ~100 tokens per expert the x traffic from L2 is ~12x the weight bytes.
// Here a workgroup (8 waves x 32 rows) stages the x of up to 128 tokens for a 64-wide K
// chunk in LDS once, and every wave reuses each x fragment across its two 16-row tiles.
// (256 rows per workgroup rather than 128 halve the x bytes per weight byte: the 2048-token
// step went from 3.43 to 2.76 ms.)
//
// Pipeline per K chunk: the next chunk's weight fragments (from HBM) and x (from L2) are
// loaded into registers while the current chunk's MFMAs run; x then goes to the other LDS
// buffer.  Each workgroup writes one partial row per (token, choice) -- w times its
// expert's output rows -- and a combine kernel sums a token's k partials in routing order:
// every output element has one writer and a fixed order.
//
// MFMA 16x16x32 (lane l: A[l%16][8(l/16)..+8], B[8(l/16)..+8][l%16], D[4(l/16)..+4][l%16]);
// A = 16 weight rows, B = 16 tokens.  Two operand forms:
// * up to 32 tokens per expert (a weight stream): bf16, x entering as bf16 hi + lo (two
//   MFMAs per product, ~16 significant bits of x);
// * more tokens (where the MFMAs and the staged x bound the kernel): f16, one MFMA per
//   product.  x is f16 scaled per token by a power of two chosen from the token's largest
//   |x| (largest magnitude in [2^14, 2^15)), so its rounding is 2^-11 relative to that
//   magnitude, and the scale is undone on the fp32 result.  A bf16 weight is exactly an f16
//   when 2^-14 <= |w| < 65504 (8 significant bits fit in 11); smaller ones keep their f16
//   subnormal bits (an absolute error below 2^-24).  This halves the MFMAs and the staged
//   x bytes: the 2048-token step went from 2.61 to 2.04 ms.
#include "kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kRowsW = 32;                 // rows per wave (2 MFMA row tiles)
constexpr int kRows = kWaves * kRowsW;     // rows per workgroup
constexpr int kKA = 64;                    // K per weight-fragment step (2 MFMA K-steps)
constexpr int kTokMax = 128;               // tokens per pass (8 MFMA token tiles)
constexpr int kXElems = 8192;              // staged x elements per buffer and array
constexpr int kPad = 8;                    // bf16 padding per staged x row

// K width of one staged x chunk for NT token tiles: a fixed LDS budget, so fewer tokens
// give wider chunks (fewer barriers and x round trips per pass).
template <int NT> constexpr int kx() { return kXElems / (16 * NT); }
template <int NT> constexpr int ldx() { return kx<NT>() + kPad; }
constexpr int kBufElems = kXElems + kTokMax * kPad;  // one staged array (max over NT)

struct TnArgs {
  const uint8_t* M;          // [E][I][H] bf16
  const uint16_t* xh;        // [B][H] bf16 hi of x
  const uint16_t* xl;        // [B][H] bf16 lo of x
  const uint16_t* x16;       // [B][H] f16 bits of x * 2^-e_b
  const float* xsc;          // [B] 2^e_b
  const float* w;            // [B][k]
  const int32_t* n_touched;
  const int32_t* touched;
  const int32_t* offsets;
  const int32_t* slots;
  float* part;               // [B*k][I]
  int H, I, k, slots_max;
};

// The operand form for NT token tiles (see the header).
template <int NT> constexpr bool use_f16() { return NT >= 4; }

// x of tokens tok_b[0..16NT) (padded with the first token), K [kc, kc + kx): 16NT tokens x
// kx/8 pieces of 16 bytes = kXElems / 8 pieces, per staged array (hi and lo, or the f16
// x); thread j holds pieces j, j + 512, ...
constexpr int kPP = kXElems / 8 / (kWaves * 64);
struct XRegs {
  u32x4 h[kPP], l[kPP];
};

template <int NT>
__device__ __forceinline__ void x_load(XRegs& xr, const TnArgs& a, const lds_i32* tok_b, int np,
                                       int kc) {
  constexpr int PR = kx<NT>() / 8;  // pieces per token row
#pragma unroll
  for (int i = 0; i < kPP; ++i) {
    const int p = threadIdx.x + i * kWaves * 64;
    const int tok = p / PR, q = p % PR;
    const int b = tok_b[tok < np ? tok : 0];
    const size_t off = (size_t)b * a.H + kc + 8 * q;
    if constexpr (use_f16<NT>()) {
      xr.h[i] = *reinterpret_cast<const u32x4*>(a.x16 + off);
    } else {
      xr.h[i] = *reinterpret_cast<const u32x4*>(a.xh + off);
      xr.l[i] = *reinterpret_cast<const u32x4*>(a.xl + off);
    }
  }
}

template <int NT>
__device__ __forceinline__ void x_store(const XRegs& xr, lds_u16* xs_h, lds_u16* xs_l) {
  constexpr int PR = kx<NT>() / 8;
#pragma unroll
  for (int i = 0; i < kPP; ++i) {
    const int p = threadIdx.x + i * kWaves * 64;
    const int tok = p / PR, q = p % PR;
    lds_st128(xs_h + tok * ldx<NT>() + 8 * q, xr.h[i]);
    if constexpr (!use_f16<NT>()) lds_st128(xs_l + tok * ldx<NT>() + 8 * q, xr.l[i]);
  }
}

// Weight fragments of one 64-wide K step: 2 row tiles x 2 MFMA K-steps, 16 bytes each.
struct ARegs {
  u32x4 f[2][2];
};

__device__ __forceinline__ void a_load(ARegs& ar, const uint8_t* const (&rp)[2], int kc, int g) {
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      ar.f[r][s] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(rp[r] + (size_t)(kc + 32 * s + 8 * g) * 2));
}

// bf16 weight pairs (one dword) -> f16 pairs: exact for normal f16 magnitudes.
// (The conversion's rounding mode is immaterial where it is exact; v_cvt_pkrtz packs the
// pair in one instruction.)
__device__ __forceinline__ f16x8 w_f16(const u32x4& v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v[i] << 16),
                                                         __uint_as_float(v[i] & 0xFFFF0000u)));
  return __builtin_bit_cast(f16x8, r);
}

// MFMAs of one 64-wide K step against the staged x at column offset k0.  bf16 form: all
// hi products, then all lo products, so that an accumulator's next MFMA is 2 NT issues
// away; f16 form: NT >= 4, so they are 2 NT apart anyway.
template <int NT>
__device__ __forceinline__ void step_mfma(const ARegs& ar, const lds_u16* xs_h,
                                          const lds_u16* xs_l, int k0, int l16, int g,
                                          f32x4 (&acc)[2][NT]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    u32x4 bh[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bh[t] = lds_ld128(xs_h + (16 * t + l16) * ldx<NT>() + k0 + 32 * s + 8 * g);
    if constexpr (use_f16<NT>()) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const f16x8 ar16 = w_f16(ar.f[r][s]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              ar16, __builtin_bit_cast(f16x8, bh[t]), acc[r][t], 0, 0, 0);
      }
    } else {
      u32x4 bl[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        bl[t] = lds_ld128(xs_l + (16 * t + l16) * ldx<NT>() + k0 + 32 * s + 8 * g);
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, ar.f[0][s]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, ar.f[1][s]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, bh[t]);
        acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[0][t], 0, 0, 0);
        acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[1][t], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, bl[t]);
        acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[0][t], 0, 0, 0);
        acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[1][t], 0, 0, 0);
      }
    }
  }
}

// One pass: tokens tok_*[0..np), np <= 16 NT, over all of K; writes the partial rows.
// Weight fragments run DA 64-wide steps ahead in registers (a ring); the x chunk runs one
// chunk ahead (registers, then the other LDS buffer).  nst is a multiple of the unrolled
// group (H is a multiple of 1024).
template <int NT, int DA>
__device__ __forceinline__ void tn_pass(const TnArgs& a, const uint8_t* Me, int rbase,
                                        const lds_i32* tok_b, const lds_i32* tok_slot,
                                        const lds_f32* tok_w, int np, lds_u16* xs) {
  constexpr int KX = kx<NT>();
  constexpr int SPC = KX / kKA;  // weight steps per x chunk
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const uint8_t* rp[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    int row = rbase + 16 * r + l16;
    row = row < a.I ? row : a.I - 1;  // rows past the end compute values that are dropped
    rp[r] = Me + (size_t)row * a.H * 2;
  }
  lds_u16* xs_h[2] = {xs, xs + 2 * kBufElems};
  lds_u16* xs_l[2] = {xs + kBufElems, xs + 3 * kBufElems};
  f32x4 acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = f32x4{0, 0, 0, 0};
  const int nst = a.H / kKA;  // weight steps (H is a multiple of 1024, KX divides 512)
  constexpr int G = SPC > DA ? SPC : DA;  // steps per unrolled group (both powers of two)
  ARegs ring[DA];
  XRegs xr;
  x_load<NT>(xr, a, tok_b, np, 0);
#pragma unroll
  for (int d = 0; d < DA; ++d) a_load(ring[d], rp, d * kKA, g);
  x_store<NT>(xr, xs_h[0], xs_l[0]);
  __syncthreads();
  for (int base = 0; base < nst; base += G) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int st = base + u;
      const int c = st / SPC;          // x chunk of this step
      const bool first = u % SPC == 0, last = u % SPC == SPC - 1;
      const bool more = (c + 1) * SPC < nst;
      if (first && more) x_load<NT>(xr, a, tok_b, np, (c + 1) * KX);
      step_mfma<NT>(ring[u % DA], xs_h[c & 1], xs_l[c & 1], (u % SPC) * kKA, l16, g, acc);
      // refill this ring slot DA steps ahead (refills past the end reread the last step)
      const int sn = st + DA < nst ? st + DA : nst - 1;
      a_load(ring[u % DA], rp, sn * kKA, g);
      if (last) {
        if (more) x_store<NT>(xr, xs_h[(c + 1) & 1], xs_l[(c + 1) & 1]);
        __syncthreads();
      }
    }
  }
  // partial rows: w (times the token's x scale) times the expert's output, per token
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tc = 16 * t + l16;
    if (tc >= np) continue;
    const float wt = tok_w[tc];
    float* prow = a.part + (size_t)tok_slot[tc] * a.I;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = rbase + 16 * r + 4 * g;
      const f32x4 v = acc[r][t] * wt;
      if (row + 3 < a.I) {
        *reinterpret_cast<f32x4*>(prow + row) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (row + i < a.I) prow[row + i] = v[i];
      }
    }
  }
}

// One kernel per range of token counts, so that the register allocation of the large
// token tiles does not limit the weight prefetch depth of the small ones: SMALL takes the
// experts with at most 32 tokens (deep prefetch), the other one the rest.
template <bool SMALL>
__global__ __launch_bounds__(kWaves * 64) void tn_kernel(TnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_u16* xs = (lds_u16*)smem;  // [2 buffers][hi, lo][kBufElems] (f16 form: hi only)
  __shared__ int tok_b_[kTokMax];
  __shared__ int tok_slot_[kTokMax];
  __shared__ float tok_w_[kTokMax];
  lds_i32* tok_b = (lds_i32*)tok_b_;
  lds_i32* tok_slot = (lds_i32*)tok_slot_;
  lds_f32* tok_w = (lds_f32*)tok_w_;
  // XCD-aware order: consecutive workgroups are dealt round-robin to the 8 XCDs, so
  // workgroup L runs on XCD L % 8.  Numbered this way, XCD x takes touched experts x, x + 8,
  // ... one at a time with all of an expert's row blocks together: the blocks share the
  // expert's x chunks, which then come from that XCD's L2 (the grid's y is a multiple of 8).
  const int L = blockIdx.y * gridDim.x + blockIdx.x;
  const int sq = L / 8;
  const int bx = sq % gridDim.x;
  const int t = (sq / gridDim.x) * 8 + L % 8;
  // (a whole workgroup leaves)
  if (t >= a.slots_max || t >= *a.n_touched || bx * kRows >= a.I) return;
  const int e = a.touched[t];
  const int s0 = a.offsets[e], ne = a.offsets[e + 1] - s0;
  if ((ne <= 32) != SMALL) return;  // the other kernel's expert
  const uint8_t* Me = a.M + (size_t)e * a.I * a.H * 2;
  const int rbase = bx * kRows + (threadIdx.x >> 6) * kRowsW;
  for (int p0 = 0; p0 < ne; p0 += kTokMax) {
    const int np = min(kTokMax, ne - p0);
    __syncthreads();  // the previous pass is done with the token list and x buffers
    for (int i = threadIdx.x; i < np; i += blockDim.x) {
      const int slot = a.slots[s0 + p0 + i];
      tok_b[i] = slot / a.k;
      tok_slot[i] = slot;
      tok_w[i] = SMALL ? a.w[slot] : a.w[slot] * a.xsc[slot / a.k];
    }
    __syncthreads();
    const int nt = (np + 15) / 16;
    if constexpr (SMALL) {
      if (nt <= 1) tn_pass<1, 4>(a, Me, rbase, tok_b, tok_slot, tok_w, np, xs);
      else tn_pass<2, 4>(a, Me, rbase, tok_b, tok_slot, tok_w, np, xs);
    } else {
      if (nt <= 4) tn_pass<4, 4>(a, Me, rbase, tok_b, tok_slot, tok_w, np, xs);
      else tn_pass<8, 2>(a, Me, rbase, tok_b, tok_slot, tok_w, np, xs);
    }
  }
}

// y[b][r] = sum_i part[b*k + i][r], i in routing order, over the choices that were used
// (choice_used: a skipped id's partial row was not written by this call).
constexpr int kTnCombineChunk = 8;  // choices whose partial rows are loaded together
__global__ __launch_bounds__(256) void tn_combine_kernel(const float* part, const int32_t* ids,
                                                         float* y, int B, int k, int I,
                                                         int E) {
  const int n4 = I / 4;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < (size_t)B * n4;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int b = (int)(idx / n4), c = (int)(idx % n4);
    const f32x4* P = reinterpret_cast<const f32x4*>(part);
    const f32x4 zero = {0, 0, 0, 0};
    f32x4 s = zero;
    // kTnCombineChunk rows loaded before any is added (rows past k clamped to row k - 1;
    // rows of unused choices, which hold an earlier call's data, read and dropped)
    for (int i0 = 0; i0 < k; i0 += kTnCombineChunk) {
      f32x4 v[kTnCombineChunk];
#pragma unroll
      for (int j = 0; j < kTnCombineChunk; ++j)
        v[j] = P[((size_t)b * k + min(i0 + j, k - 1)) * n4 + c];
#pragma unroll
      for (int j = 0; j < kTnCombineChunk; ++j) {
        const bool u = i0 + j < k && choice_used(ids + (size_t)b * k, min(i0 + j, k - 1), E);
        s += u ? v[j] : zero;
      }
    }
    reinterpret_cast<f32x4*>(y)[(size_t)b * n4 + c] = s;
  }
}

// Both operand forms of x, one workgroup per token: bf16 hi = RNE(x), lo = RNE(x - hi);
// and f16 of x * 2^-e_b, e_b chosen from the token's largest |x| (largest magnitude in
// [2^14, 2^15); e_b = 0 for an all-zero token, clamped to +-100), with 2^e_b.
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__global__ __launch_bounds__(256) void x_prep_kernel(const float* x, int H, uint16_t* xh,
                                                     uint16_t* xl, uint16_t* x16, float* xsc) {
  __shared__ float red[4];
  const float* xb = x + (size_t)blockIdx.x * H;
  float mx = 0.0f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) mx = fmaxf(mx, fabsf(xb[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = mx > 0.0f ? (int)((__float_as_uint(mx) >> 23) & 0xFF) - 127 - 14 : 0;
  e = e < -100 ? -100 : e > 100 ? 100 : e;
  const float inv = ldexpf(1.0f, -e);
  const size_t o = (size_t)blockIdx.x * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const float f = xb[i];
    const uint16_t h = bf16_bits_rne(f);
    xh[o + i] = h;
    xl[o + i] = bf16_bits_rne(f - __uint_as_float((uint32_t)h << 16));
    x16[o + i] = __builtin_bit_cast(uint16_t, (_Float16)(f * inv));
  }
  if (threadIdx.x == 0) xsc[blockIdx.x] = ldexpf(1.0f, e);
}

}  // namespace

int tn_lds_bytes() { return 2 * 2 * kBufElems * 2; }

hipError_t launch_linear_tiled(const void* M, const float* x, const float* w,
                               const int32_t* ids, const int32_t* n_touched, const int32_t* touched,
                               const int32_t* offsets, const int32_t* slots, uint16_t* xh,
                               uint16_t* xl, uint16_t* x16, float* xsc, float* part, float* y,
                               int H, int I, int E, int k, int B, hipStream_t s) {
  hipLaunchKernelGGL(x_prep_kernel, dim3(B), dim3(256), 0, s, x, H, xh, xl, x16, xsc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static bool lds_set = false;
  if (!lds_set) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(tn_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, tn_lds_bytes());
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(tn_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, tn_lds_bytes());
    if (e != hipSuccess) return e;
    lds_set = true;
  }
  TnArgs a{reinterpret_cast<const uint8_t*>(M), xh, xl, x16, xsc, w, n_touched, touched,
           offsets, slots, part, H, I, k, B * k < E ? B * k : E};
  const dim3 grid((I + kRows - 1) / kRows, (a.slots_max + 7) / 8 * 8);
  hipLaunchKernelGGL(tn_kernel<true>, grid, dim3(kWaves * 64), tn_lds_bytes(), s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tn_kernel<false>, grid, dim3(kWaves * 64), tn_lds_bytes(), s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_part_combine(part, ids, y, B, k, I, E, s);
}

hipError_t launch_part_combine(const float* part, const int32_t* ids, float* y, int B, int k,
                               int I, int E, hipStream_t s) {
  if (I % 4 != 0) return hipErrorInvalidValue;
  const size_t n = (size_t)B * (I / 4);
  int g = (int)((n + 255) / 256);
  g = g > 4096 ? 4096 : g;
  hipLaunchKernelGGL(tn_combine_kernel, dim3(g), dim3(256), 0, s, part, ids, y, B, k, I,
                     E);
  return hipGetLastError();
}

}  // namespace moe

// linear_mfma.hip -- experts that are one matrix each, for any batch, on MFMA.
//
// The batch-sweep workload of the "501B of which 23B are switched on" post (section 3):
// each expert is one H_out x H bf16 matrix M_e, a token picks k experts, and
// y_b = sum_i w_{b,i} M_{e_{b,i}} x_b.  A batch reads every touched expert once for all the
// tokens routed to it (the touched-expert union), which is what makes large batches
// cheaper per token: the reads are shared, not skipped (section 3[B]).
//
// Work layout: workgroup r (1024 threads, 16 waves) owns output rows [32r, 32r+32) of
// every expert, so it accumulates y[b][its rows] alone: no cross-workgroup reduction, and a
// fixed order (touched experts ascending).  Wave w takes the 16-row MFMA tile (w & 1) and
// the K slice (w >> 1) of eight; the eight K slices are summed through LDS.  For each
// touched expert the bucket's tokens go in passes of up to 128 (up to 8 MFMA N-tiles of
// 16 tokens), so each weight row is read from HBM once per pass.
//
// Precision: M is bf16; x is fp32 and enters the bf16 MFMA as x = hi + lo with hi = RNE(x)
// and lo = RNE(x - hi), both bf16 (prepared once per call by split_x_kernel): two MFMAs per
// product with fp32 accumulation, i.e. x carries ~16 significant bits.
//
// MFMA v_mfma_f32_16x16x32_bf16 lane layout (checked on gfx950): lane l holds
// A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16] and D[4*(l/16) .. +4][l%16].
#include "bf16_split.h"
#include "kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 32;   // output rows per workgroup
constexpr int kSplitK = 8;  // K slices per workgroup (waves = 2 row tiles x 8 slices)


// x [B][H] fp32 -> hi, lo [B][H] bf16 with hi + lo ~= x.
__global__ __launch_bounds__(256) void split_x_kernel(const float* x, size_t n, uint16_t* hi,
                                                      uint16_t* lo) {
  split_x_range(x, n, hi, lo, blockIdx.x * (size_t)blockDim.x + threadIdx.x,
                (size_t)gridDim.x * blockDim.x);
}

struct LinArgs {
  const void* M;             // [E][I][H] bf16
  const uint16_t* xh;        // [B][H] bf16 bits
  const uint16_t* xl;
  const float* w;            // [B][k]
  const int32_t* n_touched;  // [1]
  const int32_t* touched;    // [E]
  const int32_t* offsets;    // [E+1]
  const int32_t* slots;      // [B*k]
  float* y;                  // [B][I]
  int H, I, E, k, B;
};

// One pass over K for NT token tiles, unrolled U k-steps: all loads of an unrolled group
// are issued before its MFMAs; the 16 waves of the CU overlap each other's latency.
template <int NT, int U>
__device__ __forceinline__ void k_loop(const uint8_t* arow, const uint8_t* const (&bh)[NT],
                                       const uint8_t* const (&bl)[NT], int k0, int k1,
                                       f32x4 (&acc)[NT]) {
  for (int kk = k0; kk < k1; kk += 32 * U) {
    bf16x8 A[U], Bh[U][NT], Bl[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int off = (kk + 32 * u) * 2;
      A[u] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(arow + off));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        Bh[u][t] = *reinterpret_cast<const bf16x8*>(bh[t] + off);
        Bl[u][t] = *reinterpret_cast<const bf16x8*>(bl[t] + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[u], Bh[u][t], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[u], Bl[u][t], acc[t], 0, 0, 0);
      }
  }
}

// One pass: tokens [p0, p0+np) of expert e's bucket; accumulate into y.
template <int NT, int U>
__device__ inline void pass(const LinArgs& a, const uint8_t* Me, int np, const int* tok_b,
                            const float* tok_w, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rt = wave & 1, ks = wave >> 1;
  const int H = a.H;
  const int row = blockIdx.x * kRows + rt * 16 + (lane & 15);
  const int rowc = row < a.I ? row : a.I - 1;  // rows past the end compute garbage, unused
  const int kslice = H / kSplitK;
  const int k0 = ks * kslice, k1 = k0 + kslice;
  const int koff = 8 * (lane >> 4);
  const uint8_t* arow = Me + ((size_t)rowc * H + koff) * 2;
  const uint8_t* bh[NT];
  const uint8_t* bl[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int ti = t * 16 + (lane & 15);
    ti = ti < np ? ti : 0;  // padded token columns read token 0 and are discarded
    const size_t xo = ((size_t)tok_b[ti] * H + koff) * 2;
    bh[t] = reinterpret_cast<const uint8_t*>(a.xh) + xo;
    bl[t] = reinterpret_cast<const uint8_t*>(a.xl) + xo;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
  k_loop<NT, U>(arow, bh, bl, k0, k1, acc);
  // sum the eight K slices through LDS, tile by tile, in slice order
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    *reinterpret_cast<f32x4*>(red + ((ks * 2 + rt) * 64 + lane) * 4) = acc[t];
    __syncthreads();
    if (ks == 0) {
      f32x4 s = *reinterpret_cast<const f32x4*>(red + ((0 * 2 + rt) * 64 + lane) * 4);
#pragma unroll
      for (int q = 1; q < kSplitK; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(red + ((q * 2 + rt) * 64 + lane) * 4);
        s += v;
      }
      const int ti = t * 16 + (lane & 15);
      if (ti < np) {
        const int b = tok_b[ti];
        const float wgt = tok_w[ti];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = blockIdx.x * kRows + rt * 16 + 4 * (lane >> 4) + i;
          if (r < a.I) {
            float* yp = a.y + (size_t)b * a.I + r;
            *yp = fmaf(wgt, s[i], *yp);
          }
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(1024) void linear_kernel(LinArgs a) {
  __shared__ __attribute__((aligned(16))) float red[kSplitK * 2 * 64 * 4];
  __shared__ int tok_b[128];
  __shared__ float tok_w[128];
  const int tid = threadIdx.x;

  // this workgroup's rows of y start at zero for every token of the batch
  for (int i = tid; i < a.B * kRows; i += blockDim.x) {
    const int b = i / kRows, r = blockIdx.x * kRows + (i % kRows);
    if (r < a.I) a.y[(size_t)b * a.I + r] = 0.0f;
  }
  __syncthreads();

  const int nt = *a.n_touched;
  for (int ti = 0; ti < nt; ++ti) {
    const int e = a.touched[ti];
    const int s0 = a.offsets[e], ne = a.offsets[e + 1] - s0;
    const uint8_t* Me = reinterpret_cast<const uint8_t*>(a.M) + (size_t)e * a.I * a.H * 2;
    for (int p0 = 0; p0 < ne; p0 += 128) {
      const int np = min(128, ne - p0);
      for (int i = tid; i < 128; i += blockDim.x) {
        if (i < np) {
          const int slot = a.slots[s0 + p0 + i];
          tok_b[i] = slot / a.k;
          tok_w[i] = a.w[slot];
        }
      }
      __syncthreads();
      const int ntl = (np + 15) / 16;
      if (ntl <= 1) pass<1, 4>(a, Me, np, tok_b, tok_w, red);
      else if (ntl <= 2) pass<2, 2>(a, Me, np, tok_b, tok_w, red);
      else if (ntl <= 4) pass<4, 1>(a, Me, np, tok_b, tok_w, red);
      else pass<8, 1>(a, Me, np, tok_b, tok_w, red);
      __syncthreads();  // tok_b / tok_w reused by the next pass
    }
  }
}

}  // namespace

hipError_t launch_split_x(const float* x, size_t n, uint16_t* xh, uint16_t* xl, hipStream_t s) {
  int g = (int)((n + 255) / 256);
  g = g > 4096 ? 4096 : g;
  hipLaunchKernelGGL(split_x_kernel, dim3(g), dim3(256), 0, s, x, n, xh, xl);
  return hipGetLastError();
}

hipError_t launch_linear(const void* M, const float* x, const float* w, const int32_t* n_touched,
                         const int32_t* touched, const int32_t* offsets, const int32_t* slots,
                         uint16_t* xh, uint16_t* xl, float* y, int H, int I, int E, int k,
                         int B, hipStream_t s) {
  hipError_t e = launch_split_x(x, (size_t)B * H, xh, xl, s);
  if (e != hipSuccess) return e;
  LinArgs a{M, xh, xl, w, n_touched, touched, offsets, slots, y, H, I, E, k, B};
  hipLaunchKernelGGL(linear_kernel, dim3((I + kRows - 1) / kRows), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe

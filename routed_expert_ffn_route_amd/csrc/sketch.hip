// sketch.hip -- load-time construction of the ternary sketch of every routed channel's gate
// and up rows (the review of arXiv:2610.37386, "The weights-only reader", stage 1), and the
// two small pieces of its stage 3 (the rank-32 recovery): the coefficients b_j = U^T d_j at
// load time, and the final y += U R after the screen.
//
// Each row is rotated in blocks of 128 coordinates by a randomized Hadamard transform, kept
// unnormalized: u = H_128 (s * w) per block (s the layer's fixed random signs, H_128 the
// Sylvester-ordered Walsh-Hadamard matrix), so that g.x = sum over blocks of u.z / 128 with
// z = H_128 (s * x).  Each rotated block is stored as ternary codes in {-1, 0, 1} (the
// ternary-weight-network rule of Li and Liu, 2016: threshold 0.7 * mean |u|; the scale, the mean
// |u| over the nonzero codes, is the squared-error optimum for those codes), its scale as FP16
// and rho, the block's mean squared quantization error, as FP16.
//
// One wave per (row, block): lane l holds coordinates l and l + 64.  The butterflies run in
// stages h = 1, 2, ..., 64 on pairs (i, i + h), (a, b) -> (a + b, a - b); block sums are trees
// (lane's two values, then xor-folds 32, 16, ..., 1).  Every arithmetic step is an fp32
// operation rounded on its own: contraction into fused multiply-adds is off for these
// functions (plain operators under the pragma; the rounding intrinsics come from header
// functions outside its scope and were still fused: a square fed to a sum became one fma and
// moved rho by an FP16 ulp), so the result is one defined fp32 computation.
//
// Layout: codes [rows][H/16] 32-bit words, coordinate i of a row at bits 2 (i % 16) of word
// i / 16 (0 -> 00, +1 -> 01, -1 -> 11); alpha and rho [rows][nbp] FP16 bits, nbp = H/128
// rounded up to a multiple of 8 (16-byte rows; the padding holds zeros).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

template <DT dt>
__device__ inline float load_elem(const void* base, size_t i) {
  if constexpr (dt == DT::BF16)
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
  else
    return reinterpret_cast<const float*>(base)[i];
}

__device__ __forceinline__ float xor_lane(float v, int m) {
  return __shfl_xor(v, m, kWave);
}

// sum of the 128 values (two per lane) in the fixed tree order, in every lane
__device__ __forceinline__ float tree_sum128(float a, float b) {
#pragma clang fp contract(off)
  float s = a + b;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s = s + xor_lane(s, m);
  return s;
}

template <DT dt>
__global__ __launch_bounds__(256) void sketch_build_kernel(const void* rows, size_t nrows, int H,
                                                           const int8_t* signs, uint32_t* codes,
                                                           uint16_t* alpha, uint16_t* rho) {
  // no fused multiply-adds: each product below is rounded on its own, as stated
#pragma clang fp contract(off)
  const int lane = threadIdx.x & (kWave - 1);
  const int nb = H / 128, nbp = (nb + 7) & ~7;
  const size_t task = (size_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (task >= nrows * (size_t)nb) return;  // whole waves leave together
  const size_t r = task / nb;
  const int b = (int)(task - r * nb);
  const size_t base = r * (size_t)H + (size_t)b * 128;
  // s * w for coordinates l and l + 64 (multiplying by +-1 is exact)
  float lo = load_elem<dt>(rows, base + lane) * (float)signs[b * 128 + lane];
  float hi = load_elem<dt>(rows, base + lane + 64) * (float)signs[b * 128 + lane + 64];
  // butterflies across lanes: stages h = 1 .. 32 (pairs (i, i + h) with bit h of i clear)
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float plo = xor_lane(lo, h), phi = xor_lane(hi, h);
    const bool upper = (lane & h) != 0;
    lo = upper ? plo - lo : lo + plo;
    hi = upper ? phi - hi : hi + phi;
  }
  // stage h = 64 inside the lane
  const float u0 = lo + hi, u1 = lo - hi;
  const float a0 = fabsf(u0), a1 = fabsf(u1);
  const float mean = tree_sum128(a0, a1) * (1.0f / 128.0f);
  const float thr = 0.7f * mean;
  const int c0 = a0 > thr ? (u0 < 0.0f ? -1 : 1) : 0;
  const int c1 = a1 > thr ? (u1 < 0.0f ? -1 : 1) : 0;
  const int nnz = __popcll(__ballot(c0 != 0)) + __popcll(__ballot(c1 != 0));
  const float sabs = tree_sum128(c0 ? a0 : 0.0f, c1 ? a1 : 0.0f);
  const float al = nnz ? sabs / (float)nnz : 0.0f;
  const __half a16 = __float2half_rn(al);
  const float af = __half2float(a16);
  const float e0 = u0 - af * (float)c0;
  const float e1 = u1 - af * (float)c1;
  const float mse = tree_sum128(e0 * e0, e1 * e1) * (1.0f / 128.0f);
  // codes: lanes 16q .. 16q + 15 form word q (coordinates 16q ..) and word q + 4 (+ 64)
  uint32_t w0 = (uint32_t)(c0 & 3) << (2 * (lane & 15));
  uint32_t w1 = (uint32_t)(c1 & 3) << (2 * (lane & 15));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    w0 |= (uint32_t)__shfl_xor((int)w0, m, kWave);
    w1 |= (uint32_t)__shfl_xor((int)w1, m, kWave);
  }
  uint32_t* crow = codes + r * (size_t)(H / 16) + (size_t)b * 8;
  if ((lane & 15) == 0) {
    crow[lane >> 4] = w0;
    crow[4 + (lane >> 4)] = w1;
  }
  if (lane == 0) {
    alpha[r * nbp + b] = __half_as_ushort(a16);
    rho[r * nbp + b] = __half_as_ushort(__float2half_rn(mse));
  }
  if (b == 0 && lane >= nb && lane < nbp) {  // the row's padding
    alpha[r * nbp + lane] = 0;
    rho[r * nbp + lane] = 0;
  }
}

// The recovery coefficients b_j = U^T d_j of the reader's stage 3 (rank kRecRank): one thread
// per (row j of D^T, component c), an fp32 sum over h in index order, stored as FP16.
template <DT dt>
__global__ __launch_bounds__(256) void rec_build_kernel(const void* down_t, size_t nrows, int H,
                                                        const float* U, uint16_t* b) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nrows * kRecRank) return;
  const size_t j = t / kRecRank;
  const int cc = (int)(t % kRecRank);
  float acc = 0.0f;
  for (int h = 0; h < H; ++h)
    acc = fmaf(U[(size_t)h * kRecRank + cc], load_elem<dt>(down_t, j * (size_t)H + h), acc);
  b[t] = __half_as_ushort(__float2half_rn(acc));
}

// y[h] += sum_c U[h][c] R[c] with R = sum over the P workgroups' vectors r[w][c] (in workgroup
// order), the stage-3 term U sum_S w_j b_j p_j whose inner sums the screen left in r.
__global__ __launch_bounds__(256) void rec_apply_kernel(float* y, const float* U, const float* r,
                                                        int P, int H) {
  __shared__ float part[8][kRecRank];
  __shared__ float R[kRecRank];
  const int tid = threadIdx.x, cc = tid % kRecRank, g = tid / kRecRank;  // 8 groups
  // workgroups g, g + 8, ... in batches of 32 independent loads, one round trip for up to
  // 256 workgroups (a plain loop would wait for each load before issuing the next); U's row
  // is requested first
  const int h = blockIdx.x * blockDim.x + tid;
  const float4* u4 = reinterpret_cast<const float4*>(U + (size_t)min(h, H - 1) * kRecRank);
  float4 uv[kRecRank / 4];
#pragma unroll
  for (int q = 0; q < kRecRank / 4; ++q) uv[q] = u4[q];
  float s = 0.0f;
  for (int w0 = g; w0 < P; w0 += 256) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int w = min(w0 + 8 * u, P - 1);
      v[u] = r[(size_t)w * kRecRank + cc];
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) s += w0 + 8 * u < P ? v[u] : 0.0f;
  }
  part[g][cc] = s;
  __syncthreads();
  if (tid < kRecRank) {
    float t = 0.0f;
    for (int q = 0; q < 8; ++q) t += part[q][tid];
    R[tid] = t;
  }
  __syncthreads();
  if (h < H) {
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < kRecRank / 4; ++q) {
      acc = fmaf(uv[q].x, R[4 * q], acc);
      acc = fmaf(uv[q].y, R[4 * q + 1], acc);
      acc = fmaf(uv[q].z, R[4 * q + 2], acc);
      acc = fmaf(uv[q].w, R[4 * q + 3], acc);
    }
    y[h] += acc;
  }
}

}  // namespace

hipError_t launch_rec_build(const void* down_t, DT dt, size_t nrows, int H, const float* U,
                            uint16_t* b, hipStream_t s) {
  if (dt != DT::BF16 && dt != DT::F32) return hipErrorInvalidValue;
  const size_t n = nrows * kRecRank;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  if (dt == DT::BF16)
    hipLaunchKernelGGL(rec_build_kernel<DT::BF16>, dim3((unsigned)blocks), dim3(256), 0, s,
                       down_t, nrows, H, U, b);
  else
    hipLaunchKernelGGL(rec_build_kernel<DT::F32>, dim3((unsigned)blocks), dim3(256), 0, s,
                       down_t, nrows, H, U, b);
  return hipGetLastError();
}

hipError_t launch_rec_apply(float* y, const float* U, const float* r, int P, int H,
                            hipStream_t s) {
  if (H <= 0 || P <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rec_apply_kernel, dim3((H + 255) / 256), dim3(256), 0, s, y, U, r, P, H);
  return hipGetLastError();
}

hipError_t launch_sketch_build(const void* rows, DT dt, size_t nrows, int H, const int8_t* signs,
                               uint32_t* codes, uint16_t* alpha, uint16_t* rho, hipStream_t s) {
  if (H % 128 != 0 || (dt != DT::BF16 && dt != DT::F32)) return hipErrorInvalidValue;
  const size_t tasks = nrows * (size_t)(H / 128);
  if (tasks == 0) return hipSuccess;
  const size_t blocks = (tasks + 3) / 4;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  if (dt == DT::BF16)
    hipLaunchKernelGGL(sketch_build_kernel<DT::BF16>, dim3((unsigned)blocks), dim3(256), 0, s,
                       rows, nrows, H, signs, codes, alpha, rho);
  else
    hipLaunchKernelGGL(sketch_build_kernel<DT::F32>, dim3((unsigned)blocks), dim3(256), 0, s,
                       rows, nrows, H, signs, codes, alpha, rho);
  return hipGetLastError();
}

}  // namespace moe

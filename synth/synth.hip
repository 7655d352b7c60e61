// synth.hip -- host and device implementations of the seeded input generator.
// One definition of every element, shared by the host loops and the GPU kernels below
// through __host__ __device__ functions.  The contract is in synth.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <thread>
#include <vector>

#include "synth.h"

namespace {

constexpr uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;   // Philox4x32 multipliers
constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;  // key schedule increments

struct U4 { uint32_t v[4]; };

__host__ __device__ inline U4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                     uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kMul0 * c0;
    const uint64_t p1 = (uint64_t)kMul1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += kWeyl0; k1 += kWeyl1;
  }
  U4 o; o.v[0] = c0; o.v[1] = c1; o.v[2] = c2; o.v[3] = c3;
  return o;
}

// Centred Irwin-Hall(4) integer for element idx of (seed, stream); |S| < 2^23.
__host__ __device__ inline int32_t irwin_hall4(uint64_t seed, uint64_t stream, uint64_t idx) {
  const U4 r = philox((uint32_t)idx, (uint32_t)(idx >> 32), (uint32_t)stream,
                      (uint32_t)(stream >> 32), (uint32_t)seed, (uint32_t)(seed >> 32));
  const int32_t s = (int32_t)(r.v[0] >> 10) + (int32_t)(r.v[1] >> 10) +
                    (int32_t)(r.v[2] >> 10) + (int32_t)(r.v[3] >> 10);
  return s - 2 * ((1 << 22) - 1);
}

__host__ __device__ inline float normal_f32(uint64_t seed, uint64_t stream, uint64_t idx,
                                            float scale) {
  return (float)irwin_hall4(seed, stream, idx) * scale;
}

__host__ __device__ inline uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

__host__ __device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Magnitude code on the e2m1 grid {0,0.5,1,1.5,2,3,4,6}, round-to-nearest-even,
// saturating.  Ties go to the code with an even mantissa bit (codes 0,2,4,6 are even).
__host__ __device__ inline uint32_t e2m1_code(float a) {
  if (a <= 0.25f) return 0;
  if (a < 0.75f) return 1;
  if (a <= 1.25f) return 2;
  if (a < 1.75f) return 3;
  if (a <= 2.5f) return 4;
  if (a < 3.5f) return 5;
  if (a <= 5.0f) return 6;
  return 7;
}

// One 32-element MXFP4 block starting at flat element index base: 16 code bytes + scale.
__host__ __device__ inline void mxfp4_block(uint64_t seed, uint64_t stream, uint64_t base,
                                            float scale, uint8_t* codes16, uint8_t* scale1) {
  float v[32];
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    v[i] = normal_f32(seed, stream, base + i, scale);
    const float a = fabsf(v[i]);
    amax = a > amax ? a : amax;
  }
  if (amax == 0.0f) {
    for (int i = 0; i < 16; ++i) codes16[i] = 0;
    *scale1 = 0;
    return;
  }
  // floor(log2(amax)) from the exponent field (amax is a normal number here).
  const int e_amax = (int)((f32_bits(amax) >> 23) & 0xFF) - 127;
  int sb = e_amax - 2 + 127;
  sb = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
  const int e = sb - 127;
  const float inv = ldexpf(1.0f, -e);  // exact power of two
  for (int i = 0; i < 16; ++i) {
    uint32_t byte = 0;
    for (int h = 0; h < 2; ++h) {
      const float q = v[2 * i + h] * inv;
      uint32_t c = e2m1_code(fabsf(q));
      if (c != 0 && q < 0.0f) c |= 8u;
      byte |= c << (4 * h);
    }
    codes16[i] = (uint8_t)byte;
  }
  *scale1 = (uint8_t)sb;
}

template <typename F>
void parallel_for(uint64_t n, int nthreads, F f) {
  if (nthreads <= 0) nthreads = (int)std::thread::hardware_concurrency();
  if (nthreads < 1) nthreads = 1;
  if (n < 65536 || nthreads == 1) {
    f(0, n);
    return;
  }
  std::vector<std::thread> ts;
  const uint64_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    const uint64_t a = per * t, b = a + per < n ? a + per : n;
    if (a >= b) break;
    ts.emplace_back([=] { f(a, b); });
  }
  for (auto& t : ts) t.join();
}

__global__ void k_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                             float scale, float* out) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = normal_f32(seed, stream, first + i, scale);
}

__global__ void k_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                              float scale, uint16_t* out) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = bf16_rne(normal_f32(seed, stream, first + i, scale));
}

__global__ void k_mxfp4(uint64_t seed, uint64_t stream, uint64_t first_elem, uint64_t nblocks,
                        float scale, uint8_t* codes, uint8_t* scales) {
  for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
       b += (uint64_t)gridDim.x * blockDim.x) {
    uint8_t c[16], s;
    mxfp4_block(seed, stream, first_elem + 32 * b, scale, c, &s);
    uint4 w;
    memcpy(&w, c, 16);
    reinterpret_cast<uint4*>(codes)[b] = w;
    scales[b] = s;
  }
}

int grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

float synth_scale_for_sigma(double sigma) {
  return (float)(sigma * sqrt(3.0) / 4194304.0);
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const U4 r = philox(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int i = 0; i < 4; ++i) out[i] = r.v[i];
}

int synth_normal_f32_host(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                          float scale, float* out, int nthreads) {
  if (!out && n) return -1;
  parallel_for(n, nthreads, [&](uint64_t a, uint64_t b) {
    for (uint64_t i = a; i < b; ++i) out[i] = normal_f32(seed, stream, first + i, scale);
  });
  return 0;
}

int synth_normal_bf16_host(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                           float scale, uint16_t* out, int nthreads) {
  if (!out && n) return -1;
  parallel_for(n, nthreads, [&](uint64_t a, uint64_t b) {
    for (uint64_t i = a; i < b; ++i)
      out[i] = bf16_rne(normal_f32(seed, stream, first + i, scale));
  });
  return 0;
}

int synth_mxfp4_host(uint64_t seed, uint64_t stream, uint64_t row0, uint64_t rows,
                     uint64_t cols, float scale, uint8_t* codes, uint8_t* scales,
                     int nthreads) {
  if (cols % 32 != 0 || (!codes && rows) || (!scales && rows)) return -1;
  const uint64_t nblocks = rows * cols / 32, first = row0 * cols;
  parallel_for(nblocks, nthreads, [&](uint64_t a, uint64_t b) {
    for (uint64_t i = a; i < b; ++i)
      mxfp4_block(seed, stream, first + 32 * i, scale, codes + 16 * i, scales + i);
  });
  return 0;
}

int synth_normal_f32_device(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                            float scale, float* out, void* hip_stream) {
  if (!out && n) return -1;
  if (!n) return 0;
  hipLaunchKernelGGL(k_normal_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)hip_stream,
                     seed, stream, first, n, scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int synth_normal_bf16_device(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                             float scale, uint16_t* out, void* hip_stream) {
  if (!out && n) return -1;
  if (!n) return 0;
  hipLaunchKernelGGL(k_normal_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)hip_stream,
                     seed, stream, first, n, scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int synth_mxfp4_device(uint64_t seed, uint64_t stream, uint64_t row0, uint64_t rows,
                       uint64_t cols, float scale, uint8_t* codes, uint8_t* scales,
                       void* hip_stream) {
  if (cols % 32 != 0 || ((!codes || !scales) && rows)) return -1;
  if (((uintptr_t)codes & 15) != 0) return -1;
  const uint64_t nblocks = rows * cols / 32;
  if (!nblocks) return 0;
  hipLaunchKernelGGL(k_mxfp4, dim3(grid_for(nblocks)), dim3(256), 0, (hipStream_t)hip_stream,
                     seed, stream, row0 * cols, nblocks, scale, codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"

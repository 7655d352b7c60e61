// probe.hip -- measurement kernels of the benchmark (libmoe_probe.so); not part of the layer.
//
//  * a read-only stream over a buffer far larger than the 256 MB MALL, with non-temporal
//    16-byte loads: the achieved HBM read bandwidth that decode ceilings are priced against
//    (the "Code" section of "Mixture of Experts Changes the Arithmetic" derives its ceilings
//    from a measured read-only stream sum, not from the datasheet peak);
//  * an empty kernel launched with the layer kernels' geometry: graph-replayed, it gives the
//    per-launch floor that dispatch alone sets (same page, "What the Runtime Does With the
//    Promise").
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

using u32x4 = __attribute__((ext_vector_type(4))) unsigned int;

// Each thread XOR-folds 16-byte pieces i, i + S, i + 2S, ... (S = threads in the grid), four
// loads in flight per iteration; one word per workgroup is written only if the fold hits an
// impossible value, which keeps every load live.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p,
                                                          size_t n16, unsigned int* sink) {
  const size_t S = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * S < n16; i += 4 * S) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + S);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * S);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * S);
    acc ^= (a ^ b) ^ (c ^ d);
  }
  for (; i < n16; i += S) acc ^= __builtin_nontemporal_load(p + i);
  const unsigned int f = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (f == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = f;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// One read of `bytes` (a multiple of 16) at `buf` on `stream` with `blocks` x 256 threads;
// `sink` holds `blocks` words.  Returns a hipError_t.
int probe_stream_read(const void* buf, size_t bytes, int blocks, void* sink, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || blocks < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(buf), bytes / 16,
                     reinterpret_cast<unsigned int*>(sink));
  return (int)hipGetLastError();
}

// One empty kernel of `blocks` x `threads` on `stream`.
int probe_empty(int blocks, int threads, void* stream) {
  if (blocks < 1 || threads < 1 || threads > 1024) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0,
                     reinterpret_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}

}  // extern "C"

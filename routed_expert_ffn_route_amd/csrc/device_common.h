// device_common.h -- shared device helpers of the gfx950 kernels: row formats, wave
// reductions, ordered keys for exact top-k, cross-workgroup flags with bounded waits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum class DT : int { F32 = 0, BF16 = 1, MXFP4 = 2 };

constexpr int kWave = 64;
constexpr int kTeam = 256;         // threads that cover one weight row together
constexpr int kChunkElems = 8;     // elements one thread takes from a row per chunk

// ------------------------------------------------------------------------------------
// Row formats.  A row of H elements is read in chunks of 8 consecutive elements; lane i
// of a team takes chunks i, i+256, ... so a wave's loads of one row are contiguous.
//   F32:   32 bytes per chunk (two 16-byte loads)
//   BF16:  16 bytes per chunk (one 16-byte load)
//   MXFP4:  4 bytes per chunk (8 e2m1 codes) + the e8m0 scale of its 32-element block
// ------------------------------------------------------------------------------------
template <DT dt> struct Fmt;

template <> struct Fmt<DT::F32> {
  struct Raw { u32x4 a, b; };
  static __device__ __forceinline__ Raw load(const void* row, const uint8_t*, int c) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + 2 * c;
    Raw r;
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
    return r;
  }
  static __device__ __forceinline__ void decode(const Raw& r, float v[8]) {
    v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
    v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
    v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
    v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H * 4; }
};

template <> struct Fmt<DT::BF16> {
  struct Raw { u32x4 a; };
  static __device__ __forceinline__ Raw load(const void* row, const uint8_t*, int c) {
    Raw r;
    r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
    return r;
  }
  static __device__ __forceinline__ void decode(const Raw& r, float v[8]) {
    v[0] = __uint_as_float(r.a.x << 16); v[1] = __uint_as_float(r.a.x & 0xFFFF0000u);
    v[2] = __uint_as_float(r.a.y << 16); v[3] = __uint_as_float(r.a.y & 0xFFFF0000u);
    v[4] = __uint_as_float(r.a.z << 16); v[5] = __uint_as_float(r.a.z & 0xFFFF0000u);
    v[6] = __uint_as_float(r.a.w << 16); v[7] = __uint_as_float(r.a.w & 0xFFFF0000u);
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H * 2; }
};

template <> struct Fmt<DT::MXFP4> {
  struct Raw { uint32_t q; uint32_t s; };
  static __device__ __forceinline__ Raw load(const void* row, const uint8_t* srow, int c) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row) + c);
    r.s = __builtin_nontemporal_load(srow + (c >> 2));
    return r;
  }
  // value = e2m1(code) * 2^(scale - 127): the hardware conversion applies the fp32
  // scale 2^(scale-127), built from the e8m0 byte (a zero byte gives 0, not 2^-127).
  static __device__ __forceinline__ void decode(const Raw& r, float v[8]) {
    const float sc = __uint_as_float(r.s << 23);
    f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 0);
    f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 1);
    f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 2);
    f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.q, sc, 3);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
    v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H / 2; }
  static __host__ __device__ constexpr size_t scale_row_bytes(int H) { return (size_t)H / 32; }
};

// A pointer every lane of the wave holds the same value of, moved to scalar registers so
// that loads use a scalar base plus a per-lane 32-bit offset (one offset register serves
// every row of a batch instead of a 64-bit address register pair per row).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Address of row r of a stacked [rows][H] tensor, and of its MXFP4 scale row.
template <DT dt>
__device__ __forceinline__ const void* row_ptr(const void* base, size_t r, int H) {
  return reinterpret_cast<const uint8_t*>(base) + r * Fmt<dt>::row_bytes(H);
}
__device__ __forceinline__ const uint8_t* scale_row_ptr(const uint8_t* base, size_t r, int H) {
  return base ? base + r * (size_t)(H / 32) : nullptr;
}

// ------------------------------------------------------------------------------------
// Reductions
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Reduce N values held by every lane of a wave.  On return, lane l holds the wave total of
// value (l % N) in v[0] (N a power of two <= 64).  Uses N-1 + log2(64/N) exchanges
// instead of N*6.
template <int N>
__device__ __forceinline__ float wave_multi_sum(float (&v)[N], int lane) {
  // halving steps: at width w, lanes with bit set keep the upper half of the values
#pragma unroll
  for (int w = N; w > 1; w >>= 1) {
    const int half = w >> 1;
    const bool upper = (lane & half) != 0;   // which half this lane keeps
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? v[i] : v[i + half];
      const float keep = upper ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, half, kWave);
    }
  }
  float r = v[0];
#pragma unroll
  for (int m = N; m < kWave; m <<= 1) r += __shfl_xor(r, m, kWave);
  return r;  // lane l: total of value index (l & (N-1))
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ------------------------------------------------------------------------------------
// Exact top-k keys: descending float, ties to the lower index.
// key = (order-preserving bits of the value) << 32 | (0xFFFFFFFF - index)
// ------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 compare equal
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  return ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) {
  return 0xFFFFFFFFu - (uint32_t)k;
}
__device__ __forceinline__ float key_value(uint64_t k) {
  return from_ordered_bits((uint32_t)(k >> 32));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((unsigned)(uint32_t)v, m, kWave);
  const uint32_t hi = __shfl_xor((unsigned)(uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one key per lane across the 64 lanes, descending (lane 0 = largest).
__device__ __forceinline__ uint64_t wave_bitonic_desc(uint64_t key, int lane) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t other = shfl_xor_u64(key, j);
      const bool desc = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      const uint64_t mx = key > other ? key : other;
      const uint64_t mn = key > other ? other : key;
      key = (lower == desc) ? mx : mn;
    }
  }
  return key;
}

// Top-k of n keys held in LDS `buf` (capacity >= n), by the whole workgroup.  Each level
// sorts groups of 64 keys with one wave each and keeps the k best of every group, until at
// most 64 remain.  Requires k <= 32 when n > 64 (each level then at least halves the
// candidates).  On return buf[0..k) holds the k largest keys in descending order.
// `tmp` must hold at least ceil(n/64)*k keys.  All threads of the workgroup must call.
__device__ inline void wg_topk_keys(uint64_t* buf, uint64_t* tmp, int n, int k) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  uint64_t* src = buf;
  uint64_t* dst = tmp;
  while (true) {
    const int groups = (n + kWave - 1) / kWave;
    const int keep = k < kWave ? k : kWave;
    for (int g = wave; g < groups; g += nwaves) {
      const int i = g * kWave + lane;
      uint64_t key = i < n ? src[i] : 0ull;
      key = wave_bitonic_desc(key, lane);
      if (lane < keep) dst[g * keep + lane] = key;
    }
    __syncthreads();
    n = groups * keep;
    uint64_t* t = src; src = dst; dst = t;
    if (groups == 1) break;
  }
  if (src != buf) {
    for (int i = threadIdx.x; i < k; i += blockDim.x) buf[i] = src[i];
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
// Cross-workgroup signalling (device scope) with bounded waits.
//
// A release fence at device scope writes back the whole L2 of the issuing XCD, and those
// write-backs serialise across the chip (measured: one fence per workgroup of a 256-WG
// launch adds ~59 us); acquire fences invalidate L2 and serialise too.  So the kernels issue
// neither.  Data handed to other workgroups is written with device-scope atomic stores
// (st_dev); the writer waits for its stores to complete (s_waitcnt) and then bumps a flag
// or counter with a relaxed device-scope atomic.  A reader spins on the flag with relaxed
// device-scope loads and, once it has seen it, reads the data with device-scope loads
// (ld_dev), which do not hit stale cached copies; those loads are issued only after the
// flag load has returned, and the data was complete in memory before the flag was written.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t load_relaxed_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-coherent stores of values other workgroups will read.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-coherent loads of values other workgroups wrote with st_dev.
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this thread issued has completed.
__device__ __forceinline__ void stores_complete() { __builtin_amdgcn_s_waitcnt(0); }
// Make data that other workgroups completed before their flag visible to this one.
__device__ __forceinline__ void acquire_dev() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

constexpr uint64_t kWaitTicks = 100000000ull;  // 1 s of the 100 MHz constant clock


// Control block at the start of every layer workspace (device memory, cleared at layer
// creation).  Hand-offs between workgroups use arrival counters that only ever grow: launch
// number n (= the epoch read at the start of the launch) is complete for a counter group
// when the group reads (n + 1) * (its participant count).  Every launch increments every
// counter family once per participating workgroup (also families its kernel does not
// wait on), so the expected values stay in step across kernels sharing a workspace.  The
// counters of one family are split over kGroups cache lines, so that arrivals contend in
// groups of P/kGroups instead of all P on one address.
constexpr int kGroups = 16;
struct Ctrl {
  uint32_t epoch;               // launches completed on this workspace
  uint32_t err;                 // sticky error bits (read and cleared by moe_layer_check)
  uint32_t pad0[30];
  uint32_t router[kGroups][32]; // router workgroups that published their logits
  uint32_t done[kGroups][32];   // workgroups that published their partial output
  uint32_t phase2[kGroups][32]; // workgroups that published their channel scores
};
static_assert(sizeof(Ctrl) == 128 + 3 * kGroups * 128, "counter groups are 128-byte lines");

enum : uint32_t {
  kErrRouteWait = 1u, kErrReduceWait = 2u, kErrBadId = 4u, kErrPhaseWait = 8u,
};

__device__ __forceinline__ void arrive(uint32_t (*family)[32], int wg) {
  add_relaxed_dev(&family[wg % kGroups][0], 1u);
}

// Participants of group g when workgroups 0..n-1 take part.
__device__ __forceinline__ uint32_t group_count(int n, int g) {
  return (uint32_t)(n / kGroups + (g < n % kGroups ? 1 : 0));
}

// One thread: wait until every group of `family` has seen all of launch `epoch`'s
// arrivals from workgroups 0..n-1 (bounded; an expired wait sets `errbit`).
__device__ inline bool wait_family(uint32_t (*family)[32], int n, uint32_t epoch,
                                   uint32_t* err, uint32_t errbit) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    bool all = true;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t target = (epoch + 1u) * group_count(n, g);
      all &= (int32_t)(load_relaxed_dev(&family[g][0]) - target) >= 0;
    }
    if (all) return true;
    __builtin_amdgcn_s_sleep(1);
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      __hip_atomic_fetch_or(err, errbit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
}

}  // namespace moe

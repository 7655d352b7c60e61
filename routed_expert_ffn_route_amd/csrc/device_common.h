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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Pointers typed as LDS (address space 3).  Buffers chosen at run time among several LDS
// arrays can otherwise reach the accesses as generic pointers, which compile to flat
// memory operations that count against the global-load counter as well: waiting for one
// of them then drains every global load in flight.
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) int lds_i32;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
// Buffer resource over `bytes` bytes from the wave-uniform address p.  Loads through it at
// byte offsets at or past `bytes` return zeros without a memory access, so a resource of
// 0 bytes serves an empty slot and the lanes past a row's end need no bounds test.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // third word: 32-bit data format, the raw-buffer setting on this architecture
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
constexpr int kNT = 2;  // cache policy of the weight streams: non-temporal
// global-memory (address space 1) views: loads through them are global_load_* (never flat)
typedef __attribute__((address_space(1))) uint8_t gbl_u8;
typedef __attribute__((address_space(1))) uint32_t gbl_u32;
typedef __attribute__((address_space(1))) u32x2 gbl_u32x2;
typedef __attribute__((address_space(1))) u32x4 gbl_u32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
__device__ __forceinline__ u32x4 lds_ld128(const lds_u16* p) {
  return *reinterpret_cast<const lds_u32x4*>(p);
}
__device__ __forceinline__ void lds_st128(lds_u16* p, const u32x4& v) {
  *reinterpret_cast<lds_u32x4*>(p) = v;
}
__device__ __forceinline__ u32x4 lds_ld128(const lds_u8* p) {
  return *reinterpret_cast<const lds_u32x4*>(p);
}

// MXFP4W is MXFP4 read in 16-element chunks (8 bytes of codes + the block's scale byte per
// thread and row) instead of 8-element ones: the same bytes, twice as many per load.
enum class DT : int { F32 = 0, BF16 = 1, MXFP4 = 2, MXFP4W = 3 };

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
  static constexpr int kE = 8;  // elements per chunk
  struct Raw { u32x4 a, b; };
  static __device__ __forceinline__ Raw load(const void* row, const uint8_t*, int c) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + 2 * c;
    Raw r;
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
    return r;
  }
  // the same through buffer resources (w: the row, s: its scales; zeros out of range) or
  // from global-memory pointers
  static __device__ __forceinline__ Raw load_b(rsrc_t w, rsrc_t, int c) {
    Raw r;
    r.a = __builtin_amdgcn_raw_buffer_load_b128(w, 32 * c, 0, kNT);
    r.b = __builtin_amdgcn_raw_buffer_load_b128(w, 32 * c + 16, 0, kNT);
    return r;
  }
  // (offsets as unsigned 32-bit byte counts: the loads take a scalar base plus a 32-bit
  // lane offset, with no 64-bit address arithmetic per lane)
  static __device__ __forceinline__ Raw load_g(const gbl_u8* row, const gbl_u8*, int c) {
    const uint32_t o = 32u * (uint32_t)c;
    Raw r;
    r.a = __builtin_nontemporal_load(reinterpret_cast<const gbl_u32x4*>(row + o));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const gbl_u32x4*>(row + o + 16u));
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
  static constexpr int kE = 8;
  struct Raw { u32x4 a; };
  static __device__ __forceinline__ Raw load(const void* row, const uint8_t*, int c) {
    Raw r;
    r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + c);
    return r;
  }
  static __device__ __forceinline__ Raw load_b(rsrc_t w, rsrc_t, int c) {
    Raw r;
    r.a = __builtin_amdgcn_raw_buffer_load_b128(w, 16 * c, 0, kNT);
    return r;
  }
  static __device__ __forceinline__ Raw load_g(const gbl_u8* row, const gbl_u8*, int c) {
    Raw r;
    r.a = __builtin_nontemporal_load(reinterpret_cast<const gbl_u32x4*>(row + 16u * (uint32_t)c));
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
  static constexpr int kE = 8;
  struct Raw { uint32_t q; uint8_t s; };  // s: kept a byte until decode (no early zero-extension)
  static __device__ __forceinline__ Raw load(const void* row, const uint8_t* srow, int c) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row) + c);
    r.s = __builtin_nontemporal_load(srow + (c >> 2));
    return r;
  }
  static __device__ __forceinline__ Raw load_b(rsrc_t w, rsrc_t s, int c) {
    Raw r;
    r.q = __builtin_amdgcn_raw_buffer_load_b32(w, 4 * c, 0, kNT);
    r.s = __builtin_amdgcn_raw_buffer_load_b8(s, c >> 2, 0, kNT);
    return r;
  }
  static __device__ __forceinline__ Raw load_g(const gbl_u8* row, const gbl_u8* srow, int c) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const gbl_u32*>(row + 4u * (uint32_t)c));
    r.s = __builtin_nontemporal_load(srow + ((uint32_t)c >> 2));
    return r;
  }
  // value = e2m1(code) * 2^(scale - 127): the hardware conversion applies the fp32
  // scale 2^(scale-127), built from the e8m0 byte (a zero byte gives 0, not 2^-127).
  static __device__ __forceinline__ void decode(const Raw& r, float v[8]) {
    const float sc = __uint_as_float((uint32_t)r.s << 23);
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

template <> struct Fmt<DT::MXFP4W> {
  static constexpr int kE = 16;
  struct Raw { u32x2 q; uint8_t s; };
  static __device__ __forceinline__ Raw load(const void* row, const uint8_t* srow, int c) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row) + c);
    r.s = __builtin_nontemporal_load(srow + (c >> 1));
    return r;
  }
  static __device__ __forceinline__ Raw load_b(rsrc_t w, rsrc_t s, int c) {
    Raw r;
    r.q = __builtin_amdgcn_raw_buffer_load_b64(w, 8 * c, 0, kNT);
    r.s = __builtin_amdgcn_raw_buffer_load_b8(s, c >> 1, 0, kNT);
    return r;
  }
  static __device__ __forceinline__ Raw load_g(const gbl_u8* row, const gbl_u8* srow, int c) {
    Raw r;
    r.q = __builtin_nontemporal_load(reinterpret_cast<const gbl_u32x2*>(row + 8u * (uint32_t)c));
    r.s = __builtin_nontemporal_load(srow + ((uint32_t)c >> 1));
    return r;
  }
  static __device__ __forceinline__ void decode(const Raw& r, float v[16]) {
    const float sc = __uint_as_float((uint32_t)r.s << 23);
    const uint32_t w[2] = {r.q.x, r.q.y};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 0);
      const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 1);
      const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 2);
      const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], sc, 3);
      v[8 * k + 0] = p0.x; v[8 * k + 1] = p0.y; v[8 * k + 2] = p1.x; v[8 * k + 3] = p1.y;
      v[8 * k + 4] = p2.x; v[8 * k + 5] = p2.y; v[8 * k + 6] = p3.x; v[8 * k + 7] = p3.y;
    }
  }
  static __host__ __device__ constexpr size_t row_bytes(int H) { return (size_t)H / 2; }
  static __host__ __device__ constexpr size_t scale_row_bytes(int H) { return (size_t)H / 32; }
};

// A pointer every lane of the wave holds the same value of, moved to scalar registers so
// that loads use a scalar base plus a per-lane 32-bit offset (one offset register serves
// every row of a batch instead of a 64-bit address register pair per row).  The result is
// typed as global memory (address space 1): an address rebuilt from integers is otherwise
// generic, and its loads become flat operations (see the LDS-typed pointers above).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* uniform_ptr(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const __attribute__((address_space(1))) T*)(((uint64_t)hi << 32) | lo);
}
typedef __attribute__((address_space(1))) float gbl_f32;

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


// Inclusive prefix sum across the 64 lanes of a wave: Hillis-Steele steps inside each row
// of 16 lanes (DPP row shifts by 1, 2, 4, 8; lanes without a source add 0), then the last
// lane of a row is broadcast into the rows above it (row_bcast:15 into rows 1 and 3,
// row_bcast:31 into rows 2 and 3).  No LDS round trips, unlike a shuffle-based scan.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// The value of lane (lane ^ M), without an LDS round trip where the hardware allows: DPP
// quad permutes for M = 1, 2; DPP row shifts (left for lanes whose bit M is clear, right
// for the others) for M = 4, 8; a swizzle (xor within 32 lanes) for M = 16; a permute for
// M = 32.
template <int M>
__device__ __forceinline__ float lane_xor(float x, int lane) {
  const int xi = __float_as_int(x);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xf, 0xf, false));
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xf, 0xf, false));
  } else if constexpr (M == 4 || M == 8) {
    const int up = __builtin_amdgcn_update_dpp(0, xi, 0x100 + M, 0xf, 0xf, false);  // lane+M
    const int dn = __builtin_amdgcn_update_dpp(0, xi, 0x110 + M, 0xf, 0xf, false);  // lane-M
    return __int_as_float((lane & M) ? dn : up);
  } else if constexpr (M == 16) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(xi, 0x401F));  // and 0x1f, xor 0x10
  } else {
    return __shfl_xor(x, M, kWave);
  }
}

// Sum over the lanes that agree with this one in the low log2(B) lane bits (B a power of
// two <= 64), in every lane: quad permutes (DPP) for lane bits 0-1, rotations within a row
// of 16 (DPP) for bits 2-3 (x + ror4(x), then + ror8: the four lanes of a residue mod 4),
// and swaps of rows (permlane16) and of wave halves (permlane32) for bits 4-5.  Each step
// is one exchange-and-add, none of them through LDS.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int B>
__device__ __forceinline__ float sum_lanes_above(float x) {
  if constexpr (B <= 1) x = add_dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (B <= 2) x = add_dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (B <= 4) x = add_dpp<0x124>(x);  // row_ror:4
  if constexpr (B <= 8) x = add_dpp<0x128>(x);  // row_ror:8
  if constexpr (B <= 16) {
    // one of the two results is this lane's value, the other its partner's in the row pair
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (B <= 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_sum(float v) { return sum_lanes_above<1>(v); }

// Reduce N values held by every lane of a wave.  On return, lane l holds the wave total of
// value (l % N) (N a power of two <= 16).  Halving steps first: at width w, a lane with bit
// w/2 set keeps the upper half of its values and adds its partner's (lane ^ w/2) upper
// half, the other lane the lower halves; N-1 exchanges instead of N*6.
template <int N>
__device__ __forceinline__ float wave_multi_sum(float (&v)[N], int lane) {
#pragma unroll
  for (int w = N; w > 1; w >>= 1) {
    const int half = w >> 1;
    const bool upper = (lane & half) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float lo = v[i], hi = v[i + half];  // values, so that the selects stay selects
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      float got;
      if (half == 1) got = lane_xor<1>(send, lane);
      else if (half == 2) got = lane_xor<2>(send, lane);
      else if (half == 4) got = lane_xor<4>(send, lane);
      else got = lane_xor<8>(send, lane);
      v[i] = keep + got;
    }
  }
  return sum_lanes_above<N>(v[0]);  // lane l: total of value index (l & (N-1))
}

// z * sigmoid(z) with the hardware exponential and reciprocal (about 1 ulp each)
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

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

// Rank of `me` among the keys [j0, j1) of `keys` (number of larger keys).  The lanes of a
// wave read the same keys (LDS broadcasts, no cross-lane shuffles), 16 reads in flight per
// batch; keys past `n` are clamped reads that count nothing.
__device__ __forceinline__ int rank_in(const uint64_t* keys, int n, int j0, int j1,
                                       uint64_t me) {
  int r = 0;
  for (int j = j0; j < j1; j += 16) {
    uint64_t kk[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) kk[u] = keys[j + u < n ? j + u : n - 1];
#pragma unroll
    for (int u = 0; u < 16; ++u) r += (j + u < j1 && kk[u] > me) ? 1 : 0;
  }
  return r;
}

// Top-k of n distinct non-zero keys held in LDS (keys[n .. n rounded up to 64) must be 0).
// Level 1: every group of 64 keys ranks its members among themselves (one wave per group)
// and keeps its min(k, 64) best as candidates -- every key of the overall top k is among
// its group's top k.  Level 2: the candidates are ranked among themselves (each rank split
// over several threads, partial ranks summed with LDS atomics).  A key's rank is the
// number of larger keys, so the keys of rank < k are the top k in descending order:
// out[0..k).  LDS scratch `tmp` of topk_scratch_bytes(n, k).  The keys must be visible to
// the whole workgroup before the call; all threads of the workgroup must call.
__host__ __device__ constexpr int topk_candidates(int n, int k) {
  return ((n + 63) / 64) * (k < 64 ? k : 64);
}
__host__ __device__ constexpr int topk_scratch_bytes(int n, int k) {
  return topk_candidates(n, k) * 12;
}
__device__ inline void wg_topk_rank(const uint64_t* keys, void* tmp, int n, int k,
                                    uint64_t* out) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = nt / kWave;
  const int kk = k < kWave ? k : kWave;
  const int groups = (n + kWave - 1) / kWave;
  const int C = groups * kk;
  uint64_t* cand = reinterpret_cast<uint64_t*>(tmp);
  int* cnt = reinterpret_cast<int*>(cand + C);
  for (int i = tid; i < C; i += nt) {
    cand[i] = 0ull;
    cnt[i] = 0;
  }
  __syncthreads();
  for (int g = wave; g < groups; g += nwaves) {
    const uint64_t me = keys[g * kWave + lane];
    const int r = rank_in(keys + g * kWave, kWave, 0, kWave, me);
    if (me != 0ull && r < kk) cand[g * kk + r] = me;
  }
  __syncthreads();
  int parts = nt / C;
  parts = parts < 1 ? 1 : parts > 16 ? 16 : parts;
  const int span = (C + parts - 1) / parts;
  for (int i = tid; i < C * parts; i += nt) {
    const int e = i % C, q = i / C;
    const int j0 = q * span, j1 = j0 + span < C ? j0 + span : C;
    const int r = rank_in(cand, C, j0, j1, cand[e]);
    if (r) atomicAdd(&cnt[e], r);
  }
  __syncthreads();
  for (int e = tid; e < C; e += nt) {
    const int r = cnt[e];
    if (r < k && cand[e] != 0ull) out[r] = cand[e];
  }
  __syncthreads();
}

// LDS bytes the callers of wg_topk_rank set aside for n keys: keys (padded to 64), 64
// selected keys, and the candidate scratch.
__host__ __device__ constexpr int topk_lds_bytes(int n, int k) {
  return ((n + 63) & ~63) * 8 + 64 * 8 + topk_scratch_bytes(n, k);
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
// 64-bit device-coherent store / load (single-copy atomic): a value and its launch tag.
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this thread issued has completed.
__device__ __forceinline__ void stores_complete() { __builtin_amdgcn_s_waitcnt(0); }
// Make data that other workgroups completed before their flag visible to this one.
__device__ __forceinline__ void acquire_dev() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

constexpr uint64_t kWaitTicks = 100000000ull;  // 1 s of the 100 MHz constant clock

// Spin until the 64-bit word at p carries `tag` in its upper half and return it: the data
// and its arrival signal travel in one store, so a reader needs one round trip, not a flag
// read followed by a data read (bounded; an expired wait sets `errbit` and returns the
// stale word).
__device__ inline uint64_t wait_tagged(const uint64_t* p, uint32_t tag, uint32_t* err,
                                       uint32_t errbit) {
  uint64_t v = ld_dev64(p);
  if ((uint32_t)(v >> 32) == tag) return v;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    v = ld_dev64(p);
    if ((uint32_t)(v >> 32) == tag) return v;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      __hip_atomic_fetch_or(err, errbit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return v;
    }
  }
}


// Control block at the start of every layer workspace (device memory, cleared at layer
// creation).  `epoch` counts the batch-1 launches completed on this workspace; a launch
// reads it at its start and tags the data it hands between workgroups (router logits,
// channel scores) with epoch + 1, so readers wait on the data itself.  The partial outputs
// are handed over with arrival counters that only ever grow: launch n is complete for a
// counter group when the group reads (n + 1) * (its participant count); the counters are
// split over kGroups cache lines, so that arrivals contend in groups of P/kGroups instead
// of all P on one address.
constexpr int kGroups = 16;
struct Ctrl {
  uint32_t epoch;               // launches completed on this workspace
  uint32_t err;                 // sticky error bits (read and cleared by moe_layer_check)
  uint32_t pad0[30];
  uint32_t done[kGroups][32];   // workgroups that published their partial output
};
static_assert(sizeof(Ctrl) == 128 + kGroups * 128, "counter groups are 128-byte lines");

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

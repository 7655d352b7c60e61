// channel_sparse.hip -- the channel-sparse batch-1 layer in one persistent launch.
//
// The fixed-count keep rule of the review of arXiv:2610.37386 ("Background: channels and
// keep rules"): of the k*I candidate channels of a token's routed experts, keep a fixed
// number K, compute those exactly from their full rows, and never read the dropped
// channels' up rows and down rows.  Channels are ranked by an output-unit score so that
// channels of different experts compare directly ("The weights-only reader", stage 2,
// eq. 1): here s_j = |silu(g_j.x)| * ||d_j||_2, optionally times the router weight, with
// the exact gate value (every gate row is read to score) and ||d_j|| precomputed at load.
//
// Phases inside the launch (one workgroup per CU):
//  1. router rows and the exact top-k in every workgroup, as in the dense kernel; once the
//     logits arrive, the workgroup's shared-expert rows are warmed into L2;
//  2. gate pass: each workgroup owns a contiguous share of the k*I candidates, reads their
//     gate rows, and publishes each score as a 32-bit word carrying the launch parity in its
//     lowest bit; the gate values and scores of its own candidates stay in LDS;
//  3. its share of the shared experts, which covers the scores' hand-off;
//  4. every workgroup gathers all k*I scores and finds the same K-th largest T, how many
//     scores equal T and how many of those are kept: a 2048-bin histogram over the score
//     range, a scan for the bin holding the K-th, and a rank count of that bin's few members
//     (a radix search on the score bits when the bin is crowded); meanwhile the up and down
//     rows of its own candidates that scored at least 0.85 of the previous launch's threshold
//     are prefetched into L2 (a hint only; it decides nothing);
//  5. each workgroup streams the up and down rows of its own kept candidates (those above T,
//     and the ties at T when all are kept; otherwise the lowest e*I + j of them, found by a
//     scan over all candidates in that order), with g from LDS;
//  6. the deterministic cross-workgroup sum of the partial outputs; after its partial is out,
//     workgroup 0 writes the kept list in ascending e*I + j and the threshold hint.
#include <hip/hip_fp16.h>

#include "layer_common.h"

namespace moe {
namespace {

using namespace lc;

constexpr int kMaxNP = 16;
constexpr int kGateBatch = 8;  // gate rows per team per batch
constexpr int kSelBins = 2048; // histogram bins of the selection
constexpr int kSelCand = 512;  // bin members ranked by brute force (else the radix search)
constexpr int kMaxSlots = 64;  // k
constexpr int kSlotPad = kMaxSlots + 4;  // slot tables of kMaxSlots + 1 ints, padded so
                                          // that the arrays after them are 16-byte aligned

struct CSLaunch {
  B1Args a;
  const float* dnorm;  // [E*I]
  // ternary sketch (null: exact gate values): codes [E*I][H/16] and FP16 scales [E*I][H/128]
  // of the gate and up rows, and the rotation's signs [H]
  const uint32_t *sk_g, *sk_v;
  const uint16_t *sk_ag, *sk_av;
  const int8_t* signs;
  uint64_t* g_ws;      // channel scores with the launch parity, one copy per XCD
  int32_t* kept_out;   // [K]
  int K, mode, R, SW, tsz;
};

// Exclusive prefix sum over the workgroup (sh: LDS of nwaves+1 ints).  *total = sum.
__device__ inline int block_excl_scan(int v, int* sh, const Ctx& c, int* total) {
  const int lane = c.lane, wave = c.tid >> 6, nw = c.nthreads >> 6;
  const int x = wave_incl_scan(v);
  if (lane == kWave - 1) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int wv = lane < nw ? sh[lane] : 0;
    const int s = wave_incl_scan(wv);
    if (lane < nw) sh[lane] = s - wv;
    if (lane == nw - 1) sh[nw] = s;
  }
  __syncthreads();
  const int res = sh[wave] + x - v;
  *total = sh[nw];
  __syncthreads();
  return res;
}

// The K-th largest of n non-negative scores (as uint32 bit patterns in `u`, which order
// like the floats), ties to the lower index: returns T (the K-th largest pattern) and, in
// *need, how many of the values equal to T are kept (the lowest-indexed ones).  T is found
// digit by digit, most significant first (11, 11 and 10 bits): a histogram of the digit
// over the values that match the digits found so far, and the digit where the running
// count from the top reaches the remaining need.  Requires 0 < K < n.  `hist` is LDS of
// kSelBins ints, `sh` of 48 ints.
__device__ inline uint32_t select_threshold(const uint32_t* u, int n, int K, int* need_out,
                                            int* ties_out, int* hist, int* sh, const Ctx& c) {
  uint32_t prefix = 0, mask = 0;
  int need = K;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    const int nb = 1 << widths[pass];
    for (int i = c.tid; i < nb; i += c.nthreads) hist[i] = 0;
    __syncthreads();
    for (int f = c.tid; f < n; f += c.nthreads) {
      const uint32_t v = u[f];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & dmask], 1);
    }
    __syncthreads();
    // thread t owns the bins nb-1-b for b in [t*per, (t+1)*per): counts from the top
    const int per = (nb + c.nthreads - 1) / c.nthreads;
    int local = 0;
    for (int b = c.tid * per; b < (c.tid + 1) * per && b < nb; ++b) local += hist[nb - 1 - b];
    int total;
    const int before0 = block_excl_scan(local, sh + 2, c, &total);
    if (before0 < need && need <= before0 + local) {
      int before = before0;
      for (int b = c.tid * per; b < (c.tid + 1) * per && b < nb; ++b) {
        const int cnt = hist[nb - 1 - b];
        if (before < need && need <= before + cnt) {
          sh[0] = nb - 1 - b;
          sh[1] = need - before;
          sh[47] = cnt;  // after the last digit: how many values equal T
        }
        before += cnt;
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)sh[0];
    need = sh[1];
    prefix |= digit << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  *need_out = need;
  *ties_out = sh[47];
  return prefix;
}


// Wave-wide minimum / maximum of an unsigned value, in every lane (DPP within rows of 16,
// then row and half swaps).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xf, 0xf, true));
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, true));
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, true));
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, true));
  x = min(x, swap_rows32<16>(x));
  return min(x, swap_rows32<32>(x));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xf, 0xf, true));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, true));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, true));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, true));
  x = max(x, swap_rows32<16>(x));
  return max(x, swap_rows32<32>(x));
}

// The K-th largest of the n score patterns (0 < K < n; non-negative floats, whose bit
// patterns order like the values; each thread holds eight of them in sb, all of them are in sv
// for the radix fallback), how many of the values equal to it are kept (*need; which ones is
// decided later, in channel order) and how many there are (*ties).  One histogram pass bins the patterns
// linearly over [lo, hi] (a monotone binning: bin order is score order); a scan over the bins
// finds the bin holding the K-th largest and its rank there; that bin's members (few for a
// spread of scores) are ranked by brute force.  A crowded bin (more than kSelCand members)
// falls back to the radix search.  lo, hi come in per wave in sh[4 + w] and sh[20 + w];
// hist (kSelBins ints) and sh[44] come in cleared; mem is LDS of kSelCand words.
__device__ inline uint32_t select_kth(const uint32_t* sv, const uint32_t (&sb)[8], bool mine,
                                      int n, int K, int* need_out, int* ties_out, int* hist,
                                      uint32_t* mem, int* sh, const Ctx& c) {
  const int nw = c.nthreads >> 6;
  // the range over all waves: lane w reads wave w's bounds, then a wave reduction
  uint32_t lo = c.lane < nw ? (uint32_t)sh[4 + c.lane] : 0xFFFFFFFFu;
  uint32_t hi = c.lane < nw ? (uint32_t)sh[20 + c.lane] : 0u;
  lo = __builtin_amdgcn_readfirstlane(wave_min_u32(lo));
  hi = __builtin_amdgcn_readfirstlane(wave_max_u32(hi));
  if (hi > lo) {
    const float inv = (float)kSelBins / ((float)(hi - lo) + 1.0f);
    auto bin = [&](uint32_t v) {
      const int b = (int)((float)(v - lo) * inv);
      return b < kSelBins - 1 ? b : kSelBins - 1;
    };
    int bins[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) bins[i] = bin(sb[i]);
    if (mine) {
#pragma unroll
      for (int i = 0; i < 8; ++i) atomicAdd(&hist[bins[i]], 1);
    }
    __syncthreads();
    MOE_STAMP(c.stamps, 17);
    // Wave 0 finds the bin where the count from the top reaches K: lane l sums super-bin l
    // (the 32 bins [2048 - 32 (l + 1), 2048 - 32 l), counted from the top), a scan over the
    // lanes finds the super-bin, and a scan over its 32 bins (lane l: the l-th from its top)
    // the bin
    if (c.tid < kWave) {
      constexpr int kSuper = kSelBins / kWave;  // 32 bins per lane
      const int4* hb = reinterpret_cast<const int4*>(hist + kSelBins - kSuper * (c.lane + 1));
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < kSuper / 4; ++u) {
        const int4 q = hb[u];
        cnt += q.x + q.y + q.z + q.w;
      }
      const int incl = wave_incl_scan(cnt);
      const int excl = incl - cnt;
      const uint64_t bal = __ballot(excl < K && K <= incl);
      const int L = (int)__builtin_ctzll(bal);
      const int before = __builtin_amdgcn_readlane(excl, L);
      const int b = kSelBins - kSuper * L - 1 - c.lane;
      const int v = c.lane < kSuper ? hist[b] : 0;
      const int incl2 = wave_incl_scan(v) + before;
      const int excl2 = incl2 - v;
      const bool here = c.lane < kSuper && excl2 < K && K <= incl2;
      if (here) {
        sh[40] = b;
        sh[41] = K - excl2;  // the rank wanted within the bin
        sh[42] = v;
      }
    }
    __syncthreads();
    MOE_STAMP(c.stamps, 18);
    const int bstar = sh[40], needb = sh[41], m = sh[42];
    if (m <= kSelCand) {
      if (mine) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (bins[i] == bstar) mem[atomicAdd(&sh[44], 1)] = sb[i];
      }
      __syncthreads();
      MOE_STAMP(c.stamps, 19);
      if (m <= kWave) {
        // wave 0: lane l holds member l; each counts the members above and at least it
        if (c.tid < kWave) {
          const uint32_t key = c.lane < m ? mem[c.lane] : 0u;
          int gt = 0, ge = 0;
          for (int j = 0; j < m; ++j) {
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
            gt += o > key ? 1 : 0;
            ge += o >= key ? 1 : 0;
          }
          if (c.lane < m && gt < needb && needb <= ge) {  // equal keys agree
            sh[45] = (int)key;
            sh[46] = needb - gt;
            sh[47] = ge - gt;  // how many values equal it (all lie in this bin)
          }
        }
      } else if (c.tid < m) {
        const uint32_t key = mem[c.tid];
        int gt = 0, ge = 0;
        int j = 0;
        for (; j + 8 <= m; j += 8) {  // eight reads in flight
          uint32_t o[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) o[u] = mem[j + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            gt += o[u] > key ? 1 : 0;
            ge += o[u] >= key ? 1 : 0;
          }
        }
        for (; j < m; ++j) {
          const uint32_t o = mem[j];
          gt += o > key ? 1 : 0;
          ge += o >= key ? 1 : 0;
        }
        if (gt < needb && needb <= ge) {  // the needb-th largest of the bin (equal keys agree)
          sh[45] = (int)key;
          sh[46] = needb - gt;
          sh[47] = ge - gt;
        }
      }
      __syncthreads();
      *need_out = sh[46];
      *ties_out = sh[47];
      return (uint32_t)sh[45];
    }
  }
  // all scores equal, or a crowded bin: the exact radix search over the bit patterns
  return select_threshold(sv, n, K, need_out, ties_out, hist, sh, c);
}

// Candidates per thread in the selection: eight consecutive ones, which lie in one slot (I
// is a multiple of 8), so their scores stay in registers.
constexpr int kCh = 8;
// Own candidates per workgroup at most (ceil(k*I / P); the host checks)
constexpr int kOwnMax = kCsOwnMax;

// The kept candidates in the output order (ascending e*I + j: slots by expert id, a slot
// without an expert after every expert, channels within a slot in order).  Candidate f of this
// thread's eight [c0, c0 + 8) (slot sl0, first channel j0) is kept if its score pattern sb is
// above T, or equals T and is among the first `need` such in that order.  Returns the kept
// mask (bit i: candidate c0 + i) and, in pos[i], each kept candidate's output position.  Runs
// a packed workgroup scan in candidate order, per-slot counts and (wave 0) the slots' ranks;
// every thread must call.  slot_* are LDS of kSlotPad ints each, sh of 96 ints.
__device__ inline uint32_t kept_in_order(const uint32_t (&sb)[kCh], bool mine, int sl0, int j0,
                                         uint32_t T, int need, bool all, bool none, int k,
                                         int E, const int* s_ids, int* sh, int* slot_gt,
                                         int* slot_eq, int* slot_tk, int* slot_base,
                                         const Ctx& c, int (&pos)[kCh]) {
  int ngt = 0, neq = 0;
  bool ab[kCh], ti[kCh];
#pragma unroll
  for (int i = 0; i < kCh; ++i) {
    ab[i] = mine && !none && (all || sb[i] > T);
    ti[i] = mine && !none && !all && sb[i] == T;
    ngt += ab[i] ? 1 : 0;
    neq += ti[i] ? 1 : 0;
  }
  int tot;
  const int ex = block_excl_scan(ngt * 65536 + neq, sh + 48, c, &tot);
  const int gtp = ex >> 16, eqp = ex & 0xFFFF;  // counts before this thread's candidates
  // the prefixes at the slot boundaries, written by the thread whose candidates start a slot
  if (mine && j0 == 0) {
    slot_gt[sl0] = gtp;
    slot_eq[sl0] = eqp;
  }
  if (c.tid == 0) {
    slot_gt[k] = tot >> 16;
    slot_eq[k] = tot & 0xFFFF;
  }
  __syncthreads();
  // Wave 0, lane s < k: the slot's rank in the output order (ranks are distinct), its counts
  // moved to lane rank, exclusive scans over the ranks give the ties kept before it and its
  // output base, moved back to lane s.
  if (c.tid < kWave) {
    const int sl = c.lane;
    const int key = sl < k ? (s_ids[sl] >= 0 ? s_ids[sl] : E + sl) : 0x7FFFFFFF;
    int rank = 0;
    for (int o = 0; o < k; ++o) {
      const int ko = __builtin_amdgcn_readlane(key, o);
      rank += ko < key ? 1 : 0;
    }
    const int dst = sl < k ? rank : sl;  // lanes past k keep their place (zero counts)
    const int eq_s = sl < k ? slot_eq[sl + 1] - slot_eq[sl] : 0;
    const int gt_s = sl < k ? slot_gt[sl + 1] - slot_gt[sl] : 0;
    const int req = __builtin_amdgcn_ds_permute(dst * 4, eq_s);
    const int rgt = __builtin_amdgcn_ds_permute(dst * 4, gt_s);
    const int eqb = wave_incl_scan(req) - req;
    const int tk = min(max(need - eqb, 0), req);
    const int kept = rgt + tk;
    const int base = wave_incl_scan(kept) - kept;
    const int tk_s = __shfl(tk, dst, kWave);
    const int base_s = __shfl(base, dst, kWave);
    if (sl < k) {
      slot_tk[sl] = tk_s;
      slot_base[sl] = base_s;
    }
  }
  __syncthreads();
  uint32_t mask = 0;
  if (mine) {
    const int tk = slot_tk[sl0], sbase = slot_base[sl0];
    int gin = gtp - slot_gt[sl0], qin = eqp - slot_eq[sl0];
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      pos[i] = sbase + gin + min(qin, tk);
      if (ab[i] || (ti[i] && qin < tk)) mask |= 1u << i;
      gin += ab[i] ? 1 : 0;
      qin += ti[i] ? 1 : 0;
    }
  }
  return mask;
}

// The token side of the sketch screen: z = H_128 (s * x) per 128-block (fp32 butterflies,
// stages h = 1 .. 64, (a, b) -> (a + b, a - b)), and per block only the 80 coordinates of
// largest |z| kept (ties to the lower coordinate), the others zeroed, into zs [H] (LDS).  One
// wave per block: lane l holds coordinates l and l + 64; the 80th largest |z| is found bit by
// bit from the top with ballot counts, the ties at it in coordinate order with lane counts.
constexpr int kScan = 80;
__device__ inline void rotate_scan(const float* x, const int8_t* signs, float* zs, int H,
                                   const Ctx& c) {
#pragma clang fp contract(off)
  const int nb = H / 128, wave = c.tid / kWave, nw = c.nthreads / kWave, lane = c.lane;
  for (int b = wave; b < nb; b += nw) {
    // the signs as 32-bit words (four per word), extracted after both loads are out
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(signs) + b * 32;
    const uint32_t wlo = s32[lane >> 2], whi = s32[16 + (lane >> 2)];
    const float xlo = x[b * 128 + lane], xhi = x[b * 128 + lane + 64];
    float lo = xlo * (float)(int8_t)(wlo >> (8 * (lane & 3)));
    float hi = xhi * (float)(int8_t)(whi >> (8 * (lane & 3)));
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      const float plo = __shfl_xor(lo, h, kWave), phi = __shfl_xor(hi, h, kWave);
      const bool upper = (lane & h) != 0;
      lo = upper ? plo - lo : lo + plo;
      hi = upper ? phi - hi : hi + phi;
    }
    const float z0 = lo + hi, z1 = lo - hi;
    const uint32_t a0 = __float_as_uint(z0) & 0x7FFFFFFFu, a1 = __float_as_uint(z1) & 0x7FFFFFFFu;
    uint32_t t = 0;  // the largest pattern with at least kScan values at or above it
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      const int cnt = __popcll(__ballot(a0 >= cand)) + __popcll(__ballot(a1 >= cand));
      t = cnt >= kScan ? cand : t;
    }
    const int need = kScan - (__popcll(__ballot(a0 > t)) + __popcll(__ballot(a1 > t)));
    const uint64_t e0 = __ballot(a0 == t), e1 = __ballot(a1 == t);
    const int r0 = __builtin_amdgcn_mbcnt_hi((uint32_t)(e0 >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)e0, 0));
    const int r1 = __popcll(e0) + __builtin_amdgcn_mbcnt_hi(
                                      (uint32_t)(e1 >> 32),
                                      __builtin_amdgcn_mbcnt_lo((uint32_t)e1, 0));
    const bool k0 = a0 > t || (a0 == t && r0 < need);
    const bool k1 = a1 > t || (a1 == t && r1 < need);
    zs[b * 128 + lane] = k0 ? z0 : 0.0f;
    zs[b * 128 + lane + 64] = k1 ? z1 : 0.0f;
  }
}

// Sketch estimate of one row for this lane's share: coordinates [32q, 32q + 32) for q = lane,
// lane + 64 (H <= 4096): the 2-bit codes (two words per q) times zs, times the block's scale.
struct SketchPiece {
  uint2 w[2];      // the 32 codes of coordinates [32q, 32q + 32)
  uint32_t a[2];   // the FP16 scale of their block in the low half (0: no contribution)
};
// All loads unconditional and at least 4 bytes wide (a narrower load, or one under a branch,
// makes the compiler wait for it at once): an invalid row reads row 0 and gets scale 0.
__device__ __forceinline__ void sketch_load(const uint32_t* codes, const uint16_t* alpha,
                                            bool valid, int H, int lane, SketchPiece& p) {
  const uint32_t* a32 = reinterpret_cast<const uint32_t*>(alpha);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = lane + kWave * h;
    const int qq = min(q, H / 32 - 1);
    p.w[h] = reinterpret_cast<const uint2*>(codes)[qq];
    const uint32_t a2 = a32[qq >> 3];
    p.a[h] = (valid && q < H / 32) ? (a2 >> (16 * ((qq >> 2) & 1))) & 0xFFFFu : 0u;
  }
}
__device__ __forceinline__ float sketch_dot(const SketchPiece& p, const float* zs, int H,
                                            int lane) {
  float part = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = lane + kWave * h;
    if (q < H / 32) {
      const f32x4* zp = reinterpret_cast<const f32x4*>(zs + 32 * q);
      float acc = 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const f32x4 z = zp[u];
        const uint32_t w = (u >> 2) ? p.w[h].y : p.w[h].x;
        const int sh = 8 * (u & 3);  // codes of coordinates 4u .. 4u + 3 of this q
        // a 2-bit field sign-extended: 00 -> 0, 01 -> +1, 11 -> -1
        acc = fmaf((float)((int)(w << (30 - sh)) >> 30), z.x, acc);
        acc = fmaf((float)((int)(w << (28 - sh)) >> 30), z.y, acc);
        acc = fmaf((float)((int)(w << (26 - sh)) >> 30), z.z, acc);
        acc = fmaf((float)((int)(w << (24 - sh)) >> 30), z.w, acc);
      }
      part = fmaf(__half2float(__ushort_as_half((uint16_t)p.a[h])), acc, part);
    }
  }
  return part;
}

template <DT ET, DT ST, DT RT, int C, int CPT, bool SK>
__global__ __launch_bounds__(1024) void cs_kernel(CSLaunch L) {
  const B1Args& a = L.a;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = blockDim.x;
  set_teams(c, L.tsz);
  c.lane = c.tid & (kWave - 1);
  c.P = gridDim.x;
  c.wg = blockIdx.x;
  c.H = a.H;
  c.nch = a.H / 8;
  c.red = reinterpret_cast<float*>(smem);
  c.red_stride = (c.nthreads / kWave) * kMaxNP;
  c.parity = 0;
  c.zrow = a.zrow;
  c.stamps = a.stamps;
  MOE_STAMP(c.stamps, kStampStart);
  MOE_CLOCK(c.stamps, kStampClk0);
  const int I = a.I, k = a.k;
  const int n = k * I;                                 // <= kCh * nthreads (host checks)
  const DivI divI(I);
  int* s_int = reinterpret_cast<int*>(c.red + 2 * c.red_stride);  // [16]
  int* s_ids = s_int + 16;                                          // [64]
  float* s_w = reinterpret_cast<float*>(s_ids + 64);                // [64]
  int* sh = reinterpret_cast<int*>(s_w + 64);                       // [96]
  int* slot_gt = sh + 96;                                           // [kMaxSlots + 1]
  int* slot_eq = slot_gt + kSlotPad;                                // [kMaxSlots + 1]
  int* hist = slot_eq + kSlotPad;                                   // [kSelBins]
  uint32_t* mem = reinterpret_cast<uint32_t*>(hist + kSelBins);     // [kSelCand]
  float* own_g = reinterpret_cast<float*>(mem + kSelCand);          // [kOwnMax] gate values
  uint32_t* own_s = reinterpret_cast<uint32_t*>(own_g + kOwnMax);   // [kOwnMax] score patterns
  float* own_dn = reinterpret_cast<float*>(own_s + kOwnMax);        // [kOwnMax] ||d_j||
  int* own_keep = reinterpret_cast<int*>(own_dn + kOwnMax);         // [kOwnMax] kept flags
  int* klist = own_keep + kOwnMax;                                  // [kOwnMax] kept, in order
  float* est = reinterpret_cast<float*>(klist + kOwnMax);           // [2 kOwnMax] sketch
  uint32_t* sv = reinterpret_cast<uint32_t*>(est + 2 * kOwnMax);    // [n] score patterns
  float* zs = reinterpret_cast<float*>(sv + ((n + 3) & ~3));        // [H] scanned R x
  float* big = zs + a.H;
  Ctrl* ctrl = a.ctrl;
  // channel-selection launches on this workspace so far: its scores carry the parity
  const uint32_t cs_ep = load_relaxed_dev(&ctrl->cs_epoch);
  const uint32_t gpar = (cs_ep + 1u) & 1u;
  const float t_prev = __uint_as_float(load_relaxed_dev(&ctrl->cs_tprev));
  // the scores, one copy per XCD (npad words each); this workgroup polls copy wg % 8
  const int npad = (n + 63) & ~63;
  uint32_t* scores = reinterpret_cast<uint32_t*>(L.g_ws);

  float xv[CPT * 8], yv[CPT * 8];
  load_x<8, CPT>(a.x, c, xv);
#pragma unroll
  for (int i = 0; i < CPT * 8; ++i) yv[i] = 0.0f;
  read_epoch(ctrl, c);

  // 1. router rows, then the routing; the shared-expert rows are warmed meanwhile
  RouterRound<RT, CPT> rr;
  router_issue<RT, CPT>(a.route_inside, a.router, a.E, c, rr);
  router_finish<RT, CPT>(rr, a.router, a.E, xv, a.rlog, big, reinterpret_cast<uint32_t*>(s_int),
                         c);
  MOE_STAMP(c.stamps, 1);
  // this workgroup's shared-expert rows are warmed into L2 by waves 1.. once every logit has
  // been read, while wave 0 finishes the top-k (earlier, the warm loads delay the polls)
  const long long nsc = (long long)a.NS * a.IS;  // flat shared channel f of [NS][IS] is row f
  const int s0 = (int)(nsc * c.wg / c.P), s1 = (int)(nsc * (c.wg + 1) / c.P);
  uint32_t warm[kWarmLoads] = {0, 0};
  auto warm_shared = [&] {
    if (a.NS > 0)
      warm_rows(reinterpret_cast<const uint8_t*>(a.sh_gate),
                reinterpret_cast<const uint8_t*>(a.sh_up),
                reinterpret_cast<const uint8_t*>(a.sh_down_t), s0, s1,
                (uint32_t)Fmt<ST>::row_bytes(a.H), kWave, c, warm);
  };
  fetch_routing(a.route_inside, a.rlog, a.ids_in, a.w_in, a.E, k, ctrl,
                reinterpret_cast<uint64_t*>(big), s_ids, s_w, a.ids_ws, a.w_ws, c, warm_shared);
  MOE_STAMP(c.stamps, 3);

  // 2. gate pass over this workgroup's own candidates [g0, g1) (flat f = slot * I + j): the
  // down-row norms and the gate rows are loaded, each score s = |silu(g)| ||d|| (times w_e)
  // is published as a 32-bit word with the launch parity in its lowest bit, and g and s stay
  // in LDS for this workgroup's own kept channels
  const int g0 = (int)((long long)n * c.wg / c.P), g1 = (int)((long long)n * (c.wg + 1) / c.P);
  const int nown = g1 - g0;
  float dnv = 0.0f;
  if (c.tid < nown) {
    const int f = g0 + c.tid, sl = divI.div(f), e = s_ids[sl];
    dnv = e >= 0 ? L.dnorm[(size_t)e * I + (f - sl * I)] : 0.0f;
  }
  auto gate_rows = [&](int base, long long (&rows)[kGateBatch]) {
#pragma unroll
    for (int q = 0; q < kGateBatch; ++q) {
      const int f = base + c.team * kGateBatch + q;
      rows[q] = -1;
      if (f < g1) {
        const int sl = divI.div(f);
        const int e = s_ids[sl];
        if (e >= 0) rows[q] = (long long)e * I + (f - sl * I);
      }
    }
  };
  auto publish = [&](int base, const float (&g)[kGateBatch]) {
    if (c.t < kGateBatch) {
      float gq = 0.0f;
#pragma unroll
      for (int q = 0; q < kGateBatch; ++q) gq = (q == c.t) ? g[q] : gq;
      const int f = base + c.team * kGateBatch + c.t;
      if (f < g1) {
        const int o = f - g0;
        const float wsl = L.mode == 1 ? s_w[divI.div(f)] : 1.0f;
        const uint32_t sp = __float_as_uint(fabsf(silu(gq)) * own_dn[o] * wsl) & ~1u;
#pragma unroll
        for (int x = 0; x < kPollCopies; ++x)
          __hip_atomic_store(scores + (size_t)x * npad + f, sp | gpar, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        own_g[o] = gq;
        own_s[o] = sp;  // the value every workgroup will see
      }
    }
  };
  if constexpr (!SK) {
    TeamRows<ET, kGateBatch, CPT> gr;
    long long rows[kGateBatch];
    gate_rows(g0, rows);
    team_dots_load<ET, kGateBatch, CPT>(a.gate, a.gate_s, rows, c, gr);
    if (c.tid < nown) own_dn[c.tid] = dnv;  // visible after the barrier of the dots below
    float g[kGateBatch];
    team_dots_compute<ET, kGateBatch, CPT>(gr, xv, c, g);
    publish(g0, g);
    for (int base = g0 + c.nteams * kGateBatch; base < g1; base += c.nteams * kGateBatch) {
      gate_rows(base, rows);
      team_dots<ET, kGateBatch, CPT>(a.gate, a.gate_s, rows, xv, c, g);
      publish(base, g);
    }
  } else {
    // the sketch screen (stage 1 of the reader): the own candidates' sketch rows of G and V
    // (one wave per row, up to four rows per wave in flight) are loaded first; x is rotated
    // and scanned meanwhile; each estimate is sum_b alpha_b sum_(scanned i) code_i z_i / 128;
    // the score is eq. 1, w_e ||d_j|| |silu(g^) v^| (without w_e in the gate-dnorm mode)
    const int nw = c.nthreads / kWave, wave = c.tid / kWave, ntask = 2 * nown;
    for (int t0 = 0; t0 < ntask; t0 += 4 * nw) {
      SketchPiece pc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int task = t0 + wave + nw * u;
        size_t row = 0;
        bool valid = false;
        if (task < ntask) {
          const int f = g0 + (task >> 1), sl = divI.div(f), e = s_ids[sl];
          valid = e >= 0;
          row = valid ? (size_t)e * I + (f - sl * I) : 0;
        }
        sketch_load(((task & 1) ? L.sk_v : L.sk_g) + row * (size_t)(a.H / 16),
                    ((task & 1) ? L.sk_av : L.sk_ag) + row * (size_t)(a.H / 128), valid, a.H,
                    c.lane, pc[u]);
      }
      if (t0 == 0) {
        if (c.tid < nown) own_dn[c.tid] = dnv;
        rotate_scan(a.x, L.signs, zs, a.H, c);
        __syncthreads();
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int task = t0 + wave + nw * u;
        const float v = wave_sum(sketch_dot(pc[u], zs, a.H, c.lane)) * (1.0f / 128.0f);
        if (task < ntask && c.lane == 0) est[task] = v;
      }
    }
    if (ntask == 0) {
      rotate_scan(a.x, L.signs, zs, a.H, c);  // (keeps the barrier count uniform)
      __syncthreads();
    }
    __syncthreads();
    if (c.tid < nown) {
      const int f = g0 + c.tid;
      const float wsl = L.mode == 1 ? s_w[divI.div(f)] : 1.0f;
      const float gh = est[2 * c.tid], vh = est[2 * c.tid + 1];
      const uint32_t sp = __float_as_uint(fabsf(silu(gh) * vh) * own_dn[c.tid] * wsl) & ~1u;
#pragma unroll
      for (int x = 0; x < kPollCopies; ++x)
        __hip_atomic_store(scores + (size_t)x * npad + f, sp | gpar, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      own_s[c.tid] = sp;
    }
  }
  __syncthreads();
  MOE_STAMP(c.stamps, 4);

  // 3. (issued after the gather below) prefetch into L2 the up and down rows of the own
  // candidates likely to be kept: scores at least 0.85 of the previous launch's threshold (a
  // hint: the keep decision does not use it).  One 4-byte load per 128-byte line; a wave per
  // candidate.
  // Up to two candidates per wave and two loads per lane and candidate (rows up to 8 KB); the
  // loaded words are kept in registers and consumed only at the end of the kernel, so no wait
  // before then covers them.
  uint32_t warm2[2][2] = {{0, 0}, {0, 0}};
  auto warm_kept = [&] {
    if (t_prev > 0.0f && L.K > 0 && L.K < n) {
      const uint32_t rb = (uint32_t)Fmt<ET>::row_bytes(a.H), lines = (rb + 127) / 128;
      const uint32_t nrow = SK ? 3u : 2u;  // (gate,) up and down rows
      const int nw = c.nthreads / kWave;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int o = c.tid / kWave + nw * u;
        if (o < nown && __uint_as_float(own_s[o]) >= 0.85f * t_prev) {
          const int f = g0 + o, sl = divI.div(f), e = s_ids[sl];
          if (e >= 0) {
            const size_t row = (size_t)e * I + (f - sl * I);
            const uint8_t* base[3] = {reinterpret_cast<const uint8_t*>(a.up) + row * rb,
                                      reinterpret_cast<const uint8_t*>(a.down_t) + row * rb,
                                      reinterpret_cast<const uint8_t*>(a.gate) + row * rb};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t l = c.lane + kWave * h;
              if (l < nrow * lines) {
                const uint32_t which = l / lines;
                warm2[u][h] = *reinterpret_cast<const uint32_t*>(
                    (which == 0 ? base[0] : which == 1 ? base[1] : base[2]) +
                    128ull * (l - which * lines));
              }
            }
          }
        }
      }
    }
  };

  // this workgroup's share of the shared experts (weight 1, warm in L2): covers the hand-off
  // of the scores
  if (a.NS > 0)
    stream_channels<ST, C, CPT, true, true>(
        a.sh_gate, a.sh_up, a.sh_down_t, nullptr, nullptr, nullptr, s0, s1,
        [](int f, long long& row, float& wt, float&) { row = f; wt = 1.0f; }, xv, yv, c);
  MOE_STAMP(c.stamps, 2);

  // 4. every score: this thread's eight as two 16-byte device-coherent loads from this XCD's
  // copy, polled again while any lacks the launch parity; the patterns to LDS (for the radix
  // fallback and the output list), the range per wave; the histogram and the selection words
  // cleared meanwhile
  const int c0 = c.tid * kCh;
  const bool mine = c0 < n;
  const int sl0 = mine ? divI.div(c0) : 0, j0 = c0 - sl0 * I;
  uint32_t sb[kCh];
  {
    const rsrc_t gsrc = make_rsrc(scores + (size_t)(c.wg % kPollCopies) * npad, (uint32_t)n * 4u);
    u32x4 w4[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w4[h] = __builtin_amdgcn_raw_buffer_load_b128(gsrc, (mine ? c0 : 0) * 4 + 16 * h, 0,
                                                     kSc1);
    auto ready = [&](const u32x4& v) {
      return ((v.x & 1u) == gpar) & ((v.y & 1u) == gpar) & ((v.z & 1u) == gpar) &
             ((v.w & 1u) == gpar);
    };
    if (mine && !(ready(w4[0]) && ready(w4[1]))) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (!(ready(w4[0]) && ready(w4[1]))) {
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          w4[h] = __builtin_amdgcn_raw_buffer_load_b128(gsrc, c0 * 4 + 16 * h, 0, kSc1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
          __hip_atomic_fetch_or(&ctrl->err, kErrPhaseWait, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    const uint32_t wr[kCh] = {w4[0].x, w4[0].y, w4[0].z, w4[0].w,
                              w4[1].x, w4[1].y, w4[1].z, w4[1].w};
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      sb[i] = mine ? wr[i] & ~1u : 0u;
      lo = mine ? min(lo, sb[i]) : lo;
      hi = mine ? max(hi, sb[i]) : hi;
    }
    MOE_STAMP_AFTER(c.stamps, 16, lo);
    if (mine) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        reinterpret_cast<u32x4*>(sv + c0)[h] = u32x4{sb[4 * h], sb[4 * h + 1], sb[4 * h + 2],
                                                     sb[4 * h + 3]};
    }
    for (int i = c.tid; i < kSelBins; i += c.nthreads) hist[i] = 0;
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (c.lane == 0) {
      sh[4 + (c.tid >> 6)] = (int)lo;
      sh[20 + (c.tid >> 6)] = (int)hi;
    }
    if (c.tid == 0) sh[44] = 0;
  }
  __syncthreads();
  MOE_STAMP(c.stamps, 5);
  warm_kept();  // its loads land in L2 during the selection, which issues no memory loads

  // 6. the threshold: T = the K-th largest score (all kept when K >= n, none when K = 0), how
  // many of the scores equal to T are kept (need) and how many there are (ties)
  uint32_t T = 0u;
  int need = 0, ties = 0;
  if (L.K > 0 && L.K < n) T = select_kth(sv, sb, mine, n, L.K, &need, &ties, hist, mem, sh, c);
  const bool all = L.K >= n, none = L.K == 0;
  MOE_STAMP(c.stamps, 6);
  // this workgroup's own kept candidates: above T, or at T when every tie is kept; when only
  // some ties are (equal scores straddling the K-th place), the lowest e*I + j of them, which
  // takes the output-order scan over all candidates
  int* slot_tk = hist;                // [k] (hist is free now)
  int* slot_base = hist + kMaxSlots;  // [k]
  if (!all && !none && need < ties) {
    int pos[kCh];
    const uint32_t m = kept_in_order(sb, mine, sl0, j0, T, need, all, none, k, a.E, s_ids, sh,
                                     slot_gt, slot_eq, slot_tk, slot_base, c, pos);
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const int f = c0 + i;
      if (mine && f >= g0 && f < g1) own_keep[f - g0] = (m >> i) & 1u;
    }
  } else if (c.tid < nown) {
    const uint32_t v = own_s[c.tid];
    own_keep[c.tid] = !none && (all || v > T || (v == T && need == ties));
  }
  __syncthreads();
  // wave 0 lists them in candidate order
  if (c.tid < kWave) {
    int nk = 0;
    for (int o0 = 0; o0 < nown; o0 += kWave) {
      const int o = o0 + c.lane;
      const bool kk = o < nown && own_keep[o];
      const uint64_t bal = __ballot(kk);
      const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (kk) klist[nk + before] = o;
      nk += __popcll(bal);
    }
    if (c.lane == 0) s_int[14] = nk;
  }
  __syncthreads();
  const int nkept = s_int[14];
  MOE_STAMP(c.stamps, 23);

  // 7. the own kept channels: up row and down row only, g from LDS
  stream_channels<ET, C, CPT, SK, false>(
      SK ? a.gate : nullptr, a.up, a.down_t, SK ? a.gate_s : nullptr, a.up_s, a.down_s, 0,
      nkept,
      [=](int i, long long& row, float& wt, float& gvv) {
        // i is wave-uniform, so are the candidate, its slot and expert: scalar arithmetic
        const int o = __builtin_amdgcn_readfirstlane(klist[i]);
        const int f = g0 + o;
        const int sl = divI.div(f);
        const int e = __builtin_amdgcn_readfirstlane(s_ids[sl]);
        if (e >= 0) {
          row = (long long)e * I + (f - sl * I);
          wt = s_w[sl];
          gvv = own_g[o];
        }
      },
      xv, yv, c);
  MOE_STAMP_AFTER(c.stamps, 7, yv[0]);
  __syncthreads();  // `big` is reused by the reduction below

  // 8. deterministic cross-workgroup sum; its first reducer also advances the count of
  // channel-selection launches
  reduce_output<CPT>(yv, a.partials, a.y, ctrl, L.R, L.SW, big, c, &ctrl->cs_epoch, cs_ep + 1u);

  // 9. workgroup 0 (not a reducer) writes the kept list after its partial output is out: every
  // kept candidate's id e*I + j at its place in ascending order (-1 for a skipped given id),
  // and the threshold as the next launch's prefetch hint
  if (c.wg == 0 && !none && L.K > 0) {
    __syncthreads();
    uint32_t sb2[kCh];
#pragma unroll
    for (int i = 0; i < kCh; ++i) sb2[i] = mine ? sv[c0 + i] : 0u;
    int pos[kCh];
    const uint32_t m = kept_in_order(sb2, mine, sl0, j0, T, need, all, none, k, a.E, s_ids, sh,
                                     slot_gt, slot_eq, slot_tk, slot_base, c, pos);
    const int e0 = mine ? s_ids[sl0] : -1;
#pragma unroll
    for (int i = 0; i < kCh; ++i)
      if ((m >> i) & 1u) L.kept_out[pos[i]] = e0 >= 0 ? e0 * I + j0 + i : -1;
    if (c.tid == 0 && !all) store_relaxed_dev(&ctrl->cs_tprev, T);
  }
  s_int[15] = (int)(warm[0] ^ warm[1] ^ warm2[0][0] ^ warm2[0][1] ^ warm2[1][0] ^
                    warm2[1][1]);  // keeps the warming loads
}

template <DT ET, DT ST, DT RT, int C, int CPT, bool SK>
hipError_t launch_t(const CSLaunch& L, int wgs, int threads, int lds, hipStream_t s,
                    int* occ) {
  auto fn = cs_kernel<ET, ST, RT, C, CPT, SK>;
  static bool lds_set = false;
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    lds_set = true;
  }
  if (occ)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, reinterpret_cast<const void*>(fn),
                                                        threads, lds);
  hipLaunchKernelGGL(fn, dim3(wgs), dim3(threads), lds, s, L);
  return hipGetLastError();
}

template <DT ET, DT ST, DT RT>
hipError_t launch_cpt(const CSLaunch& L, int wgs, int threads, int lds, hipStream_t s,
                      int* occ) {
  const int cpt = (L.a.H / 8 + L.tsz - 1) / L.tsz;
  if (cpt > 1) return hipErrorInvalidValue;
  constexpr int C = ET != DT::F32 ? 2 : 1;
  if (L.sk_g) return launch_t<ET, ST, RT, C, 1, true>(L, wgs, threads, lds, s, occ);
  return launch_t<ET, ST, RT, C, 1, false>(L, wgs, threads, lds, s, occ);
}

}  // namespace

// LDS of the channel-sparse kernel: team-reduction buffers, routing, selection words, slot
// tables, histogram, bin members, this workgroup's kept list, the gate values and score
// patterns of all k*I candidates, and the larger of the router / top-k / output scratch.
int cs_lds_bytes(int H, int threads, int E, int k, int I, int wgs, int K) {
  (void)K;
  const int nteams = threads / team_size(H);
  const int n = k * I;
  const int fixed = 2 * (threads / kWave) * kMaxNP * 4 + (16 + 64 + 64 + 96) * 4 +
                    2 * kSlotPad * 4 + kSelBins * 4 + kSelCand * 4 + 7 * kOwnMax * 4 +
                    ((n + 3) & ~3) * 4 + H * 4;
  const int ybuf = nteams * H * 4;
  const int topk = topk_lds_bytes(E, k);
  const int router = ((E + wgs - 1) / wgs) * 4;
  int big = ybuf > topk ? ybuf : topk;
  big = big > threads * 8 ? big : threads * 8;
  big = big > router ? big : router;
  return fixed + (big + 15) / 16 * 16;
}

hipError_t launch_cs(const B1Args& a, const float* dnorm, uint64_t* g_ws, int32_t* kept, int K,
                     int mode, DT et, DT st, DT rt, int wgs, int threads, hipStream_t s,
                     int* occ, const CsSketch* sketch) {
  // the selection's bin scan holds at most four bins per thread
  const long long n = (long long)a.k * a.I;
  if (a.k > kMaxSlots || n > (long long)kCh * threads || a.I % kCh != 0 ||
      threads * 4 < kSelBins || threads > 1024 || (n + wgs - 1) / wgs > kOwnMax)
    return hipErrorInvalidValue;
  CSLaunch L;
  L.a = a;
  L.dnorm = dnorm;
  L.g_ws = g_ws;
  L.kept_out = kept;
  L.K = K;
  L.mode = mode;
  L.tsz = team_size(a.H);
  L.sk_g = L.sk_v = nullptr;
  L.sk_ag = L.sk_av = nullptr;
  L.signs = nullptr;
  if (sketch) {
    if (a.H % 128 != 0 || a.H > 4096 || !sketch->g || !sketch->v || !sketch->ag ||
        !sketch->av || !sketch->signs)
      return hipErrorInvalidValue;
    L.sk_g = sketch->g;
    L.sk_v = sketch->v;
    L.sk_ag = sketch->ag;
    L.sk_av = sketch->av;
    L.signs = sketch->signs;
  }
  lc::reducer_split(a.H, wgs, &L.R, &L.SW);
  const int lds = cs_lds_bytes(a.H, threads, a.E, a.k, a.I, wgs, K);
  if (et == DT::F32 && st == DT::F32 && rt == DT::F32)
    return launch_cpt<DT::F32, DT::F32, DT::F32>(L, wgs, threads, lds, s, occ);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::BF16)
    return launch_cpt<DT::BF16, DT::BF16, DT::BF16>(L, wgs, threads, lds, s, occ);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::F32)
    return launch_cpt<DT::BF16, DT::BF16, DT::F32>(L, wgs, threads, lds, s, occ);
  return hipErrorInvalidValue;
}

}  // namespace moe

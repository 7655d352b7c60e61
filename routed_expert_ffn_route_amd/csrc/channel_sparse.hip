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
//
// With a ternary sketch of the gate and up rows ("The weights-only reader", stages 1 and 2)
// phase 2 scores from the sketch instead of the gate rows: waves 1.. rotate and scan x while
// wave 0 finishes the top-k, and each own candidate's two sketch rows give the estimates
// g^ and v^ of eq. 1.  Phase 5 then reads the gate, up and down rows of every kept channel,
// so the kept channels are shared out evenly over the workgroups rather than by owner.
#include <hip/hip_fp16.h>
#include <type_traits>

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
  // ternary sketch (null: exact gate values): codes [E*I][H/16] and FP16 scales [E*I][nbp]
  // of the gate and up rows, and the rotation's signs [H]
  const uint32_t *sk_g, *sk_v;
  const uint16_t *sk_ag, *sk_av;
  const int8_t* signs;
  uint64_t* sk_mask;   // launch-tagged scan masks, one copy per XCD (kSkMaskWords each)
  const uint16_t* rec_b;  // (reader) recovery coefficients b_j, FP16 [E*I][kRecRank]
  float* rec_r;           // (reader) this launch's per-workgroup sums r [P][kRecRank]
  uint64_t* g_ws;      // channel scores with the launch parity, one copy per XCD
  int32_t* kept_out;   // [K] ([k*I] under the threshold rule)
  int32_t* kept_count; // (threshold rule) how many were kept
  uint32_t tau;        // (threshold rule) the score threshold's bit pattern (non-negative)
  int K, mode, R, SW, tsz, thr;
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

// The token side of the sketch screen, in two steps that hide behind other waits.
// rotate_*: z = H_128 (s * x) per 128-block into zs [H] (LDS), one wave per block, lane l
// holding coordinates l and l + 64; fp32 butterflies, stages h = 1 .. 64, each pair
// (i, i + h) -> (a + b, a - b).  scan_blocks: per block only the 80 coordinates of largest |z|
// kept (ties to the lower coordinate), the others zeroed, in place.
constexpr int kScan = 80;
constexpr int kRotHeld = 2;  // blocks per wave whose x and signs are loaded ahead
struct RotIn {
  float x[kRotHeld][2];     // x at coordinates l and l + 64 of the block
  uint32_t s[kRotHeld][2];  // the sign words holding those coordinates' signs
};
// the loads for blocks wave, wave + nw (always in range: a block past the end reads the last)
__device__ inline void rotate_load(const float* x, const int8_t* signs, int H, int lane,
                                   int wave, int nw, RotIn& r) {
  const int nb = H / 128;
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(signs);
#pragma unroll
  for (int i = 0; i < kRotHeld; ++i) {
    const int b = min(wave + nw * i, nb - 1);
    r.x[i][0] = x[b * 128 + lane];
    r.x[i][1] = x[b * 128 + lane + 64];
    r.s[i][0] = s32[b * 32 + (lane >> 2)];
    r.s[i][1] = s32[b * 32 + 16 + (lane >> 2)];
  }
}
// the value of lane ^ h (the lane permutations of the top-k's xor_lane64, on 32 bits)
template <int h>
__device__ __forceinline__ float xor_lane_f32(float v) {
  const int u = __float_as_int(v);
  int r;
  if constexpr (h == 1) r = __builtin_amdgcn_mov_dpp(u, 0xB1, 0xf, 0xf, true);
  else if constexpr (h == 2) r = __builtin_amdgcn_mov_dpp(u, 0x4E, 0xf, 0xf, true);
  else if constexpr (h == 4)
    r = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(u, 0x1B, 0xf, 0xf, true), 0x141, 0xf,
                                 0xf, true);
  else if constexpr (h == 8) r = __builtin_amdgcn_mov_dpp(u, 0x128, 0xf, 0xf, true);
  else r = (int)swap_rows32<h>((uint32_t)u);
  return __int_as_float(r);
}
template <int h>
__device__ __forceinline__ void butterfly_stage(float& lo, float& hi, int lane) {
#pragma clang fp contract(off)
  const bool upper = (lane & h) != 0;
  const float plo = xor_lane_f32<h>(lo), phi = xor_lane_f32<h>(hi);
  lo = upper ? plo - lo : lo + plo;
  hi = upper ? phi - hi : hi + phi;
}
__device__ inline void rotate_block(float xlo, float xhi, uint32_t wlo, uint32_t whi, int lane,
                                    float* zb) {
#pragma clang fp contract(off)
  float lo = xlo * (float)(int8_t)(wlo >> (8 * (lane & 3)));  // s * x (exact)
  float hi = xhi * (float)(int8_t)(whi >> (8 * (lane & 3)));
  butterfly_stage<1>(lo, hi, lane);
  butterfly_stage<2>(lo, hi, lane);
  butterfly_stage<4>(lo, hi, lane);
  butterfly_stage<8>(lo, hi, lane);
  butterfly_stage<16>(lo, hi, lane);
  butterfly_stage<32>(lo, hi, lane);
  zb[lane] = lo + hi;  // stage h = 64 inside the lane
  zb[lane + 64] = lo - hi;
}
__device__ inline void rotate_compute(const RotIn& r, const float* x, const int8_t* signs,
                                      float* zs, int H, int lane, int wave, int nw) {
  const int nb = H / 128;
#pragma unroll
  for (int i = 0; i < kRotHeld; ++i) {
    const int b = wave + nw * i;
    if (b < nb) rotate_block(r.x[i][0], r.x[i][1], r.s[i][0], r.s[i][1], lane, zs + b * 128);
  }
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(signs);
  for (int b = wave + nw * kRotHeld; b < nb; b += nw)  // more blocks than loaded ahead
    rotate_block(x[b * 128 + lane], x[b * 128 + lane + 64], s32[b * 32 + (lane >> 2)],
                 s32[b * 32 + 16 + (lane >> 2)], lane, zs + b * 128);
}
// The 80th largest |z| of a block is found bit by bit from the top with ballot counts (a
// pattern with exactly 80 values at or above it already separates them, so the search stops
// there), the ties at it in coordinate order with lane counts.  Two blocks' searches run
// interleaved (`two`: the second is live).
__device__ inline void search_two(uint32_t aA0, uint32_t aA1, uint32_t aB0, uint32_t aB1,
                                  bool two, uint32_t& tA, uint32_t& tB) {
  tA = 0;  // the largest pattern with at least kScan values at or above it
  tB = 0;
  bool dA = false, dB = !two;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cA = tA | (1u << bit), cB = tB | (1u << bit);
    const int nA = __popcll(__ballot(aA0 >= cA)) + __popcll(__ballot(aA1 >= cA));
    const int nB = __popcll(__ballot(aB0 >= cB)) + __popcll(__ballot(aB1 >= cB));
    tA = !dA && nA >= kScan ? cA : tA;
    tB = !dB && nB >= kScan ? cB : tB;
    dA = dA || nA == kScan;
    dB = dB || nB == kScan;
    if (dA && dB) break;
  }
}
// which of this lane's two coordinates (l, l + 64) are kept, given the 80th largest pattern t
__device__ inline void keep_bits(uint32_t a0, uint32_t a1, uint32_t t, bool& k0, bool& k1) {
  const int need = kScan - (__popcll(__ballot(a0 > t)) + __popcll(__ballot(a1 > t)));
  const uint64_t e0 = __ballot(a0 == t), e1 = __ballot(a1 == t);
  const int r0 = __builtin_amdgcn_mbcnt_hi((uint32_t)(e0 >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)e0, 0));
  const int r1 = __popcll(e0) + __builtin_amdgcn_mbcnt_hi(
                                    (uint32_t)(e1 >> 32),
                                    __builtin_amdgcn_mbcnt_lo((uint32_t)e1, 0));
  k0 = a0 > t || (a0 == t && r0 < need);
  k1 = a1 > t || (a1 == t && r1 < need);
}
__device__ __forceinline__ uint32_t abs_bits(float z) { return __float_as_uint(z) & 0x7FFFFFFFu; }
// Block b of z, its kept coordinates given, to 24-bit fixed point in place: each kept value
// times 2^e (e[b] = 148 - the biased exponent of the largest kept |z|, so that every scaled
// value is below 2^22 in magnitude), rounded to the nearest integer; the others 0.  The
// estimates then add codes times these integers exactly (24-bit multiply-adds) and scale by
// 2^-e once per block.
__device__ inline void finish_block(float* zs, int* ebs, int b, int lane, float z0, float z1,
                                    bool k0, bool k1) {
  const float v0 = k0 ? z0 : 0.0f, v1 = k1 ? z1 : 0.0f;
  const uint32_t mb = wave_max_u32(max(abs_bits(v0), abs_bits(v1)));
  const int e = 148 - max((int)(mb >> 23), 1);
  int* zi = reinterpret_cast<int*>(zs) + b * 128;
  zi[lane] = (int)rintf(ldexpf(v0, e));
  zi[lane + 64] = (int)rintf(ldexpf(v1, e));
  if (lane == 0) ebs[b] = e;
}
// Scan and finish blocks bA and bB (bB >= nb: none; bA >= nb: nothing to do) in place.
__device__ inline void scan_finish_two(float* zs, int* ebs, int lane, int bA, int bB, int nb) {
  if (bA >= nb) return;
  const bool two = bB < nb;
  const int b2 = two ? bB : bA;
  const float zA0 = zs[bA * 128 + lane], zA1 = zs[bA * 128 + lane + 64];
  const float zB0 = zs[b2 * 128 + lane], zB1 = zs[b2 * 128 + lane + 64];
  const uint32_t aA0 = abs_bits(zA0), aA1 = abs_bits(zA1), aB0 = abs_bits(zB0), aB1 = abs_bits(zB1);
  uint32_t tA, tB;
  search_two(aA0, aA1, aB0, aB1, two, tA, tB);
  bool k0, k1;
  keep_bits(aA0, aA1, tA, k0, k1);
  finish_block(zs, ebs, bA, lane, zA0, zA1, k0, k1);
  if (two) {
    keep_bits(aB0, aB1, tB, k0, k1);
    finish_block(zs, ebs, bB, lane, zB0, zB1, k0, k1);
  }
}
// The scan of block b, computed once per launch (by workgroup b) and handed to every
// workgroup: its keep mask as four 32-bit words (coordinates 0-31, 32-63, 64-95, 96-127),
// each in a 64-bit word whose upper half is the launch tag, written to every per-XCD copy.
__device__ inline void scan_publish(const float* zs, int lane, int b, uint64_t* mask,
                                    uint32_t tag) {
  const uint32_t a0 = abs_bits(zs[b * 128 + lane]), a1 = abs_bits(zs[b * 128 + lane + 64]);
  uint32_t t, t_unused;
  search_two(a0, a1, a0, a1, false, t, t_unused);
  bool k0, k1;
  keep_bits(a0, a1, t, k0, k1);
  const uint64_t m0 = __ballot(k0), m1 = __ballot(k1);
  if (lane < 4 * kPollCopies) {
    const int word = lane & 3;
    const uint64_t m = word < 2 ? m0 : m1;
    const uint32_t v = (word & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
    st_dev64(mask + (size_t)(lane >> 2) * kSkMaskWords + 4 * b + word,
             ((uint64_t)tag << 32) | v);
  }
}
// Block b's published mask (every lane holds word lane % 4 of this workgroup's copy, `w`,
// loaded ahead; re-polled if it is not this launch's yet) and block b finished with it.
__device__ inline void consume_finish(float* zs, int* ebs, int lane, int b, uint64_t w,
                                      const uint64_t* mcopy, uint32_t tag, uint32_t* err) {
  if ((uint32_t)(w >> 32) != tag) w = wait_tagged(mcopy + 4 * b + (lane & 3), tag, err, kErrPhaseWait);
  const uint32_t mw0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)w, 0);
  const uint32_t mw1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)w, 1);
  const uint32_t mw2 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)w, 2);
  const uint32_t mw3 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)w, 3);
  const bool k0 = (((lane < 32 ? mw0 : mw1) >> (lane & 31)) & 1u) != 0;
  const bool k1 = (((lane < 32 ? mw2 : mw3) >> (lane & 31)) & 1u) != 0;
  finish_block(zs, ebs, b, lane, zs[b * 128 + lane], zs[b * 128 + lane + 64], k0, k1);
}

// Sketch staging in LDS: the codes of each task's row (task 2o + t: own candidate o, t = 0
// gate, 1 up), H/4 bytes each, then their FP16 scales, nbp (the scale row stride) each.
__host__ __device__ constexpr int sketch_nbp(int H) { return (H / 128 + 7) & ~7; }
__host__ __device__ constexpr int sketch_stage_bytes(int H, int ntask) {
  return ntask * (H / 4 + 2 * sketch_nbp(H));
}
// a * b + c on 24-bit signed a and b in one instruction (as an integer sum the compiler would
// otherwise regroup into separate multiplies and three-way adds)
__device__ __forceinline__ int mad24(int a, int b, int c) {
  int d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
// The estimates sum_b alpha_b sum_(scanned i in b) code_i z_i / 128 of G staged rows (tasks
// t0, t0 + step, ...; those past ntask are computed for task t0 and not used), in every lane:
// lane l takes coordinates [32q, 32q + 32) for q = l, l + 64 (H <= 4096), each piece of z read
// once for all G rows; z as the fixed-point integers of finish_block (zi) with their block
// exponents (ebs).
template <int G>
__device__ inline void sketch_estimates(const uint8_t* st_codes, const uint16_t* st_alpha,
                                        int nbp, int t0, int step, int ntask, const int* zi,
                                        const int* ebs, int H, int lane, float (&out)[G]) {
  const int nq = H / 32;
  // the eight 16-byte pieces of zi in an order rotated by lane: lanes 32 words apart taking
  // the same piece would all hit the same LDS banks; the codes are rotated to match
  const int rot = (lane + (lane >> 3)) & 7;
  float part[G];
#pragma unroll
  for (int g = 0; g < G; ++g) part[g] = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = lane + kWave * h;
    if (q < nq) {
      uint64_t wr[G];
      float al[G];
      int acc[G];  // |acc| < 32 * 2^22
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int t = t0 + g * step < ntask ? t0 + g * step : t0;
        const uint2 w = reinterpret_cast<const uint2*>(st_codes + (size_t)t * (H / 4))[q];
        wr[g] = __builtin_rotateright64(((uint64_t)w.y << 32) | w.x, 8 * rot);
        al[g] = __half2float(__ushort_as_half(st_alpha[t * nbp + (q >> 2)]));
        acc[g] = 0;
      }
      const i32x4* zp = reinterpret_cast<const i32x4*>(zi + 32 * q);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const i32x4 z = zp[(u + rot) & 7];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          // the codes of that piece's four coordinates; a 2-bit field sign-extended:
          // 00 -> 0, 01 -> +1, 11 -> -1
          const int b = (int)(uint32_t)(wr[g] >> (8 * u));
          acc[g] = mad24(__builtin_amdgcn_sbfe(b, 0, 2), z.x, acc[g]);
          acc[g] = mad24(__builtin_amdgcn_sbfe(b, 2, 2), z.y, acc[g]);
          acc[g] = mad24(__builtin_amdgcn_sbfe(b, 4, 2), z.z, acc[g]);
          acc[g] = mad24(__builtin_amdgcn_sbfe(b, 6, 2), z.w, acc[g]);
        }
      }
      const int e = ebs[q >> 2];
#pragma unroll
      for (int g = 0; g < G; ++g) part[g] = fmaf(al[g], ldexpf((float)acc[g], -e), part[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) out[g] = wave_sum(part[g]) * (1.0f / 128.0f);
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
  int* ebs = reinterpret_cast<int*>(est + 2 * kOwnMax);             // [32] block exponents
  uint32_t* sv = reinterpret_cast<uint32_t*>(ebs + 32);             // [n] score patterns
  float* zs = reinterpret_cast<float*>(sv + ((n + 3) & ~3));        // [H] R x, then scanned
                                                                    // (fixed point)
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
  RotIn rin;  // (sketch) x and the signs for the rotation, loaded ahead of the router rows
  if constexpr (SK) rotate_load(a.x, L.signs, a.H, c.lane, c.tid / kWave, c.nthreads / kWave, rin);
  read_epoch(ctrl, c);

  // 1. router rows, then the routing; the shared-expert rows are warmed meanwhile.  (Sketch:
  // z = R x is computed while the router rows are in flight, and scanned during the top-k.)
  RouterRound<RT, CPT> rr;
  router_issue<RT, CPT>(a.route_inside, a.router, a.E, c, rr);
  if constexpr (SK)
    rotate_compute(rin, a.x, L.signs, zs, a.H, c.lane, c.tid / kWave, c.nthreads / kWave);
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
  // (sketch) the scan of z.  With the router inside and P >= H/128 workgroups, block b is
  // scanned once per launch, by workgroup b in a wave that reads no router keys, and its mask
  // handed to every workgroup (read while the sketch rows load).  Otherwise each workgroup
  // scans every block itself in the top-k's idle moments: blocks [0, sb_pre) by the waves that
  // read no keys, two each; [sb_pre, sb_hook) by waves 1.., one each, before they warm the
  // shared rows; the rest while the sketch rows load.
  const int nbk = a.H / 128, nwv = c.nthreads / kWave;
  const int nidle = SK && a.route_inside ? max(0, nwv - (a.E + kWave - 1) / kWave) : 0;
  const bool pub = nidle >= 1 && c.P >= nbk;
  const int sb_pre = pub ? 0 : min(nbk, 2 * nidle);
  const int sb_hook = SK && a.route_inside && !pub ? min(nbk, sb_pre + nwv - 1) : 0;
  auto hooks = topk_hooks(
      [&] {
        if constexpr (SK)
          scan_finish_two(zs, ebs, c.lane, sb_pre + c.tid / kWave - 1, sb_hook, sb_hook);
        warm_shared();
      },
      [&](int i, int ni) {
        if constexpr (SK) {
          if (pub) {
            if (i == 0 && c.wg < nbk) scan_publish(zs, c.lane, c.wg, L.sk_mask, c.epoch + 1u);
          } else {
            scan_finish_two(zs, ebs, c.lane, i, i + ni, sb_pre);
          }
        }
      });
  fetch_routing(a.route_inside, a.rlog, a.ids_in, a.w_in, a.E, k, ctrl,
                reinterpret_cast<uint64_t*>(big), s_ids, s_w, a.ids_ws, a.w_ws, c, hooks);
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
    // the sketch screen (stage 1 of the reader): the sketch rows of G and V of the own
    // candidates are staged in LDS (`big`, free until the output reduction) by the whole
    // workgroup, 16 bytes a thread and load; then one wave per row forms its estimate
    // sum_b alpha_b sum_(scanned i) code_i z_i / 128; the score is eq. 1,
    // w_e ||d_j|| |silu(g^) v^| (without w_e in the gate-dnorm mode)
    const int ntask = 2 * nown, nbp = sketch_nbp(a.H);
    const int cpr = a.H / 64, ppr = cpr + nbp / 8;  // 16-byte pieces per row: codes, all
    const int npieces = ntask * ppr;
    uint8_t* st_codes = reinterpret_cast<uint8_t*>(big);
    uint8_t* st_alpha = st_codes + (size_t)ntask * (a.H / 4);
    const DivI divP(ppr);
    const int wave = c.tid / kWave;
    // (the published masks of this wave's blocks are requested first, one word a lane, so
    // that waiting for them does not wait for the sketch rows requested after them; the loads
    // are made in either case, from the workspace's mask words)
    const uint64_t* mcopy = L.sk_mask + (size_t)(c.wg % kPollCopies) * kSkMaskWords;
    uint64_t mw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) mw[i] = ld_dev64(mcopy + 4 * min(wave + nwv * i, nbk - 1) + (c.lane & 3));
    // every sketch-row load and LDS store unconditional (a load or store under a branch makes
    // the compiler's later waits wait for every load in flight): a piece past the end is the
    // last one again, stored twice with the same bytes; a slot without an expert reads row 0
    // and stores zeros
    const int np1 = max(npieces, 1);
    auto issue = [&](int p0, u32x4(&v)[2], bool(&ok)[2], int(&dst)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = p0 + c.tid + u * c.nthreads, pc = min(p, np1 - 1);
        const int task = divP.div(pc), piece = pc - task * ppr;
        const int f = g0 + (task >> 1), sl = divI.div(f), e = s_ids[sl];
        const size_t row = e >= 0 ? (size_t)e * I + (f - sl * I) : 0;
        const bool code = piece < cpr;
        const uint8_t* src =
            code ? reinterpret_cast<const uint8_t*>((task & 1) ? L.sk_v : L.sk_g) +
                       row * (size_t)(a.H / 4) + 16 * piece
                 : reinterpret_cast<const uint8_t*>((task & 1) ? L.sk_av : L.sk_ag) +
                       row * (size_t)(2 * nbp) + 16 * (piece - cpr);
        v[u] = *reinterpret_cast<const u32x4*>(src);
        ok[u] = e >= 0 && npieces > 0;
        dst[u] = code ? task * (a.H / 4) + 16 * piece
                      : ntask * (a.H / 4) + task * 2 * nbp + 16 * (piece - cpr);
      }
    };
    auto store = [&](const u32x4(&v)[2], const bool(&ok)[2], const int(&dst)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<u32x4*>(st_codes + dst[u]) = ok[u] ? v[u] : u32x4{0u, 0u, 0u, 0u};
    };
    u32x4 v[2];
    bool ok[2];
    int dst[2];
    issue(0, v, ok, dst);
    // (reader) the own candidates' recovery coefficients: 64 bytes each, four 16-byte pieces
    const bool rec = L.rec_b != nullptr;
    uint8_t* st_b = st_alpha + (size_t)ntask * 2 * nbp;
    u32x4 bv = u32x4{0u, 0u, 0u, 0u};
    bool bok = false;
    if (rec) {
      const int o = min(c.tid >> 2, max(nown - 1, 0));
      const int f = g0 + o, sl = divI.div(f), e = s_ids[sl];
      const size_t row = e >= 0 ? (size_t)e * I + (f - sl * I) : 0;
      bv = reinterpret_cast<const u32x4*>(L.rec_b + row * kRecRank)[c.tid & 3];
      bok = e >= 0 && (c.tid >> 2) < nown;
    }
    // the blocks of z not finished during the top-k, while the sketch rows are in flight
    if (pub) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (wave + nwv * i < nbk)
          consume_finish(zs, ebs, c.lane, wave + nwv * i, mw[i], mcopy, c.epoch + 1u, &ctrl->err);
      for (int b = wave + 2 * nwv; b < nbk; b += nwv)  // (fewer than 16 waves)
        consume_finish(zs, ebs, c.lane, b, ld_dev64(mcopy + 4 * b + (c.lane & 3)), mcopy,
                       c.epoch + 1u, &ctrl->err);
    } else {
      for (int b = sb_hook + wave; b < nbk; b += 2 * nwv)
        scan_finish_two(zs, ebs, c.lane, b, b + nwv, nbk);
    }
    store(v, ok, dst);
    if (rec && (c.tid >> 2) < nown)
      reinterpret_cast<u32x4*>(st_b)[c.tid] = bok ? bv : u32x4{0u, 0u, 0u, 0u};
    for (int p0 = 2 * c.nthreads; p0 < npieces; p0 += 2 * c.nthreads) {
      issue(p0, v, ok, dst);
      store(v, ok, dst);
    }
    if (c.tid < nown) own_dn[c.tid] = dnv;
    __syncthreads();
    // one wave per row, up to four rows of a wave at once (each piece of z read once for
    // them); the group is as large as the rows per wave, as every row in it is computed
    auto estimates = [&](auto gtag) {
      constexpr int G = decltype(gtag)::value;
      for (int t0 = wave; t0 < ntask; t0 += G * nwv) {
        float ev[G];
        sketch_estimates<G>(st_codes, reinterpret_cast<const uint16_t*>(st_alpha), nbp, t0, nwv,
                            ntask, reinterpret_cast<const int*>(zs), ebs, a.H, c.lane, ev);
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (c.lane == 0 && t0 + g * nwv < ntask) est[t0 + g * nwv] = ev[g];
      }
    };
    const int per_wave = (ntask + nwv - 1) / nwv;
    if (per_wave <= 1) estimates(std::integral_constant<int, 1>{});
    else if (per_wave == 2) estimates(std::integral_constant<int, 2>{});
    else if (per_wave == 3) estimates(std::integral_constant<int, 3>{});
    else estimates(std::integral_constant<int, 4>{});
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
  auto gather = [&] {
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
      __syncthreads();
  };
  // (threshold rule: a workgroup's own kept channels follow from its own scores, so only
  // workgroup 0 gathers them, after its partial output is out, for the kept list)
  const bool thr = L.thr != 0;
  if (!thr) {
    gather();
    MOE_STAMP(c.stamps, 5);
    warm_kept();  // its loads land in L2 during the selection, which issues no memory loads
  }

  // 6. the threshold: T = the K-th largest score (all kept when K >= n, none when K = 0), how
  // many of the scores equal to T are kept (need) and how many there are (ties); under the
  // threshold rule T = tau and every score at or above it is kept
  uint32_t T = 0u;
  int need = 0, ties = 0;
  if (thr) {
    T = L.tau;
    need = ties = n;
  } else if (L.K > 0 && L.K < n) {
    T = select_kth(sv, sb, mine, n, L.K, &need, &ties, hist, mem, sh, c);
  }
  const bool all = !thr && L.K >= n, none = !thr && L.K == 0;
  MOE_STAMP(c.stamps, 6);
  // this workgroup's own kept candidates: above T, or at T when every tie is kept; when only
  // some ties are (equal scores straddling the K-th place), the lowest e*I + j of them, which
  // takes the output-order scan over all candidates
  int* slot_tk = hist;                // [k] (hist is free now)
  int* slot_base = hist + kMaxSlots;  // [k]
  int nkept = 0;
  if constexpr (SK) {
    // with the sketch every kept channel is computed from its full rows, so any workgroup
    // can take it: the kept candidates are shared out evenly instead, workgroup w taking
    // those of ranks [N w / P, N (w + 1) / P) in candidate order (N kept in all); klist
    // holds their flat candidate indices
    uint32_t m = 0;
    if (!all && !none && need < ties) {
      int pos[kCh];
      m = kept_in_order(sb, mine, sl0, j0, T, need, all, none, k, a.E, s_ids, sh, slot_gt,
                        slot_eq, slot_tk, slot_base, c, pos);
    } else {
#pragma unroll
      for (int i = 0; i < kCh; ++i)
        if (mine && !none && (all || sb[i] > T || (sb[i] == T && need == ties))) m |= 1u << i;
    }
    int tot;
    int r = block_excl_scan(__popc(m), sh + 48, c, &tot);
    const int p0 = (int)((long long)tot * c.wg / c.P);
    const int p1 = (int)((long long)tot * (c.wg + 1) / c.P);
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      if ((m >> i) & 1u) {
        if (r >= p0 && r < p1) klist[r - p0] = c0 + i;
        ++r;
      }
    }
    nkept = p1 - p0;  // at most ceil(n / P) <= kOwnMax
    if (L.rec_b) {  // (reader) which own candidates were dropped
#pragma unroll
      for (int i = 0; i < kCh; ++i) {
        const int f = c0 + i;
        if (mine && f >= g0 && f < g1) own_keep[f - g0] = (int)((m >> i) & 1u);
      }
    }
    __syncthreads();
    if (L.rec_b && c.tid < kWave) {
      // (reader, stage 3) r = sum over the own dropped candidates of w_e b_j p_j, with p_j =
      // silu(g^_j) v^_j the screen's estimates; lane q < kRecRank holds component q
      const uint16_t* sb16 = reinterpret_cast<const uint16_t*>(
          reinterpret_cast<const uint8_t*>(big) + (size_t)(2 * nown) * (a.H / 4) +
          (size_t)(2 * nown) * 2 * sketch_nbp(a.H));
      float rq = 0.0f;
      for (int o = 0; o < nown; ++o) {
        if (own_keep[o]) continue;  // (uniform)
        const float p = silu(est[2 * o]) * est[2 * o + 1];
        const float we = s_w[divI.div(g0 + o)];
        const float bq = c.lane < kRecRank
                             ? __half2float(__ushort_as_half(sb16[o * kRecRank + c.lane]))
                             : 0.0f;
        rq = fmaf(we * p, bq, rq);
      }
      if (c.lane < kRecRank) L.rec_r[(size_t)c.wg * kRecRank + c.lane] = rq;
    }
  } else {
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
  nkept = s_int[14];
  }
  MOE_STAMP(c.stamps, 23);

  // 7. the kept channels: the own ones' up and down rows with g from LDS, or (sketch) this
  // workgroup's share's gate, up and down rows
  stream_channels<ET, C, CPT, SK, false>(
      SK ? a.gate : nullptr, a.up, a.down_t, SK ? a.gate_s : nullptr, a.up_s, a.down_s, 0,
      nkept,
      [=](int i, long long& row, float& wt, float& gvv) {
        // i is wave-uniform, so are the candidate, its slot and expert: scalar arithmetic
        const int o = __builtin_amdgcn_readfirstlane(klist[i]);
        const int f = SK ? o : g0 + o;
        const int sl = divI.div(f);
        const int e = __builtin_amdgcn_readfirstlane(s_ids[sl]);
        if (e >= 0) {
          row = (long long)e * I + (f - sl * I);
          wt = s_w[sl];
          if constexpr (!SK) gvv = own_g[o];
        }
      },
      xv, yv, c);
  MOE_STAMP_AFTER(c.stamps, 24, yv[0]);  // (7 is the reducers' all-polled stamp)
  __syncthreads();  // `big` is reused by the reduction below

  // 8. deterministic cross-workgroup sum; its first reducer also advances the count of
  // channel-selection launches
  reduce_output<CPT>(yv, a.partials, a.y, ctrl, L.R, L.SW, big, c, &ctrl->cs_epoch, cs_ep + 1u);

  // 9. workgroup 0 (not a reducer) writes the kept list after its partial output is out: every
  // kept candidate's id e*I + j at its place in ascending order (-1 for a skipped given id),
  // and the threshold as the next launch's prefetch hint
  if (c.wg == 0 && (thr || (!none && L.K > 0))) {
    __syncthreads();
    if (thr) gather();
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
    if (thr) {  // how many the threshold kept
      int tot;
      (void)block_excl_scan(__popc(m), sh + 48, c, &tot);
      if (c.tid == 0) *L.kept_count = tot;
    }
    if (c.tid == 0 && !all && !thr) store_relaxed_dev(&ctrl->cs_tprev, T);
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

// ------------------------------------------------------------------------------------
// Batch-wide channel selection (the review's "Limits": choosing the whole batch's channels at
// once is the authors' future work).  For B tokens routed independently, the candidates are
// the channels of the touched experts (candidate index t*I + j: channel j of the t-th touched
// expert, ascending expert id, so ascending e*I + j); a channel's batch score is the sum over
// the tokens routed to its expert of w_{b,e} |silu(g_j.x_b)|, times ||d_j||; the `keep` best
// are computed exactly for every token routed to their expert, each row read once for the
// batch, and the shared experts for every token.  Five launches after the routing and the
// union: scores (each gate row read once for all its tokens; the gate values kept), selection
// (one workgroup), activations (the kept up rows and the shared experts' rows), down products
// (channel chunks x column blocks, partial rows) and their sum in chunk order.
struct BselArgs {
  const float* x;                                     // [B][H]
  const int32_t* ids;                                 // [B][k]
  const float* w;                                     // [B][k]
  const int32_t *n_touched, *touched, *offsets, *slots;  // the union
  const void *gate, *up, *down_t, *sh_gate, *sh_up, *sh_down_t;
  const float* dnorm;                                 // [E*I]
  float* S;                                           // [n_t*I] batch scores
  float* G;                                           // [n_t*I][B] gate values, by slot rank
  i32x4* desc;  // [keep] per kept channel: row e*I + j, candidate, first slot, slots (-1 past)
  int32_t* kept_out;                                  // [keep] kept ids e*I + j
  int32_t* nkept;                                     // [1]
  int32_t* sel;  // [4] T's score pattern, need, K, every; then [chunks][2] above, tie counts
  float* A;                                           // [NS*IS + keep][B] activations x w
  float* part;                                        // [nchunk][B][H]
  float* y;                                           // [B][H]
  int H, I, E, k, B, NS, IS, keep, nchunk;
  int nkmax;  // min(keep, min(E, B*k)*I): descriptors written
};
constexpr int kBselMaxB = kBselMaxBatch;
constexpr int kBselChunks = kBselPartChunks;

// Eight consecutive weights of a row (BF16: one 16-byte load; F32: two), as raw words.
template <DT dt>
struct Row8 {
  u32x4 a, b;
};
template <DT dt>
__device__ __forceinline__ Row8<dt> ld_row8(const void* base, size_t e) {
  Row8<dt> r;
  if constexpr (dt == DT::BF16) {
    r.a = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + e);
    r.b = r.a;
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(base) + e);
    r.a = p[0];
    r.b = p[1];
  }
  return r;
}
// sum over the eight of weight * x
template <DT dt>
__device__ __forceinline__ float dot_row8(const Row8<dt>& r, f32x4 x0, f32x4 x1, float acc) {
  if constexpr (dt == DT::BF16) {
    acc = fmaf(__uint_as_float(r.a.x << 16), x0.x, acc);
    acc = fmaf(__uint_as_float(r.a.x & 0xFFFF0000u), x0.y, acc);
    acc = fmaf(__uint_as_float(r.a.y << 16), x0.z, acc);
    acc = fmaf(__uint_as_float(r.a.y & 0xFFFF0000u), x0.w, acc);
    acc = fmaf(__uint_as_float(r.a.z << 16), x1.x, acc);
    acc = fmaf(__uint_as_float(r.a.z & 0xFFFF0000u), x1.y, acc);
    acc = fmaf(__uint_as_float(r.a.w << 16), x1.z, acc);
    acc = fmaf(__uint_as_float(r.a.w & 0xFFFF0000u), x1.w, acc);
  } else {
    acc = fmaf(__uint_as_float(r.a.x), x0.x, acc);
    acc = fmaf(__uint_as_float(r.a.y), x0.y, acc);
    acc = fmaf(__uint_as_float(r.a.z), x0.z, acc);
    acc = fmaf(__uint_as_float(r.a.w), x0.w, acc);
    acc = fmaf(__uint_as_float(r.b.x), x1.x, acc);
    acc = fmaf(__uint_as_float(r.b.y), x1.y, acc);
    acc = fmaf(__uint_as_float(r.b.z), x1.z, acc);
    acc = fmaf(__uint_as_float(r.b.w), x1.w, acc);
  }
  return acc;
}
// Chunks of eight per lane per pass over a row (registers of NR rows in flight).
template <DT dt>
constexpr int bsel_cpl() { return dt == DT::BF16 ? 4 : 2; }

// Dots of NR rows (row r: element offset ro[r] in tensor w[r]) with up to four tokens' x (xb[i],
// nt of them), over H: acc[r][i], summed over the wave (every lane).  Each lane takes chunks
// of eight, CPL per pass, rows loaded once per pass for all tokens.
template <DT dt, int NR>
__device__ __forceinline__ void bsel_dots(const void* const (&w)[NR], const size_t (&ro)[NR],
                                          const float* const (&xb)[4], int nt, int H, int lane,
                                          float (&acc)[NR][4]) {
  constexpr int CPL = bsel_cpl<dt>();
  const int nch = H / 8;
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += kWave * CPL) {
    Row8<dt> rv[NR][CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int ch = min(c0 + kWave * q + lane, nch - 1);
#pragma unroll
      for (int r = 0; r < NR; ++r) rv[r][q] = ld_row8<dt>(w[r], ro[r] + 8 * (size_t)ch);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nt) {
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int chr = c0 + kWave * q + lane;
          const int ch = min(chr, nch - 1);
          f32x4 x0 = reinterpret_cast<const f32x4*>(xb[i])[2 * ch];
          f32x4 x1 = reinterpret_cast<const f32x4*>(xb[i])[2 * ch + 1];
          if (chr >= nch) x0 = x1 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int r = 0; r < NR; ++r) acc[r][i] = dot_row8<dt>(rv[r][q], x0, x1, acc[r][i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < nt) {
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r][i] = wave_sum(acc[r][i]);
    }
}

// Scores: workgroup = 4 waves x 4 consecutive channels of one touched expert; each gate row is
// read once for all the expert's tokens (groups of four).  S[c] = ||d_j|| sum w |silu(g)|;
// G[c][r] = g for the expert's r-th slot (slot order of the union).
constexpr int kBselScoreRows = 16;  // channels per workgroup
template <DT ET>
__global__ __launch_bounds__(256) void bsel_score_kernel(BselArgs a) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nblk = (a.I + kBselScoreRows - 1) / kBselScoreRows;
  const int t = blockIdx.x / nblk, blk = blockIdx.x - t * nblk;
  if (t >= *a.n_touched) return;  // whole workgroups
  const int e = a.touched[t];
  const int s0 = a.offsets[e], ne = a.offsets[e + 1] - s0;
  const int j0 = blk * kBselScoreRows + wave * 4;
  size_t ro[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) ro[r] = ((size_t)e * a.I + min(j0 + r, a.I - 1)) * a.H;
  float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int tg = 0; tg < ne; tg += 4) {
    const int nt = min(4, ne - tg);
    int slot[4];
    const float* xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      slot[i] = a.slots[s0 + tg + min(i, nt - 1)];
      xb[i] = a.x + (size_t)(slot[i] / a.k) * a.H;
    }
    float acc[4][4];
    const void* const wr[4] = {a.gate, a.gate, a.gate, a.gate};
    bsel_dots<ET, 4>(wr, ro, xb, nt, a.H, lane, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nt) {
        const float wi = a.w[slot[i]];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[r] = fmaf(wi, fabsf(silu(acc[r][i])), sc[r]);
          if (lane == r && j0 + r < a.I)
            a.G[((size_t)t * a.I + j0 + r) * a.B + tg + i] = acc[r][i];
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (lane == r && j0 + r < a.I)
      a.S[(size_t)t * a.I + j0 + r] = sc[r] * a.dnorm[(size_t)e * a.I + j0 + r];
}

// One wave (every lane): over nb LDS bins (nb = 64 times a power of two; lane l sums the nb/64
// bins [nb - seg (l + 1), nb - seg l), counted from the top), the bin where the count from the
// top reaches Kp (0 < Kp <= the total) and Kp minus the count above that bin.
__device__ __forceinline__ void wave_find_digit(const int* hist, int nb, int Kp, int lane,
                                                int* bin, int* rem) {
  const int seg = nb / kWave;
  const int top = nb - seg * (lane + 1);
  int cnt = 0;
  for (int q = 0; q < seg; ++q) cnt += hist[top + ((q + lane) & (seg - 1))];  // rotated reads
  const int incl = wave_incl_scan(cnt);
  const int excl = incl - cnt;
  const uint64_t bal = __ballot(excl < Kp && Kp <= incl);
  const int L = (int)__builtin_ctzll(bal);
  const int before = __builtin_amdgcn_readlane(excl, L);
  const int b = nb - seg * L - 1 - lane;
  const int hv = lane < seg ? hist[b] : 0;
  const int incl2 = wave_incl_scan(hv) + before;
  const int excl2 = incl2 - hv;
  const uint64_t bal2 = __ballot(lane < seg && excl2 < Kp && Kp <= incl2);
  const int L2 = (int)__builtin_ctzll(bal2);
  *bin = nb - seg * L - 1 - L2;
  *rem = Kp - __builtin_amdgcn_readlane(excl2, L2);
}

// One workgroup: K = min(keep, m) kept and T the K-th largest batch score.  Thread t holds
// the scores of candidates [NV t, NV t + NV) in registers, as offsets o = pattern - lo (lo,
// hi: the smallest and largest pattern).  The offset of T is found digit by digit: the first
// digit is o >> s1, s1 the smallest shift with (hi - lo) >> s1 < 2048 (the scores spread over
// at least 1024 bins); each later digit holds the next (up to) 11 bits; each digit comes from
// an LDS histogram of the offsets that match the digits found so far, and the rank left after
// the last digit is how many of the values equal to T are kept.  The kept list itself is
// written by bsel_count_kernel and bsel_write_kernel over many workgroups: one workgroup
// walking every candidate again to compact them took longer than finding T.
constexpr uint32_t kNoScore = 0xFFFFFFFFu;
template <int NV>
__global__ __launch_bounds__(1024) void bsel_select_kernel(BselArgs a) {
  static_assert(NV % 4 == 0, "scores are loaded four at a time");
  constexpr int kT = 1024, kNW = kT / kWave;
  __shared__ int hist[2048];
  __shared__ int sh[96];
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = kT;
  c.lane = c.tid & (kWave - 1);
  const int wave = c.tid / kWave;
  const int nt = *a.n_touched;
  const int m = nt * a.I;  // a multiple of 8
  const int K = min(a.keep, m);
  const bool every = K >= m;
  const int f0 = c.tid * NV;
  uint32_t v[NV];
  {
    const u32x4* u4 = reinterpret_cast<const u32x4*>(a.S);  // non-negative: patterns order
#pragma unroll
    for (int q = 0; q < NV / 4; ++q) {
      const u32x4 x = u4[min(f0 / 4 + q, m / 4 - 1)];
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)  // past m: a pattern no score has (a negative NaN)
      if (f0 + i >= m) v[i] = kNoScore;
  }
  // the scores' range; each value becomes its offset from the smallest (past m: above span)
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    lo = min(lo, v[i]);
    hi = max(hi, v[i] != kNoScore ? v[i] : 0u);
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (c.lane == 0) {
    sh[4 + wave] = (int)lo;
    sh[20 + wave] = (int)hi;
  }
  __syncthreads();
  lo = c.lane < kNW ? (uint32_t)sh[4 + c.lane] : 0xFFFFFFFFu;
  hi = c.lane < kNW ? (uint32_t)sh[20 + c.lane] : 0u;
  lo = __builtin_amdgcn_readfirstlane(wave_min_u32(lo));
  hi = __builtin_amdgcn_readfirstlane(wave_max_u32(hi));
  const uint32_t span = hi - lo;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] -= lo;
  // (a score is finite and non-negative, so lo <= 0x7FC00000 and a missing value's offset,
  // at least 0x803FFFFF, exceeds span; shifted right by at most 21 it still exceeds it)
  uint32_t To = 0;  // the offset of T
  int need = 0;
  if (K > 0 && !every) {
    int shift = 0;
    while (shift < 32 && (span >> shift) >= 2048u) ++shift;
    // the first digit: offsets >> shift (below 2048)
    for (int i = c.tid; i < 2048; i += kT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (v[i] <= span) atomicAdd(&hist[v[i] >> shift], 1);
    // P: the offset of T shifted right by `prev` (the digits found so far)
    uint32_t P = 0;
    int prev = shift;
    int rem = K;
    for (;;) {
      __syncthreads();
      if (c.tid < kWave) {
        int d, r;
        wave_find_digit(hist, 2048, rem, c.lane, &d, &r);
        if (c.lane == 0) {
          sh[0] = d;
          sh[1] = r;
        }
      }
      __syncthreads();
      P += (uint32_t)sh[0];
      rem = sh[1];
      if (prev == 0) break;
      // the next digit: bits [shift, prev) of the offsets whose bits from prev up are P's
      shift = prev > 11 ? prev - 11 : 0;
      const uint32_t base = P << (prev - shift);
      for (int i = c.tid; i < 2048; i += kT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if ((v[i] >> prev) == P) atomicAdd(&hist[(v[i] >> shift) - base], 1);
      P = base;
      prev = shift;
    }
    To = P;
    need = rem;
  }
  // the threshold for the kept-list kernels: T's score pattern, how many scores equal to T
  // are kept, K, and whether every candidate is
  if (c.tid == 0) {
    a.sel[0] = (int32_t)(To + lo);
    a.sel[1] = need;
    a.sel[2] = K;
    a.sel[3] = every ? 1 : 0;
  }
  for (int i = K + c.tid; i < a.keep; i += kT) {
    a.kept_out[i] = -1;
    a.desc[i] = i32x4{-1, -1, 0, 0};
  }
  if (c.tid == 0) *a.nkept = K;
}

// The kept list in candidate order (ties to the lower candidate), over chunks of
// kBselChunkCand candidates, one workgroup of 256 threads (four candidates each) per chunk.
// bsel_count_kernel: how many of the chunk's candidates are above T and how many equal it.
__global__ __launch_bounds__(256) void bsel_count_kernel(BselArgs a) {
  __shared__ int sh[2][8];
  const int m = *a.n_touched * a.I;  // a multiple of 8
  const uint32_t T = (uint32_t)a.sel[0];
  const int K = a.sel[2];
  const bool every = a.sel[3] != 0;
  const int f0 = blockIdx.x * kBselChunkCand + threadIdx.x * 4;
  int above = 0, tie = 0;
  if (K > 0 && f0 < m) {
    const u32x4 v = reinterpret_cast<const u32x4*>(a.S)[f0 / 4];
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      above += every || p[q] > T ? 1 : 0;
      tie += !every && p[q] == T ? 1 : 0;
    }
  }
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = blockDim.x;
  c.lane = c.tid & (kWave - 1);
  int na, nq;
  (void)block_excl_scan(above, sh[0], c, &na);
  (void)block_excl_scan(tie, sh[1], c, &nq);
  if (c.tid == 0) {
    a.sel[4 + 2 * blockIdx.x] = na;
    a.sel[5 + 2 * blockIdx.x] = nq;
  }
}

// bsel_write_kernel: the counts of the chunks before this one give its first places; within
// the chunk, block scans give each thread's; a kept candidate's place is (kept above T
// before it) + min(equal to T before it, need), and it is kept when above T or one of the
// first `need` equal to T.  It writes the id e*I + j and the descriptor (row, candidate, first
// slot, slots) of each kept candidate.
__global__ __launch_bounds__(256) void bsel_write_kernel(BselArgs a) {
  __shared__ int sh[2][8];
  const int m = *a.n_touched * a.I;
  const uint32_t T = (uint32_t)a.sel[0];
  const int need = a.sel[1], K = a.sel[2];
  const bool every = a.sel[3] != 0;
  if (K <= 0 || blockIdx.x * kBselChunkCand >= m) return;  // (uniform)
  Ctx c;
  c.tid = threadIdx.x;
  c.nthreads = blockDim.x;
  c.lane = c.tid & (kWave - 1);
  int ba = 0, bt = 0;
  for (int i = c.tid; i < (int)blockIdx.x; i += c.nthreads) {
    ba += a.sel[4 + 2 * i];
    bt += a.sel[5 + 2 * i];
  }
  int tot;
  ba = block_excl_scan(ba, sh[0], c, &tot);
  ba = tot;
  bt = block_excl_scan(bt, sh[1], c, &tot);
  bt = tot;
  const int f0 = blockIdx.x * kBselChunkCand + c.tid * 4;
  bool up[4] = {false, false, false, false}, eq[4] = {false, false, false, false};
  if (f0 < m) {
    const u32x4 v = reinterpret_cast<const u32x4*>(a.S)[f0 / 4];
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      up[q] = every || p[q] > T;
      eq[q] = !every && p[q] == T;
    }
  }
  int gb = block_excl_scan((int)up[0] + up[1] + up[2] + up[3], sh[0], c, &tot) + ba;
  int eb = block_excl_scan((int)eq[0] + eq[1] + eq[2] + eq[3], sh[1], c, &tot) + bt;
  if (f0 < m) {
    int t = f0 / a.I, j = f0 - t * a.I;
    int e = a.touched[t], s0 = a.offsets[e], ne = a.offsets[e + 1] - s0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (up[q] || (eq[q] && eb < need)) {
        const int pos = gb + min(eb, need);
        a.kept_out[pos] = e * a.I + j;
        a.desc[pos] = i32x4{e * a.I + j, f0 + q, s0, ne};
      }
      gb += up[q] ? 1 : 0;
      eb += eq[q] ? 1 : 0;
      if (++j == a.I && q < 3) {  // (I is a multiple of 8: f0 + q + 1 < m)
        j = 0;
        ++t;
        e = a.touched[t];
        s0 = a.offsets[e];
        ne = a.offsets[e + 1] - s0;
      }
    }
  }
}

// One wave per channel: the shared experts' channels first (gate and up rows, every token;
// these waves depend on nothing else and are the longest), then the kept routed channels (from
// their descriptors: the up row, the gate values kept by the scores; waves past the kept
// count exit).  Channel c (shared: c < NS*IS; kept: NS*IS + its rank) ends with lane b < B
// holding w_{b,e} silu(g.x_b) (v.x_b) (0 for a token not routed to the channel's expert) and
// writing A[c][b].
template <DT ET, DT ST>
__global__ __launch_bounds__(256) void bsel_act_kernel(BselArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int ch = blockIdx.x * 4 + threadIdx.x / kWave;
  const int NSI = a.NS * a.IS;
  float val = 0.0f;
  if (ch < NSI) {
    const size_t ro[2] = {(size_t)ch * a.H, (size_t)ch * a.H};
    const void* const wr[2] = {a.sh_gate, a.sh_up};
    for (int tg = 0; tg < a.B; tg += 4) {
      const int nt = min(4, a.B - tg);
      const float* xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xb[i] = a.x + (size_t)(tg + min(i, nt - 1)) * a.H;
      float gv[2][4];
      bsel_dots<ST, 2>(wr, ro, xb, nt, a.H, lane, gv);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nt && lane == tg + i) val = silu(gv[0][i]) * gv[1][i];
    }
  } else {
    // past the descriptors written (the grid's last workgroup), or past the kept count
    if (ch - NSI >= a.nkmax) return;  // whole waves
    const i32x4 d = a.desc[ch - NSI];
    if (d.x < 0) return;
    const int f = d.y, s0 = d.z, ne = d.w;
    const size_t ro[1] = {(size_t)d.x * a.H};
    const void* const wr[1] = {a.up};
    for (int tg = 0; tg < ne; tg += 4) {
      const int nt = min(4, ne - tg);
      int slot[4];
      const float* xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        slot[i] = a.slots[s0 + tg + min(i, nt - 1)];
        xb[i] = a.x + (size_t)(slot[i] / a.k) * a.H;
      }
      float acc[1][4];
      bsel_dots<ET, 1>(wr, ro, xb, nt, a.H, lane, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nt && lane == slot[i] / a.k) {
          const float g = a.G[(size_t)f * a.B + tg + i];
          val = a.w[slot[i]] * silu(g) * acc[0][i];
        }
      }
    }
  }
  if (lane < a.B) a.A[(size_t)ch * a.B + lane] = val;
}

// Down products: workgroup = 16 waves over one column block of 256 (lane: four consecutive
// columns) and channel chunk q of kBselChunks (channels in A's order: the shared ones, then the
// kept ones); wave w takes the w-th sixteenth of the chunk (in order), its A rows and row
// offsets staged in LDS by the workgroup; tokens in blocks of eight; the 16 waves' sums are
// added in wave order through LDS, every wave adding its share of the outputs.
// part[q][b][h] = that chunk's sum of A[c][b] d_c[h].
constexpr int kBselDownWaves = 16;
constexpr int kBselStage = 256;   // channels staged at a time
constexpr int kBselTB = 8;        // tokens per block
constexpr int kBselDownU = 8;     // rows in flight per lane
template <DT dt>
__device__ __forceinline__ f32x4 ld4(const void* base, size_t e) {
  if constexpr (dt == DT::BF16) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(base) + e);
    return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                 __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
  } else {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + e);
  }
}
template <DT ET, DT ST>
__global__ __launch_bounds__(1024) void bsel_down_kernel(BselArgs a) {
  __shared__ float As[kBselStage * kBselMaxB];
  __shared__ uint64_t rows[kBselStage];
  __shared__ f32x4 red[kBselDownWaves * kBselTB * kWave];  // [wave][token][lane]
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int h0 = (blockIdx.x * kWave + lane) * 4;
  const int hh = min(h0, a.H - 4);
  const int q = blockIdx.y;
  const int NSI = a.NS * a.IS;
  const int C = NSI + *a.nkept;
  const int c0 = (int)((long long)C * q / a.nchunk), c1 = (int)((long long)C * (q + 1) / a.nchunk);
  constexpr uint64_t kShared = (uint64_t)1 << 62;  // marks a shared expert's row
  for (int tb = 0; tb < a.B; tb += kBselTB) {
    const int nb = min(kBselTB, a.B - tb);
    f32x4 acc[kBselTB];
#pragma unroll
    for (int b = 0; b < kBselTB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int base = c0; base < c1; base += kBselStage) {
      const int nc = min(kBselStage, c1 - base);
      __syncthreads();
      for (int i = threadIdx.x; i < nc * a.B; i += blockDim.x) As[i] = a.A[(size_t)base * a.B + i];
      for (int i = threadIdx.x; i < nc; i += blockDim.x) {
        const int c = base + i;
        rows[i] = c < NSI ? ((uint64_t)c * a.H) | kShared
                          : (uint64_t)a.kept_out[c - NSI] * a.H;
      }
      __syncthreads();
      const int i0 = nc * wave / kBselDownWaves, i1 = nc * (wave + 1) / kBselDownWaves;
      for (int i = i0; i < i1; i += kBselDownU) {
        f32x4 d[kBselDownU];
#pragma unroll
        for (int u = 0; u < kBselDownU; ++u) {
          const uint64_t r = rows[min(i + u, i1 - 1)];
          d[u] = (r & kShared) ? ld4<ST>(a.sh_down_t, (r & (kShared - 1)) + hh)
                               : ld4<ET>(a.down_t, r + hh);
        }
#pragma unroll
        for (int u = 0; u < kBselDownU; ++u) {
          if (i + u < i1) {
#pragma unroll
            for (int b = 0; b < kBselTB; ++b) {
              if (b < nb) {
                const float av = As[(i + u) * a.B + tb + b];
                acc[b].x = fmaf(av, d[u].x, acc[b].x);
                acc[b].y = fmaf(av, d[u].y, acc[b].y);
                acc[b].z = fmaf(av, d[u].z, acc[b].z);
                acc[b].w = fmaf(av, d[u].w, acc[b].w);
              }
            }
          }
        }
      }
    }
    // the waves' sums in wave order: every wave writes its sums, then wave w adds, for token
    // w % 8 and lanes of half w / 8, the 16 partials
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kBselTB; ++b) red[(wave * kBselTB + b) * kWave + lane] = acc[b];
    __syncthreads();
    {
      const int b = wave % kBselTB, l0 = (wave / kBselTB) * (kWave / 2);
      if (lane < kWave / 2 && b < nb) {
        const int l = l0 + lane;
        f32x4 s4 = red[b * kWave + l];
#pragma unroll
        for (int w2 = 1; w2 < kBselDownWaves; ++w2) {
          const f32x4 o = red[(w2 * kBselTB + b) * kWave + l];
          s4.x += o.x;
          s4.y += o.y;
          s4.z += o.z;
          s4.w += o.w;
        }
        const int hcol = (blockIdx.x * kWave + l) * 4;
        if (hcol < a.H)
          *reinterpret_cast<f32x4*>(a.part + ((size_t)q * a.B + tb + b) * a.H + hcol) = s4;
      }
    }
  }
}

// y = the sum over the chunks, in chunk order (one element per thread, the loads in flight
// together).
__global__ __launch_bounds__(256) void bsel_sum_kernel(BselArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)a.B * a.H;
  if (i >= n) return;
  float v[kBselChunks];
#pragma unroll
  for (int q = 0; q < kBselChunks; ++q) v[q] = a.part[(size_t)q * n + i];
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kBselChunks; ++q) s += v[q];
  a.y[i] = s;
}

template <DT ET, DT ST>
hipError_t launch_bsel_t(const BselArgs& a, int maxcand, hipStream_t s) {
  const int nblk = (a.I + kBselScoreRows - 1) / kBselScoreRows;
  const int maxt = maxcand / a.I;
  hipLaunchKernelGGL(bsel_score_kernel<ET>, dim3(maxt * nblk), dim3(256), 0, s, a);
  const int nv = (maxcand + 1023) / 1024;
  if (nv <= 8)
    hipLaunchKernelGGL(bsel_select_kernel<8>, dim3(1), dim3(1024), 0, s, a);
  else if (nv <= 24)
    hipLaunchKernelGGL(bsel_select_kernel<24>, dim3(1), dim3(1024), 0, s, a);
  else if (nv <= 48)
    hipLaunchKernelGGL(bsel_select_kernel<48>, dim3(1), dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL(bsel_select_kernel<96>, dim3(1), dim3(1024), 0, s, a);
  const int nchunks = (maxcand + kBselChunkCand - 1) / kBselChunkCand;
  hipLaunchKernelGGL(bsel_count_kernel, dim3(nchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(bsel_write_kernel, dim3(nchunks), dim3(256), 0, s, a);
  const int cmax = a.NS * a.IS + min(a.keep, maxcand);
  if (cmax > 0)
    hipLaunchKernelGGL((bsel_act_kernel<ET, ST>), dim3((cmax + 3) / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL((bsel_down_kernel<ET, ST>), dim3((a.H + 255) / 256, a.nchunk),
                     dim3(kBselDownWaves * kWave), 0, s, a);
  hipLaunchKernelGGL(bsel_sum_kernel, dim3((a.B * a.H + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bsel(const BselLaunch& L, DT et, DT st, hipStream_t s) {
  BselArgs a;
  a.x = L.x; a.ids = L.ids; a.w = L.w;
  a.n_touched = L.n_touched; a.touched = L.touched; a.offsets = L.offsets; a.slots = L.slots;
  a.gate = L.gate; a.up = L.up; a.down_t = L.down_t;
  a.sh_gate = L.sh_gate; a.sh_up = L.sh_up; a.sh_down_t = L.sh_down_t;
  a.dnorm = L.dnorm; a.S = L.S; a.G = L.G; a.desc = reinterpret_cast<i32x4*>(L.desc); a.kept_out = L.kept_out; a.nkept = L.nkept;
  a.sel = L.sel;
  a.A = L.A; a.part = L.part; a.y = L.y;
  a.H = L.H; a.I = L.I; a.E = L.E; a.k = L.k; a.B = L.B; a.NS = L.NS; a.IS = L.IS;
  a.keep = L.keep; a.nchunk = kBselChunks;
  if (a.B < 1 || a.B > kBselMaxB || a.H % 8 != 0 || a.H < 8 || a.keep < 0)
    return hipErrorInvalidValue;
  const int maxcand = min(a.E, a.B * a.k) * a.I;
  if (maxcand > kBselMaxCandidates || a.keep > maxcand) return hipErrorInvalidValue;
  a.nkmax = min(a.keep, maxcand);
  if (et == DT::BF16 && st == DT::BF16) return launch_bsel_t<DT::BF16, DT::BF16>(a, maxcand, s);
  if (et == DT::BF16 && st == DT::F32) return launch_bsel_t<DT::BF16, DT::F32>(a, maxcand, s);
  if (et == DT::F32 && st == DT::F32) return launch_bsel_t<DT::F32, DT::F32>(a, maxcand, s);
  if (et == DT::F32 && st == DT::BF16) return launch_bsel_t<DT::F32, DT::BF16>(a, maxcand, s);
  return hipErrorInvalidValue;
}

// LDS of the channel-sparse kernel: team-reduction buffers, routing, selection words, slot
// tables, histogram, bin members, this workgroup's kept list, the gate values and score
// patterns of all k*I candidates, and the larger of the router / top-k / output scratch.
int cs_lds_bytes(int H, int threads, int E, int k, int I, int wgs, int K, bool sketch) {
  (void)K;
  const int nteams = threads / team_size(H);
  const int n = k * I;
  const int fixed = 2 * (threads / kWave) * kMaxNP * 4 + (16 + 64 + 64 + 96) * 4 +
                    2 * kSlotPad * 4 + kSelBins * 4 + kSelCand * 4 + 7 * kOwnMax * 4 + 32 * 4 +
                    ((n + 3) & ~3) * 4 + H * 4;
  const int ybuf = nteams * H * 4;
  const int topk = topk_lds_bytes(E, k);
  const int router = ((E + wgs - 1) / wgs) * 4;
  int big = ybuf > topk ? ybuf : topk;
  big = big > threads * 8 ? big : threads * 8;
  big = big > router ? big : router;
  // (sketch) the own candidates' sketch rows staged
  const int stage = sketch ? sketch_stage_bytes(H, 2 * ((n + wgs - 1) / wgs)) +
                                 ((n + wgs - 1) / wgs) * kRecRank * 2
                           : 0;
  big = big > stage ? big : stage;
  return fixed + (big + 15) / 16 * 16;
}

hipError_t launch_cs(const B1Args& a, const float* dnorm, uint64_t* g_ws, int32_t* kept, int K,
                     int mode, DT et, DT st, DT rt, int wgs, int threads, hipStream_t s,
                     int* occ, const CsSketch* sketch, const CsThreshold* thr) {
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
  L.thr = thr != nullptr;
  L.tau = thr ? thr->tau_bits : 0u;
  L.kept_count = thr ? thr->count : nullptr;
  if (thr && (sketch || !kept || !thr->count)) return hipErrorInvalidValue;
  L.tsz = team_size(a.H);
  L.sk_g = L.sk_v = nullptr;
  L.sk_ag = L.sk_av = nullptr;
  L.signs = nullptr;
  L.sk_mask = nullptr;
  L.rec_b = nullptr;
  L.rec_r = nullptr;
  if (sketch) {
    if (a.H % 128 != 0 || a.H > 4096 || !sketch->g || !sketch->v || !sketch->ag ||
        !sketch->av || !sketch->signs || !sketch->mask)
      return hipErrorInvalidValue;
    L.sk_g = sketch->g;
    L.sk_v = sketch->v;
    L.sk_ag = sketch->ag;
    L.sk_av = sketch->av;
    L.signs = sketch->signs;
    L.sk_mask = sketch->mask;
    L.rec_b = sketch->rec_b;
    L.rec_r = sketch->rec_r;
    if ((L.rec_b == nullptr) != (L.rec_r == nullptr)) return hipErrorInvalidValue;
  }
  lc::reducer_split(a.H, wgs, &L.R, &L.SW);
  const int lds = cs_lds_bytes(a.H, threads, a.E, a.k, a.I, wgs, K, sketch != nullptr);
  if (et == DT::F32 && st == DT::F32 && rt == DT::F32)
    return launch_cpt<DT::F32, DT::F32, DT::F32>(L, wgs, threads, lds, s, occ);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::BF16)
    return launch_cpt<DT::BF16, DT::BF16, DT::BF16>(L, wgs, threads, lds, s, occ);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::F32)
    return launch_cpt<DT::BF16, DT::BF16, DT::F32>(L, wgs, threads, lds, s, occ);
  return hipErrorInvalidValue;
}

}  // namespace moe

// expert_b1.hip -- the batch-1 layer in one persistent launch.
//
// Per token and layer the layer reads the router, the k routed experts and the shared
// experts once each, so its time is the weight bytes over the bandwidth; launching one
// small kernel per expert instead makes per-launch overhead the floor ("Mixture of
// Experts Changes the Arithmetic", section "What the Runtime Does With the Promise").
// This kernel therefore does the whole layer in one launch of one workgroup per CU:
//
//  1. router rows are spread over the first workgroups (one team of 256 threads per
//     row) and published; once all are in, every workgroup selects the top-k itself
//     (exact, on ordered 64-bit keys) with the softmax over the selected logits;
//  2. meanwhile every workgroup streams its share of the shared experts' channels,
//     which do not depend on routing;
//  3. with the routing known, every workgroup streams its contiguous share of the
//     k*I routed channels.  For a channel j it reads row j of G_e and V_e and row j of
//     D_e^T (the review of arXiv:2610.37386, "Background: channels and keep rules":
//     channel j owns those rows/columns; D is stored transposed so d_j is contiguous),
//     forms a_j = silu(g_j.x)(v_j.x) w_e and accumulates a_j d_j into registers;
//  4. each workgroup writes one partial H-vector; R fixed workgroups each sum an H/R
//     slice over all partials in a fixed order (deterministic, no float atomics).
//
// All cross-workgroup waits are on work of workgroups that never wait before producing
// it, and every wait is bounded in time (an expired wait sets an error bit).
#include "layer_common.h"

namespace moe {
namespace {

using namespace lc;

constexpr int kMaxNP = 16;
#ifndef MOE_B1_BF16_C
#define MOE_B1_BF16_C 1
#endif

struct B1Launch {
  B1Args a;
  int R;    // reducers
  int SW;   // slice width of each reducer (columns of y)
  int tsz;  // threads per team (one weight row) in 8-element chunks
  int tsz_r;  // threads per team of the routed experts' layout
  int big_floats;  // floats of the general LDS scratch (a second H-vector region follows
                   // when the routed experts use their own layout)
};

template <DT ET, DT ST, DT RT, int CR, int CS, int CPT>
__global__ __launch_bounds__(1024) void b1_kernel(B1Launch L) {
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
  int* s_int = reinterpret_cast<int*>(c.red + 2 * c.red_stride);  // [16]
  int* s_ids = s_int + 16;                                          // [64]
  float* s_w = reinterpret_cast<float*>(s_ids + 64);                // [64]
  float* big = s_w + 64;
  Ctrl* ctrl = a.ctrl;

  // router and shared experts in 8-element chunks (layout c); the routed experts in the
  // chunks of their format (layout cr: the same as c unless the chunks are wider)
  constexpr int ER = kE<ET>;
  constexpr bool kTwo = ER != 8;
  float xv[CPT * 8], yv[CPT * 8];
  load_x<8, CPT>(a.x, c, xv);
#pragma unroll
  for (int i = 0; i < CPT * 8; ++i) yv[i] = 0.0f;

  read_epoch(ctrl, c);

  // 1. router rows, spread over all workgroups (one row each at E <= P)
  RouterRound<RT, CPT> rr;
  router_issue<RT, CPT>(a.route_inside, a.router, a.E, c, rr);
  auto finish_router = [&] {
    router_finish<RT, CPT>(rr, a.router, a.E, xv, a.rlog, reinterpret_cast<float*>(big),
                           reinterpret_cast<uint32_t*>(s_int), c);
    MOE_STAMP(c.stamps, 1);
  };

  // The shared experts do not depend on routing.  With one row format for every expert they
  // are the leading slots of the routed stream below, read after the routing is known: the
  // router's loads then have the memory to themselves, and the stream has no gap between
  // shared and routed rows.  With two formats (MXFP4 routed experts, bf16 shared ones) they
  // stream before the routing, their first loads queued right behind the router rows', and
  // their output moves to LDS (ysh: nteams * H floats), freeing its registers.
  float* ysh = big + L.big_floats;
  if constexpr (kTwo) {
    if (a.NS > 0) {
      const long long nsc = (long long)a.NS * a.IS;  // flat channel f of [NS][IS] is row f
      stream_channels<ST, CS, CPT, true, true>(
          a.sh_gate, a.sh_up, a.sh_down_t, nullptr, nullptr, nullptr, (int)(nsc * c.wg / c.P),
          (int)(nsc * (c.wg + 1) / c.P),
          [](int f, long long& row, float& wt, float&) { row = f; wt = 1.0f; }, xv, yv, c,
          finish_router);
    } else {
      finish_router();
    }
    teams_to_lds<8, CPT>(yv, ysh, c);
    MOE_STAMP(c.stamps, 2);
  } else {
    finish_router();
  }

  SlotSet ss;
  ss.G = reinterpret_cast<const uint8_t*>(a.gate);
  ss.V = reinterpret_cast<const uint8_t*>(a.up);
  ss.D = reinterpret_cast<const uint8_t*>(a.down_t);
  ss.Gs = a.gate_s;
  ss.Vs = a.up_s;
  ss.Ds = a.down_s;
  ss.SG = reinterpret_cast<const uint8_t*>(a.sh_gate);
  ss.SV = reinterpret_cast<const uint8_t*>(a.sh_up);
  ss.SD = reinterpret_cast<const uint8_t*>(a.sh_down_t);
  ss.I = a.I;
  ss.IS = a.IS > 0 ? a.IS : 1;
  ss.NS = kTwo ? 0 : a.NS;
  ss.k = a.k;
  ss.s_ids = s_ids;
  ss.s_w = s_w;
  const SlotShare share = slot_share(ss, c, L.R);

  // 2. the routing (top-k of the published logits, or the given ids) in LDS.  Once every logit
  // has been read, waves 1.. warm L2 with this workgroup's shared-expert rows while wave 0
  // finishes the top-k, so the stream reads those from there and the memory's bandwidth goes
  // to the routed rows.  (Issued together with the logit polls, the 9 MB of warm loads of a
  // layer queued ahead of them and stretched the router hand-off from 0.9 to 2.3 us.)
  uint32_t warm[kWarmLoads] = {0, 0};
  auto warm_shared = [&] {
    if (!kTwo)
      warm_rows(ss.SG, ss.SV, ss.SD, share.s0, share.s1, (uint32_t)Fmt<ST>::row_bytes(a.H),
                kWave, c, warm);
  };
  fetch_routing(a.route_inside, a.rlog, a.ids_in, a.w_in, a.E, a.k, ctrl,
                reinterpret_cast<uint64_t*>(big), s_ids, s_w, a.ids_ws, a.w_ws, c, warm_shared);
  MOE_STAMP(c.stamps, 3);

  // 3. the slot stream: [shared slots,] routed slots; flat channel f, contiguous shares
  Ctx cr = c;
  if constexpr (kTwo) {
    set_teams(cr, L.tsz_r);
    cr.nch = a.H / ER;
  }
  // the routed layout's x as f16 pairs (MXFP4 dot products), its outputs in fp32
  XHalf<CPT> xr;
  float yr[kTwo ? CPT * ER : 1];
  if constexpr (kTwo) {
    load_x_half<CPT>(a.x, cr, xr);
#pragma unroll
    for (int i = 0; i < CPT * ER; ++i) yr[i] = 0.0f;
  }
  if constexpr (kTwo)
    stream_routed_flat<ET, CR, CPT>(a.gate, a.up, a.down_t, a.gate_s, a.up_s, a.down_s,
                                    share.r0, share.r1, a.I, a.k, s_ids, s_w, xr, yr, cr);
  else
    stream_routed<ET, CR, CPT>(ss, share, xv, yv, c);

  // 4. deterministic cross-workgroup sum of the partial outputs
  if constexpr (kTwo) MOE_STAMP_AFTER(c.stamps, 4, yr[0]);
  else MOE_STAMP_AFTER(c.stamps, 4, yv[0]);
  if constexpr (kTwo) {
    // the routed teams' vectors to big (one H-vector each); the publish adds them to the
    // shared output in ysh, in team order
    teams_to_lds_split<ER, CPT>(yr, big, cr);
    publish_and_reduce(a.partials, a.y, ctrl, L.R, L.SW, big, c, ysh, nullptr, 0, big,
                       cr.nteams);
  } else {
    teams_to_lds<8, CPT>(yv, big, c);
    MOE_STAMP(c.stamps, 5);
    publish_and_reduce(a.partials, a.y, ctrl, L.R, L.SW, big, c);
  }
  s_int[15] = (int)(warm[0] ^ warm[1]);  // keeps the warming loads (see warm_rows)
}

template <DT ET, DT ST, DT RT, int CR, int CS, int CPT>
hipError_t launch_t(const B1Launch& L, int wgs, int threads, int lds, hipStream_t s,
                    int* occ) {
  auto fn = b1_kernel<ET, ST, RT, CR, CS, CPT>;
  // Raise the dynamic-LDS limit once per instantiation (kept out of the per-launch path
  // so that graph capture records only the launch).
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

// Channels per team and pipeline stage: enough bytes in flight without spilling the two
// register stages (a bf16 or fp32 chunk holds 4 or 8 registers per row, an MXFP4 chunk 2,
// a wide MXFP4 chunk 3, and its layout keeps 32 x and output values per thread).
template <DT dt> constexpr int channels_per_batch() {
  return dt == DT::MXFP4W ? 2 : dt == DT::MXFP4 ? 2 : dt == DT::BF16 ? MOE_B1_BF16_C : 1;
}

template <DT ET, DT ST, DT RT>
hipError_t launch_cpt(const B1Launch& L, int wgs, int threads, int lds, hipStream_t s,
                      int* occ) {
  // the shared experts stream on their own before the routing when the formats differ (two
  // channels per team there, as the routed MXFP4 rows); otherwise they are slots of the
  // routed stream and CS is unused
  constexpr int CR = channels_per_batch<ET>(), CS = ET == DT::MXFP4W ? 2 : CR;
  // team_size gives one chunk per thread for every H the host admits (H <= 8192)
  if (L.a.H / 8 > L.tsz) return hipErrorInvalidValue;
  return launch_t<ET, ST, RT, CR, CS, 1>(L, wgs, threads, lds, s, occ);
}

}  // namespace

// Threads per team: the smallest of 256/512/1024 that covers a row in one chunk per thread.
int team_size(int H) {
  const int nch = H / 8;
  return nch <= 256 ? 256 : nch <= 512 ? 512 : 1024;
}

// Threads per team for rows of nch chunks: the smallest power of two of whole waves.
static int team_threads(int nch) {
  int t = 64;
  while (t < nch && t < 1024) t <<= 1;
  return t;
}

static int b1_big_floats(int H, int threads, int E, int k, bool two_layouts) {
  const int nteams = threads / team_size(H);
  const int ybuf = nteams * H * 4;
  const int topk = topk_lds_bytes(E, k);
  const int reduce = threads * 8;  // the reducers' two floats per thread
  // MXFP4: the routed layout's teams, one H-vector each (16 values per thread at most)
  const int routed = two_layouts ? threads * 16 * 4 : 0;
  int big = ybuf > topk ? ybuf : topk;
  big = big > reduce ? big : reduce;
  big = big > routed ? big : routed;
  return (big + 15) / 16 * 4;
}

int b1_lds_bytes(int H, int threads, int E, int k, bool two_layouts) {
  const int red = 2 * (threads / kWave) * kMaxNP * 4;
  const int small = (16 + 64 + 64) * 4;
  const int ysh = two_layouts ? (threads / team_size(H)) * H * 4 : 0;
  return red + small + b1_big_floats(H, threads, E, k, two_layouts) * 4 + ysh;
}

hipError_t launch_b1(const B1Args& a, DT et, DT st, DT rt, int wgs, int threads,
                     hipStream_t s, int* occ) {
  B1Launch L;
  L.a = a;
  L.tsz = team_size(a.H);
  L.tsz_r = L.tsz;
  reducer_split(a.H, wgs, &L.R, &L.SW);
  const int lds = b1_lds_bytes(a.H, threads, a.E, a.k, et == DT::MXFP4);
  L.big_floats = b1_big_floats(a.H, threads, a.E, a.k, et == DT::MXFP4);
  if (et == DT::F32 && st == DT::F32 && rt == DT::F32)
    return launch_cpt<DT::F32, DT::F32, DT::F32>(L, wgs, threads, lds, s, occ);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::BF16)
    return launch_cpt<DT::BF16, DT::BF16, DT::BF16>(L, wgs, threads, lds, s, occ);
  if (et == DT::BF16 && st == DT::BF16 && rt == DT::F32)
    return launch_cpt<DT::BF16, DT::BF16, DT::F32>(L, wgs, threads, lds, s, occ);
  if (et == DT::MXFP4 && st == DT::BF16 && rt == DT::BF16) {
    // routed MXFP4 rows in 16-element chunks: 8 bytes of codes per thread and row
    L.tsz_r = team_threads(a.H / kE<DT::MXFP4W>);
    return launch_cpt<DT::MXFP4W, DT::BF16, DT::BF16>(L, wgs, threads, lds, s, occ);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe

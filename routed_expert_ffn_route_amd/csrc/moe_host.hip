// moe_host.hip -- the C ABI: argument validation, workspace layout, launch selection.
// Validation happens on the host before any HIP call; no call allocates device memory.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <string>

#include "../../include/moe_ffn.h"
#include "kernels.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status device_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int kMaxWorkgroups = 512;   // partial-sum rows reserved in the workspace
#ifndef MOE_B1_LOOP_MAX
#define MOE_B1_LOOP_MAX 2
#endif
constexpr int kB1LoopMax = MOE_B1_LOOP_MAX;  // batches run token by token on the batch-1 kernel
constexpr int kThreads = 1024;
// From this batch size on, linear experts use the tiled kernel (x staged in LDS, many tokens
// per expert); below it the row-owner kernel, which needs no partial rows.
constexpr int kLinearTiledMinBatch = 32;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Layout {
  size_t ctrl, rlog, zrow, logits, ids, w, dnorm, partials, union_n, union_touched, union_offsets,
      union_slots, cs_s, sk_mask, cs_y, rec_r, bsel_s, bsel_g, bsel_desc, bsel_nk, bsel_sel, bsel_a, bsel_part, xh,
      xl, x16, xsc, act, part, total;
};

bool desc_valid(const moe_layer_desc* d, std::string* why) {
  char buf[256];
  auto bad = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (!d) return bad("null descriptor");
  if (d->hidden < 32 || d->hidden % 32 != 0 || d->hidden > 16384)
    return bad("hidden must be a multiple of 32 in [32, 16384]");
  if (d->n_experts < 1 || d->n_experts > 4096) return bad("n_experts must be in [1, 4096]");
  if (d->top_k < 1 || d->top_k > d->n_experts) return bad("top_k must be in [1, n_experts]");
  if (d->top_k > 32 && d->n_experts > 64)
    return bad("top_k above 32 needs n_experts <= 64");
  if (d->inter < 8 || d->inter % 8 != 0) return bad("inter must be a positive multiple of 8");
  // channel indices of the batch-1 kernels are 32-bit
  if ((long long)d->n_experts * d->inter > 0x7FFFFFFFll)
    return bad("n_experts * inter must be below 2^31");
  // one expert's rows are addressed with 32-bit byte offsets
  if ((long long)d->inter * d->hidden * 4 >= (1ll << 32))
    return bad("inter * hidden must be below 2^30");
  if (d->kind != MOE_EXPERT_SWIGLU && d->kind != MOE_EXPERT_LINEAR) return bad("bad kind");
  if (d->max_batch < 1 || d->max_batch > 4096) return bad("max_batch must be in [1, 4096]");
  if (d->router_dtype != MOE_DTYPE_NONE && d->router_dtype != MOE_F32 &&
      d->router_dtype != MOE_BF16)
    return bad("router_dtype must be NONE, F32 or BF16");
  if (d->expert_dtype != MOE_F32 && d->expert_dtype != MOE_BF16 && d->expert_dtype != MOE_MXFP4)
    return bad("expert_dtype must be F32, BF16 or MXFP4");
  if (d->kind == MOE_EXPERT_SWIGLU) {
    if (d->n_shared < 0 || d->n_shared > 4) return bad("n_shared must be in [0, 4]");
    if (d->n_shared > 0) {
      if (d->shared_inter < 8 || d->shared_inter % 8 != 0)
        return bad("shared_inter must be a positive multiple of 8");
      if ((long long)d->n_shared * d->shared_inter + (long long)d->top_k * d->inter >
          0x7FFFFFFFll)
        return bad("n_shared * shared_inter + top_k * inter must be below 2^31");
      if ((long long)d->shared_inter * d->hidden * 4 >= (1ll << 32))
        return bad("shared_inter * hidden must be below 2^30");
      if (d->shared_dtype != MOE_F32 && d->shared_dtype != MOE_BF16)
        return bad("shared_dtype must be F32 or BF16");
    }
  } else {
    if (d->n_shared != 0) return bad("LINEAR experts take no shared experts");
    if (d->expert_dtype != MOE_BF16) return bad("LINEAR experts are BF16");
    if (d->hidden % 1024 != 0) return bad("LINEAR experts need hidden to be a multiple of 1024");
  }
  (void)buf;
  return true;
}

Layout layout_of(const moe_layer_desc* d, bool with_dnorm = true) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t B = (size_t)d->max_batch, E = (size_t)d->n_experts, k = (size_t)d->top_k;
  L.ctrl = take(sizeof(Ctrl));
  L.rlog = take((size_t)kPollCopies * ((E + 15) & ~(size_t)15) * 8);  // a copy per XCD
  // zeros that empty slots of the batch-1 streams read in place of a weight row
  L.zrow = take((size_t)d->hidden * 4);
  L.logits = take(B * E * 4);
  L.ids = take(B * k * 4);
  L.w = take(B * k * 4);
  L.dnorm = take(d->kind == MOE_EXPERT_SWIGLU && with_dnorm ? E * (size_t)d->inter * 4 : 0);
  L.partials = take((size_t)kMaxWorkgroups * (size_t)d->hidden * 4);
  L.union_n = take(4);
  L.union_touched = take(E * 4);
  L.union_offsets = take((E + 1) * 4);
  L.union_slots = take(B * k * 4);
  const size_t kI = d->kind == MOE_EXPERT_SWIGLU ? k * (size_t)d->inter : 0;
  // channel selection: the launch-tagged scores [k*I] (32-bit), one copy per XCD, each padded
  // to 64 words
  L.cs_s = take(kI ? (size_t)kPollCopies * ((kI + 63) / 64) * 64 * 4 : 0);
  // the sketch screen's launch-tagged scan masks (4 words per 128-block), one copy per XCD
  L.sk_mask = take(kI && d->hidden % 128 == 0 && d->hidden <= 4096
                       ? (size_t)kPollCopies * kSkMaskWords * 8
                       : 0);
  L.cs_y = take(d->kind == MOE_EXPERT_SWIGLU ? (size_t)d->hidden * 4 : 0);
  // the reader's per-workgroup recovery sums [workgroups][kRecRank] (written every launch)
  L.rec_r = take(kI ? (size_t)kMaxWorkgroups * kRecRank * 4 : 0);
  // batch-wide channel selection (up to kBselMaxBatch tokens): batch scores [min(E, mb*k)*I],
  // the gate values [min(E, mb*k)*I][mb], kept-channel descriptors [min(E, mb*k)*I][4], the
  // kept count, activations [(NS*IS + min(E, mb*k)*I)][mb] and partial outputs
  // [kBselPartChunks][mb][H]
  const size_t mb = B < (size_t)kBselMaxBatch ? B : (size_t)kBselMaxBatch;
  const size_t bcand =
      kI && with_dnorm ? (E < mb * k ? E : mb * k) * (size_t)d->inter : 0;
  const size_t bsh = (size_t)d->n_shared * (size_t)(d->n_shared > 0 ? d->shared_inter : 0);
  L.bsel_s = take(bcand * 4);
  L.bsel_g = take(bcand * mb * 4);
  L.bsel_desc = take(bcand * 16);
  L.bsel_nk = take(bcand ? 4 : 0);
  L.bsel_sel = take(bsel_sel_bytes(bcand));
  L.bsel_a = take(bcand ? (bcand + bsh) * mb * 4 : 0);
  L.bsel_part = take(bcand ? (size_t)kBselPartChunks * mb * d->hidden * 4 : 0);
  const bool batched_swiglu = d->kind == MOE_EXPERT_SWIGLU && B > 1;
  const size_t xs =
      d->kind == MOE_EXPERT_LINEAR || batched_swiglu ? B * (size_t)d->hidden * 2 : 0;
  L.xh = take(xs);
  L.xl = take(xs);
  // linear experts at larger batches: x as scaled f16 and the per-token scales
  const bool lin_tiled = d->kind == MOE_EXPERT_LINEAR && B >= kLinearTiledMinBatch;
  L.x16 = take(lin_tiled ? B * (size_t)d->hidden * 2 : 0);
  L.xsc = take(lin_tiled ? B * (size_t)4 : 0);
  // batched SwiGLU: activations and partial outputs of every (token, choice) and every
  // (shared expert, token)
  const size_t pairs = batched_swiglu ? B * k + (size_t)d->n_shared * B : 0;
  const size_t ia = (size_t)(d->inter > d->shared_inter ? d->inter : d->shared_inter);
  L.act = take(pairs * ia * 4);
  // partial outputs: batched SwiGLU [kDownRowSlices][pairs][H]; linear experts above
  // kGemvMaxBatch tokens [B*k][I]
  const size_t lin_part = d->kind == MOE_EXPERT_LINEAR && B > kGemvMaxBatch
                              ? B * k * (size_t)d->inter * 4
                              : 0;
  const size_t sw_part = kDownRowSlices * pairs * (size_t)d->hidden * 4;
  L.part = take(lin_part > sw_part ? lin_part : sw_part);
  L.total = o;
  return L;
}

DT to_dt(int32_t v) { return v == MOE_BF16 ? DT::BF16 : v == MOE_MXFP4 ? DT::MXFP4 : DT::F32; }

}  // namespace

struct moe_layer_s {
  moe_layer_desc d;
  moe_weights w;
  unsigned char* ws;
  Layout L;
  int device;
  int workgroups;
  int threads;
  uint32_t magic;
  CsSketch sketch{};  // bound by moe_layer_build_sketch (all null until then)
  const float* rec_U = nullptr;     // bound by moe_layer_build_recovery: U [H][kRecRank]
  const uint16_t* rec_b = nullptr;  // and b [E*I][kRecRank] FP16
  template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  Ctrl* ctrl() const { return at<Ctrl>(L.ctrl); }
};

static constexpr uint32_t kMagic = 0x4D6F4546u;

// Phase-timeline buffer of the single-launch kernels ([workgroups][kStamps] uint64 device
// memory), set by moe_debug_set_stamps in the timeline build only.
static uint64_t* g_stamps = nullptr;

static moe_status check_layer(moe_layer l) {
  if (!l || l->magic != kMagic) return fail(MOE_ERR_ARG, "invalid or destroyed layer handle");
  return MOE_OK;
}

static moe_status b1_types(moe_layer layer, DT* et, DT* st, DT* rt) {
  const moe_layer_desc& d = layer->d;
  *et = to_dt(d.expert_dtype);
  *st = d.n_shared > 0 ? to_dt(d.shared_dtype) : (*et == DT::MXFP4 ? DT::BF16 : *et);
  *rt = d.router_dtype == MOE_DTYPE_NONE ? *st : to_dt(d.router_dtype);
  const bool combo_ok = (*et == DT::F32 && *st == DT::F32 && *rt == DT::F32) ||
                        (*et == DT::BF16 && *st == DT::BF16 && *rt == DT::BF16) ||
                        (*et == DT::BF16 && *st == DT::BF16 && *rt == DT::F32) ||
                        (*et == DT::MXFP4 && *st == DT::BF16 && *rt == DT::BF16);
  if (!combo_ok) return fail(MOE_ERR_UNSUPPORTED, "expert/shared/router dtype combination");
  return MOE_OK;
}

static B1Args b1_args(moe_layer layer, const float* x, const int32_t* ids, const float* w,
                      float* y) {
  const moe_layer_desc& d = layer->d;
  B1Args a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.router = layer->w.router;
  a.gate = layer->w.gate;
  a.up = layer->w.up;
  a.down_t = layer->w.down_t;
  a.gate_s = layer->w.gate_scale;
  a.up_s = layer->w.up_scale;
  a.down_s = layer->w.down_scale;
  a.sh_gate = layer->w.sh_gate;
  a.sh_up = layer->w.sh_up;
  a.sh_down_t = layer->w.sh_down_t;
  a.ids_in = ids;
  a.w_in = w;
  a.rlog = layer->at<uint64_t>(layer->L.rlog);
  a.zrow = layer->at<uint8_t>(layer->L.zrow);
  a.ids_ws = layer->at<int32_t>(layer->L.ids);
  a.w_ws = layer->at<float>(layer->L.w);
  a.partials = layer->at<float>(layer->L.partials);
  a.y = y;
  a.ctrl = layer->ctrl();
  a.H = d.hidden;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.I = d.inter;
  a.NS = d.n_shared;
  a.IS = d.shared_inter;
  a.route_inside = ids == nullptr;
  a.stamps = g_stamps;
  return a;
}

// Host-side checks of the weight pointers against a valid descriptor.
static moe_status validate_weights(const moe_layer_desc& d, const moe_weights& w) {
  if ((d.router_dtype == MOE_DTYPE_NONE) != (w.router == nullptr))
    return fail(MOE_ERR_ARG, "router pointer must be given iff router_dtype is not NONE");
  if (w.router && !aligned16(w.router)) return fail(MOE_ERR_ARG, "router is not 16-byte aligned");
  if (d.kind == MOE_EXPERT_SWIGLU) {
    if (!w.gate || !w.up || !w.down_t) return fail(MOE_ERR_ARG, "gate/up/down_t must be given");
    if (!aligned16(w.gate) || !aligned16(w.up) || !aligned16(w.down_t))
      return fail(MOE_ERR_ARG, "expert tensors must be 16-byte aligned");
    const bool mx = d.expert_dtype == MOE_MXFP4;
    if (mx != (w.gate_scale != nullptr) || mx != (w.up_scale != nullptr) ||
        mx != (w.down_scale != nullptr))
      return fail(MOE_ERR_ARG, "scales must be given iff expert_dtype is MXFP4");
    if (mx && (!aligned16(w.gate_scale) || !aligned16(w.up_scale) || !aligned16(w.down_scale)))
      return fail(MOE_ERR_ARG, "scale tensors must be 16-byte aligned");
    if (d.n_shared > 0) {
      if (!w.sh_gate || !w.sh_up || !w.sh_down_t)
        return fail(MOE_ERR_ARG, "shared expert tensors must be given");
      if (!aligned16(w.sh_gate) || !aligned16(w.sh_up) || !aligned16(w.sh_down_t))
        return fail(MOE_ERR_ARG, "shared tensors must be 16-byte aligned");
    }
  } else {
    if (!w.linear || !aligned16(w.linear))
      return fail(MOE_ERR_ARG, "linear must be given and 16-byte aligned");
  }
  return MOE_OK;
}

// ------------------------------------------------------------------------------------
// Static scratch for moe_ffn_forward_noalloc: the workspace of one call at a time per GPU,
// in the code object's own device memory (every GPU the library runs on holds its copy until
// the process ends).  Host code reaches it only through the address hipGetSymbolAddress
// returns for the current device; the array's name in host code is a stand-in, not a device
// address.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];
static int g_scratch_cus[kMaxDevices];

// The scratch's device address and the compute-unit count of device `dev`, looked up once per
// device (with that device current).
static moe_status scratch_for(int dev, void** ptr, int* cus) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_fail(e, "hipGetSymbolAddress(scratch)");
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return device_fail(e, "hipDeviceGetAttribute");
    g_scratch_cus[dev] = n;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *cus = g_scratch_cus[dev];
  return MOE_OK;
}

// Zero `words` 32-bit words (a fill kernel, so that the clearing can be captured in a graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The batch-1 kernels are persistent: their workgroups wait on one another's results (router
// logits, gate values, partial outputs), so all of them -- one per CU -- must be resident at
// once.  The occupancy the runtime computes from the kernel's registers and this layer's LDS
// must allow one workgroup of `threads` per CU; a kernel that needs more would hang on its own
// bounded waits instead.  Shapes or types the kernels do not take are left to the calls, which
// reject them.
static moe_status check_residency(moe_layer l) {
  const moe_layer_desc& d = l->d;
  if (d.kind != MOE_EXPERT_SWIGLU) return ok();
  DT et = to_dt(d.expert_dtype), st, rt;
  st = d.n_shared > 0 ? to_dt(d.shared_dtype) : (et == DT::MXFP4 ? DT::BF16 : et);
  rt = d.router_dtype == MOE_DTYPE_NONE ? st : to_dt(d.router_dtype);
  B1Args a = b1_args(l, nullptr, nullptr, nullptr, nullptr);
  if (d.hidden <= 8192 && b1_lds_bytes(d.hidden, l->threads, d.n_experts, d.top_k,
                                       et == DT::MXFP4) <= 160 * 1024) {
    int occ = 0;
    const hipError_t e = launch_b1(a, et, st, rt, l->workgroups, l->threads, nullptr, &occ);
    if (e == hipSuccess && occ < 1)
      return fail(MOE_ERR_UNSUPPORTED, "the batch-1 kernel cannot keep a workgroup of %d "
                  "threads resident on every CU (occupancy %d)", l->threads, occ);
  }
  if (et != DT::MXFP4 && d.hidden <= 4096 && d.top_k <= 64 &&
      (long long)d.top_k * d.inter <= (long long)kCsMaxPerThread * l->threads) {
    int occ = 0;
    const hipError_t e = launch_cs(a, nullptr, nullptr, nullptr, 0, 0, et, st, rt,
                                   l->workgroups, l->threads, nullptr, &occ);
    if (e == hipSuccess && occ < 1)
      return fail(MOE_ERR_UNSUPPORTED, "the channel-sparse kernel cannot keep a workgroup of "
                  "%d threads resident on every CU (occupancy %d)", l->threads, occ);
  }
  return ok();
}

// moe_ffn_forward on a checked handle (also serves moe_ffn_forward_noalloc, whose handle
// lives on the stack and binds the library's static scratch).
static moe_status forward_impl(moe_layer layer, const float* x, int32_t B, const int32_t* ids,
                               const float* w, float* y, void* stream) {
  const moe_layer_desc& d = layer->d;
  if (!x || !y) return fail(MOE_ERR_ARG, "x and y must be given");
  if (!aligned16(x) || !aligned16(y)) return fail(MOE_ERR_ARG, "x and y must be 16-byte aligned");
  if (B < 1 || B > d.max_batch) return fail(MOE_ERR_ARG, "B=%d outside [1, max_batch]", B);
  if ((ids == nullptr) != (w == nullptr))
    return fail(MOE_ERR_ARG, "ids and w must both be given or both be null");
  if (!ids && d.router_dtype == MOE_DTYPE_NONE)
    return fail(MOE_ERR_ARG, "routing inside the call needs a router");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Up to kB1LoopMax tokens run as that many launches of the single-launch layer, one token
  // each (its routing inside or the token's row of ids and w): below that batch the batched
  // path's separate routing, union and product launches cost more than the second token saves.
  if (d.kind == MOE_EXPERT_SWIGLU && (B == 1 || (B <= kB1LoopMax && d.hidden <= 8192))) {
    DT et, st, rt;
    if (moe_status e = b1_types(layer, &et, &st, &rt)) return e;
    if (d.hidden > 8192) return fail(MOE_ERR_UNSUPPORTED, "batch-1 kernel needs hidden <= 8192");
    if (b1_lds_bytes(d.hidden, layer->threads, d.n_experts, d.top_k, et == DT::MXFP4) >
        160 * 1024)
      return fail(MOE_ERR_UNSUPPORTED, "batch-1 kernel LDS exceeds 160 KiB");
    for (int b = 0; b < B; ++b) {
      const size_t xo = (size_t)b * d.hidden, ro = (size_t)b * d.top_k;
      B1Args a = b1_args(layer, x + xo, ids ? ids + ro : nullptr, w ? w + ro : nullptr, y + xo);
      a.ids_ws += ro;  // the routing read back: row b
      a.w_ws += ro;
      hipError_t e = launch_b1(a, et, st, rt, layer->workgroups, layer->threads, s);
      if (e != hipSuccess) return device_fail(e, "batch-1 layer launch");
    }
    return ok();
  }
  if (d.kind == MOE_EXPERT_SWIGLU) {
    DT et, st, rt;
    if (moe_status e = b1_types(layer, &et, &st, &rt)) return e;
    if (et == DT::F32 || st != DT::BF16)
      return fail(MOE_ERR_UNSUPPORTED, "batched SwiGLU needs BF16 or MXFP4 experts and BF16 "
                                       "shared experts");
    if (union_lds_bytes(B, d.n_experts) > kUnionMaxLds)
      return fail(MOE_ERR_UNSUPPORTED, "E*(ceil(B/32)|1)*8 + 8E bytes exceed the union LDS budget (144 KiB)");
    const int32_t* rid = ids;
    const float* rw = w;
    hipError_t e = hipSuccess;
    if (!ids) {
      RouteArgs r;
      r.x = x;
      r.logits_in = nullptr;
      r.router = layer->w.router;
      r.logits = layer->at<float>(layer->L.logits);
      r.ids = layer->at<int32_t>(layer->L.ids);
      r.w = layer->at<float>(layer->L.w);
      r.H = d.hidden;
      r.E = d.n_experts;
      r.k = d.top_k;
      r.B = B;
      e = launch_route(r, rt, s);
      rid = r.ids;
      rw = r.w;
    }
    BsArgs a;
    memset(&a, 0, sizeof(a));
    a.gate = layer->w.gate;
    a.up = layer->w.up;
    a.down_t = layer->w.down_t;
    a.gate_s = layer->w.gate_scale;
    a.up_s = layer->w.up_scale;
    a.down_s = layer->w.down_scale;
    a.sh_gate = layer->w.sh_gate;
    a.sh_up = layer->w.sh_up;
    a.sh_down_t = layer->w.sh_down_t;
    a.xh = layer->at<uint16_t>(layer->L.xh);
    a.xl = layer->at<uint16_t>(layer->L.xl);
    a.w = rw;
    a.ids = rid;
    a.n_touched = layer->at<int32_t>(layer->L.union_n);
    a.touched = layer->at<int32_t>(layer->L.union_touched);
    a.offsets = layer->at<int32_t>(layer->L.union_offsets);
    a.slots = layer->at<int32_t>(layer->L.union_slots);
    a.act = layer->at<float>(layer->L.act);
    a.part = layer->at<float>(layer->L.part);
    a.y = y;
    a.H = d.hidden;
    a.I = d.inter;
    a.IS = d.n_shared > 0 ? d.shared_inter : 0;
    a.IA = d.inter > a.IS ? d.inter : a.IS;
    a.E = d.n_experts;
    a.k = d.top_k;
    a.B = B;
    a.NS = d.n_shared;
    a.pairs = B * d.top_k + d.n_shared * B;
    a.slots_max = B * d.top_k < d.n_experts ? B * d.top_k : d.n_experts;
    if (e == hipSuccess)
      e = launch_union(rid, B, d.top_k, d.n_experts, layer->at<int32_t>(layer->L.union_n),
                       layer->at<int32_t>(layer->L.union_touched),
                       layer->at<int32_t>(layer->L.union_offsets),
                       layer->at<int32_t>(layer->L.union_slots), layer->ctrl(), s, x,
                       (size_t)B * d.hidden, layer->at<uint16_t>(layer->L.xh),
                       layer->at<uint16_t>(layer->L.xl));
    if (e == hipSuccess) e = launch_batched_swiglu(a, et, st, s);
    if (e != hipSuccess) return device_fail(e, "batched SwiGLU layer launch");
    return ok();
  }
  if (d.kind == MOE_EXPERT_LINEAR) {
    if (union_lds_bytes(B, d.n_experts) > kUnionMaxLds)
      return fail(MOE_ERR_UNSUPPORTED, "E*(ceil(B/32)|1)*8 + 8E bytes exceed the union LDS budget (144 KiB)");
    const int32_t* rid = ids;
    const float* rw = w;
    hipError_t e = hipSuccess;
    if (!ids) {
      RouteArgs r;
      r.x = x;
      r.logits_in = nullptr;
      r.router = layer->w.router;
      r.logits = layer->at<float>(layer->L.logits);
      r.ids = layer->at<int32_t>(layer->L.ids);
      r.w = layer->at<float>(layer->L.w);
      r.H = d.hidden;
      r.E = d.n_experts;
      r.k = d.top_k;
      r.B = B;
      e = launch_route(r, to_dt(d.router_dtype), s);
      rid = r.ids;
      rw = r.w;
    }
    int32_t* n_t = layer->at<int32_t>(layer->L.union_n);
    int32_t* touched = layer->at<int32_t>(layer->L.union_touched);
    int32_t* offsets = layer->at<int32_t>(layer->L.union_offsets);
    int32_t* slots = layer->at<int32_t>(layer->L.union_slots);
    // up to kGemvMaxBatch tokens: the VALU kernel builds the touched list from the ids itself
    const bool gemv = B < kLinearTiledMinBatch && linear_gemv_fits(d.hidden, d.inter, B) &&
                      B * d.top_k <= 256;
    if (e == hipSuccess && gemv) {
      e = launch_linear_gemv(layer->w.linear, x, rid, rw, &layer->ctrl()->err,
                             layer->at<uint8_t>(layer->L.zrow), y, d.hidden, d.inter,
                             d.n_experts, d.top_k, B, layer->workgroups, s);
    } else if (e == hipSuccess) {
      e = launch_union(rid, B, d.top_k, d.n_experts, n_t, touched, offsets, slots,
                       layer->ctrl(), s);
      if (e == hipSuccess && B >= kLinearTiledMinBatch)
        e = launch_linear_tiled(layer->w.linear, x, rw, rid, n_t, touched, offsets, slots,
                                layer->at<uint16_t>(layer->L.xh),
                                layer->at<uint16_t>(layer->L.xl),
                                layer->at<uint16_t>(layer->L.x16),
                                layer->at<float>(layer->L.xsc), layer->at<float>(layer->L.part),
                                y, d.hidden, d.inter, d.n_experts, d.top_k, B, s);
      else if (e == hipSuccess && linear_pass_fits(d.hidden, d.inter, B, d.top_k))
        e = launch_linear_pass(layer->w.linear, x, rw, rid, n_t, touched, offsets, slots,
                               layer->at<uint8_t>(layer->L.zrow),
                               layer->at<float>(layer->L.part), y, d.hidden, d.inter,
                               d.n_experts, d.top_k, B, layer->workgroups, s);
      else if (e == hipSuccess)
        e = launch_linear(layer->w.linear, x, rw, n_t, touched, offsets, slots,
                          layer->at<uint16_t>(layer->L.xh), layer->at<uint16_t>(layer->L.xl),
                          y, d.hidden, d.inter, d.n_experts, d.top_k, B, s);
    }
    if (e != hipSuccess) return device_fail(e, "linear-expert layer launch");
    return ok();
  }
  return fail(MOE_ERR_UNSUPPORTED, "unknown expert kind");
}

extern "C" {

const char* moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

#ifdef MOE_TIMELINE
// Timeline build only (not part of the product ABI): every later batch-1 launch records its
// phase clock into `stamps` (device memory of at least 512 * kStamps uint64), or stops
// recording when it is null.  Returns kStamps.
int moe_debug_set_stamps(void* stamps) {
  g_stamps = reinterpret_cast<uint64_t*>(stamps);
  return (int)kStamps;
}
#endif

size_t moe_layer_workspace_bytes(const moe_layer_desc* desc) {
  if (!desc_valid(desc, nullptr)) return 0;
  return layout_of(desc).total;
}

moe_status moe_layer_create(const moe_layer_desc* desc, const moe_weights* weights,
                            void* workspace, size_t workspace_bytes, void* stream,
                            moe_layer* out) {
  std::string why;
  if (!out) return fail(MOE_ERR_ARG, "out is null");
  if (!desc_valid(desc, &why)) return fail(MOE_ERR_ARG, "descriptor: %s", why.c_str());
  if (!weights) return fail(MOE_ERR_ARG, "weights is null");
  const moe_layer_desc& d = *desc;
  const moe_weights& w = *weights;
  if (moe_status st = validate_weights(d, w)) return st;
  const Layout L = layout_of(&d);
  if (!workspace || ((uintptr_t)workspace % kAlign) != 0)
    return fail(MOE_ERR_WORKSPACE, "workspace must be non-null and 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                L.total);

  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_fail(e, "hipDeviceGetAttribute");
  moe_layer l = new (std::nothrow) moe_layer_s;
  if (!l) return fail(MOE_ERR_ARG, "out of host memory");
  l->d = d;
  l->w = w;
  l->ws = reinterpret_cast<unsigned char*>(workspace);
  l->L = L;
  l->device = dev;
  l->workgroups = cus < kMaxWorkgroups ? cus : kMaxWorkgroups;
  l->threads = kThreads;
  l->magic = kMagic;
  if (moe_status st = check_residency(l)) {
    l->magic = 0;
    delete l;
    return st;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Everything from the control block (offset 0) through the tagged channel scores starts
  // at zero: the epoch and arrival counters, the zero row, and every word that carries a
  // launch tag (router logits, channel scores; tag 0 is never a launch's).  Memory reused
  // from an earlier layer could otherwise hold words with the tag of this layer's first
  // launch.
  e = hipMemsetAsync(l->ctrl(), 0, L.cs_y, s);
  if (e == hipSuccess && d.kind == MOE_EXPERT_SWIGLU)
    e = launch_row_norms(w.down_t, w.down_scale, to_dt(d.expert_dtype),
                         (size_t)d.n_experts * d.inter, d.hidden, l->at<float>(L.dnorm), s);
  if (e != hipSuccess) {
    l->magic = 0;
    delete l;
    return device_fail(e, "layer preparation");
  }
  *out = l;
  return ok();
}

moe_status moe_layer_destroy(moe_layer layer) {
  if (moe_status st = check_layer(layer)) return st;
  layer->magic = 0;
  delete layer;
  return ok();
}

moe_status moe_layer_geometry(moe_layer layer, int32_t* workgroups, int32_t* threads) {
  if (moe_status st = check_layer(layer)) return st;
  if (workgroups) *workgroups = layer->workgroups;
  if (threads) *threads = layer->threads;
  return ok();
}

moe_status moe_layer_check(moe_layer layer, void* stream, int32_t* device_error) {
  if (moe_status st = check_layer(layer)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t err = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&err, &layer->ctrl()->err, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && err) e = hipMemset(&layer->ctrl()->err, 0, 4);
  if (e != hipSuccess) return device_fail(e, "moe_layer_check");
  if (device_error) *device_error = (int32_t)err;
  return ok();
}

moe_status moe_layer_routing(moe_layer layer, int32_t B, int32_t* ids, float* w,
                             void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const moe_layer_desc& d = layer->d;
  if (B < 1 || B > d.max_batch) return fail(MOE_ERR_ARG, "B=%d outside [1, max_batch]", B);
  if (!ids || !w) return fail(MOE_ERR_ARG, "ids and w must be given");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t n = (size_t)B * d.top_k * 4;
  hipError_t e = hipMemcpyAsync(ids, layer->at<int32_t>(layer->L.ids), n,
                                hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(w, layer->at<float>(layer->L.w), n, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return device_fail(e, "moe_layer_routing copy");
  return ok();
}

moe_status moe_route(moe_layer layer, const float* x, const float* logits_in, int32_t B,
                     int32_t* ids, float* w, float* logits_out, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const moe_layer_desc& d = layer->d;
  if (B < 1 || B > d.max_batch) return fail(MOE_ERR_ARG, "B=%d outside [1, max_batch]", B);
  if ((x == nullptr) == (logits_in == nullptr))
    return fail(MOE_ERR_ARG, "exactly one of x and logits_in must be given");
  if (x && d.router_dtype == MOE_DTYPE_NONE)
    return fail(MOE_ERR_ARG, "routing from x needs a router");
  if (!ids || !w) return fail(MOE_ERR_ARG, "ids and w must be given");
  if ((x && !aligned16(x)) || (logits_in && !aligned16(logits_in)))
    return fail(MOE_ERR_ARG, "x and logits_in must be 16-byte aligned");
  RouteArgs a;
  a.x = x;
  a.logits_in = logits_in;
  a.router = layer->w.router;
  a.logits = logits_out ? logits_out : layer->at<float>(layer->L.logits);
  a.ids = ids;
  a.w = w;
  a.H = d.hidden;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.B = B;
  hipError_t e = launch_route(a, to_dt(d.router_dtype), reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "moe_route launch");
  return ok();
}

moe_status moe_ffn_forward(moe_layer layer, const float* x, int32_t B, const int32_t* ids,
                           const float* w, float* y, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  return forward_impl(layer, x, B, ids, w, y, stream);
}

moe_status moe_ffn_forward_noalloc(const moe_layer_desc* desc, const moe_weights* weights,
                                   const float* x, int32_t B, const int32_t* ids,
                                   const float* w, float* y, void* stream) {
  std::string why;
  if (!desc_valid(desc, &why)) return fail(MOE_ERR_ARG, "descriptor: %s", why.c_str());
  if (!weights) return fail(MOE_ERR_ARG, "weights is null");
  if (moe_status st = validate_weights(*desc, *weights)) return st;
  // the layer's workspace without the down-norm table (only channel selection reads it)
  const Layout L = layout_of(desc, /*with_dnorm=*/false);
  if (L.total > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "needs %zu bytes of scratch; the static scratch holds %zu",
                L.total, kScratchBytes);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  void* ptr = nullptr;
  if (moe_status st = scratch_for(dev, &ptr, &cus)) return st;
  moe_layer_s l;
  l.d = *desc;
  l.w = *weights;
  l.ws = reinterpret_cast<unsigned char*>(ptr);
  l.L = L;
  l.device = dev;
  l.workgroups = cus < kMaxWorkgroups ? cus : kMaxWorkgroups;
  l.threads = kThreads;
  l.magic = kMagic;
  if (moe_status st = check_residency(&l)) return st;
  // Everything that must start at zero, as at layer creation: the control block (epoch,
  // error word), the tagged words, the zero row and the partial rows, through the channel
  // scores.  The previous call on this GPU left its own contents there.
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t words = L.cs_y / 4;
  const int grid = (int)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(ptr), words);
  e = hipGetLastError();
  if (e != hipSuccess) return device_fail(e, "scratch clear");
  return forward_impl(&l, x, B, ids, w, y, stream);
}

static moe_status channel_select_impl(moe_layer layer, const float* x, const int32_t* ids,
                                      const float* w, int32_t keep, int32_t mode, int32_t* kept,
                                      float* y, void* stream, const CsSketch* sketch,
                                      const CsThreshold* thr = nullptr) {
  const moe_layer_desc& d = layer->d;
  if (d.kind != MOE_EXPERT_SWIGLU) return fail(MOE_ERR_ARG, "channel selection needs SWIGLU experts");
  if (!x || !aligned16(x)) return fail(MOE_ERR_ARG, "x must be given and 16-byte aligned");
  if (y && !aligned16(y)) return fail(MOE_ERR_ARG, "y must be 16-byte aligned");
  const long long n = (long long)d.top_k * d.inter;
  if (thr) {
    if (!kept || !thr->count) return fail(MOE_ERR_ARG, "kept and kept_count must be given");
    keep = (int32_t)n;  // (the kept list's capacity)
  }
  if (keep < 0 || keep > n) return fail(MOE_ERR_ARG, "keep=%d outside [0, k*I=%lld]", keep, n);
  if (keep > 0 && !kept) return fail(MOE_ERR_ARG, "kept must be given when keep > 0");
  if (mode != MOE_SCORE_GATE_DNORM && mode != MOE_SCORE_ROUTER_WEIGHTED)
    return fail(MOE_ERR_ARG, "mode must be GATE_DNORM or ROUTER_WEIGHTED");
  if ((ids == nullptr) != (w == nullptr))
    return fail(MOE_ERR_ARG, "ids and w must both be given or both be null");
  if (!ids && d.router_dtype == MOE_DTYPE_NONE)
    return fail(MOE_ERR_ARG, "routing inside the call needs a router");
  DT et, st, rt;
  if (moe_status e = b1_types(layer, &et, &st, &rt)) return e;
  if (et == DT::MXFP4) return fail(MOE_ERR_UNSUPPORTED, "channel selection for MXFP4 experts");
  if (d.hidden > 4096) return fail(MOE_ERR_UNSUPPORTED, "channel selection needs hidden <= 4096");
  if (d.top_k > 64 || n > (long long)kCsMaxPerThread * layer->threads ||
      (n + layer->workgroups - 1) / layer->workgroups > kCsOwnMax)
    return fail(MOE_ERR_UNSUPPORTED, "channel selection needs k <= 64, k*I <= %d and at most "
                "%d candidates per workgroup", kCsMaxPerThread * layer->threads, kCsOwnMax);
  if (cs_lds_bytes(d.hidden, layer->threads, d.n_experts, d.top_k, d.inter, layer->workgroups,
                   keep, sketch != nullptr) > 160 * 1024)
    return fail(MOE_ERR_UNSUPPORTED, "k*I=%lld candidates exceed the selection LDS budget", n);
  B1Args a = b1_args(layer, x, ids, w, y ? y : layer->at<float>(layer->L.cs_y));
  CsSketch sk{};
  if (sketch) {
    sk = *sketch;
    sk.mask = layer->at<uint64_t>(layer->L.sk_mask);
  }
  hipError_t e = launch_cs(a, layer->at<float>(layer->L.dnorm),
                           layer->at<uint64_t>(layer->L.cs_s), kept, keep, mode, et, st, rt,
                           layer->workgroups, layer->threads, reinterpret_cast<hipStream_t>(stream),
                           nullptr, sketch ? &sk : nullptr, thr);
  if (e != hipSuccess) return device_fail(e, "channel-sparse layer launch");
  return ok();
}

moe_status moe_channel_select(moe_layer layer, const float* x, const int32_t* ids,
                              const float* w, int32_t keep, int32_t mode, int32_t* kept,
                              float* y, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  return channel_select_impl(layer, x, ids, w, keep, mode, kept, y, stream, nullptr);
}

moe_status moe_channel_select_threshold(moe_layer layer, const float* x, const int32_t* ids,
                                        const float* w, float tau, int32_t mode, int32_t* kept,
                                        int32_t* kept_count, float* y, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  if (!(tau == tau)) return fail(MOE_ERR_ARG, "tau is NaN");
  // scores are non-negative: their bit patterns order like the values, and a tau at or below
  // zero keeps every candidate
  uint32_t bits;
  const float t = tau > 0.0f ? tau : 0.0f;
  memcpy(&bits, &t, 4);
  CsThreshold thr{bits, kept_count};
  return channel_select_impl(layer, x, ids, w, 0, mode, kept, y, stream, nullptr, &thr);
}

__global__ void scores_copy_kernel(const uint32_t* src, float* dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = __uint_as_float(src[i] & ~1u);
}

moe_status moe_layer_scores(moe_layer layer, float* scores, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const moe_layer_desc& d = layer->d;
  if (d.kind != MOE_EXPERT_SWIGLU) return fail(MOE_ERR_ARG, "channel scores need SWIGLU experts");
  if (!scores) return fail(MOE_ERR_ARG, "scores must be given");
  const int n = d.top_k * d.inter;
  hipLaunchKernelGGL(scores_copy_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream),
                     layer->at<uint32_t>(layer->L.cs_s), scores, n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return device_fail(e, "moe_layer_scores copy");
  return ok();
}

// Sketch buffer layout: codes of G then V [E*I][H/16] uint32, then alpha of G, alpha of V,
// rho of G, rho of V [E*I][nbp] FP16 (nbp = H/128 rounded up to a multiple of 8); each region
// 256-byte aligned.
struct SketchLayout {
  size_t cg, cv, ag, av, rg, rv, total;
};
static bool sketch_layout(const moe_layer_desc* d, SketchLayout* S) {
  if (!desc_valid(d, nullptr) || d->kind != MOE_EXPERT_SWIGLU || d->expert_dtype == MOE_MXFP4 ||
      d->hidden % 128 != 0 || d->hidden > 4096)
    return false;
  const size_t rows = (size_t)d->n_experts * d->inter;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  S->cg = take(rows * (d->hidden / 16) * 4);
  S->cv = take(rows * (d->hidden / 16) * 4);
  const size_t nbp = (size_t)((d->hidden / 128 + 7) & ~7);
  S->ag = take(rows * nbp * 2);
  S->av = take(rows * nbp * 2);
  S->rg = take(rows * nbp * 2);
  S->rv = take(rows * nbp * 2);
  S->total = o;
  return true;
}

size_t moe_sketch_bytes(const moe_layer_desc* desc) {
  SketchLayout S;
  return sketch_layout(desc, &S) ? S.total : 0;
}

moe_status moe_layer_build_sketch(moe_layer layer, const int8_t* signs, void* sketch,
                                  size_t sketch_bytes, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const moe_layer_desc& d = layer->d;
  SketchLayout S;
  if (!sketch_layout(&d, &S))
    return fail(MOE_ERR_UNSUPPORTED, "the sketch needs SWIGLU experts in BF16 or F32 and hidden "
                "a multiple of 128, at most 4096");
  if (!signs || !sketch) return fail(MOE_ERR_ARG, "signs and sketch must be given");
  if (((uintptr_t)signs % 4) != 0) return fail(MOE_ERR_ARG, "signs must be 4-byte aligned");
  if (((uintptr_t)sketch % kAlign) != 0)
    return fail(MOE_ERR_WORKSPACE, "the sketch buffer must be 256-byte aligned");
  if (sketch_bytes < S.total)
    return fail(MOE_ERR_WORKSPACE, "sketch buffer has %zu bytes, needs %zu", sketch_bytes, S.total);
  unsigned char* base = reinterpret_cast<unsigned char*>(sketch);
  CsSketch sk{};
  sk.g = reinterpret_cast<const uint32_t*>(base + S.cg);
  sk.v = reinterpret_cast<const uint32_t*>(base + S.cv);
  sk.ag = reinterpret_cast<const uint16_t*>(base + S.ag);
  sk.av = reinterpret_cast<const uint16_t*>(base + S.av);
  sk.signs = signs;
  sk.mask = nullptr;  // the layer workspace's, bound at each launch
  const size_t rows = (size_t)d.n_experts * d.inter;
  const DT et = to_dt(d.expert_dtype);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_sketch_build(layer->w.gate, et, rows, d.hidden, signs,
                                     reinterpret_cast<uint32_t*>(base + S.cg),
                                     reinterpret_cast<uint16_t*>(base + S.ag),
                                     reinterpret_cast<uint16_t*>(base + S.rg), s);
  if (e == hipSuccess)
    e = launch_sketch_build(layer->w.up, et, rows, d.hidden, signs,
                            reinterpret_cast<uint32_t*>(base + S.cv),
                            reinterpret_cast<uint16_t*>(base + S.av),
                            reinterpret_cast<uint16_t*>(base + S.rv), s);
  if (e != hipSuccess) return device_fail(e, "sketch construction");
  layer->sketch = sk;
  return ok();
}

// Recovery buffer layout: U [H][kRecRank] fp32, then b [E*I][kRecRank] FP16, 256-byte aligned.
static bool recovery_layout(const moe_layer_desc* d, size_t* b_off, size_t* total) {
  SketchLayout S;
  if (!sketch_layout(d, &S)) return false;
  *b_off = align_up((size_t)d->hidden * kRecRank * 4);
  *total = align_up(*b_off + (size_t)d->n_experts * d->inter * kRecRank * 2);
  return true;
}

size_t moe_recovery_bytes(const moe_layer_desc* desc) {
  size_t b_off, total;
  return recovery_layout(desc, &b_off, &total) ? total : 0;
}

moe_status moe_layer_build_recovery(moe_layer layer, const float* U, int32_t rank, void* rec,
                                    size_t rec_bytes, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const moe_layer_desc& d = layer->d;
  size_t b_off, total;
  if (!recovery_layout(&d, &b_off, &total))
    return fail(MOE_ERR_UNSUPPORTED, "the recovery map needs a layer with a sketch form");
  if (rank != kRecRank) return fail(MOE_ERR_UNSUPPORTED, "rank must be %d", kRecRank);
  if (!U || !rec) return fail(MOE_ERR_ARG, "U and rec must be given");
  if (((uintptr_t)U % 4) != 0) return fail(MOE_ERR_ARG, "U must be 4-byte aligned");
  if (((uintptr_t)rec % kAlign) != 0)
    return fail(MOE_ERR_WORKSPACE, "the recovery buffer must be 256-byte aligned");
  if (rec_bytes < total)
    return fail(MOE_ERR_WORKSPACE, "recovery buffer has %zu bytes, needs %zu", rec_bytes, total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* base = reinterpret_cast<unsigned char*>(rec);
  hipError_t e = hipMemcpyAsync(base, U, (size_t)d.hidden * kRecRank * 4,
                                hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_rec_build(layer->w.down_t, to_dt(d.expert_dtype),
                         (size_t)d.n_experts * d.inter, d.hidden,
                         reinterpret_cast<const float*>(base),
                         reinterpret_cast<uint16_t*>(base + b_off), s);
  if (e != hipSuccess) return device_fail(e, "recovery map construction");
  layer->rec_U = reinterpret_cast<const float*>(base);
  layer->rec_b = reinterpret_cast<const uint16_t*>(base + b_off);
  return ok();
}

moe_status moe_channel_select_reader(moe_layer layer, const float* x, const int32_t* ids,
                                     const float* w, int32_t keep, int32_t mode, int32_t* kept,
                                     float* y, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  if (!layer->sketch.g)
    return fail(MOE_ERR_ARG, "no sketch: call moe_layer_build_sketch first");
  if (!layer->rec_b)
    return fail(MOE_ERR_ARG, "no recovery map: call moe_layer_build_recovery first");
  CsSketch sk = layer->sketch;
  sk.rec_b = layer->rec_b;
  sk.rec_r = layer->at<float>(layer->L.rec_r);
  float* yy = y ? y : layer->at<float>(layer->L.cs_y);
  if (moe_status st = channel_select_impl(layer, x, ids, w, keep, mode, kept, yy, stream, &sk))
    return st;
  const hipError_t e = launch_rec_apply(yy, layer->rec_U, layer->at<float>(layer->L.rec_r),
                                        layer->workgroups, layer->d.hidden,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "recovery launch");
  return ok();
}

moe_status moe_channel_select_sketch(moe_layer layer, const float* x, const int32_t* ids,
                                     const float* w, int32_t keep, int32_t mode, int32_t* kept,
                                     float* y, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  if (!layer->sketch.g)
    return fail(MOE_ERR_ARG, "no sketch: call moe_layer_build_sketch first");
  return channel_select_impl(layer, x, ids, w, keep, mode, kept, y, stream, &layer->sketch);
}

moe_status moe_channel_select_batch(moe_layer layer, const float* x, int32_t B,
                                    const int32_t* ids, const float* w, int32_t keep,
                                    int32_t* kept, int32_t* kept_count, float* y, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const moe_layer_desc& d = layer->d;
  if (d.kind != MOE_EXPERT_SWIGLU) return fail(MOE_ERR_ARG, "channel selection needs SWIGLU experts");
  if (!x || !y || !aligned16(x) || !aligned16(y))
    return fail(MOE_ERR_ARG, "x and y must be given and 16-byte aligned");
  const int mb = d.max_batch < kBselMaxBatch ? d.max_batch : kBselMaxBatch;
  if (B < 1 || B > mb) return fail(MOE_ERR_ARG, "B=%d outside [1, min(max_batch, %d)=%d]", B,
                                   kBselMaxBatch, mb);
  if ((ids == nullptr) != (w == nullptr))
    return fail(MOE_ERR_ARG, "ids and w must both be given or both be null");
  if (!ids && d.router_dtype == MOE_DTYPE_NONE)
    return fail(MOE_ERR_ARG, "routing inside the call needs a router");
  const long long maxcand =
      (long long)(d.n_experts < B * d.top_k ? d.n_experts : B * d.top_k) * d.inter;
  if (keep < 0 || keep > maxcand)
    return fail(MOE_ERR_ARG, "keep=%d outside [0, min(E, B*k)*I=%lld]", keep, maxcand);
  if (keep > 0 && !kept) return fail(MOE_ERR_ARG, "kept must be given when keep > 0");
  DT et, st, rt;
  if (moe_status e = b1_types(layer, &et, &st, &rt)) return e;
  if (et == DT::MXFP4) return fail(MOE_ERR_UNSUPPORTED, "channel selection for MXFP4 experts");
  if (maxcand > kBselMaxCandidates)
    return fail(MOE_ERR_UNSUPPORTED, "min(E, B*k)*I=%lld candidates exceed %d", maxcand,
                kBselMaxCandidates);
  if (union_lds_bytes(B, d.n_experts) > kUnionMaxLds)
    return fail(MOE_ERR_UNSUPPORTED, "E*(ceil(B/32)|1)*8 + 8E bytes exceed the union LDS budget (144 KiB)");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int32_t* rid = ids;
  const float* rw = w;
  hipError_t e = hipSuccess;
  if (!ids) {
    RouteArgs r;
    r.x = x;
    r.logits_in = nullptr;
    r.router = layer->w.router;
    r.logits = layer->at<float>(layer->L.logits);
    r.ids = layer->at<int32_t>(layer->L.ids);
    r.w = layer->at<float>(layer->L.w);
    r.H = d.hidden;
    r.E = d.n_experts;
    r.k = d.top_k;
    r.B = B;
    e = launch_route(r, rt, s);
    rid = r.ids;
    rw = r.w;
  }
  BselLaunch L;
  L.x = x;
  L.ids = rid;
  L.w = rw;
  L.n_touched = layer->at<int32_t>(layer->L.union_n);
  L.touched = layer->at<int32_t>(layer->L.union_touched);
  L.offsets = layer->at<int32_t>(layer->L.union_offsets);
  L.slots = layer->at<int32_t>(layer->L.union_slots);
  L.gate = layer->w.gate;
  L.up = layer->w.up;
  L.down_t = layer->w.down_t;
  L.sh_gate = layer->w.sh_gate;
  L.sh_up = layer->w.sh_up;
  L.sh_down_t = layer->w.sh_down_t;
  L.dnorm = layer->at<float>(layer->L.dnorm);
  L.S = layer->at<float>(layer->L.bsel_s);
  L.G = layer->at<float>(layer->L.bsel_g);
  L.desc = layer->at<int32_t>(layer->L.bsel_desc);
  L.kept_out = kept;
  L.nkept = kept_count ? kept_count : layer->at<int32_t>(layer->L.bsel_nk);
  L.sel = layer->at<int32_t>(layer->L.bsel_sel);
  L.A = layer->at<float>(layer->L.bsel_a);
  L.part = layer->at<float>(layer->L.bsel_part);
  L.y = y;
  L.H = d.hidden;
  L.I = d.inter;
  L.E = d.n_experts;
  L.k = d.top_k;
  L.B = B;
  L.NS = d.n_shared;
  L.IS = d.n_shared > 0 ? d.shared_inter : 0;
  L.keep = keep;
  if (e == hipSuccess)
    e = launch_union(rid, B, d.top_k, d.n_experts, layer->at<int32_t>(layer->L.union_n),
                     layer->at<int32_t>(layer->L.union_touched),
                     layer->at<int32_t>(layer->L.union_offsets),
                     layer->at<int32_t>(layer->L.union_slots), layer->ctrl(), s);
  if (e == hipSuccess) e = launch_bsel(L, et, st, s);
  if (e != hipSuccess) return device_fail(e, "batch channel selection launch");
  return ok();
}

moe_status moe_union_experts(const int32_t* ids, int32_t B, int32_t k, int32_t E,
                             int32_t* n_touched, int32_t* touched, int32_t* offsets,
                             int32_t* slots, void* stream) {
  if (!ids || !n_touched || !touched || !offsets || !slots)
    return fail(MOE_ERR_ARG, "null pointer");
  if (E < 1 || E > 4096 || k < 1 || k > E || B < 1 || B > 4096)
    return fail(MOE_ERR_ARG, "sizes out of range");
  if (union_lds_bytes(B, E) > kUnionMaxLds)
    return fail(MOE_ERR_UNSUPPORTED, "E*(ceil(B/32)|1)*8 + 8E bytes exceed the union LDS budget (144 KiB)");
  hipError_t e = launch_union(ids, B, k, E, n_touched, touched, offsets, slots, nullptr,
                              reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "union launch");
  return ok();
}

}  // extern "C"

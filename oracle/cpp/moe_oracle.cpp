// moe_oracle.cpp -- CPU oracle of the routed-expert FFN layer in plain C++17.
// TEST INFRASTRUCTURE ONLY: built for the host, loaded by the tests, the smoke check and the
// CPU-baseline leg of the benchmark through oracle/cpp_oracle.py; the GPU library never links
// or calls it, and it shares no code with it.
//
// Plain loops, every weight widened exactly from its storage type to double and every sum
// accumulated in double, in index order.  The optional thread split only divides independent
// outputs (router logits by expert, activations by channel, the output vector by coordinate);
// each output is summed by one thread in the same order, so results do not depend on the
// thread count.  Sources (cited by page title and section):
//
//  [MoE-arith]   "Mixture of Experts Changes the Arithmetic", section "Two Numbers Instead of
//                One": each token picks k of E experts, re-chosen in every layer; shared
//                experts are read by every token.
//  [Reader]      the jaehun.me review of arXiv:2610.37386, section "Background: channels and
//                keep rules" (channel j of expert e owns row j of G_e and V_e and column j of
//                D_e; a_j = phi(g_j . x)(v_j . x); the fixed-count top-K keep rule) and
//                "The weights-only reader" stage 2 (||d_j|| precomputed at load; eq. 1 output
//                units let channels of different experts compare).
//  [Sparse-501B] "501B of which 23B are switched on", section 2 (the experts a batch touches)
//                and section 3 (one matrix per expert for the linear sweep).
//
// Readings where the pages leave a step open: phi is silu; the router weights are a softmax
// over the k selected logits; ties in any top-k go to the lower index (for channels, the lower
// id e*I + j); shared experts carry weight 1 and are never channel candidates; MXFP4 is the OCP
// Microscaling v1.0 e2m1 element with an e8m0 scale per 32 elements.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- storage decoding (exact)
enum { OC_F64 = 0, OC_F32 = 1, OC_BF16 = 2, OC_MXFP4 = 3 };

struct Tensor {  // one row-major [rows][cols] tensor in its storage form
  int32_t dtype;
  const void* data;       // f64 / f32 / bf16 bits / MXFP4 codes (two per byte, even low)
  const uint8_t* scales;  // MXFP4: e8m0 per 32 consecutive elements of a row
};

double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// e2m1: sign, 2-bit exponent, 1-bit mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
double e2m1_value(unsigned code) {
  const unsigned e = (code >> 1) & 3u, m = code & 1u;
  const double mag = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, (int)e - 1);
  return (code & 8u) ? -mag : mag;
}

double elem(const Tensor& t, long row, long col, long cols) {
  const long i = row * cols + col;
  switch (t.dtype) {
    case OC_F64: return static_cast<const double*>(t.data)[i];
    case OC_F32: return (double)static_cast<const float*>(t.data)[i];
    case OC_BF16: return bf16_value(static_cast<const uint16_t*>(t.data)[i]);
    default: {
      const uint8_t byte = static_cast<const uint8_t*>(t.data)[i >> 1];
      const unsigned code = (i & 1) ? (byte >> 4) : (byte & 0xF);
      const int scale = (int)t.scales[row * (cols / 32) + col / 32];
      return std::ldexp(e2m1_value(code), scale - 127);
    }
  }
}

// dot of row r of t with x (double accumulation, index order)
double row_dot(const Tensor& t, long r, const double* x, long H) {
  double s = 0.0;
  for (long h = 0; h < H; ++h) s += elem(t, r, h, H) * x[h];
  return s;
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// run body(lo, hi) over [0, n) split in `threads` contiguous pieces
template <class F>
void split(long n, int threads, F body) {
  if (threads <= 1 || n < 2) {
    body(0L, n);
    return;
  }
  const int t = (int)std::min<long>(threads, n);
  std::vector<std::thread> pool;
  for (int i = 0; i < t; ++i) {
    const long lo = n * i / t, hi = n * (i + 1) / t;
    pool.emplace_back([=] { body(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

// indices of the k largest of v[0..n), largest first, ties to the lower index
std::vector<long> topk(const double* v, long n, long k) {
  std::vector<long> idx(n);
  for (long i = 0; i < n; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](long a, long b) { return v[a] > v[b]; });
  idx.resize(std::min(k, n));
  return idx;
}

// sum_j a_j d_j of one gated-MLP expert, scaled and added to y [Reader, "Background"]
void expert_add(const double* x, long H, long I, const Tensor& G, const Tensor& V,
                const Tensor& Dt, double scale, int threads, double* y) {
  std::vector<double> a(I);
  split(I, threads, [&](long j0, long j1) {
    for (long j = j0; j < j1; ++j) a[j] = silu(row_dot(G, j, x, H)) * row_dot(V, j, x, H);
  });
  split(H, threads, [&](long h0, long h1) {
    for (long h = h0; h < h1; ++h) {
      double s = 0.0;
      for (long j = 0; j < I; ++j) s += a[j] * elem(Dt, j, h, H);
      y[h] += scale * s;
    }
  });
}

}  // namespace

extern "C" {

// Widen rows x cols elements of a stored tensor to double (exact).
int oc_widen(const Tensor* t, long rows, long cols, double* out) {
  for (long r = 0; r < rows; ++r)
    for (long c = 0; c < cols; ++c) out[r * cols + c] = elem(*t, r, c, cols);
  return 0;
}

// Router logits l = W_r x for B tokens: x [B][H], W_r [E][H] -> out [B][E] [MoE-arith].
int oc_router_logits(const double* x, long B, long H, const Tensor* wr, long E, int threads,
                     double* out) {
  for (long b = 0; b < B; ++b)
    split(E, threads, [&](long e0, long e1) {
      for (long e = e0; e < e1; ++e) out[b * E + e] = row_dot(*wr, e, x + b * H, H);
    });
  return 0;
}

// Top-k of each token's logits in routing order (descending, ties to the lower id) and the
// softmax over the selected logits [MoE-arith; Reader].  logits [B][E] -> ids, w [B][k].
int oc_route(const double* logits, long B, long E, long k, int64_t* ids, double* w) {
  if (k < 1 || k > E) return 1;
  for (long b = 0; b < B; ++b) {
    const double* l = logits + b * E;
    const std::vector<long> sel = topk(l, E, k);
    double m = l[sel[0]];
    for (long i = 1; i < k; ++i) m = std::max(m, l[sel[i]]);
    double z = 0.0;
    for (long i = 0; i < k; ++i) z += std::exp(l[sel[i]] - m);
    for (long i = 0; i < k; ++i) {
      ids[b * k + i] = sel[i];
      w[b * k + i] = std::exp(l[sel[i]] - m) / z;
    }
  }
  return 0;
}

// a_j = silu(g_j . x) (v_j . x) for every channel of one expert -> a [I] [Reader].
int oc_expert_activations(const double* x, long H, long I, const Tensor* G, const Tensor* V,
                          int threads, double* a) {
  split(I, threads, [&](long j0, long j1) {
    for (long j = j0; j < j1; ++j) a[j] = silu(row_dot(*G, j, x, H)) * row_dot(*V, j, x, H);
  });
  return 0;
}

// The layer for one token with a given routing: y = sum_i w_i sum_j a_j d_j over the n listed
// experts (G[i], V[i], Dt[i], each [I][H]) + sum over the ns shared experts (weight 1, each
// [Is][H]) [Reader, "Background"; MoE-arith].  y [H] is overwritten.
int oc_layer_given(const double* x, long H, long I, long n, const double* w, const Tensor* G,
                   const Tensor* V, const Tensor* Dt, long ns, long Is, const Tensor* SG,
                   const Tensor* SV, const Tensor* SD, int threads, double* y) {
  for (long h = 0; h < H; ++h) y[h] = 0.0;
  for (long i = 0; i < n; ++i) expert_add(x, H, I, G[i], V[i], Dt[i], w[i], threads, y);
  for (long s = 0; s < ns; ++s) expert_add(x, H, Is, SG[s], SV[s], SD[s], 1.0, threads, y);
  return 0;
}

// ||d_j||_2 of every row of D^T [I][H] [Reader, "The weights-only reader", stage 2].
int oc_down_norms(const Tensor* Dt, long I, long H, double* out) {
  for (long j = 0; j < I; ++j) {
    double s = 0.0;
    for (long h = 0; h < H; ++h) {
      const double d = elem(*Dt, j, h, H);
      s += d * d;
    }
    out[j] = std::sqrt(s);
  }
  return 0;
}

// Fixed-count top-K channel keep rule for one token [Reader, "Background"; stage 2, eq. 1].
// Candidates: the k*I channels of the routed experts (slot i holds expert ids[i]; G/V/Dt[i]
// its tensors; dnorm [k][I] their down-row norms).  Score s = |silu(g_j . x)| * ||d_j||, times
// w_i when mode = 1.  The `keep` best (ties to the lower id e*I + j) are computed from their full
// rows; the rest are never read.  kept [keep] receives their ids ascending; y [H] = kept sum +
// shared experts.
int oc_channel_select(const double* x, long H, long I, long k, const int64_t* ids,
                      const double* w, const Tensor* G, const Tensor* V, const Tensor* Dt,
                      const double* dnorm, long keep, int mode, long ns, long Is,
                      const Tensor* SG, const Tensor* SV, const Tensor* SD, int threads,
                      int64_t* kept, double* y) {
  const long n = k * I;
  if (keep < 0 || keep > n) return 1;
  std::vector<double> g(n), s(n);
  split(n, threads, [&](long f0, long f1) {
    for (long f = f0; f < f1; ++f) {
      const long i = f / I, j = f % I;
      g[f] = row_dot(G[i], j, x, H);
      s[f] = std::fabs(silu(g[f])) * dnorm[f] * (mode == 1 ? w[i] : 1.0);
    }
  });
  std::vector<long> order(n);
  for (long f = 0; f < n; ++f) order[f] = f;
  auto cid = [&](long f) { return ids[f / I] * I + f % I; };
  std::sort(order.begin(), order.end(), [&](long a, long b) {
    return s[a] != s[b] ? s[a] > s[b] : cid(a) < cid(b);
  });
  order.resize(keep);
  std::vector<double> a(keep);
  split(keep, threads, [&](long q0, long q1) {
    for (long q = q0; q < q1; ++q) {
      const long f = order[q], i = f / I, j = f % I;
      a[q] = w[i] * silu(g[f]) * row_dot(V[i], j, x, H);
    }
  });
  for (long h = 0; h < H; ++h) y[h] = 0.0;
  split(H, threads, [&](long h0, long h1) {
    for (long h = h0; h < h1; ++h) {
      double acc = 0.0;
      for (long q = 0; q < keep; ++q) {
        const long f = order[q];
        acc += a[q] * elem(Dt[f / I], f % I, h, H);
      }
      y[h] = acc;
    }
  });
  for (long sidx = 0; sidx < ns; ++sidx)
    expert_add(x, H, Is, SG[sidx], SV[sidx], SD[sidx], 1.0, threads, y);
  std::vector<int64_t> out(keep);
  for (long q = 0; q < keep; ++q) out[q] = cid(order[q]);
  std::sort(out.begin(), out.end());
  for (long q = 0; q < keep; ++q) kept[q] = out[q];
  return 0;
}

// The distinct experts a batch touches and each one's (token, slot) list [Sparse-501B, 2]:
// ids [B][k] in [0, E) -> n_touched, touched (ascending), offsets [E+1] (prefix sum of
// per-expert counts), slots [B*k] (flat b*k+i grouped by expert, ascending within one).
int oc_union_experts(const int64_t* ids, long B, long k, long E, int64_t* n_touched,
                     int64_t* touched, int64_t* offsets, int64_t* slots) {
  std::vector<long> count(E, 0);
  for (long f = 0; f < B * k; ++f) {
    if (ids[f] < 0 || ids[f] >= E) return 1;
    ++count[ids[f]];
  }
  offsets[0] = 0;
  for (long e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + count[e];
  std::vector<long> fill(offsets, offsets + E);
  for (long f = 0; f < B * k; ++f) slots[fill[ids[f]]++] = f;
  long nt = 0;
  for (long e = 0; e < E; ++e)
    if (count[e]) touched[nt++] = e;
  *n_touched = nt;
  return 0;
}

// Linear experts: Y[b] = sum_i w[b][i] M_{ids[b][i]} X[b], M stacked [E][I][H] [Sparse-501B, 3].
int oc_linear_moe(const double* X, long B, long H, long I, long k, const int64_t* ids,
                  const double* w, const Tensor* M, long E, int threads, double* Y) {
  for (long b = 0; b < B; ++b) {
    for (long i = 0; i < k; ++i)
      if (ids[b * k + i] < 0 || ids[b * k + i] >= E) return 1;
    split(I, threads, [&](long r0, long r1) {
      for (long r = r0; r < r1; ++r) {
        double acc = 0.0;
        for (long i = 0; i < k; ++i)
          acc += w[b * k + i] * row_dot(*M, ids[b * k + i] * I + r, X + b * H, H);
        Y[b * I + r] = acc;
      }
    });
  }
  return 0;
}

}  // extern "C"

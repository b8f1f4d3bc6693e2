// C ABI of the LaCT layer: host-side validation, launch planning and the
// stream-ordered chunk scan.  Declarations and conventions: include/lact.h.
#include "lact.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "lact_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(LACT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------------ profiling
struct ProfRec {
  int phase;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// RAII bracket around one phase's launches on a stream.
struct PhaseTimer {
  int phase;
  hipStream_t stream;
  hipEvent_t start = nullptr;
  PhaseTimer(int p, hipStream_t s) : phase(p), stream(s) {
    if (!g_prof_on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    start = prof_event();
    if (start) (void)hipEventRecord(start, stream);
  }
  ~PhaseTimer() {
    if (!g_prof_on || start == nullptr) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t stop = prof_event();
    if (stop == nullptr) return;
    (void)hipEventRecord(stop, stream);
    g_prof_recs.push_back({phase, start, stop});
  }
};

// ------------------------------------------------------------------- planning
struct Plan {
  int P = 0, d = 0, h = 0;
  bool bf16 = false;
  bool mfma = false;
  bool momentum = false;
  bool muon = false;
  bool split = false;  // bf16 inputs, ~fp32 derived operands
  bool linear = false; // linear fast net (one d x d matrix per pair)
  bool pm = false;     // a learning rate per token and matrix
  int norm = 0;        // lact_norm_mode
};

// Token splits of one chunk's gradient.  Derived from the shapes only (not
// from the device), so results are reproducible on any GPU.
struct Splits {
  int S;
  int64_t tps;
};

struct SplitRule {
  int64_t wgs_per_split;  // workgroups launched per split
  int64_t target_wgs;     // aim for about this many workgroups in total
  int64_t min_tokens;     // never split below this many tokens
  int64_t align;          // tokens per split are a multiple of this
};

// Upper bound of the split count for n tokens; non-decreasing in n, and
// plan_splits never exceeds it (the workspace is sized with it).
int64_t split_bound(const SplitRule& r, int64_t n) {
  int64_t S = (r.target_wgs + r.wgs_per_split - 1) / r.wgs_per_split;
  const int64_t by_size = (n + r.min_tokens - 1) / r.min_tokens;
  if (S > by_size) S = by_size;
  if (S > 4096) S = 4096;
  if (S < 1) S = 1;
  return S;
}

Splits plan_splits(const SplitRule& r, int64_t n) {
  int64_t S = split_bound(r, n);
  int64_t tps = (n + S - 1) / S;
  tps = (tps + r.align - 1) / r.align * r.align;
  S = (n + tps - 1) / tps;
  return {static_cast<int>(S), tps};
}

// Generic kernel: one workgroup per (split, 32 hidden units, pair).
SplitRule generic_rule(const Plan& p) {
  return {static_cast<int64_t>(p.P) * (p.h / 32), 1024, 256, 128};
}

// Linear fast net: one workgroup per (split, pair), 64-token tiles.
SplitRule linear_rule(const Plan& p) { return {static_cast<int64_t>(p.P), 1024, 256, 64}; }

// Which chunk-gradient kernel runs.  The MFMA kernels read 16-byte rows with
// 32-bit offsets inside a pair's rows: they need aligned K, V and strides and
// n d < 2^31.  With split products the d = 64 kernel runs one workgroup per
// CU (one wavefront per SIMD); the d = 128 kernel one workgroup of eight
// wavefronts (a 128-unit hidden slice) per CU.
enum class GradKind { Generic, D64, D128W };

// Above this many token splits the Muon tail's partial sum runs as a
// separate all-CU kernel.
constexpr int kTailSplitsInline = 8;

struct GradChoice {
  GradKind kind;
  int stage;        // token splits are multiples of this
  int wgs_per_cu;   // resident workgroups per CU
  int hid_per_wg;   // hidden units per workgroup
};

GradChoice grad_choice(const Plan& p, bool aligned, int64_t n) {
  const bool fits = aligned && n * p.d < (static_cast<int64_t>(1) << 31);
  if (p.mfma && fits) {
    if (lact::grad_d64_shape_ok(p.d, p.h)) return {GradKind::D64, 128, p.split ? 1 : 2, 128};
    // d = 128: 16 hidden units per wavefront, two wavefronts per SIMD
    if (lact::grad_d128w_shape_ok(p.d, p.h))
      return {GradKind::D128W, lact::grad_d128w_stage_tokens(p.split), lact::grad_d128w_workgroups_per_cu(),
              lact::grad_d128w_hidden_per_workgroup()};
  }
  return {GradKind::Generic, 1, 0, 0};
}

// MFMA kernels: one workgroup per (split, hidden slice, pair), sized to
// one round of resident workgroups on 256 CUs, rounding the split count
// down so no second round is started.
SplitRule mfma_rule(const Plan& p, const GradChoice& k) {
  const int64_t per_split = static_cast<int64_t>(p.P) * (p.h / k.hid_per_wg);
  const int64_t resident = 256 * k.wgs_per_cu;
  int64_t target = (resident / per_split) * per_split;
  if (target < per_split) target = per_split;
  return {per_split, target, 4 * static_cast<int64_t>(k.stage), k.stage};
}

bool finite(float x) { return std::isfinite(x); }

int check_config(const lact_config* c, Plan* p) {
  if (c == nullptr) return fail(LACT_ERR_INVALID_ARG, "config is NULL");
  if (c->B < 1 || c->H < 1) return fail(LACT_ERR_INVALID_ARG, "B=%d H=%d must be >= 1", c->B, c->H);
  if (static_cast<int64_t>(c->B) * c->H > 65535)
    return fail(LACT_ERR_UNSUPPORTED, "B*H=%lld above 65535", (long long)c->B * c->H);
  if (c->net != LACT_NET_SWIGLU && c->net != LACT_NET_LINEAR)
    return fail(LACT_ERR_INVALID_ARG, "net %d unknown", c->net);
  const bool linear = c->net == LACT_NET_LINEAR;
  if (c->d < 1 || (!linear && c->h < 1))
    return fail(LACT_ERR_INVALID_ARG, "d=%d h=%d must be >= 1", c->d, c->h);
  if (c->io_dtype != LACT_F32 && c->io_dtype != LACT_BF16)
    return fail(LACT_ERR_INVALID_ARG, "io_dtype %d unknown", c->io_dtype);
  if (c->opt != LACT_OPT_GD && c->opt != LACT_OPT_MOMENTUM && c->opt != LACT_OPT_MUON)
    return fail(LACT_ERR_INVALID_ARG, "opt %d unknown", c->opt);
  if (!finite(c->beta) || c->beta < 0.f || c->beta >= 1.f)
    return fail(LACT_ERR_INVALID_ARG, "beta %g outside [0, 1)", c->beta);
  if (c->opt == LACT_OPT_MUON) {
    if (c->ns_iters < 0 || c->ns_iters > 32)
      return fail(LACT_ERR_INVALID_ARG, "ns_iters %d outside [0, 32]", c->ns_iters);
    if (!finite(c->ns_a) || !finite(c->ns_b) || !finite(c->ns_c) || !finite(c->ns_eps) || c->ns_eps < 0.f)
      return fail(LACT_ERR_INVALID_ARG, "Newton-Schulz coefficients must be finite, eps >= 0");
  }
  if (!finite(c->step)) return fail(LACT_ERR_INVALID_ARG, "step must be finite");
  if (c->products != LACT_PRODUCTS_BF16 && c->products != LACT_PRODUCTS_SPLIT &&
      c->products != LACT_PRODUCTS_AUTO)
    return fail(LACT_ERR_INVALID_ARG, "products %d unknown", c->products);
  if (!finite(c->norm_eps) || c->norm_eps <= 0.f)
    return fail(LACT_ERR_INVALID_ARG, "norm_eps %g must be finite and > 0", c->norm_eps);
  if (c->norm_mode != LACT_NORM_UNIT && c->norm_mode != LACT_NORM_KEEP && c->norm_mode != LACT_NORM_NONE)
    return fail(LACT_ERR_INVALID_ARG, "norm_mode %d unknown", c->norm_mode);
  if (c->eta_mode != LACT_ETA_SHARED && c->eta_mode != LACT_ETA_PER_MATRIX)
    return fail(LACT_ERR_INVALID_ARG, "eta_mode %d unknown", c->eta_mode);
  if (linear) {
    if (!lact::linear_shape_ok(c->d))
      return fail(LACT_ERR_UNSUPPORTED, "linear fast net: d=%d not in {16, 32, 64, 128}", c->d);
    if (c->eta_mode != LACT_ETA_SHARED)
      return fail(LACT_ERR_UNSUPPORTED, "linear fast net: one rate per token (eta_mode 0)");
    p->P = c->B * c->H;
    p->d = c->d;
    p->h = c->d;
    p->bf16 = c->io_dtype == LACT_BF16;
    p->momentum = c->opt == LACT_OPT_MOMENTUM || (c->opt == LACT_OPT_MUON && c->beta > 0.f);
    p->muon = c->opt == LACT_OPT_MUON;
    p->linear = true;
    p->norm = c->norm_mode;
    return LACT_OK;
  }
  if (c->norm_mode == LACT_NORM_NONE)
    return fail(LACT_ERR_UNSUPPORTED, "norm_mode LACT_NORM_NONE is built for the linear fast net only");
  const int mf = lact_mfma_path(c->d, c->h, c->io_dtype);
  if (mf < 0)
    return fail(LACT_ERR_UNSUPPORTED,
                "(d, h) = (%d, %d) not supported: d in {32, 64, 128}, h a multiple of 32 in [32, 1024]",
                c->d, c->h);
  p->P = c->B * c->H;
  p->d = c->d;
  p->h = c->h;
  p->bf16 = c->io_dtype == LACT_BF16;
  p->mfma = mf == 1;
  p->momentum = c->opt == LACT_OPT_MOMENTUM || (c->opt == LACT_OPT_MUON && c->beta > 0.f);
  p->muon = c->opt == LACT_OPT_MUON;
  p->split = p->bf16 && c->products == LACT_PRODUCTS_SPLIT;
  p->norm = c->norm_mode;
  p->pm = c->eta_mode == LACT_ETA_PER_MATRIX;
  return LACT_OK;
}

// bf16 operand products under Muon.  Newton-Schulz maps every singular value
// of the gradient towards one, so operand rounding that moves the small
// singular directions moves the update as much as the large ones: on chunks
// of ~100 keys bf16 operands alone change the result by ~7e-2, and over a scan
// the change compounds by ~1.4x per chunk (3e-3 after one chunk of 4096
// keys, 1.5e-2 after five, 0.25 after fourteen).  Inside these limits bf16
// products stay within 2e-2 of the exact result; outside them AUTO keeps the
// derived operands split and an explicit request for bf16 is refused.
constexpr int64_t kMuonBf16MinKeys = 1024;
constexpr int64_t kMuonBf16MaxChunks = 4;

// Settles the product precision of a run of `chunks` chunks of `n` keys.
int resolve_products(const lact_config* c, Plan* p, int64_t n, int64_t chunks) {
  if (!p->bf16 || p->linear) {
    p->split = false;
    return LACT_OK;
  }
  const bool bf16_ok = !p->muon || (n >= kMuonBf16MinKeys && chunks <= kMuonBf16MaxChunks);
  if (c->products == LACT_PRODUCTS_SPLIT) {
    p->split = true;
  } else if (c->products == LACT_PRODUCTS_AUTO) {
    p->split = !bf16_ok;
  } else if (!bf16_ok) {
    return fail(LACT_ERR_UNSUPPORTED,
                "bf16 operand products with Muon need chunks of >= %lld keys and at most %lld chunks "
                "(got %lld keys x %lld chunks): use LACT_PRODUCTS_SPLIT or LACT_PRODUCTS_AUTO",
                (long long)kMuonBf16MinKeys, (long long)kMuonBf16MaxChunks, (long long)n,
                (long long)chunks);
  } else {
    p->split = false;
  }
  return LACT_OK;
}

int check_state(const Plan& p, const lact_state* st, bool need_m) {
  if (st == nullptr) return fail(LACT_ERR_INVALID_ARG, "state is NULL");
  if (p.linear) {
    if (!st->W1) return fail(LACT_ERR_INVALID_ARG, "linear fast net: W1 must be non-NULL");
    if (need_m && p.momentum && !st->M1)
      return fail(LACT_ERR_INVALID_ARG, "this optimizer keeps momentum: M1 must be non-NULL");
    return LACT_OK;
  }
  if (!st->W1 || !st->W2 || !st->W3) return fail(LACT_ERR_INVALID_ARG, "W1, W2, W3 must be non-NULL");
  if (need_m && p.momentum && (!st->M1 || !st->M2 || !st->M3))
    return fail(LACT_ERR_INVALID_ARG, "this optimizer keeps momentum: M1, M2, M3 must be non-NULL");
  return LACT_OK;
}

// Workspace sections (bytes), each 256-byte aligned.
struct WsLayout {
  size_t partials = 0, dir = 0, ns = 0, wb = 0, wb2 = 0, total = 0;
  bool has_wb = false;  // section for bf16 copies of W1, W2, W3 (P 3 h d values)
  bool has_wb2 = false;  // a second such section (Muon: the copy of chunk c is read while the next is written)
};

WsLayout ws_layout(const Plan& p, int64_t max_chunk_kv) {
  WsLayout w;
  const int64_t n = max_chunk_kv < 1 ? 1 : max_chunk_kv;
  if (p.linear) {
    // partials [P, S, d d] | dir [P, d d] | Newton-Schulz scratch [P, 4 d d]
    const size_t dd = static_cast<size_t>(p.d) * p.d;
    const int64_t S = split_bound(linear_rule(p), n);
    size_t off = 0;
    w.partials = off;
    off += align_up(sizeof(float) * dd * p.P * static_cast<size_t>(S));
    w.dir = off;
    off += align_up(sizeof(float) * dd * p.P);
    w.ns = off;
    if (p.muon) off += align_up(sizeof(float) * 4 * dd * p.P);
    w.wb = off;
    w.total = off;
    return w;
  }
  const size_t per = static_cast<size_t>(3) * p.h * p.d;
  // every kernel the update may pick for up to n tokens
  // (for either product precision: AUTO settles it per call)
  int64_t S = split_bound(generic_rule(p), n);
  for (int split = 0; split < 2; ++split) {
    Plan q = p;
    q.split = q.bf16 && split;
    const GradChoice k = grad_choice(q, true, 0);
    if (k.kind != GradKind::Generic) {
      const int64_t sm = split_bound(mfma_rule(q, k), n);
      if (sm > S) S = sm;
    }
  }
  size_t off = 0;
  w.partials = off;
  off += align_up(sizeof(float) * per * p.P * static_cast<size_t>(S));
  w.dir = off;
  off += align_up(sizeof(float) * per * p.P);
  w.ns = off;
  if (p.muon) off += align_up(sizeof(float) * lact::ns_simple_scratch_floats(p.P, p.d, p.h));
  // the chunk scan hands the updated weights to the next query read as bf16
  // operands (written by the update tail), where the MFMA query read runs
  w.wb = off;
  w.has_wb = p.bf16 && lact::apply_mfma_shape_ok(p.d, p.h);
  if (w.has_wb) off += align_up(sizeof(uint16_t) * per * p.P);
  // with Muon the update tail of chunk c and the query read of chunk c can
  // share a launch (the read takes the CUs the tail leaves): the read's
  // copy and the tail's new one alternate between two sections
  w.wb2 = off;
  w.has_wb2 = w.has_wb && p.muon && lact::muon_tail_apply_ok(p.d, p.h, p.P);
  if (w.has_wb2) off += align_up(sizeof(uint16_t) * per * p.P);
  w.total = off;
  return w;
}

int check_ws(const Plan& p, int64_t max_chunk_kv, void* ws, size_t ws_bytes, WsLayout* out) {
  *out = ws_layout(p, max_chunk_kv);
  if (ws_bytes < out->total)
    return fail(LACT_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes needed", ws_bytes,
                out->total);
  if (out->total > 0 && ws == nullptr) return fail(LACT_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(LACT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return LACT_OK;
}

size_t io_bytes(const Plan& p) { return p.bf16 ? 2 : 4; }

// One update on validated arguments (steps 2-4).  With wb non-NULL the
// update tail also stores the new W1, W2, W3 as bf16 there (three arrays of
// P h d values) where its kernels support it; *wb_written says whether it did.
// The chunk gradient's split partials (the kernel chosen by shape, alignment
// and product precision); *sp receives the split plan.
int launch_gradient(const lact_config* c, const Plan& p, const lact_state* st, const void* K, const void* V,
                    const float* eta, int64_t n, int64_t kv_stride, int64_t eta_stride, float* partials,
                    hipStream_t s, Splits* sp_out) {
  const bool aligned = (reinterpret_cast<uintptr_t>(K) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(V) % 16 == 0) && (kv_stride % 8 == 0);
  const GradChoice gk = grad_choice(p, aligned, n);
  const Splits sp = plan_splits(gk.kind == GradKind::Generic ? generic_rule(p) : mfma_rule(p, gk), n);
  *sp_out = sp;
  PhaseTimer t(0, s);
  lact::GradArgs g{};
  g.K = K;
  g.V = V;
  g.eta = eta;
  g.n = n;
  g.kv_stride = kv_stride;
  g.eta_stride = eta_stride;
  // per-matrix rates: three blocks of P pairs each
  g.eta_mat = c->eta_mode == LACT_ETA_PER_MATRIX ? static_cast<int64_t>(p.P) * eta_stride : 0;
  g.W1 = st->W1;
  g.W2 = st->W2;
  g.W3 = st->W3;
  g.partials = partials;
  g.P = p.P;
  g.d = p.d;
  g.h = p.h;
  g.S = sp.S;
  g.tps = sp.tps;
  g.bf16 = p.bf16;
  hipError_t e;
  switch (gk.kind) {
    case GradKind::D64: e = lact::launch_grad_d64(g, p.split, s); break;
    case GradKind::D128W: e = lact::launch_grad_d128w(g, p.split, s); break;
    default: e = lact::launch_grad_simple(g, s); break;
  }
  if (e != hipSuccess) return hip_fail(e, "gradient kernel");
  return LACT_OK;
}

// One update of the linear fast net: split-K gradient, then reduction with
// momentum, Newton-Schulz (Muon) and the step with the row rule.
int run_update_linear(const lact_config* c, const Plan& p, const lact_state* st, const void* K,
                      const void* V, const float* eta, int64_t n, int64_t kv_stride, int64_t eta_stride,
                      char* ws, const WsLayout& L, hipStream_t s) {
  const Splits sp = plan_splits(linear_rule(p), n);
  float* partials = reinterpret_cast<float*>(ws + L.partials);
  hipError_t e;
  {
    PhaseTimer t(0, s);
    lact::LinGradArgs g{};
    g.K = K;
    g.V = V;
    g.eta = eta;
    g.n = n;
    g.kv_stride = kv_stride;
    g.eta_stride = eta_stride;
    g.partials = partials;
    g.P = p.P;
    g.d = p.d;
    g.S = sp.S;
    g.tps = sp.tps;
    g.bf16 = p.bf16;
    e = lact::launch_lin_grad(g, s);
    if (e != hipSuccess) return hip_fail(e, "linear gradient kernel");
  }
  PhaseTimer t(1, s);
  lact::LinTailArgs a{};
  a.partials = partials;
  a.splits = sp.S;
  a.dir = reinterpret_cast<float*>(ws + L.dir);
  a.scratch = reinterpret_cast<float*>(ws + L.ns);
  a.W = st->W1;
  a.M = p.momentum ? st->M1 : nullptr;
  a.beta = c->beta;
  a.step = c->step;
  a.norm_eps = c->norm_eps;
  a.norm = p.norm;
  a.muon = p.muon;
  a.iters = c->ns_iters;
  a.a = c->ns_a;
  a.b = c->ns_b;
  a.c = c->ns_c;
  a.ns_eps = c->ns_eps;
  a.P = p.P;
  a.d = p.d;
  e = lact::launch_lin_tail(a, s);
  if (e != hipSuccess) return hip_fail(e, "linear update-tail kernels");
  return LACT_OK;
}

// Whether a Muon update runs the bf16-mode matrix-core tail (which also
// writes the bf16 weight copy): bf16 mode, a supported shape, and W and M
// 16-byte aligned (the tail moves them in 16-byte pieces).
bool muon_mfma_tail(const Plan& p, const lact_state* st) {
  const bool state_aligned =
      ((reinterpret_cast<uintptr_t>(st->W1) | reinterpret_cast<uintptr_t>(st->W2) |
        reinterpret_cast<uintptr_t>(st->W3) | reinterpret_cast<uintptr_t>(st->M1) |
        reinterpret_cast<uintptr_t>(st->M2) | reinterpret_cast<uintptr_t>(st->M3)) & 15) == 0;
  return p.muon && !p.linear && p.bf16 && lact::ns_mfma_shape_ok(p.d, p.h) && state_aligned;
}

int run_update(const lact_config* c, const Plan& p, const lact_state* st, const void* K,
               const void* V, const float* eta, int64_t n, int64_t kv_stride,
               int64_t eta_stride, char* ws, const WsLayout& L, hipStream_t s,
               uint16_t* wb = nullptr, bool* wb_written = nullptr,
               const lact::ApplyArgs* fused_read = nullptr) {
  if (wb_written != nullptr) *wb_written = false;
  if (p.linear) return run_update_linear(c, p, st, K, V, eta, n, kv_stride, eta_stride, ws, L, s);
  float* partials = reinterpret_cast<float*>(ws + L.partials);
  float* dir = reinterpret_cast<float*>(ws + L.dir);
  Splits sp;
  int rc = launch_gradient(c, p, st, K, V, eta, n, kv_stride, eta_stride, partials, s, &sp);
  if (rc) return rc;
  hipError_t e;
  lact::TailArgs ta{};
  ta.partials = partials;
  ta.splits = sp.S;
  if (p.momentum) {
    ta.M1 = st->M1;
    ta.M2 = st->M2;
    ta.M3 = st->M3;
  }
  ta.beta = c->beta;
  ta.W1 = st->W1;
  ta.W2 = st->W2;
  ta.W3 = st->W3;
  ta.step = c->step;
  ta.norm_eps = c->norm_eps;
  ta.norm_keep = c->norm_mode == LACT_NORM_KEEP;
  ta.P = p.P;
  ta.d = p.d;
  ta.h = p.h;
  ta.iters = c->ns_iters;
  ta.a = c->ns_a;
  ta.b = c->ns_b;
  ta.c = c->ns_c;
  ta.eps = c->ns_eps;
  const int64_t phd = static_cast<int64_t>(p.P) * p.h * p.d;
  auto with_wb = [&]() {
    if (wb == nullptr) return;
    ta.Wb1 = wb;
    ta.Wb2 = wb + phd;
    ta.Wb3 = wb + 2 * phd;
    if (wb_written != nullptr) *wb_written = true;
  };
  if (!p.muon) {
    // GD / momentum: one row-wise kernel for reduction, momentum, step, unit rows
    PhaseTimer t(1, s);
    with_wb();
    if (fused_read != nullptr) return fail(LACT_ERR_HIP, "internal: fused query read without the Muon tail");
    e = lact::launch_reduce_step(ta, s);
    if (e != hipSuccess) return hip_fail(e, "update-tail kernel");
    return LACT_OK;
  }
  if (muon_mfma_tail(p, st)) {
    // bf16 mode Muon: one kernel per matrix for reduction, momentum,
    // split-bf16 MFMA Newton-Schulz, step and unit rows.  With many splits
    // the partial sum goes first to a kernel that spreads it over every CU
    // (the tail then reads one reduced gradient per matrix).
    PhaseTimer t(1, s);
    if (sp.S > kTailSplitsInline) {
      lact::ReduceArgs r{};
      r.partials = partials;
      r.dir = dir;
      if (p.momentum) {
        r.M1 = st->M1;
        r.M2 = st->M2;
        r.M3 = st->M3;
      }
      r.beta = c->beta;
      r.P = p.P;
      r.d = p.d;
      r.h = p.h;
      r.S = sp.S;
      e = lact::launch_reduce(r, s);
      if (e != hipSuccess) return hip_fail(e, "reduction kernel");
      ta.partials = dir;
      ta.splits = 1;
      ta.M1 = ta.M2 = ta.M3 = nullptr;
    }
    with_wb();
    if (fused_read != nullptr) {
      e = lact::launch_muon_tail_apply(ta, *fused_read, s);
      if (e != hipSuccess) return hip_fail(e, "Muon update-tail + query-read kernel");
      return LACT_OK;
    }
    e = lact::launch_muon_tail(ta, s);
    if (e != hipSuccess) return hip_fail(e, "Muon update-tail kernel");
    return LACT_OK;
  }
  if (fused_read != nullptr) return fail(LACT_ERR_HIP, "internal: fused query read without the matrix-core Muon tail");
  // fp32 arithmetic Muon: reduction (+momentum), Newton-Schulz, step + unit rows
  {
    PhaseTimer t(1, s);
    lact::ReduceArgs r{};
    r.partials = partials;
    r.dir = dir;
    if (p.momentum) {
      r.M1 = st->M1;
      r.M2 = st->M2;
      r.M3 = st->M3;
    }
    r.beta = c->beta;
    r.P = p.P;
    r.d = p.d;
    r.h = p.h;
    r.S = sp.S;
    e = lact::launch_reduce(r, s);
    if (e != hipSuccess) return hip_fail(e, "reduction kernel");
  }
  {
    PhaseTimer t(2, s);
    lact::NSArgs a{};
    a.dir = dir;
    a.scratch = reinterpret_cast<float*>(ws + L.ns);
    a.P = p.P;
    a.d = p.d;
    a.h = p.h;
    a.iters = c->ns_iters;
    a.a = c->ns_a;
    a.b = c->ns_b;
    a.c = c->ns_c;
    a.eps = c->ns_eps;
    e = lact::launch_ns_simple(a, s);
    if (e != hipSuccess) return hip_fail(e, "Newton-Schulz kernel");
  }
  {
    PhaseTimer t(3, s);
    lact::StepArgs a{};
    a.W1 = st->W1;
    a.W2 = st->W2;
    a.W3 = st->W3;
    a.dir = dir;
    a.step = c->step;
    a.norm_eps = c->norm_eps;
    a.norm_keep = c->norm_mode == LACT_NORM_KEEP;
    a.P = p.P;
    a.d = p.d;
    a.h = p.h;
    e = lact::launch_step_norm(a, s);
    if (e != hipSuccess) return hip_fail(e, "step/normalise kernel");
  }
  return LACT_OK;
}

// Query read; wb (or NULL): bf16 copies of the current W1, W2, W3 as the
// update tail stores them.
// Arguments of the SwiGLU query read; *mfma: the matrix-core kernel applies
// (bf16, a supported shape, 16-byte aligned Q and O rows); only then is the
// bf16 copy wb (or NULL) used.
lact::ApplyArgs apply_args(const Plan& p, const lact_state* st, const void* Q, void* O, int64_t m,
                           int64_t q_stride, const uint16_t* wb, bool* mfma) {
  lact::ApplyArgs a{};
  a.Q = Q;
  a.O = O;
  a.m = m;
  a.q_stride = q_stride;
  a.W1 = st->W1;
  a.W2 = st->W2;
  a.W3 = st->W3;
  a.P = p.P;
  a.d = p.d;
  a.h = p.h;
  a.bf16 = p.bf16;
  a.w_vec = ((reinterpret_cast<uintptr_t>(st->W1) | reinterpret_cast<uintptr_t>(st->W2) |
              reinterpret_cast<uintptr_t>(st->W3)) & 15) == 0;
  *mfma = p.bf16 && lact::apply_mfma_shape_ok(p.d, p.h) && reinterpret_cast<uintptr_t>(Q) % 16 == 0 &&
          reinterpret_cast<uintptr_t>(O) % 16 == 0 && q_stride % 8 == 0;
  if (*mfma && wb != nullptr) {
    const int64_t phd = static_cast<int64_t>(p.P) * p.h * p.d;
    a.Wb1 = wb;
    a.Wb2 = wb + phd;
    a.Wb3 = wb + 2 * phd;
  }
  return a;
}

int run_apply(const Plan& p, const lact_state* st, const void* Q, void* O, int64_t m,
              int64_t q_stride, hipStream_t s, const uint16_t* wb = nullptr) {
  PhaseTimer t(4, s);
  if (p.linear) {
    lact::LinApplyArgs a{};
    a.Q = Q;
    a.O = O;
    a.m = m;
    a.q_stride = q_stride;
    a.W = st->W1;
    a.P = p.P;
    a.d = p.d;
    a.bf16 = p.bf16;
    hipError_t e = lact::launch_lin_apply(a, s);
    if (e != hipSuccess) return hip_fail(e, "linear query-read kernel");
    return LACT_OK;
  }
  bool use_mfma = false;
  const lact::ApplyArgs a = apply_args(p, st, Q, O, m, q_stride, wb, &use_mfma);
  hipError_t e = use_mfma ? lact::launch_apply_mfma(a, s) : lact::launch_apply_simple(a, s);
  if (e != hipSuccess) return hip_fail(e, "query-read kernel");
  return LACT_OK;
}

// ------------------------------------------------------------------ backward
// Workspace of the backward pass (bytes, 256-byte aligned sections).
struct BwLayout {
  WsLayout fwd;           // the forward update's own workspace, at offset 0
  size_t ckW = 0, ckM = 0;  // N + 1 slots of W1 | W2 | W3 (and of M1 | M2 | M3)
  size_t cot = 0, dM = 0, g = 0, dir = 0, ddir = 0, pc = 0, t = 0;  // [P, 3hd] each
  size_t X = 0;           // three [P, max(chunk_kv, chunk_q), h] factor arrays
  size_t part = 0, part2 = 0;  // contraction partials [P, S, 3hd] (chunk gradient's, query read's)
  size_t ns = 0;          // Newton-Schulz VJP scratch
  size_t op = 0;          // bf16 hi | lo operands of the matrix-core token kernels [P][6][2][h][d]
  size_t total = 0;
  int64_t rows = 0;       // max(chunk_kv, chunk_q)
  int S = 1;
};

SplitRule backward_rule(const Plan& p) { return {static_cast<int64_t>(p.P) * (p.h / 32), 1024, 256, 32}; }

BwLayout bw_layout(const lact_config* c, const Plan& p, int64_t N, int64_t chunk_kv, int64_t chunk_q) {
  BwLayout b;
  b.fwd = ws_layout(p, chunk_kv);
  const size_t per = static_cast<size_t>(3) * p.h * p.d * p.P;  // floats of one state
  b.rows = chunk_kv > chunk_q ? chunk_kv : chunk_q;
  b.S = static_cast<int>(split_bound(backward_rule(p), b.rows));
  size_t off = b.fwd.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  b.ckW = take(sizeof(float) * per * static_cast<size_t>(N + 1));
  b.ckM = take(p.momentum ? sizeof(float) * per * static_cast<size_t>(N + 1) : 0);
  b.cot = take(sizeof(float) * per);
  b.dM = take(sizeof(float) * per);
  b.g = take(sizeof(float) * per);
  b.dir = take(sizeof(float) * per);
  b.ddir = take(sizeof(float) * per);
  b.pc = take(sizeof(float) * per);
  b.t = take(sizeof(float) * per);
  b.X = take(sizeof(float) * 3 * static_cast<size_t>(p.P) * static_cast<size_t>(b.rows) * p.h);
  b.part = take(sizeof(float) * per * static_cast<size_t>(b.S));
  b.part2 = take(sizeof(float) * per * static_cast<size_t>(b.S));
  b.op = take(p.bf16 && (p.d == 64 || p.d == 128) ? sizeof(uint16_t) * 4 * per : 0);
  b.ns = take(p.muon ? sizeof(float) * 3 * static_cast<size_t>(p.P) *
                           static_cast<size_t>(lact::bw_ns_floats_per_matrix(p.d, p.h, c->ns_iters))
                     : 0);
  b.total = off;
  return b;
}

int check_backward(const lact_config* c, const Plan& p) {
  if (p.linear) return fail(LACT_ERR_UNSUPPORTED, "backward: SwiGLU fast net only");
  if (p.norm != LACT_NORM_UNIT) return fail(LACT_ERR_UNSUPPORTED, "backward: unit rows (norm_mode 0) only");
  if (c->eta_mode != LACT_ETA_SHARED) return fail(LACT_ERR_UNSUPPORTED, "backward: one rate per token only");
  if (!lact::backward_shape_ok(p.d, p.h))
    return fail(LACT_ERR_UNSUPPORTED, "backward: (d, h) = (%d, %d): d in {32, 64, 128}, h a multiple of 32",
                p.d, p.h);
  return LACT_OK;
}

// The backward pass on validated arguments (see include/lact.h).
int run_backward(const lact_config* c, const Plan& p, const lact_state* st0, const char* Q, const char* K,
                 const char* V, const float* eta, const char* dO, const lact_state* dWf, const lact_grads* out,
                 int64_t T_kv, int64_t T_q, int64_t chunk_kv, int64_t chunk_q, int32_t order, char* ws,
                 const BwLayout& L, hipStream_t s) {
  using lact::MatRef;
  const int64_t N = T_kv / chunk_kv;
  const int64_t hd = static_cast<int64_t>(p.h) * p.d;
  const int64_t per = 3 * hd * p.P;  // floats of one state
  const size_t eb = io_bytes(p);
  float* ckW = reinterpret_cast<float*>(ws + L.ckW);
  float* ckM = reinterpret_cast<float*>(ws + L.ckM);
  float* cot = reinterpret_cast<float*>(ws + L.cot);
  float* dM = reinterpret_cast<float*>(ws + L.dM);
  float* gb = reinterpret_cast<float*>(ws + L.g);
  float* dirb = reinterpret_cast<float*>(ws + L.dir);
  float* ddir = reinterpret_cast<float*>(ws + L.ddir);
  float* pc = reinterpret_cast<float*>(ws + L.pc);
  float* tb = reinterpret_cast<float*>(ws + L.t);
  float* X = reinterpret_cast<float*>(ws + L.X);
  // split partials of the last contractions (0: chunk gradient, 1: query
  // read), summed into the cotangent by the next step kernel or at the end
  float* const partbuf[2] = {reinterpret_cast<float*>(ws + L.part), reinterpret_cast<float*>(ws + L.part2)};
  const float* pend[2] = {nullptr, nullptr};
  int pend_S[2] = {0, 0};
  const int64_t xs = L.rows * p.h;  // pair stride of a factor array
  hipError_t e;
  // slot c of the checkpoints as a state: W1 | W2 | W3, each [P, ...]
  auto slot = [&](int64_t cidx) {
    lact_state x{};
    x.W1 = ckW + cidx * per;
    x.W2 = x.W1 + hd * p.P;
    x.W3 = x.W2 + hd * p.P;
    if (p.momentum) {
      x.M1 = ckM + cidx * per;
      x.M2 = x.M1 + hd * p.P;
      x.M3 = x.M2 + hd * p.P;
    }
    return x;
  };
  auto refs = [&](float* a, float* b, float* d3, int64_t stride, MatRef* r) {
    r[0] = {a, stride};
    r[1] = {b, stride};
    r[2] = {d3, stride};
  };
  const size_t state_bytes = sizeof(float) * hd * p.P;
  // ---- forward: the weights (and momentum) entering every chunk
  {
    lact_state s0 = slot(0);
    if ((e = hipMemcpyAsync(s0.W1, st0->W1, state_bytes, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(s0.W2, st0->W2, state_bytes, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(s0.W3, st0->W3, state_bytes, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "initial weights copy");
    if (p.momentum) {
      MatRef z{nullptr, 0};
      if ((e = lact::launch_bw_copy(s0.M1, z, z, z, p.P, p.d, p.h, true, s)) != hipSuccess)
        return hip_fail(e, "momentum zero");
    }
  }
  for (int64_t cidx = 0; cidx < N; ++cidx) {
    const size_t bytes = sizeof(float) * per * (p.momentum ? 1 : 1);
    if ((e = hipMemcpyAsync(ckW + (cidx + 1) * per, ckW + cidx * per, bytes, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "checkpoint copy");
    if (p.momentum &&
        (e = hipMemcpyAsync(ckM + (cidx + 1) * per, ckM + cidx * per, bytes, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "checkpoint copy");
    lact_state sn = slot(cidx + 1);
    const char* Kp = K + static_cast<size_t>(cidx * chunk_kv * p.d) * eb;
    const char* Vp = V + static_cast<size_t>(cidx * chunk_kv * p.d) * eb;
    int rc = run_update(c, p, &sn, Kp, Vp, eta + cidx * chunk_kv, chunk_kv, T_kv * p.d, T_kv, ws, L.fwd, s);
    if (rc) return rc;
  }
  // ---- cotangents of the final state and of the momentum
  {
    MatRef f1{dWf ? dWf->W1 : nullptr, hd}, f2{dWf ? dWf->W2 : nullptr, hd}, f3{dWf ? dWf->W3 : nullptr, hd};
    MatRef z{nullptr, 0};
    if ((e = lact::launch_bw_copy(cot, f1, f2, f3, p.P, p.d, p.h, true, s)) != hipSuccess ||
        (e = lact::launch_bw_copy(dM, z, z, z, p.P, p.d, p.h, true, s)) != hipSuccess)
      return hip_fail(e, "cotangent init");
  }
  // token-local VJP + weight contraction; its split partials stay pending
  // (added into cot by the next step kernel, or at the end)
  // (ops_ready: the operand region already holds W's operands, written by the
  // previous call with the same weights)
  auto tok_and_contract = [&](bool apply, const lact_state& W, const char* A, const char* B, const float* et,
                              int64_t n, int64_t in_stride, char* dA, char* dB, float* de, bool ops_ready) -> int {
    lact::BwTokArgs a{};
    a.A = A;
    a.B = B;
    a.eta = et;
    a.n = n;
    a.in_stride = in_stride;
    a.eta_stride = T_kv;
    a.W1 = {W.W1, hd};
    a.W2 = {W.W2, hd};
    a.W3 = {W.W3, hd};
    a.P1 = {pc, 3 * hd};
    a.P2 = {pc + hd, 3 * hd};
    a.P3 = {pc + 2 * hd, 3 * hd};
    a.X1 = X;
    a.X2 = X + xs * p.P;
    a.X3 = X + 2 * xs * p.P;
    a.x_stride = xs;
    a.dA = dA;
    a.dB = dB;
    a.out_stride = in_stride;
    a.deta = de;
    a.deta_stride = T_kv;
    a.P = p.P;
    a.d = p.d;
    a.h = p.h;
    a.bf16 = p.bf16;
    // the matrix-core kernels follow the layer's product precision: hi + lo
    // operands with split products, plain bf16 operands with bf16 products
    a.split = p.split;
    hipError_t err;
    if (p.bf16 && (p.d == 64 || p.d == 128)) {  // (the operand region exists exactly then)
      // operands of the matrix-core token kernels as bf16 hi | lo: W1, W3, W2^T
      // (and for the chunk gradient's VJP P1, P3, P2^T)
      lact::BwOpsArgs o{};
      o.m[0] = a.W1;
      o.m[1] = a.W3;
      o.m[2] = a.W2;
      o.m[3] = a.P1;
      o.m[4] = a.P3;
      o.m[5] = a.P2;
      o.nm = apply ? 3 : 6;
      o.op = reinterpret_cast<uint16_t*>(ws + L.op);
      o.op_stride = 12 * hd;
      o.P = p.P;
      o.d = p.d;
      o.h = p.h;
      o.hi_only = !p.split;
      if (!ops_ready && (err = lact::launch_bw_ops(o, s)) != hipSuccess)
        return hip_fail(err, "backward operand kernel");
      a.op = o.op;
      a.op_stride = o.op_stride;
    }
    const Splits sp = plan_splits(backward_rule(p), n);
    lact::BwContractArgs b{};
    b.A = A;
    b.B = B;
    b.eta = apply ? nullptr : et;
    b.n = n;
    b.in_stride = in_stride;
    b.eta_stride = T_kv;
    b.X1 = a.X1;
    b.X2 = a.X2;
    b.X3 = a.X3;
    b.x_stride = xs;
    b.partials = partbuf[apply ? 1 : 0];
    b.P = p.P;
    b.d = p.d;
    b.h = p.h;
    b.S = sp.S;
    b.tps = sp.tps;
    b.bf16 = p.bf16;
    b.split = p.split;
    // with plain bf16 products and matrix-core kernels on both sides the
    // factors travel as bf16 (half the bytes; the contraction rounds them to
    // bf16 operands either way), X2 of the chunk gradient already times -eta
    a.x_bf16 = b.x_bf16 = !p.split && lact::bw_tok_mfma_ok(a, apply) && lact::bw_contract_mfma_ok(b);
    {
      PhaseTimer t(apply ? 6 : 5, s);
      err = lact::launch_bw_tok(a, apply, s);
    }
    if (err != hipSuccess) return hip_fail(err, "backward token kernel");
    PhaseTimer tc(7, s);
    if ((err = lact::launch_bw_contract(b, s)) != hipSuccess) return hip_fail(err, "backward contraction kernel");
    pend[apply ? 1 : 0] = b.partials;
    pend_S[apply ? 1 : 0] = sp.S;
    return LACT_OK;
  };
  char* dQ = static_cast<char*>(out->dQ);
  char* dK = static_cast<char*>(out->dK);
  char* dV = static_cast<char*>(out->dV);
  // ---- chunks in reverse order
  for (int64_t cidx = N - 1; cidx >= 0; --cidx) {
    const lact_state Win = slot(cidx), Wout = slot(cidx + 1);
    const size_t ko = static_cast<size_t>(cidx * chunk_kv * p.d) * eb;
    const size_t qo = static_cast<size_t>(cidx * chunk_q * p.d) * eb;
    const float* ec = eta + cidx * chunk_kv;
    int rc;
    if (order == LACT_UPDATE_THEN_APPLY &&
        (rc = tok_and_contract(true, Wout, Q + qo, dO + qo, nullptr, chunk_q, T_q * p.d, dQ + qo, nullptr, nullptr,
                               false)))
      return rc;
    // the update's direction, recomputed: g (GD, Muon without momentum) or
    // the new momentum M_{c+1}; through Newton-Schulz for Muon
    // (momentum without Newton-Schulz: the step kernel reads M_{c+1} from its
    // checkpoint and runs the momentum VJP in the same pass)
    const bool mom_in_step = p.momentum && !p.muon;
    if (p.momentum) {
      MatRef m1{Wout.M1, hd}, m2{Wout.M2, hd}, m3{Wout.M3, hd};
      if (!mom_in_step && (e = lact::launch_bw_copy(gb, m1, m2, m3, p.P, p.d, p.h, true, s)) != hipSuccess)
        return hip_fail(e, "momentum gather");
    } else {
      Splits sp;
      if ((rc = launch_gradient(c, p, &Win, K + ko, V + ko, ec, chunk_kv, T_kv * p.d, T_kv,
                                reinterpret_cast<float*>(ws + L.fwd.partials), s, &sp)))
        return rc;
      lact::ReduceArgs r{};
      r.partials = reinterpret_cast<float*>(ws + L.fwd.partials);
      r.dir = gb;
      r.P = p.P;
      r.d = p.d;
      r.h = p.h;
      r.S = sp.S;
      if ((e = lact::launch_reduce(r, s)) != hipSuccess) return hip_fail(e, "gradient reduction");
    }
    const float* direction = gb;
    if (p.muon) {
      // Newton-Schulz forward: the direction, with the iterates kept in the
      // VJP's scratch
      lact::BwNSArgs nf{};
      nf.g = gb;
      nf.out = dirb;
      nf.scratch = reinterpret_cast<float*>(ws + L.ns);
      nf.per_mat = lact::bw_ns_floats_per_matrix(p.d, p.h, c->ns_iters);
      nf.P = p.P;
      nf.d = p.d;
      nf.h = p.h;
      nf.iters = c->ns_iters;
      nf.a = c->ns_a;
      nf.b = c->ns_b;
      nf.c = c->ns_c;
      nf.eps = c->ns_eps;
      nf.bf16_split = p.bf16;  // (bf16 I/O: split-bf16 products; fp32 I/O: fp32 products)
      PhaseTimer tn(8, s);
      if ((e = lact::launch_bw_ns_fwd(nf, s)) != hipSuccess) return hip_fail(e, "Newton-Schulz kernel");
      direction = dirb;
    }
    // through the step and the row normalisation
    lact::BwStepArgs sa{};
    refs(Win.W1, Win.W2, Win.W3, hd, sa.W_in);
    refs(Wout.W1, Wout.W2, Wout.W3, hd, sa.W_out);
    sa.dir = mom_in_step ? nullptr : direction;
    if (mom_in_step) {
      refs(Wout.M1, Wout.M2, Wout.M3, hd, sa.dir_m);
      sa.dM = dM;
      sa.pc = pc;
      sa.beta = c->beta;
    }
    sa.cot = cot;
    sa.ddir = (p.momentum || p.muon) ? ddir : pc;
    for (int q = 0; q < 2; ++q) {
      sa.pend[q] = pend[q];
      sa.pend_S[q] = pend_S[q];
      pend[q] = nullptr;
    }
    sa.step = c->step;
    sa.norm_eps = c->norm_eps;
    sa.P = p.P;
    sa.d = p.d;
    sa.h = p.h;
    if ((e = lact::launch_bw_step(sa, s)) != hipSuccess) return hip_fail(e, "backward step kernel");
    // through the optimizer: the cotangent of the chunk gradient into pc
    const float* t_in = ddir;
    if (p.muon) {
      lact::BwNSArgs na{};
      na.g = gb;
      na.dx = ddir;
      na.out = p.momentum ? tb : pc;
      na.scratch = reinterpret_cast<float*>(ws + L.ns);
      na.per_mat = lact::bw_ns_floats_per_matrix(p.d, p.h, c->ns_iters);
      na.P = p.P;
      na.d = p.d;
      na.h = p.h;
      na.iters = c->ns_iters;
      na.a = c->ns_a;
      na.b = c->ns_b;
      na.c = c->ns_c;
      na.eps = c->ns_eps;
      na.bf16_split = p.bf16;  // (bf16 I/O: split-bf16 products; fp32 I/O: fp32 products)
      PhaseTimer tn(8, s);
      if ((e = lact::launch_bw_ns(na, s)) != hipSuccess) return hip_fail(e, "Newton-Schulz VJP kernel");
      t_in = tb;
    }
    // (plain GD: the step kernel wrote the direction's cotangent into pc itself)
    if (p.momentum && !mom_in_step &&
        (e = lact::launch_bw_momentum(t_in, dM, pc, c->beta, per, s)) != hipSuccess)
      return hip_fail(e, "momentum VJP kernel");
    // through the chunk gradient
    if ((rc = tok_and_contract(false, Win, K + ko, V + ko, ec, chunk_kv, T_kv * p.d, dK + ko, dV + ko,
                               out->deta + cidx * chunk_kv, false)))
      return rc;
    // (the chunk gradient's call has just converted W_in, the read's weights here)
    if (order == LACT_APPLY_THEN_UPDATE &&
        (rc = tok_and_contract(true, Win, Q + qo, dO + qo, nullptr, chunk_q, T_q * p.d, dQ + qo, nullptr, nullptr,
                               true)))
      return rc;
  }
  for (int q = 0; q < 2; ++q) {
    if (pend[q] != nullptr && (e = lact::launch_bw_reduce_add(cot, pend[q], pend_S[q], 3 * hd, p.P, s)) != hipSuccess)
      return hip_fail(e, "backward reduction kernel");
  }
  MatRef o1{out->dW1, hd}, o2{out->dW2, hd}, o3{out->dW3, hd};
  if ((e = lact::launch_bw_copy(cot, o1, o2, o3, p.P, p.d, p.h, false, s)) != hipSuccess)
    return hip_fail(e, "cotangent store");
  return LACT_OK;
}

// ------------------------------------------------- allocation-free entry point
// Scratch of lact_chunked_forward_noalloc: a fixed array in the code object,
// one copy per GPU the library runs on, held until the process ends.  Host
// code must not use the array's name as an address (on the host it is only a
// stand-in): each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that pointer is passed on.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the scratch array (looked up on the first call made
// with the device current).
int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LACT_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % kAlign != 0)
      return fail(LACT_ERR_HIP, "scratch array at an unusable address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LACT_OK;
}

}  // namespace

extern "C" {

void lact_config_default(lact_config* c) {
  if (c == nullptr) return;
  std::memset(c, 0, sizeof(*c));
  c->io_dtype = LACT_BF16;
  c->opt = LACT_OPT_GD;
  c->beta = 0.f;
  c->ns_iters = 5;
  c->ns_a = 3.4445f;
  c->ns_b = -4.7750f;
  c->ns_c = 2.0315f;
  c->ns_eps = 1e-7f;
  c->step = 1.f;
  c->norm_eps = 1e-12f;
  c->products = LACT_PRODUCTS_AUTO;
  c->norm_mode = LACT_NORM_UNIT;
  c->eta_mode = LACT_ETA_SHARED;
  c->net = LACT_NET_SWIGLU;
}

int lact_mfma_path(int32_t d, int32_t h, int32_t io_dtype) {
  if (!lact::simple_shape_ok(d, h)) return -1;
  return (io_dtype == LACT_BF16 && (lact::grad_d64_shape_ok(d, h) || lact::d128_mfma_shape_ok(d, h))) ? 1 : 0;
}

size_t lact_workspace_bytes(const lact_config* cfg, int64_t max_chunk_kv, int64_t max_chunk_q) {
  (void)max_chunk_q;
  Plan p;
  if (check_config(cfg, &p) != LACT_OK) return 0;
  if (max_chunk_kv < 1) return 0;
  return ws_layout(p, max_chunk_kv).total;
}

int lact_update(const lact_config* cfg, const lact_state* st, const void* K, const void* V,
                const float* eta, int64_t n, int64_t kv_stride_bh, int64_t eta_stride_bh,
                void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan p;
  int rc = check_config(cfg, &p);
  if (rc) return rc;
  if ((rc = check_state(p, st, true))) return rc;
  if (!K || !V || !eta) return fail(LACT_ERR_INVALID_ARG, "K, V, eta must be non-NULL");
  if (n < 1) return fail(LACT_ERR_INVALID_ARG, "n=%lld must be >= 1", (long long)n);
  if (kv_stride_bh < n * p.d)
    return fail(LACT_ERR_INVALID_ARG, "kv_stride_bh %lld below n*d", (long long)kv_stride_bh);
  if (eta_stride_bh < n) return fail(LACT_ERR_INVALID_ARG, "eta_stride_bh %lld below n", (long long)eta_stride_bh);
  if ((rc = resolve_products(cfg, &p, n, 1))) return rc;
  WsLayout L;
  if ((rc = check_ws(p, n, ws, ws_bytes, &L))) return rc;
  return run_update(cfg, p, st, K, V, eta, n, kv_stride_bh, eta_stride_bh, static_cast<char*>(ws), L,
                    static_cast<hipStream_t>(stream));
}

int lact_apply(const lact_config* cfg, const lact_state* st, const void* Q, void* O, int64_t m,
               int64_t q_stride_bh, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  (void)ws;
  (void)ws_bytes;
  Plan p;
  int rc = check_config(cfg, &p);
  if (rc) return rc;
  if ((rc = check_state(p, st, false))) return rc;
  if (!Q || !O) return fail(LACT_ERR_INVALID_ARG, "Q, O must be non-NULL");
  if (m < 1) return fail(LACT_ERR_INVALID_ARG, "m=%lld must be >= 1", (long long)m);
  if (q_stride_bh < m * p.d) return fail(LACT_ERR_INVALID_ARG, "q_stride_bh %lld below m*d", (long long)q_stride_bh);
  return run_apply(p, st, Q, O, m, q_stride_bh, static_cast<hipStream_t>(stream));
}

int lact_chunked_forward(const lact_config* cfg, const lact_state* st, const void* Q, const void* K,
                         const void* V, const float* eta, void* O, int64_t T_kv, int64_t T_q,
                         int64_t chunk_kv, int64_t chunk_q, int32_t order, void* ws, size_t ws_bytes,
                         void* stream) {
  g_last_error.clear();
  Plan p;
  int rc = check_config(cfg, &p);
  if (rc) return rc;
  if ((rc = check_state(p, st, true))) return rc;
  if (!Q || !K || !V || !eta || !O) return fail(LACT_ERR_INVALID_ARG, "Q, K, V, eta, O must be non-NULL");
  if (T_kv < 1 || T_q < 1 || chunk_kv < 1 || chunk_q < 1)
    return fail(LACT_ERR_INVALID_ARG, "sequence lengths and chunk sizes must be >= 1");
  if (T_kv % chunk_kv || T_q % chunk_q)
    return fail(LACT_ERR_INVALID_ARG, "chunk sizes (%lld, %lld) must divide T_kv=%lld and T_q=%lld",
                (long long)chunk_kv, (long long)chunk_q, (long long)T_kv, (long long)T_q);
  const int64_t N = T_kv / chunk_kv;
  if (T_q / chunk_q != N)
    return fail(LACT_ERR_INVALID_ARG, "key chunks (%lld) and query chunks (%lld) differ", (long long)N,
                (long long)(T_q / chunk_q));
  if (order != LACT_APPLY_THEN_UPDATE && order != LACT_UPDATE_THEN_APPLY)
    return fail(LACT_ERR_INVALID_ARG, "order %d unknown", order);
  if ((rc = resolve_products(cfg, &p, chunk_kv, N))) return rc;
  WsLayout L;
  if ((rc = check_ws(p, chunk_kv, ws, ws_bytes, &L))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t eb = io_bytes(p);
  const char* Qc = static_cast<const char*>(Q);
  const char* Kc = static_cast<const char*>(K);
  const char* Vc = static_cast<const char*>(V);
  char* Oc = static_cast<char*>(O);
  // bf16 copy of the weights as the last update left them (none before it)
  uint16_t* wb = L.has_wb ? reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + L.wb) : nullptr;
  bool wb_valid = false;
  // Apply-then-update with a matrix-core query read: the bf16 copy of the
  // initial weights is made first (one small kernel), so every query read,
  // the first one included, loads the copy instead of converting the fp32
  // weights.
  bool read_mfma = false;
  if (order == LACT_APPLY_THEN_UPDATE && L.has_wb && !p.linear)
    (void)apply_args(p, st, Qc, Oc, chunk_q, T_q * p.d, nullptr, &read_mfma);
  const bool w_aligned = ((reinterpret_cast<uintptr_t>(st->W1) | reinterpret_cast<uintptr_t>(st->W2) |
                           reinterpret_cast<uintptr_t>(st->W3)) & 15) == 0;
  // With the matrix-core Muon tail the tail of chunk c and the query read of
  // chunk c also share one launch (the read takes the CUs the 3P tail
  // workgroups leave); the read loads the copy of W_c while the tail writes
  // W_c+1 and the other copy.
  const bool fuse = read_mfma && L.has_wb2 && muon_mfma_tail(p, st);
  if (read_mfma && w_aligned) {
    PhaseTimer t(4, s);
    hipError_t e = lact::launch_wb_copy(st->W1, st->W2, st->W3, wb, p.P, p.d, p.h, s);
    if (e != hipSuccess) return hip_fail(e, "bf16 weight-copy kernel");
    wb_valid = true;
  }
  if (fuse && wb_valid) {
    uint16_t* cp[2] = {wb, reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + L.wb2)};
    for (int64_t c = 0; c < N; ++c) {
      const void* Kp = Kc + static_cast<size_t>(c * chunk_kv * p.d) * eb;
      const void* Vp = Vc + static_cast<size_t>(c * chunk_kv * p.d) * eb;
      const float* ep = eta + c * chunk_kv;
      const void* Qp = Qc + static_cast<size_t>(c * chunk_q * p.d) * eb;
      void* Op = Oc + static_cast<size_t>(c * chunk_q * p.d) * eb;
      bool mfma = false;
      const lact::ApplyArgs aa = apply_args(p, st, Qp, Op, chunk_q, T_q * p.d, cp[c & 1], &mfma);
      if ((rc = run_update(cfg, p, st, Kp, Vp, ep, chunk_kv, T_kv * p.d, T_kv, static_cast<char*>(ws), L, s,
                           cp[(c + 1) & 1], &wb_valid, &aa)))
        return rc;
    }
    return LACT_OK;
  }
  for (int64_t c = 0; c < N; ++c) {
    const void* Kp = Kc + static_cast<size_t>(c * chunk_kv * p.d) * eb;
    const void* Vp = Vc + static_cast<size_t>(c * chunk_kv * p.d) * eb;
    const float* ep = eta + c * chunk_kv;
    const void* Qp = Qc + static_cast<size_t>(c * chunk_q * p.d) * eb;
    void* Op = Oc + static_cast<size_t>(c * chunk_q * p.d) * eb;
    if (order == LACT_APPLY_THEN_UPDATE &&
        (rc = run_apply(p, st, Qp, Op, chunk_q, T_q * p.d, s, wb_valid ? wb : nullptr)))
      return rc;
    if ((rc = run_update(cfg, p, st, Kp, Vp, ep, chunk_kv, T_kv * p.d, T_kv, static_cast<char*>(ws), L, s,
                         wb, &wb_valid)))
      return rc;
    if (order == LACT_UPDATE_THEN_APPLY &&
        (rc = run_apply(p, st, Qp, Op, chunk_q, T_q * p.d, s, wb_valid ? wb : nullptr)))
      return rc;
  }
  return LACT_OK;
}

int lact_chunked_forward_noalloc(const lact_config* cfg, const lact_state* st, const void* Q,
                                 const void* K, const void* V, const float* eta, void* O, int64_t T_kv,
                                 int64_t T_q, int64_t chunk_kv, int64_t chunk_q, int32_t order,
                                 void* stream) {
  g_last_error.clear();
  Plan p;
  int rc = check_config(cfg, &p);
  if (rc) return rc;
  if (chunk_kv < 1) return fail(LACT_ERR_INVALID_ARG, "chunk sizes must be >= 1");
  const size_t need = lact_workspace_bytes(cfg, chunk_kv, chunk_q);
  if (need > kNoallocScratchBytes)
    return fail(LACT_ERR_WORKSPACE,
                "chunks of %lld keys need %zu bytes of scratch, above the %zu bytes of the "
                "allocation-free entry point (use lact_chunked_forward with a workspace)",
                (long long)chunk_kv, need, kNoallocScratchBytes);
  void* ws = nullptr;
  if ((rc = noalloc_scratch(&ws))) return rc;
  return lact_chunked_forward(cfg, st, Q, K, V, eta, O, T_kv, T_q, chunk_kv, chunk_q, order, ws,
                              kNoallocScratchBytes, stream);
}

size_t lact_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

int lact_window_attention(const lact_config* cfg, const void* Q, const void* K, const void* V, void* O, int64_t T,
                          int64_t window, float scale, int32_t accumulate, void* stream) {
  g_last_error.clear();
  if (cfg == nullptr) return fail(LACT_ERR_INVALID_ARG, "config is NULL");
  if (cfg->B < 1 || cfg->H < 1) return fail(LACT_ERR_INVALID_ARG, "B=%d H=%d must be >= 1", cfg->B, cfg->H);
  if (static_cast<int64_t>(cfg->B) * cfg->H > 65535)
    return fail(LACT_ERR_UNSUPPORTED, "B*H=%lld above 65535", (long long)cfg->B * cfg->H);
  if (cfg->io_dtype != LACT_F32 && cfg->io_dtype != LACT_BF16)
    return fail(LACT_ERR_INVALID_ARG, "io_dtype %d unknown", cfg->io_dtype);
  if (!lact::window_shape_ok(cfg->d))
    return fail(LACT_ERR_UNSUPPORTED, "window attention: d=%d not in {32, 64, 128}", cfg->d);
  if (!Q || !K || !V || !O) return fail(LACT_ERR_INVALID_ARG, "Q, K, V, O must be non-NULL");
  if (T < 1 || window < 1) return fail(LACT_ERR_INVALID_ARG, "T and window must be >= 1");
  if (!finite(scale)) return fail(LACT_ERR_INVALID_ARG, "scale must be finite");
  if (accumulate != 0 && accumulate != 1) return fail(LACT_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  lact::WindowArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.T = T;
  a.stride = T * cfg->d;
  a.window = window;
  a.scale = scale > 0.f ? scale : 1.f / std::sqrt(static_cast<float>(cfg->d));
  a.accumulate = accumulate;
  a.P = cfg->B * cfg->H;
  a.d = cfg->d;
  a.bf16 = cfg->io_dtype == LACT_BF16;
  hipError_t e;
  {
    PhaseTimer t(9, static_cast<hipStream_t>(stream));
    e = lact::launch_window_attn(a, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return hip_fail(e, "window-attention kernel");
  return LACT_OK;
}

int lact_block_forward(const lact_config* cfg, const lact_state* st, const void* Q, const void* K, const void* V,
                       const float* eta, void* O, int64_t T, int64_t chunk, int64_t window, float scale,
                       int32_t order, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (cfg == nullptr) return fail(LACT_ERR_INVALID_ARG, "config is NULL");
  if (!lact::window_shape_ok(cfg->d))
    return fail(LACT_ERR_UNSUPPORTED, "window attention: d=%d not in {32, 64, 128}", cfg->d);
  if (window < 1) return fail(LACT_ERR_INVALID_ARG, "window must be >= 1");
  if (!finite(scale)) return fail(LACT_ERR_INVALID_ARG, "scale must be finite");
  int rc = lact_chunked_forward(cfg, st, Q, K, V, eta, O, T, T, chunk, chunk, order, ws, ws_bytes, stream);
  if (rc) return rc;
  return lact_window_attention(cfg, Q, K, V, O, T, window, scale, 1, stream);
}

size_t lact_backward_workspace_bytes(const lact_config* cfg, int64_t T_kv, int64_t chunk_kv, int64_t chunk_q) {
  Plan p;
  if (check_config(cfg, &p) != LACT_OK || check_backward(cfg, p) != LACT_OK) return 0;
  if (T_kv < 1 || chunk_kv < 1 || chunk_q < 1 || T_kv % chunk_kv) return 0;
  return bw_layout(cfg, p, T_kv / chunk_kv, chunk_kv, chunk_q).total;
}

int lact_chunked_backward(const lact_config* cfg, const lact_state* st, const void* Q, const void* K,
                          const void* V, const float* eta, const void* dO, const lact_state* dW_final,
                          const lact_grads* out, int64_t T_kv, int64_t T_q, int64_t chunk_kv, int64_t chunk_q,
                          int32_t order, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan p;
  int rc = check_config(cfg, &p);
  if (rc) return rc;
  if ((rc = check_backward(cfg, p))) return rc;
  if (st == nullptr || !st->W1 || !st->W2 || !st->W3)
    return fail(LACT_ERR_INVALID_ARG, "initial W1, W2, W3 must be non-NULL");
  if (dW_final != nullptr && (!dW_final->W1 || !dW_final->W2 || !dW_final->W3))
    return fail(LACT_ERR_INVALID_ARG, "dW_final: W1, W2, W3 must be non-NULL");
  if (!Q || !K || !V || !eta || !dO || out == nullptr)
    return fail(LACT_ERR_INVALID_ARG, "Q, K, V, eta, dO, out must be non-NULL");
  if (!out->dQ || !out->dK || !out->dV || !out->deta || !out->dW1 || !out->dW2 || !out->dW3)
    return fail(LACT_ERR_INVALID_ARG, "every output of lact_grads must be non-NULL");
  if (T_kv < 1 || T_q < 1 || chunk_kv < 1 || chunk_q < 1)
    return fail(LACT_ERR_INVALID_ARG, "sequence lengths and chunk sizes must be >= 1");
  if (T_kv % chunk_kv || T_q % chunk_q)
    return fail(LACT_ERR_INVALID_ARG, "chunk sizes (%lld, %lld) must divide T_kv=%lld and T_q=%lld",
                (long long)chunk_kv, (long long)chunk_q, (long long)T_kv, (long long)T_q);
  const int64_t N = T_kv / chunk_kv;
  if (T_q / chunk_q != N)
    return fail(LACT_ERR_INVALID_ARG, "key chunks (%lld) and query chunks (%lld) differ", (long long)N,
                (long long)(T_q / chunk_q));
  if (order != LACT_APPLY_THEN_UPDATE && order != LACT_UPDATE_THEN_APPLY)
    return fail(LACT_ERR_INVALID_ARG, "order %d unknown", order);
  if ((rc = resolve_products(cfg, &p, chunk_kv, N))) return rc;
  const BwLayout L = bw_layout(cfg, p, N, chunk_kv, chunk_q);
  if (ws_bytes < L.total)
    return fail(LACT_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes needed", ws_bytes, L.total);
  if (ws == nullptr || reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(LACT_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  return run_backward(cfg, p, st, static_cast<const char*>(Q), static_cast<const char*>(K),
                      static_cast<const char*>(V), eta, static_cast<const char*>(dO), dW_final, out, T_kv, T_q,
                      chunk_kv, chunk_q, order, static_cast<char*>(ws), L, static_cast<hipStream_t>(stream));
}

const char* lact_status_string(int status) {
  switch (status) {
    case LACT_OK: return "ok";
    case LACT_ERR_INVALID_ARG: return "invalid argument";
    case LACT_ERR_UNSUPPORTED: return "unsupported configuration";
    case LACT_ERR_WORKSPACE: return "workspace too small or misaligned";
    case LACT_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* lact_last_error(void) { return g_last_error.c_str(); }

int lact_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return LACT_OK;
}

int lact_profile_read(double* ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int rc = LACT_OK;
  for (const ProfRec& r : g_prof_recs) {
    hipError_t e = hipEventSynchronize(r.stop);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) {
      rc = hip_fail(e, "profile event");
    } else if (r.phase >= 0 && r.phase < LACT_PROFILE_PHASES) {
      if (ms) ms[r.phase] += t;
      if (launches) launches[r.phase] += 1;
    }
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
  return rc;
}

int lact_version(void) { return 3; }

}  // extern "C"

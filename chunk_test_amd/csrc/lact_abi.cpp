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

// Which chunk-gradient kernel runs.  The MFMA kernels read 16-byte rows with
// 32-bit offsets inside a pair's rows: they need aligned K, V and strides and
// n d < 2^31.  Split products run on MFMA at d = 128 only.
enum class GradKind { Generic, D64, D128 };

// Above this many token splits the Muon tail's partial sum runs as a
// separate all-CU kernel.
constexpr int kTailSplitsInline = 8;

struct GradChoice {
  GradKind kind;
  int stage;        // token splits are multiples of this
  int wgs_per_cu;   // resident workgroups per CU
};

GradChoice grad_choice(const Plan& p, bool aligned, int64_t n) {
  const bool fits = aligned && n * p.d < (static_cast<int64_t>(1) << 31);
  if (p.mfma && fits) {
    if (!p.split && lact::grad_d64_shape_ok(p.d, p.h)) return {GradKind::D64, 128, 2};
    if (lact::grad_d128_shape_ok(p.d, p.h))
      return {GradKind::D128, lact::grad_d128_stage_tokens(p.split), 1};
  }
  return {GradKind::Generic, 1, 0};
}

// MFMA kernels: one workgroup per (split, 128 hidden units, pair), sized to
// one round of resident workgroups on 256 CUs, rounding the split count
// down so no second round is started.
SplitRule mfma_rule(const Plan& p, const GradChoice& k) {
  const int64_t per_split = static_cast<int64_t>(p.P) * (p.h / 128);
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
  if (c->d < 1 || c->h < 1) return fail(LACT_ERR_INVALID_ARG, "d=%d h=%d must be >= 1", c->d, c->h);
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
  if (c->products != LACT_PRODUCTS_BF16 && c->products != LACT_PRODUCTS_SPLIT)
    return fail(LACT_ERR_INVALID_ARG, "products %d unknown", c->products);
  if (!finite(c->norm_eps) || c->norm_eps <= 0.f)
    return fail(LACT_ERR_INVALID_ARG, "norm_eps %g must be finite and > 0", c->norm_eps);
  if (c->norm_mode != LACT_NORM_UNIT && c->norm_mode != LACT_NORM_KEEP)
    return fail(LACT_ERR_INVALID_ARG, "norm_mode %d unknown", c->norm_mode);
  if (c->eta_mode != LACT_ETA_SHARED && c->eta_mode != LACT_ETA_PER_MATRIX)
    return fail(LACT_ERR_INVALID_ARG, "eta_mode %d unknown", c->eta_mode);
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
  return LACT_OK;
}

int check_state(const Plan& p, const lact_state* st, bool need_m) {
  if (st == nullptr) return fail(LACT_ERR_INVALID_ARG, "state is NULL");
  if (!st->W1 || !st->W2 || !st->W3) return fail(LACT_ERR_INVALID_ARG, "W1, W2, W3 must be non-NULL");
  if (need_m && p.momentum && (!st->M1 || !st->M2 || !st->M3))
    return fail(LACT_ERR_INVALID_ARG, "this optimizer keeps momentum: M1, M2, M3 must be non-NULL");
  return LACT_OK;
}

// Workspace sections (bytes), each 256-byte aligned.
struct WsLayout {
  size_t partials = 0, dir = 0, ns = 0, wb = 0, total = 0;
  bool has_wb = false;  // section for bf16 copies of W1, W2, W3 (P 3 h d values)
};

WsLayout ws_layout(const Plan& p, int64_t max_chunk_kv) {
  WsLayout w;
  const size_t per = static_cast<size_t>(3) * p.h * p.d;
  const int64_t n = max_chunk_kv < 1 ? 1 : max_chunk_kv;
  // every kernel the update may pick for up to n tokens
  int64_t S = split_bound(generic_rule(p), n);
  const GradChoice k = grad_choice(p, true, 0);
  if (k.kind != GradKind::Generic) {
    const int64_t sm = split_bound(mfma_rule(p, k), n);
    if (sm > S) S = sm;
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
int run_update(const lact_config* c, const Plan& p, const lact_state* st, const void* K,
               const void* V, const float* eta, int64_t n, int64_t kv_stride,
               int64_t eta_stride, char* ws, const WsLayout& L, hipStream_t s,
               uint16_t* wb = nullptr, bool* wb_written = nullptr) {
  if (wb_written != nullptr) *wb_written = false;
  const bool aligned = (reinterpret_cast<uintptr_t>(K) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(V) % 16 == 0) && (kv_stride % 8 == 0);
  const GradChoice gk = grad_choice(p, aligned, n);
  const Splits sp = plan_splits(gk.kind == GradKind::Generic ? generic_rule(p) : mfma_rule(p, gk), n);
  float* partials = reinterpret_cast<float*>(ws + L.partials);
  float* dir = reinterpret_cast<float*>(ws + L.dir);
  hipError_t e;
  {
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
    switch (gk.kind) {
      case GradKind::D64: e = lact::launch_grad_d64(g, s); break;
      case GradKind::D128: e = lact::launch_grad_d128(g, p.split, s); break;
      default: e = lact::launch_grad_simple(g, s); break;
    }
    if (e != hipSuccess) return hip_fail(e, "gradient kernel");
  }
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
    e = lact::launch_reduce_step(ta, s);
    if (e != hipSuccess) return hip_fail(e, "update-tail kernel");
    return LACT_OK;
  }
  // (the MFMA tail moves W and M in 16-byte pieces)
  const bool state_aligned =
      ((reinterpret_cast<uintptr_t>(st->W1) | reinterpret_cast<uintptr_t>(st->W2) |
        reinterpret_cast<uintptr_t>(st->W3) | reinterpret_cast<uintptr_t>(st->M1) |
        reinterpret_cast<uintptr_t>(st->M2) | reinterpret_cast<uintptr_t>(st->M3)) & 15) == 0;
  if (p.bf16 && lact::ns_mfma_shape_ok(p.d, p.h) && state_aligned) {
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
    e = lact::launch_muon_tail(ta, s);
    if (e != hipSuccess) return hip_fail(e, "Muon update-tail kernel");
    return LACT_OK;
  }
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
int run_apply(const Plan& p, const lact_state* st, const void* Q, void* O, int64_t m,
              int64_t q_stride, hipStream_t s, const uint16_t* wb = nullptr) {
  PhaseTimer t(4, s);
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
  const bool use_mfma = p.bf16 && lact::apply_mfma_shape_ok(p.d, p.h) &&
                        reinterpret_cast<uintptr_t>(Q) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(O) % 16 == 0 && q_stride % 8 == 0;
  if (use_mfma && wb != nullptr) {
    const int64_t phd = static_cast<int64_t>(p.P) * p.h * p.d;
    a.Wb1 = wb;
    a.Wb2 = wb + phd;
    a.Wb3 = wb + 2 * phd;
  }
  hipError_t e = use_mfma ? lact::launch_apply_mfma(a, s) : lact::launch_apply_simple(a, s);
  if (e != hipSuccess) return hip_fail(e, "query-read kernel");
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
  c->products = LACT_PRODUCTS_BF16;
  c->norm_mode = LACT_NORM_UNIT;
  c->eta_mode = LACT_ETA_SHARED;
}

int lact_mfma_path(int32_t d, int32_t h, int32_t io_dtype) {
  if (!lact::simple_shape_ok(d, h)) return -1;
  return (io_dtype == LACT_BF16 && (lact::grad_d64_shape_ok(d, h) || lact::grad_d128_shape_ok(d, h))) ? 1 : 0;
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

int lact_version(void) { return 1; }

}  // extern "C"

// Backward pass of the LaCT layer (training): the vector-Jacobian products of
// every forward step, run chunk by chunk in reverse order over fast weights
// recomputed by a forward pass.  The layer is trained through its outputs
// ("LaCT: Large Chunk Test-Time Training" review, section "Language
// modelling: quality and throughput differ"); per chunk the forward is
//   H1 = K W1^T, H3 = K W3^T, A = silu(H1), G = A H3, U = -eta V,
//   dG = U W2, dH3 = dG A, dH1 = dG H3 silu'(H1),
//   g = (dH1^T K, U^T G, dH3^T K),  direction = opt(g),
//   W' = rows(W - step * direction),  O = W2 (silu(W1 q) (W3 q)),
// and the kernels here take the cotangents back through it.  All arithmetic
// is fp32 (bf16 inputs are widened exactly; bf16 outputs rounded once).
//
//   k_bw_grad_tok   token-local part of the chunk gradient's VJP: given the
//                   cotangents P of g, per key token the cotangents of k, v
//                   and eta, and per (token, hidden unit) the three factors
//                   of the weight cotangents (H1bar, dGbar, H3bar)
//   k_bw_apply_tok  the same for the query read: dq, and (H1bar, G, H3bar)
//   k_bw_contract   weight cotangents as token contractions of those
//                   factors: X1^T A, B^T X2, X3^T A, split over tokens
//   k_bw_reduce_add fixed-order sum of the splits into the running cotangent
//   k_bw_step       through W' = rows(W - step d): the row normalisation's
//                   VJP, giving the cotangents of W and of the direction
//   k_bw_momentum   the momentum buffer's cotangent carried to the earlier
//                   chunk
//   k_bw_ns_fwd     Newton-Schulz's forward (iterates and A, B kept)
//   k_bw_ns         its VJP through every iteration and the Frobenius
//                   pre-scaling
//   k_bw_copy       layout moves between separate W1 | W2 | W3 arrays and the
//                   per-pair [W1 | W2 | W3] blocks
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 32;  // tokens per tile
constexpr int kHS = 32;   // hidden units per slice

__device__ __forceinline__ float silu_d1(float z, float s) { return s * (1.f + z * (1.f - s)); }
__device__ __forceinline__ float silu_d2(float z, float s) { return s * (1.f - s) * (2.f + z * (1.f - 2.f * s)); }

template <int D>
__device__ __forceinline__ float dot_row(const float (*a)[D + 1], int i, const float (*b)[D + 1], int j) {
  float s = 0.f;
#pragma unroll 8
  for (int e = 0; e < D; ++e) s = fmaf(a[i][e], b[j][e], s);
  return s;
}

// Loads a 32 x D slice of a matrix stored [rows, D] (hidden units of W1, W3, or of
// their cotangents) and, transposed, a D x 32 slice of one stored [D, h] (W2).
template <int D>
__device__ __forceinline__ void load_slices(const MatRef& r1, const MatRef& r3, const MatRef& r2, int pair, int j0,
                                            int h, float (*s1)[D + 1], float (*s3)[D + 1], float (*s2t)[D + 1]) {
  const float* m1 = r1.p + pair * r1.pair_stride;
  const float* m3 = r3.p + pair * r3.pair_stride;
  const float* m2 = r2.p + pair * r2.pair_stride;
  for (int i = threadIdx.x; i < kHS * D; i += kThreads) {
    const int jj = i / D, e = i % D;
    s1[jj][e] = m1[static_cast<int64_t>(j0 + jj) * D + e];
    s3[jj][e] = m3[static_cast<int64_t>(j0 + jj) * D + e];
  }
  for (int i = threadIdx.x; i < kHS * D; i += kThreads) {
    const int e = i / kHS, jj = i % kHS;
    s2t[jj][e] = m2[static_cast<int64_t>(e) * h + j0 + jj];
  }
}

// ---------------------------------------------------------------------------
// Token-local VJP of the chunk gradient.  Grid (key tiles of 32, P pairs).
// With p1 = P1[j] k, p3 = P3[j] k, gb = (U P2)_j (the cotangents reaching
// dH1, dH3, G), per (token, hidden unit j):
//   dGbar = p3 a + p1 h3 s1,         Abar = p3 dg + gb h3,
//   H3bar = p1 dg s1 + gb a,         H1bar = p1 dg h3 s2 + Abar s1
// (s1 = silu'(h1), s2 = silu''(h1)), and per token
//   Ubar = P2 g + W2 dGbar,   kbar = P1^T dh1 + P3^T dh3 + W1^T H1bar + W3^T H3bar,
//   vbar = -eta Ubar,  etabar = -Ubar . v.
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_bw_grad_tok(BwTokArgs a) {
  __shared__ float sK[kTok][D + 1];
  __shared__ float sU[kTok][D + 1];
  __shared__ float sW1[kHS][D + 1], sW3[kHS][D + 1], sW2t[kHS][D + 1];
  __shared__ float sP1[kHS][D + 1], sP3[kHS][D + 1], sP2t[kHS][D + 1];
  __shared__ float sDH1[kTok][kHS + 1], sDH3[kTok][kHS + 1], sG[kTok][kHS + 1];
  __shared__ float sHB1[kTok][kHS + 1], sHB3[kTok][kHS + 1], sDGB[kTok][kHS + 1];
  const int pair = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int tid = threadIdx.x;
  const int h = a.h;
  const int64_t kv = static_cast<int64_t>(pair) * a.in_stride;
  const float* eta = a.eta + static_cast<int64_t>(pair) * a.eta_stride;
  for (int i = tid; i < kTok * D; i += kThreads) {
    const int t = i / D, e = i % D;
    const int64_t tok = t0 + t;
    float k = 0.f, u = 0.f;
    if (tok < a.n) {
      k = load_io<BF16>(a.A, kv + tok * D + e);
      u = -eta[tok] * load_io<BF16>(a.B, kv + tok * D + e);
    }
    sK[t][e] = k;
    sU[t][e] = u;
  }
  constexpr int NE = kTok * D / kThreads;  // owned (token, feature) entries
  float ub[NE], kb[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) ub[q] = kb[q] = 0.f;
  float* X1 = a.X1 + static_cast<int64_t>(pair) * a.x_stride;
  float* X2 = a.X2 + static_cast<int64_t>(pair) * a.x_stride;
  float* X3 = a.X3 + static_cast<int64_t>(pair) * a.x_stride;
  for (int j0 = 0; j0 < h; j0 += kHS) {
    __syncthreads();
    load_slices<D>(a.W1, a.W3, a.W2, pair, j0, h, sW1, sW3, sW2t);
    load_slices<D>(a.P1, a.P3, a.P2, pair, j0, h, sP1, sP3, sP2t);
    __syncthreads();
    for (int idx = tid; idx < kTok * kHS; idx += kThreads) {
      const int t = idx / kHS, jj = idx % kHS;
      const float h1 = dot_row<D>(sK, t, sW1, jj);
      const float h3 = dot_row<D>(sK, t, sW3, jj);
      const float dg = dot_row<D>(sU, t, sW2t, jj);
      const float p1 = dot_row<D>(sK, t, sP1, jj);
      const float p3 = dot_row<D>(sK, t, sP3, jj);
      const float gb = dot_row<D>(sU, t, sP2t, jj);
      const float s = sigmoid_f(h1);
      const float act = h1 * s;
      const float s1 = silu_d1(h1, s);
      const float s2 = silu_d2(h1, s);
      const float dgb = p3 * act + p1 * h3 * s1;
      const float ab = p3 * dg + gb * h3;
      const float h3b = p1 * dg * s1 + gb * act;
      const float h1b = p1 * dg * h3 * s2 + ab * s1;
      sDH1[t][jj] = dg * h3 * s1;
      sDH3[t][jj] = dg * act;
      sG[t][jj] = act * h3;
      sHB1[t][jj] = h1b;
      sHB3[t][jj] = h3b;
      sDGB[t][jj] = dgb;
      const int64_t tok = t0 + t;
      if (tok < a.n) {
        X1[tok * h + j0 + jj] = h1b;
        X2[tok * h + j0 + jj] = dgb;
        X3[tok * h + j0 + jj] = h3b;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int idx = tid + kThreads * q;
      const int t = idx / D, e = idx % D;
      float u = ub[q], k = kb[q];
      for (int jj = 0; jj < kHS; ++jj) {
        u = fmaf(sP2t[jj][e], sG[t][jj], u);
        u = fmaf(sW2t[jj][e], sDGB[t][jj], u);
        k = fmaf(sP1[jj][e], sDH1[t][jj], k);
        k = fmaf(sP3[jj][e], sDH3[t][jj], k);
        k = fmaf(sW1[jj][e], sHB1[t][jj], k);
        k = fmaf(sW3[jj][e], sHB3[t][jj], k);
      }
      ub[q] = u;
      kb[q] = k;
    }
  }
  __syncthreads();
  // outputs; the rate cotangent -Ubar . v summed per token in feature order
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int idx = tid + kThreads * q;
    const int t = idx / D, e = idx % D;
    const int64_t tok = t0 + t;
    float prod = 0.f;
    if (tok < a.n) {
      const float v = load_io<BF16>(a.B, kv + tok * D + e);
      store_io<BF16>(a.dA, static_cast<int64_t>(pair) * a.out_stride + tok * D + e, kb[q]);
      store_io<BF16>(a.dB, static_cast<int64_t>(pair) * a.out_stride + tok * D + e, -eta[tok] * ub[q]);
      prod = -ub[q] * v;
    }
    sU[t][e] = prod;
  }
  __syncthreads();
  if (tid < kTok && t0 + tid < a.n) {
    float s = 0.f;
    for (int e = 0; e < D; ++e) s += sU[tid][e];
    a.deta[static_cast<int64_t>(pair) * a.deta_stride + t0 + tid] = s;
  }
}

// ---------------------------------------------------------------------------
// Token-local VJP of the query read O = W2 (silu(W1 q) (W3 q)).  Grid (query
// tiles of 32, P pairs).  Per (query, hidden unit j): ob = (dO W2)_j,
//   H3bar = ob a,  H1bar = ob h3 silu'(h1),  G = a h3;
// per query qbar = W1^T H1bar + W3^T H3bar.
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_bw_apply_tok(BwTokArgs a) {
  __shared__ float sQ[kTok][D + 1];
  __shared__ float sO[kTok][D + 1];
  __shared__ float sW1[kHS][D + 1], sW3[kHS][D + 1], sW2t[kHS][D + 1];
  __shared__ float sHB1[kTok][kHS + 1], sHB3[kTok][kHS + 1];
  const int pair = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int tid = threadIdx.x;
  const int h = a.h;
  const int64_t qb = static_cast<int64_t>(pair) * a.in_stride;
  for (int i = tid; i < kTok * D; i += kThreads) {
    const int t = i / D, e = i % D;
    const int64_t tok = t0 + t;
    sQ[t][e] = tok < a.n ? load_io<BF16>(a.A, qb + tok * D + e) : 0.f;
    sO[t][e] = tok < a.n ? load_io<BF16>(a.B, qb + tok * D + e) : 0.f;
  }
  constexpr int NE = kTok * D / kThreads;
  float qacc[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) qacc[q] = 0.f;
  float* X1 = a.X1 + static_cast<int64_t>(pair) * a.x_stride;
  float* X2 = a.X2 + static_cast<int64_t>(pair) * a.x_stride;
  float* X3 = a.X3 + static_cast<int64_t>(pair) * a.x_stride;
  for (int j0 = 0; j0 < h; j0 += kHS) {
    __syncthreads();
    load_slices<D>(a.W1, a.W3, a.W2, pair, j0, h, sW1, sW3, sW2t);
    __syncthreads();
    for (int idx = tid; idx < kTok * kHS; idx += kThreads) {
      const int t = idx / kHS, jj = idx % kHS;
      const float h1 = dot_row<D>(sQ, t, sW1, jj);
      const float h3 = dot_row<D>(sQ, t, sW3, jj);
      const float ob = dot_row<D>(sO, t, sW2t, jj);
      const float s = sigmoid_f(h1);
      const float act = h1 * s;
      const float h3b = ob * act;
      const float h1b = ob * h3 * silu_d1(h1, s);
      sHB1[t][jj] = h1b;
      sHB3[t][jj] = h3b;
      const int64_t tok = t0 + t;
      if (tok < a.n) {
        X1[tok * h + j0 + jj] = h1b;
        X2[tok * h + j0 + jj] = act * h3;
        X3[tok * h + j0 + jj] = h3b;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int idx = tid + kThreads * q;
      const int t = idx / D, e = idx % D;
      float acc = qacc[q];
      for (int jj = 0; jj < kHS; ++jj) {
        acc = fmaf(sW1[jj][e], sHB1[t][jj], acc);
        acc = fmaf(sW3[jj][e], sHB3[t][jj], acc);
      }
      qacc[q] = acc;
    }
  }
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int idx = tid + kThreads * q;
    const int t = idx / D, e = idx % D;
    const int64_t tok = t0 + t;
    if (tok < a.n) store_io<BF16>(a.dA, static_cast<int64_t>(pair) * a.out_stride + tok * D + e, qacc[q]);
  }
}

// ---------------------------------------------------------------------------
// Weight cotangents as token contractions, split over tokens.  Grid (S
// splits, h/32 hidden slices, P pairs).  Over the split's tokens:
//   out1[j][e] += X1[t][j] A[t][e],  out3[j][e] += X3[t][j] A[t][e],
//   out2[e][j] += b_t B[t][e] X2[t][j]   (b_t = -eta_t, or 1 without rates),
// written to partials[pair][split] in the [W1 | W2 | W3] block order.
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_bw_contract(BwContractArgs a) {
  constexpr int NACC = 3 * kHS * D / kThreads;
  __shared__ float sA[kTok][D + 1];
  __shared__ float sB[kTok][D + 1];
  __shared__ float sX1[kTok][kHS + 1], sX2[kTok][kHS + 1], sX3[kTok][kHS + 1];
  const int split = blockIdx.x;
  const int j0 = blockIdx.y * kHS;
  const int pair = blockIdx.z;
  const int tid = threadIdx.x;
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int64_t base = static_cast<int64_t>(pair) * a.in_stride;
  const float* X1 = a.X1 + static_cast<int64_t>(pair) * a.x_stride;
  const float* X2 = a.X2 + static_cast<int64_t>(pair) * a.x_stride;
  const float* X3 = a.X3 + static_cast<int64_t>(pair) * a.x_stride;
  const float* eta = a.eta ? a.eta + static_cast<int64_t>(pair) * a.eta_stride : nullptr;
  float acc[NACC];
#pragma unroll
  for (int q = 0; q < NACC; ++q) acc[q] = 0.f;
  const int64_t t_begin = static_cast<int64_t>(split) * a.tps;
  const int64_t t_end = min(a.n, t_begin + a.tps);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTok) {
    __syncthreads();
    for (int i = tid; i < kTok * D; i += kThreads) {
      const int t = i / D, e = i % D;
      const int64_t tok = t0 + t;
      float av = 0.f, bv = 0.f;
      if (tok < t_end) {
        av = load_io<BF16>(a.A, base + tok * D + e);
        bv = (eta ? -eta[tok] : 1.f) * load_io<BF16>(a.B, base + tok * D + e);
      }
      sA[t][e] = av;
      sB[t][e] = bv;
    }
    for (int i = tid; i < kTok * kHS; i += kThreads) {
      const int t = i / kHS, jj = i % kHS;
      const int64_t tok = t0 + t;
      const bool ok = tok < t_end;
      sX1[t][jj] = ok ? X1[tok * h + j0 + jj] : 0.f;
      sX2[t][jj] = ok ? X2[tok * h + j0 + jj] : 0.f;
      sX3[t][jj] = ok ? X3[tok * h + j0 + jj] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      const int idx = tid + kThreads * q;
      float s = 0.f;
      if (idx < kHS * D) {
        const int jj = idx / D, e = idx % D;
        for (int t = 0; t < kTok; ++t) s = fmaf(sX1[t][jj], sA[t][e], s);
      } else if (idx < 2 * kHS * D) {
        const int i2 = idx - kHS * D;
        const int jj = i2 / D, e = i2 % D;
        for (int t = 0; t < kTok; ++t) s = fmaf(sX3[t][jj], sA[t][e], s);
      } else {
        const int i3 = idx - 2 * kHS * D;
        const int e = i3 / kHS, jj = i3 % kHS;
        for (int t = 0; t < kTok; ++t) s = fmaf(sB[t][e], sX2[t][jj], s);
      }
      acc[q] += s;
    }
  }
  float* out = a.partials + (static_cast<int64_t>(pair) * a.S + split) * 3 * hd;
#pragma unroll
  for (int q = 0; q < NACC; ++q) {
    const int idx = tid + kThreads * q;
    if (idx < kHS * D) {
      const int jj = idx / D, e = idx % D;
      out[(j0 + jj) * D + e] = acc[q];
    } else if (idx < 2 * kHS * D) {
      const int i2 = idx - kHS * D;
      const int jj = i2 / D, e = i2 % D;
      out[2 * hd + (j0 + jj) * D + e] = acc[q];
    } else {
      const int i3 = idx - 2 * kHS * D;
      const int e = i3 / kHS, jj = i3 % kHS;
      out[hd + e * h + j0 + jj] = acc[q];
    }
  }
}

// dst[pair][e] += sum_s partials[pair][s][e], splits in order.
__global__ __launch_bounds__(kThreads) void k_bw_reduce_add(float* dst, const float* partials, int S, int64_t per,
                                                            int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int64_t pair = i / per, e = i % per;
  const float* src = partials + pair * S * per + e;
  float g = 0.f;
  for (int s = 0; s < S; ++s) g += src[static_cast<int64_t>(s) * per];
  dst[i] += g;
}

// ---------------------------------------------------------------------------
// Through W' = rows(W - step d) for every stored row (one wavefront per row):
// R = W - step d recomputed, Y = W' (checkpoint), dY the running cotangent
// (plus the split sums of the contractions still pending, in the order a
// separate reduction pass would have added them);
//   dR = (dY - Y (Y . dY)) / ||R||   (dY / norm_eps where ||R|| <= norm_eps),
// then the running cotangent becomes dR (W enters R directly) and the
// direction's cotangent is -step dR.
// ---------------------------------------------------------------------------
constexpr int kMaxRowPerLane = 16;

__global__ __launch_bounds__(kThreads) void k_bw_step(BwStepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int R = 2 * a.h + a.d;
  const int64_t pair = row / R;
  if (pair >= a.P) return;
  const int r = static_cast<int>(row % R);
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  int m, len;
  int64_t off;  // offset of the row inside its matrix
  if (r < a.h) {
    m = 0;
    len = a.d;
    off = static_cast<int64_t>(r) * a.d;
  } else if (r < 2 * a.h) {
    m = 2;
    len = a.d;
    off = static_cast<int64_t>(r - a.h) * a.d;
  } else {
    m = 1;
    len = a.h;
    off = static_cast<int64_t>(r - 2 * a.h) * a.h;
  }
  const float* W = a.W_in[m].p + pair * a.W_in[m].pair_stride + off;
  const float* Y = a.W_out[m].p + pair * a.W_out[m].pair_stride + off;
  const int64_t blk = pair * 3 * hd + m * hd + off;  // [W1 | W2 | W3] block layout
  float dy[kMaxRowPerLane], y[kMaxRowPerLane];
  float ss = 0.f, yd = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxRowPerLane; ++k) {
    const int e = lane + 64 * k;
    dy[k] = y[k] = 0.f;
    if (e < len) {
      const float dv = a.dir != nullptr ? a.dir[blk + e] : a.dir_m[m].p[pair * a.dir_m[m].pair_stride + off + e];
      const float rr = W[e] - a.step * dv;
      ss += rr * rr;
      y[k] = Y[e];
      dy[k] = a.cot[blk + e];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (a.pend[q] != nullptr) {
          const float* src = a.pend[q] + pair * a.pend_S[q] * 3 * hd + m * hd + off + e;
          float g = 0.f;
          for (int sp = 0; sp < a.pend_S[q]; ++sp) g += src[sp * 3 * hd];
          dy[k] += g;
        }
      }
      yd += y[k] * dy[k];
    }
  }
  ss = wave_sum(ss);
  yd = wave_sum(yd);
  const float nrm = sqrtf(ss);
  const bool big = nrm > a.norm_eps;
#pragma unroll
  for (int k = 0; k < kMaxRowPerLane; ++k) {
    const int e = lane + 64 * k;
    if (e < len) {
      const float dr = big ? (dy[k] - y[k] * yd) / nrm : dy[k] / a.norm_eps;
      a.cot[blk + e] = dr;
      const float dd = __fmul_rn(-a.step, dr);
      if (a.dM != nullptr) {
        const float v = __fadd_rn(dd, a.dM[blk + e]);
        a.pc[blk + e] = v;
        a.dM[blk + e] = __fmul_rn(a.beta, v);
      } else {
        a.ddir[blk + e] = dd;
      }
    }
  }
}

// dM_new = t + dM;  P = dM_new;  dM = beta dM_new   (elementwise, block layout)
__global__ __launch_bounds__(kThreads) void k_bw_momentum(const float* t, float* dM, float* Pout, float beta,
                                                          int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const float v = t[i] + dM[i];
  Pout[i] = v;
  dM[i] = beta * v;
}

// ---------------------------------------------------------------------------
// Newton-Schulz and its VJP, one workgroup per matrix (3P of them, block
// layout), in two kernels around the step's VJP.  On X (s x l,
// s = min(rows, cols), G transposed when rows > cols):
//   forward   X0 = G / (||G||_F + eps);  A_k = X_k X_k^T;  B_k = b A_k + c A_k A_k;
//             X_{k+1} = a X_k + B_k X_k   (iterates, A_k, B_k kept in scratch;
//             X_I, in G's orientation, is the update direction);
//   reverse   k = I-1 .. 0 with dY the cotangent of X_{k+1}:
//             dB = dY X_k^T,  dA = b dB + c (dB A_k^T + A_k^T dB),
//             dX_k = a dY + B_k^T dY + (dA + dA^T) X_k;
//   then dG = dX_0 / (n + eps) - (<dX_0, G> / (n + eps)^2) G / n.
// Every product runs on fp32 MFMA (v_mfma_f32_32x32x2_f32: products and sums
// in fp32; fp32 I/O) or as three bf16 MFMAs on hi + lo parts (wg_mm_bf; bf16
// I/O), 32 x 32 output tiles spread over the eight wavefronts, the operands
// staged through LDS 32 k values at a time.
// ---------------------------------------------------------------------------
constexpr int kNSThreads = 512;
constexpr int kNB = 256;  // output columns per block of a product

typedef __attribute__((ext_vector_type(16))) float ns_f32x16;

struct MOp {  // element (i, k) of a matrix operand at p[i * rs + k * cs]
  const float* p;
  int rs, cs;
};

// C (M x N) = sum over the terms t < NTERM of op(P_t) (M x K_t) op(Q_t) (K_t x N),
// handed to epi(i, j, value) element by element.  M <= 128, M, N, K_t
// multiples of 32.  The operands move through LDS 32 k values at a time,
// double-buffered: while the wavefronts multiply one chunk (Ps: 32 x (M + 1),
// Qs: 32 x (kNB + 1) floats per buffer), every thread holds its share of the
// next chunk's global loads in registers and then stores it into the other
// buffer.  Each thread's share is fixed per term (its LDS slots and element
// offsets), so only the chunk offset changes from chunk to chunk.
template <int NTERM, class Epi>
__device__ __forceinline__ void wg_mm(int M, int N, const int (&K)[NTERM], const MOp (&P)[NTERM],
                                      const MOp (&Q)[NTERM], float* Ps, float* Qs, Epi epi) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, ln = lane & 31;
  const int ps = M + 1;
  constexpr int PSZ = 32 * 129, QSZ = 32 * (kNB + 1);                        // floats per buffer
  constexpr int MP = 32 * 128 / kNSThreads, MQ = 32 * kNB / kNSThreads;  // staged values per thread
  for (int nb = 0; nb < N; nb += kNB) {
    const int NB = min(kNB, N - nb), qs = NB + 1;
    const int ntl = NB / 32, tiles = (M / 32) * ntl;  // <= 32: at most four per wave
    ns_f32x16 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
    }
#pragma unroll 1
    for (int t = 0; t < NTERM; ++t) {
      const MOp p = P[t], q = Q[t];
      // this thread's share of a chunk: element e is idx = tid + 512 e of the
      // chunk (in the order of the operand's contiguous index), at LDS slot
      // *l and offset *o from the chunk's first k (recomputed where used:
      // a few integer operations, where keeping them would cost registers)
      auto pslot = [&](int e, int& l, int& o) {
        int t2 = tid;
        asm volatile("" : "+v"(t2));  // (not hoisted out of the chunk loop)
        const int idx = t2 + kNSThreads * e;
        int i, k;
        if (p.cs == 1) {
          k = idx & 31;
          i = idx >> 5;
        } else {
          i = idx % M;
          k = idx / M;
        }
        l = k * ps + i;
        o = i * p.rs + k * p.cs;
        return idx < 32 * M;
      };
      auto qslot = [&](int e, int& l, int& o) {
        int t2 = tid;
        asm volatile("" : "+v"(t2));
        const int idx = t2 + kNSThreads * e;
        int j, k;
        if (q.cs == 1) {
          j = idx % NB;
          k = idx / NB;
        } else {
          k = idx & 31;
          j = idx >> 5;
        }
        l = k * qs + j;
        o = k * q.rs + (nb + j) * q.cs;
        return idx < 32 * NB;
      };
      float vp[MP], vq[MQ];
      auto load = [&](int kc) {
        const float* bp = p.p + static_cast<int64_t>(kc) * p.cs;
        const float* bq = q.p + static_cast<int64_t>(kc) * q.rs;
#pragma unroll
        for (int e = 0; e < MP; ++e) {
          int l, o;
          vp[e] = pslot(e, l, o) ? bp[o] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < MQ; ++e) {
          int l, o;
          vq[e] = qslot(e, l, o) ? bq[o] : 0.f;
        }
      };
      auto store = [&](int b) {
#pragma unroll
        for (int e = 0; e < MP; ++e) {
          int l, o;
          if (pslot(e, l, o)) Ps[b * PSZ + l] = vp[e];
        }
#pragma unroll
        for (int e = 0; e < MQ; ++e) {
          int l, o;
          if (qslot(e, l, o)) Qs[b * QSZ + l] = vq[e];
        }
      };
      const int nc = K[t] / 32;
      load(0);
      __syncthreads();  // the previous readers of both buffers are done
      store(0);
      __syncthreads();
      for (int c = 0; c < nc; ++c) {
        const int b = c & 1;
        if (c + 1 < nc) load(32 * (c + 1));
        const float* pb = Ps + b * PSZ;
        const float* qb = Qs + b * QSZ;
#pragma unroll 4
        for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int tt = wave + 8 * u;
            if (tt < tiles) {
              const int ti = tt / ntl, tj = tt % ntl;
              const float av = pb[(2 * ks + g) * ps + 32 * ti + ln];
              const float bv = qb[(2 * ks + g) * qs + 32 * tj + ln];
              acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[u], 0, 0, 0);
            }
          }
        }
        if (c + 1 < nc) store(b ^ 1);
        __syncthreads();
      }
    }
    // acc[u][r] = C[32 ti + 8 (r / 4) + 4 g + r % 4][nb + 32 tj + ln]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tt = wave + 8 * u;
      if (tt < tiles) {
        const int ti = tt / ntl, tj = tt % ntl;
#pragma unroll
        for (int r = 0; r < 16; ++r) epi(32 * ti + 8 * (r >> 2) + 4 * g + (r & 3), nb + 32 * tj + ln, acc[u][r]);
      }
    }
  }
  __syncthreads();  // every element of C written (global, visible to the workgroup)
}

// The same products with every fp32 operand value x split into bf16 parts
// hi = bf16(x), lo = bf16(x - hi) and the three products hi hi + hi lo + lo hi
// on v_mfma_f32_32x32x16_bf16 (fp32 sums; the dropped lo lo term is ~2^-16 of
// a product): about five times the fp32 matrix-core rate.  LDS holds 32 k
// values per operand row as bf16 (hi and lo arrays), rows of 80 bytes, so the
// 16-byte operand reads of 16 consecutive rows fall into distinct banks.
// Each thread stages eight k values of one operand row per task (one task of
// the M x 32 chunk of op(P), two of the NB x 32 chunk of op(Q)), loading
// along whichever index is contiguous in memory.
typedef __attribute__((ext_vector_type(8))) __bf16 nsb_bf16x8;
typedef __attribute__((ext_vector_type(4))) float nsb_f32x4;
constexpr int kBRow = 40;                   // bf16 per LDS row (32 + 8 padding)
constexpr int kBP = 128 * kBRow;            // bf16 of one P part (hi or lo)
constexpr int kBQ = kNB * kBRow;            // bf16 of one Q part
constexpr int kBBuf = 2 * kBP + 2 * kBQ;    // one stage: P hi, P lo, Q hi, Q lo
constexpr int kNSBfLds = 2 * kBBuf * 2;     // bytes, two stages
constexpr int kNSF32Lds = (2 * 32 * 129 + 2 * 32 * (kNB + 1)) * 4;

__device__ __forceinline__ void nsb_split(const float (&v)[8], nsb_bf16x8& hi, nsb_bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = static_cast<__bf16>(v[e]);
    lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(hi[e]));
  }
}

// eight values of a matrix starting at src with element stride st (16-byte
// aligned vector loads where st == 1)
__device__ __forceinline__ void nsb_load8(const float* src, int st, float (&v)[8]) {
  if (st == 1) {
    const nsb_f32x4 a = *reinterpret_cast<const nsb_f32x4*>(src);
    const nsb_f32x4 b = *reinterpret_cast<const nsb_f32x4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[static_cast<int64_t>(e) * st];
  }
}

template <int NTERM, class Epi>
__device__ __forceinline__ void wg_mm_bf(int M, int N, const int (&K)[NTERM], const MOp (&P)[NTERM],
                                         const MOp (&Q)[NTERM], uint16_t* lds, Epi epi) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, ln = lane & 31;
  for (int nb = 0; nb < N; nb += kNB) {
    const int NB = min(kNB, N - nb);
    const int ntl = NB / 32, tiles = (M / 32) * ntl;  // <= 32: at most four per wave
    ns_f32x16 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
    }
#pragma unroll 1
    for (int t = 0; t < NTERM; ++t) {
      const MOp p = P[t], q = Q[t];
      // tasks: (row, octet of k); rows follow the contiguous index when k is not it
      int pi, po, qj[2], qo[2];
      if (p.cs == 1) {
        pi = tid >> 2;
        po = tid & 3;
      } else {
        pi = tid % M;
        po = tid / M;
      }
      const bool pv = tid < 4 * M;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int task = tid + kNSThreads * u;
        if (q.rs == 1) {
          qj[u] = task >> 2;
          qo[u] = task & 3;
        } else {
          qj[u] = task % NB;
          qo[u] = task / NB;
        }
      }
      float vp[8], vq[2][8];
      auto load = [&](int kc) {
        if (pv) nsb_load8(p.p + static_cast<int64_t>(pi) * p.rs + static_cast<int64_t>(kc + 8 * po) * p.cs, p.cs, vp);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (tid + kNSThreads * u < 4 * NB)
            nsb_load8(q.p + static_cast<int64_t>(kc + 8 * qo[u]) * q.rs + static_cast<int64_t>(nb + qj[u]) * q.cs,
                      q.rs, vq[u]);
        }
      };
      auto store = [&](int b) {
        uint16_t* base = lds + b * kBBuf;
        nsb_bf16x8 hi, lo;
        if (pv) {
          nsb_split(vp, hi, lo);
          *reinterpret_cast<nsb_bf16x8*>(base + pi * kBRow + 8 * po) = hi;
          *reinterpret_cast<nsb_bf16x8*>(base + kBP + pi * kBRow + 8 * po) = lo;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (tid + kNSThreads * u < 4 * NB) {
            nsb_split(vq[u], hi, lo);
            *reinterpret_cast<nsb_bf16x8*>(base + 2 * kBP + qj[u] * kBRow + 8 * qo[u]) = hi;
            *reinterpret_cast<nsb_bf16x8*>(base + 2 * kBP + kBQ + qj[u] * kBRow + 8 * qo[u]) = lo;
          }
        }
      };
      const int nc = K[t] / 32;
      load(0);
      __syncthreads();  // the previous readers of both buffers are done
      store(0);
      __syncthreads();
      for (int c = 0; c < nc; ++c) {
        const int b = c & 1;
        if (c + 1 < nc) load(32 * (c + 1));
        const uint16_t* base = lds + b * kBBuf;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int tt = wave + 8 * u;
            if (tt < tiles) {
              const int ti = tt / ntl, tj = tt % ntl;
              const int pa = (32 * ti + ln) * kBRow + 16 * ks + 8 * g;
              const int qa = 2 * kBP + (32 * tj + ln) * kBRow + 16 * ks + 8 * g;
              const nsb_bf16x8 ah = *reinterpret_cast<const nsb_bf16x8*>(base + pa);
              const nsb_bf16x8 al = *reinterpret_cast<const nsb_bf16x8*>(base + kBP + pa);
              const nsb_bf16x8 bh = *reinterpret_cast<const nsb_bf16x8*>(base + qa);
              const nsb_bf16x8 bl = *reinterpret_cast<const nsb_bf16x8*>(base + kBQ + qa);
              acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[u], 0, 0, 0);
              acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[u], 0, 0, 0);
              acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[u], 0, 0, 0);
            }
          }
        }
        if (c + 1 < nc) store(b ^ 1);
        __syncthreads();
      }
    }
    // acc[u][r] = C[32 ti + 8 (r / 4) + 4 g + r % 4][nb + 32 tj + ln]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tt = wave + 8 * u;
      if (tt < tiles) {
        const int ti = tt / ntl, tj = tt % ntl;
#pragma unroll
        for (int r = 0; r < 16; ++r) epi(32 * ti + 8 * (r >> 2) + 4 * g + (r & 3), nb + 32 * tj + ln, acc[u][r]);
      }
    }
  }
  __syncthreads();  // every element of C written (global, visible to the workgroup)
}

// the products of one Newton-Schulz kernel: fp32 or split-bf16 matrix cores
template <bool BF, int NTERM, class Epi>
__device__ __forceinline__ void ns_mm(int M, int N, const int (&K)[NTERM], const MOp (&P)[NTERM],
                                     const MOp (&Q)[NTERM], unsigned char* lds, Epi epi) {
  if constexpr (BF) {
    wg_mm_bf(M, N, K, P, Q, reinterpret_cast<uint16_t*>(lds), epi);
  } else {
    float* f = reinterpret_cast<float*>(lds);
    wg_mm(M, N, K, P, Q, f, f + 2 * 32 * 129, epi);
  }
}

// One matrix's geometry and scratch (floats): iterates X_0 .. X_I (s l each),
// dY and dX (s l), A_0 .. A_{I-1}, B_0 .. B_{I-1} (s s each), dB, dA (s s).
struct NSMat {
  int mat, pair, which, rows, cols, s, l;
  bool tr;
  int64_t hd, sl, ss;
  float *xs, *dY, *dX, *As, *Bs, *dB, *dA;
  __device__ NSMat(const BwNSArgs& a) {
    mat = blockIdx.x;
    pair = mat / 3;
    which = mat % 3;  // 0: W1, 1: W2, 2: W3
    hd = static_cast<int64_t>(a.h) * a.d;
    rows = (which == 1) ? a.d : a.h;
    cols = (which == 1) ? a.h : a.d;
    tr = rows > cols;
    s = tr ? cols : rows;
    l = tr ? rows : cols;
    sl = static_cast<int64_t>(s) * l;
    ss = static_cast<int64_t>(s) * s;
    xs = a.scratch + static_cast<int64_t>(mat) * a.per_mat;
    dY = xs + (a.iters + 1) * sl;
    dX = dY + sl;
    As = dX + sl;
    Bs = As + a.iters * ss;
    dB = Bs + a.iters * ss;
    dA = dB + ss;
  }
  __device__ int64_t gidx(int i, int j) const {  // element (i, j) of the s x l orientation in G's storage
    return tr ? static_cast<int64_t>(j) * cols + i : static_cast<int64_t>(i) * cols + j;
  }
};

__device__ __forceinline__ float ns_block_sum(float v, float* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int w = kNSThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

template <bool BF>
__global__ __launch_bounds__(kNSThreads) void k_bw_ns_fwd(BwNSArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[BF ? kNSBfLds : kNSF32Lds];
  __shared__ float red[kNSThreads];
  const NSMat m(a);
  const int tid = threadIdx.x;
  const float ca = a.a, cb = a.b, cc = a.c;
  const float* G = a.g + m.pair * 3 * m.hd + m.which * m.hd;
  float* dir = a.out + m.pair * 3 * m.hd + m.which * m.hd;
  float part = 0.f;
  for (int64_t i = tid; i < m.sl; i += kNSThreads) {
    const float v = G[i];
    part += v * v;
  }
  const float den = sqrtf(ns_block_sum(part, red)) + a.eps;
  for (int64_t idx = tid; idx < m.sl; idx += kNSThreads) {
    const int i = static_cast<int>(idx / m.l), j = static_cast<int>(idx % m.l);
    m.xs[idx] = G[m.gidx(i, j)] / den;
  }
  __syncthreads();
  const int s = m.s, l = m.l;
  for (int it = 0; it < a.iters; ++it) {
    const float* X = m.xs + it * m.sl;
    float* Xn = m.xs + (it + 1) * m.sl;
    float* A = m.As + it * m.ss;
    float* B = m.Bs + it * m.ss;
    {  // A = X X^T
      const int K[1] = {l};
      const MOp P[1] = {{X, l, 1}}, Q[1] = {{X, 1, l}};
      ns_mm<BF>(s, s, K, P, Q, lds, [&](int i, int j, float v) { A[i * s + j] = v; });
    }
    {  // B = b A + c A A
      const int K[1] = {s};
      const MOp P[1] = {{A, s, 1}}, Q[1] = {{A, s, 1}};
      ns_mm<BF>(s, s, K, P, Q, lds, [&](int i, int j, float v) { B[i * s + j] = cb * A[i * s + j] + cc * v; });
    }
    {  // X <- a X + B X
      const int K[1] = {s};
      const MOp P[1] = {{B, s, 1}}, Q[1] = {{X, l, 1}};
      ns_mm<BF>(s, l, K, P, Q, lds,
            [&](int i, int j, float v) { Xn[static_cast<int64_t>(i) * l + j] = ca * X[static_cast<int64_t>(i) * l + j] + v; });
    }
  }
  const float* XI = m.xs + a.iters * m.sl;
  for (int64_t idx = tid; idx < m.sl; idx += kNSThreads) {
    const int i = static_cast<int>(idx / l), j = static_cast<int>(idx % l);
    dir[m.gidx(i, j)] = XI[idx];
  }
}

template <bool BF>
__global__ __launch_bounds__(kNSThreads) void k_bw_ns(BwNSArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[BF ? kNSBfLds : kNSF32Lds];
  __shared__ float red[kNSThreads];
  const NSMat m(a);
  const int tid = threadIdx.x;
  const float ca = a.a, cb = a.b, cc = a.c;
  const float* G = a.g + m.pair * 3 * m.hd + m.which * m.hd;
  const float* dXin = a.dx + m.pair * 3 * m.hd + m.which * m.hd;
  float* dG = a.out + m.pair * 3 * m.hd + m.which * m.hd;
  const int s = m.s, l = m.l;
  float* dY = m.dY;
  float* dXn = m.dX;
  for (int64_t idx = tid; idx < m.sl; idx += kNSThreads) {
    const int i = static_cast<int>(idx / l), j = static_cast<int>(idx % l);
    dY[idx] = dXin[m.gidx(i, j)];
  }
  __syncthreads();
  for (int it = a.iters - 1; it >= 0; --it) {
    const float* X = m.xs + it * m.sl;
    const float* A = m.As + it * m.ss;
    const float* B = m.Bs + it * m.ss;
    {  // dB = dY X^T
      const int K[1] = {l};
      const MOp P[1] = {{dY, l, 1}}, Q[1] = {{X, 1, l}};
      ns_mm<BF>(s, s, K, P, Q, lds, [&](int i, int j, float v) { m.dB[i * s + j] = v; });
    }
    {  // dA = b dB + c (dB A^T + A^T dB)
      const int K[2] = {s, s};
      const MOp P[2] = {{m.dB, s, 1}, {A, 1, s}}, Q[2] = {{A, 1, s}, {m.dB, s, 1}};
      ns_mm<BF>(s, s, K, P, Q, lds, [&](int i, int j, float v) { m.dA[i * s + j] = cb * m.dB[i * s + j] + cc * v; });
    }
    {  // dX = a dY + B^T dY + dA X + dA^T X
      const int K[3] = {s, s, s};
      const MOp P[3] = {{B, 1, s}, {m.dA, s, 1}, {m.dA, 1, s}}, Q[3] = {{dY, l, 1}, {X, l, 1}, {X, l, 1}};
      ns_mm<BF>(s, l, K, P, Q, lds, [&](int i, int j, float v) {
        dXn[static_cast<int64_t>(i) * l + j] = ca * dY[static_cast<int64_t>(i) * l + j] + v;
      });
    }
    float* t = dY;
    dY = dXn;
    dXn = t;
  }
  // through X0 = G / (n + eps)
  float part = 0.f, dot = 0.f;
  for (int64_t idx = tid; idx < m.sl; idx += kNSThreads) {
    const int i = static_cast<int>(idx / l), j = static_cast<int>(idx % l);
    const float gv = G[m.gidx(i, j)];
    part += gv * gv;
    dot += dY[idx] * gv;
  }
  const float nrm = sqrtf(ns_block_sum(part, red));
  dot = ns_block_sum(dot, red);
  const float den = nrm + a.eps;
  const float coef = nrm > 0.f ? dot / (den * den * nrm) : 0.f;
  for (int64_t idx = tid; idx < m.sl; idx += kNSThreads) {
    const int i = static_cast<int>(idx / l), j = static_cast<int>(idx % l);
    const int64_t gi = m.gidx(i, j);
    dG[gi] = dY[idx] / den - coef * G[gi];
  }
}

// Moves between separate W1 | W2 | W3 arrays (pair stride h d each) and the
// per-pair [W1 | W2 | W3] blocks; to_blocks = 1: separate -> blocks.  With a
// NULL source the destination is zeroed.
__global__ __launch_bounds__(kThreads) void k_bw_copy(float* blocks, MatRef m1, MatRef m2, MatRef m3, int64_t hd,
                                                      int64_t total, int to_blocks) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int64_t pair = i / (3 * hd), e = i % (3 * hd);
  const MatRef& r = e < hd ? m1 : (e < 2 * hd ? m2 : m3);
  const int64_t off = e % hd;
  if (to_blocks) {
    blocks[i] = r.p ? r.p[pair * r.pair_stride + off] : 0.f;
  } else {
    r.p[pair * r.pair_stride + off] = blocks[i];
  }
}

template <int D>
hipError_t launch_tok_d(const BwTokArgs& a, bool apply, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.n + kTok - 1) / kTok), a.P);
  if (apply) {
    if (a.bf16) hipLaunchKernelGGL((k_bw_apply_tok<true, D>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_bw_apply_tok<false, D>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (a.bf16) hipLaunchKernelGGL((k_bw_grad_tok<true, D>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_bw_grad_tok<false, D>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_contract_d(const BwContractArgs& a, hipStream_t s) {
  const dim3 grid(a.S, a.h / kHS, a.P);
  if (a.bf16) hipLaunchKernelGGL((k_bw_contract<true, D>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_bw_contract<false, D>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool backward_shape_ok(int d, int h) { return (d == 32 || d == 64 || d == 128) && h % kHS == 0 && h >= kHS && h <= 1024; }

hipError_t launch_bw_tok(const BwTokArgs& a, bool apply, hipStream_t s) {
  if (bw_tok_mfma_ok(a, apply)) return launch_bw_tok_mfma(a, apply, s);
  if (a.x_bf16) return hipErrorInvalidValue;  // (bf16 factors only from the matrix-core kernels)
  switch (a.d) {
    case 32: return launch_tok_d<32>(a, apply, s);
    case 64: return launch_tok_d<64>(a, apply, s);
    case 128: return launch_tok_d<128>(a, apply, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bw_contract(const BwContractArgs& a, hipStream_t s) {
  if (bw_contract_mfma_ok(a)) return launch_bw_contract_mfma(a, s);
  if (a.x_bf16) return hipErrorInvalidValue;  // (bf16 factors only for the matrix-core contraction)
  switch (a.d) {
    case 32: return launch_contract_d<32>(a, s);
    case 64: return launch_contract_d<64>(a, s);
    case 128: return launch_contract_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bw_reduce_add(float* dst, const float* partials, int S, int64_t per, int P, hipStream_t s) {
  const int64_t total = per * P;
  hipLaunchKernelGGL(k_bw_reduce_add, dim3(static_cast<unsigned>((total + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, s, dst, partials, S, per, total);
  return hipGetLastError();
}

hipError_t launch_bw_step(const BwStepArgs& a, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.P) * (2 * a.h + a.d);
  hipLaunchKernelGGL(k_bw_step, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bw_momentum(const float* t, float* dM, float* Pout, float beta, int64_t total, hipStream_t s) {
  hipLaunchKernelGGL(k_bw_momentum, dim3(static_cast<unsigned>((total + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     s, t, dM, Pout, beta, total);
  return hipGetLastError();
}

int64_t bw_ns_floats_per_matrix(int d, int h, int iters) {
  const int64_t s = d < h ? d : h, l = d < h ? h : d;
  return (iters + 3) * s * l + (2 * iters + 2) * s * s;
}

hipError_t launch_bw_ns(const BwNSArgs& a, hipStream_t s) {
  if (a.d % 32 != 0 || a.h % 32 != 0 || (a.d < a.h ? a.d : a.h) > 128) return hipErrorInvalidValue;
  if (a.bf16_split)
    hipLaunchKernelGGL(k_bw_ns<true>, dim3(3 * a.P), dim3(kNSThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_bw_ns<false>, dim3(3 * a.P), dim3(kNSThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bw_ns_fwd(const BwNSArgs& a, hipStream_t s) {
  if (a.d % 32 != 0 || a.h % 32 != 0 || (a.d < a.h ? a.d : a.h) > 128) return hipErrorInvalidValue;
  if (a.bf16_split)
    hipLaunchKernelGGL(k_bw_ns_fwd<true>, dim3(3 * a.P), dim3(kNSThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_bw_ns_fwd<false>, dim3(3 * a.P), dim3(kNSThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bw_copy(float* blocks, const MatRef& m1, const MatRef& m2, const MatRef& m3, int P, int d, int h,
                          bool to_blocks, hipStream_t s) {
  const int64_t hd = static_cast<int64_t>(h) * d;
  const int64_t total = 3 * hd * P;
  hipLaunchKernelGGL(k_bw_copy, dim3(static_cast<unsigned>((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     blocks, m1, m2, m3, hd, total, to_blocks ? 1 : 0);
  return hipGetLastError();
}

}  // namespace lact

// Generic kernels of the LaCT layer: fp32 arithmetic for every supported
// (d, h), fp32 or bf16 activations.  They serve the fp32 I/O mode and any
// shape that has no MFMA kernel; every step of the layer has one here:
//   chunk gradient (split over tokens), fixed-order split reduction with
//   fused momentum, Newton-Schulz, step + row L2 normalisation, query read.
// The method is the one of "LaCT: Large Chunk Test-Time Training"
// (iplexlaw.co.kr review), section "Local attention and nonlinear memory
// work together".
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

constexpr int kThreads = 256;
constexpr int kTok = 32;  // tokens per LDS tile
constexpr int kHS = 32;   // hidden units per workgroup

// ---------------------------------------------------------------------------
// Chunk gradient.  Grid (S splits, h/32 hidden slices, P pairs).  Each
// workgroup owns 32 hidden units j and the tokens of one split:
//   h1 = k.W1[j], h3 = k.W3[j], dg = u.W2[:, j]  (u = -eta v)
//   a = silu(h1), g = a h3, dh3 = dg a, dh1 = dg h3 silu'(h1)
//   dW1[j] += dh1 k,  dW3[j] += dh3 k,  dW2[:, j] += g u.
// Tokens past the split end load as zero and contribute nothing.  PM: a rate
// per token and matrix (rows for W1, W2, W3, a.eta_mat elements apart): u = v
// is staged unscaled, dg of W1 / W3 takes -eta1 / -eta3 and g takes -eta2.
// ---------------------------------------------------------------------------
template <bool BF16, int D, bool PM>
__global__ __launch_bounds__(kThreads) void k_grad_generic(GradArgs a) {
  constexpr int NACC = 3 * kHS * D / kThreads;
  __shared__ float sW1[kHS][D + 1];
  __shared__ float sW3[kHS][D + 1];
  __shared__ float sW2[D][kHS + 1];
  __shared__ float sK[kTok][D + 1];
  __shared__ float sU[kTok][D + 1];
  __shared__ float sdh1[kTok][kHS + 1];
  __shared__ float sdh3[kTok][kHS + 1];
  __shared__ float sg[kTok][kHS + 1];
  __shared__ float sE[PM ? 3 : 1][kTok];  // with PM: -eta of W1, W2, W3 per token

  const int split = blockIdx.x;
  const int j0 = blockIdx.y * kHS;
  const int pair = blockIdx.z;
  const int tid = threadIdx.x;
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;

  const float* W1 = a.W1 + pair * hd;
  const float* W2 = a.W2 + pair * hd;
  const float* W3 = a.W3 + pair * hd;
  for (int i = tid; i < kHS * D; i += kThreads) {
    const int jj = i / D, e = i % D;
    sW1[jj][e] = W1[(j0 + jj) * D + e];
    sW3[jj][e] = W3[(j0 + jj) * D + e];
  }
  for (int i = tid; i < D * kHS; i += kThreads) {
    const int e = i / kHS, jj = i % kHS;
    sW2[e][jj] = W2[e * h + j0 + jj];
  }

  float acc[NACC];
#pragma unroll
  for (int q = 0; q < NACC; ++q) acc[q] = 0.f;

  const int64_t t_begin = static_cast<int64_t>(split) * a.tps;
  const int64_t t_end = min(a.n, t_begin + a.tps);
  const int64_t kv_base = static_cast<int64_t>(pair) * a.kv_stride;
  const float* eta = a.eta + static_cast<int64_t>(pair) * a.eta_stride;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTok) {
    __syncthreads();
    for (int i = tid; i < kTok * D; i += kThreads) {
      const int t = i / D, e = i % D;
      const int64_t tok = t0 + t;
      float kv = 0.f, u = 0.f;
      if (tok < t_end) {
        kv = load_io<BF16>(a.K, kv_base + tok * D + e);
        u = (PM ? 1.f : -eta[tok]) * load_io<BF16>(a.V, kv_base + tok * D + e);
      }
      sK[t][e] = kv;
      sU[t][e] = u;
    }
    if constexpr (PM) {
      for (int i = tid; i < 3 * kTok; i += kThreads) {
        const int m = i / kTok, t = i % kTok;
        const int64_t tok = t0 + t;
        sE[m][t] = tok < t_end ? -eta[m * a.eta_mat + tok] : 0.f;
      }
    }
    __syncthreads();
    {
      const int jj = tid % kHS;
      const int tb = tid / kHS;
#pragma unroll
      for (int r = 0; r < kTok / (kThreads / kHS); ++r) {
        const int t = tb + (kThreads / kHS) * r;
        float h1 = 0.f, h3 = 0.f, dg = 0.f;
        for (int e = 0; e < D; ++e) {
          const float k = sK[t][e];
          h1 += k * sW1[jj][e];
          h3 += k * sW3[jj][e];
          dg += sU[t][e] * sW2[e][jj];
        }
        const float s = sigmoid_f(h1);
        const float act = h1 * s;
        float dg1 = dg, dg3 = dg, gv = act * h3;
        if constexpr (PM) {
          dg1 = sE[0][t] * dg;
          gv = sE[1][t] * gv;
          dg3 = sE[2][t] * dg;
        }
        sg[t][jj] = gv;
        sdh3[t][jj] = dg3 * act;
        sdh1[t][jj] = dg1 * h3 * (s * (1.f + h1 * (1.f - s)));
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      const int idx = tid + kThreads * q;
      float s = 0.f;
      if (idx < kHS * D) {
        const int jj = idx / D, e = idx % D;
        for (int t = 0; t < kTok; ++t) s += sdh1[t][jj] * sK[t][e];
      } else if (idx < 2 * kHS * D) {
        const int i2 = idx - kHS * D;
        const int jj = i2 / D, e = i2 % D;
        for (int t = 0; t < kTok; ++t) s += sdh3[t][jj] * sK[t][e];
      } else {
        const int i3 = idx - 2 * kHS * D;
        const int e = i3 / kHS, jj = i3 % kHS;
        for (int t = 0; t < kTok; ++t) s += sU[t][e] * sg[t][jj];
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

// ---------------------------------------------------------------------------
// Split reduction in fixed order s = 0..S-1, momentum fused.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_reduce(ReduceArgs a) {
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  const int64_t per = 3 * hd;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= per * a.P) return;
  const int64_t pair = i / per, e = i % per;
  const float* src = a.partials + pair * a.S * per + e;
  float g = 0.f;
  int s = 0;
  for (; s + 8 <= a.S; s += 8) {  // eight loads in flight, summed in split order
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = src[static_cast<int64_t>(s + u) * per];
#pragma unroll
    for (int u = 0; u < 8; ++u) g += t[u];
  }
  for (; s < a.S; ++s) g += src[static_cast<int64_t>(s) * per];
  if (a.M1 != nullptr) {
    float* M;
    int64_t off;
    if (e < hd) {
      M = a.M1;
      off = e;
    } else if (e < 2 * hd) {
      M = a.M2;
      off = e - hd;
    } else {
      M = a.M3;
      off = e - 2 * hd;
    }
    const float m = a.beta * M[pair * hd + off] + g;
    M[pair * hd + off] = m;
    g = m;
  }
  a.dir[i] = g;
}

// The same sum on 16-byte groups of four consecutive elements (every sum
// still runs over the splits in order, so the result is the same bit for
// bit); 3 h d is a multiple of 4 and no group straddles two matrices.  The
// caller checks that every pointer is 16-byte aligned.
__global__ __launch_bounds__(kThreads) void k_reduce_v4(ReduceArgs a) {
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  const int64_t per4 = 3 * hd / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= per4 * a.P) return;
  const int64_t pair = i / per4, e4 = i % per4;
  const float4* src = reinterpret_cast<const float4*>(a.partials) + pair * a.S * per4 + e4;
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
  // the splits in rounds of 16: every load of a round is issued before the
  // first add (the last round masked), and the adds run in split order
  constexpr int U = 16;
  for (int s = 0; s < a.S; s += U) {
    float4 t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < a.S) t[u] = src[static_cast<int64_t>(s + u) * per4];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < a.S) {
        g.x += t[u].x;
        g.y += t[u].y;
        g.z += t[u].z;
        g.w += t[u].w;
      }
    }
  }
  if (a.M1 != nullptr) {
    const int64_t e = 4 * e4;
    float* M;
    int64_t off;
    if (e < hd) {
      M = a.M1;
      off = e;
    } else if (e < 2 * hd) {
      M = a.M2;
      off = e - hd;
    } else {
      M = a.M3;
      off = e - 2 * hd;
    }
    float4* mp = reinterpret_cast<float4*>(M + pair * hd + off);
    const float4 m = *mp;
    g.x = a.beta * m.x + g.x;
    g.y = a.beta * m.y + g.y;
    g.z = a.beta * m.z + g.z;
    g.w = a.beta * m.w + g.w;
    *mp = g;
  }
  reinterpret_cast<float4*>(a.dir)[i] = g;
}

// ---------------------------------------------------------------------------
// Newton-Schulz, one workgroup per matrix, operands in global scratch.
// X is s x l with s = min(rows, cols); X0 = G / (||G||_F + eps);
//   A = X X^T;  B = b A + c A A;  X <- a X + B X.
// ---------------------------------------------------------------------------
constexpr int kNSThreads = 512;

__global__ __launch_bounds__(kNSThreads) void k_ns_generic(NSArgs a) {
  __shared__ float red[kNSThreads];
  const int mat = blockIdx.x;
  const int pair = mat / 3, which = mat % 3;  // 0: W1, 1: W2, 2: W3
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  float* G = a.dir + pair * 3 * hd + which * hd;
  const int rows = (which == 1) ? a.d : a.h;
  const int cols = (which == 1) ? a.h : a.d;
  const bool tr = rows > cols;
  const int s = tr ? cols : rows;
  const int l = tr ? rows : cols;
  const int64_t sl = static_cast<int64_t>(s) * l, ss = static_cast<int64_t>(s) * s;
  float* X = a.scratch + static_cast<int64_t>(mat) * (2 * sl + 2 * ss);
  float* Xn = X + sl;
  float* A = Xn + sl;
  float* Bm = A + ss;
  const int tid = threadIdx.x;

  float part = 0.f;
  for (int64_t i = tid; i < sl; i += kNSThreads) part += G[i] * G[i];
  red[tid] = part;
  __syncthreads();
  for (int w = kNSThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float denom = sqrtf(red[0]) + a.eps;
  for (int64_t idx = tid; idx < sl; idx += kNSThreads) {
    const int i = static_cast<int>(idx / l), j = static_cast<int>(idx % l);
    X[idx] = (tr ? G[static_cast<int64_t>(j) * cols + i] : G[static_cast<int64_t>(i) * cols + j]) / denom;
  }
  __syncthreads();
  for (int it = 0; it < a.iters; ++it) {
    for (int64_t idx = tid; idx < ss; idx += kNSThreads) {
      const int i = static_cast<int>(idx / s), k = static_cast<int>(idx % s);
      const float* xi = X + static_cast<int64_t>(i) * l;
      const float* xk = X + static_cast<int64_t>(k) * l;
      float acc = 0.f;
      for (int j = 0; j < l; ++j) acc += xi[j] * xk[j];
      A[idx] = acc;
    }
    __syncthreads();
    for (int64_t idx = tid; idx < ss; idx += kNSThreads) {
      const int i = static_cast<int>(idx / s), k = static_cast<int>(idx % s);
      float acc = 0.f;
      for (int m = 0; m < s; ++m) acc += A[static_cast<int64_t>(i) * s + m] * A[static_cast<int64_t>(m) * s + k];
      Bm[idx] = a.b * A[idx] + a.c * acc;
    }
    __syncthreads();
    for (int64_t idx = tid; idx < sl; idx += kNSThreads) {
      const int i = static_cast<int>(idx / l), j = static_cast<int>(idx % l);
      float acc = 0.f;
      for (int m = 0; m < s; ++m) acc += Bm[static_cast<int64_t>(i) * s + m] * X[static_cast<int64_t>(m) * l + j];
      Xn[idx] = a.a * X[idx] + acc;
    }
    __syncthreads();
    float* t = X;
    X = Xn;
    Xn = t;
  }
  for (int64_t idx = tid; idx < sl; idx += kNSThreads) {
    const int i = static_cast<int>(idx / l), j = static_cast<int>(idx % l);
    if (tr) {
      G[static_cast<int64_t>(j) * cols + i] = X[idx];
    } else {
      G[static_cast<int64_t>(i) * cols + j] = X[idx];
    }
  }
}

// ---------------------------------------------------------------------------
// W <- W - step * dir, then every row to unit L2 norm (or, with norm_keep,
// back to its length before the step).  One wavefront per row; rows of W1
// and W3 have d entries, rows of W2 have h (<= 1024).
// ---------------------------------------------------------------------------
constexpr int kMaxRowPerLane = 16;

__global__ __launch_bounds__(kThreads) void k_step_norm(StepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int R = 2 * a.h + a.d;
  const int64_t pair = row / R;
  if (pair >= a.P) return;
  const int r = static_cast<int>(row % R);
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  float* W;
  const float* dr;
  int len;
  if (r < a.h) {
    W = a.W1 + pair * hd + static_cast<int64_t>(r) * a.d;
    dr = a.dir + pair * 3 * hd + static_cast<int64_t>(r) * a.d;
    len = a.d;
  } else if (r < 2 * a.h) {
    W = a.W3 + pair * hd + static_cast<int64_t>(r - a.h) * a.d;
    dr = a.dir + pair * 3 * hd + 2 * hd + static_cast<int64_t>(r - a.h) * a.d;
    len = a.d;
  } else {
    W = a.W2 + pair * hd + static_cast<int64_t>(r - 2 * a.h) * a.h;
    dr = a.dir + pair * 3 * hd + hd + static_cast<int64_t>(r - 2 * a.h) * a.h;
    len = a.h;
  }
  float v[kMaxRowPerLane];
  float ss = 0.f, ss_old = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxRowPerLane; ++k) {
    const int e = lane + 64 * k;
    v[k] = 0.f;
    if (e < len) {
      const float w = W[e];
      ss_old += w * w;
      v[k] = w - a.step * dr[e];
      ss += v[k] * v[k];
    }
  }
  ss = wave_sum(ss);
  const float den = fmaxf(sqrtf(ss), a.norm_eps);
  const float len_new = a.norm_keep ? sqrtf(wave_sum(ss_old)) : 1.f;
#pragma unroll
  for (int k = 0; k < kMaxRowPerLane; ++k) {
    const int e = lane + 64 * k;
    if (e < len) W[e] = len_new * (v[k] / den);
  }
}

// ---------------------------------------------------------------------------
// GD / momentum update tail, one wavefront per stored row: fixed-order sum of
// the split partials, M <- beta M + g (when kept), W <- W - step g, unit row
// (or, with norm_keep, the row back to its length before the step).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_reduce_step(TailArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int R = 2 * a.h + a.d;
  const int64_t pair = row / R;
  if (pair >= a.P) return;
  const int r = static_cast<int>(row % R);
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  float* W;
  float* M;
  uint16_t* Wb;
  int64_t po;
  int len;
  if (r < a.h) {
    W = a.W1;
    M = a.M1;
    Wb = a.Wb1;
    po = static_cast<int64_t>(r) * a.d;
    len = a.d;
  } else if (r < 2 * a.h) {
    W = a.W3;
    M = a.M3;
    Wb = a.Wb3;
    po = 2 * hd + static_cast<int64_t>(r - a.h) * a.d;
    len = a.d;
  } else {
    W = a.W2;
    M = a.M2;
    Wb = a.Wb2;
    po = hd + static_cast<int64_t>(r - 2 * a.h) * a.h;
    len = a.h;
  }
  const int64_t wo = pair * hd + (po % hd);  // offset of this row inside its matrix
  const float* part = a.partials + pair * a.splits * 3 * hd + po;
  float v[kMaxRowPerLane];
  float ss = 0.f, ss_old = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxRowPerLane; ++k) {
    const int e = lane + 64 * k;
    v[k] = 0.f;
    if (e < len) {
      float g = 0.f;
      int sp = 0;
      for (; sp + 8 <= a.splits; sp += 8) {  // eight loads in flight, summed in split order
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = part[static_cast<int64_t>(sp + u) * 3 * hd + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) g += t[u];
      }
      for (; sp < a.splits; ++sp) g += part[static_cast<int64_t>(sp) * 3 * hd + e];
      if (M != nullptr) {
        g = a.beta * M[wo + e] + g;
        M[wo + e] = g;
      }
      const float w = W[wo + e];
      ss_old += w * w;
      v[k] = w - a.step * g;
      ss += v[k] * v[k];
    }
  }
  ss = wave_sum(ss);
  const float den = fmaxf(sqrtf(ss), a.norm_eps);
  const float len_new = a.norm_keep ? sqrtf(wave_sum(ss_old)) : 1.f;
#pragma unroll
  for (int k = 0; k < kMaxRowPerLane; ++k) {
    const int e = lane + 64 * k;
    if (e < len) {
      const float x = len_new * (v[k] / den);
      W[wo + e] = x;
      if (Wb != nullptr)
        Wb[pair * hd + wb_tiled(static_cast<int>((po % hd) / len), e, len)] =
            __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    }
  }
}

// ---------------------------------------------------------------------------
// The same tail with 16-byte accesses (W, M 16-byte aligned): each stored row
// of length L is handled by min(64, L/4) lanes, four floats per lane per
// chunk, so a wavefront covers 256 floats (several short rows) per access.
// Rows of W1 and W3 (length d) come first in the grid, then rows of W2
// (length h).  The row norm is a reduction over the lanes of a row (their
// count is a power of two).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_reduce_step_v4(TailArgs a, int64_t blocks_a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool part_a = blockIdx.x < blocks_a;   // rows of W1 / W3, else of W2
  const int len = part_a ? a.d : a.h;
  const int lpr = len / 4 < 64 ? len / 4 : 64;  // lanes per row
  const int rpw = 64 / lpr;                    // rows per wavefront
  const int cpl = len / 4 / lpr;               // 16-byte chunks per lane
  const int64_t blk = part_a ? blockIdx.x : blockIdx.x - blocks_a;
  const int64_t grow = (blk * (kThreads / 64) + wave) * rpw + lane / lpr;  // global row of this part
  const int64_t rows_per_pair = part_a ? 2 * static_cast<int64_t>(a.h) : a.d;
  const int64_t pair = grow / rows_per_pair;
  const bool live = pair < a.P;
  const int r = static_cast<int>(grow % rows_per_pair);
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  float* W;
  float* M;
  uint16_t* Wb;
  int64_t po;  // offset of the row inside its pair's [W1 | W2 | W3] partial block
  if (part_a) {
    const bool w3 = r >= a.h;
    W = w3 ? a.W3 : a.W1;
    M = w3 ? a.M3 : a.M1;
    Wb = w3 ? a.Wb3 : a.Wb1;
    po = (w3 ? 2 * hd : 0) + static_cast<int64_t>(w3 ? r - a.h : r) * a.d;
  } else {
    W = a.W2;
    M = a.M2;
    Wb = a.Wb2;
    po = hd + static_cast<int64_t>(r) * a.h;
  }
  const int64_t wo = pair * hd + (po % hd);
  const float4* part = reinterpret_cast<const float4*>(a.partials + pair * a.splits * 3 * hd + po);
  const int64_t sstride = 3 * hd / 4;
  const int c0 = lane % lpr;
  float4 v[4];
  float ss = 0.f, ss_old = 0.f;
  for (int k = 0; k < cpl; ++k) {
    const int c = c0 + lpr * k;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
      int sp = 0;
      for (; sp + 4 <= a.splits; sp += 4) {  // four loads in flight, summed in split order
        float4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = part[(sp + u) * sstride + c];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          g.x += t[u].x;
          g.y += t[u].y;
          g.z += t[u].z;
          g.w += t[u].w;
        }
      }
      for (; sp < a.splits; ++sp) {
        const float4 t = part[sp * sstride + c];
        g.x += t.x;
        g.y += t.y;
        g.z += t.z;
        g.w += t.w;
      }
      if (M != nullptr) {
        float4* mp = reinterpret_cast<float4*>(M + wo) + c;
        const float4 m = *mp;
        g.x = a.beta * m.x + g.x;
        g.y = a.beta * m.y + g.y;
        g.z = a.beta * m.z + g.z;
        g.w = a.beta * m.w + g.w;
        *mp = g;
      }
      const float4 w = reinterpret_cast<const float4*>(W + wo)[c];
      ss_old += w.x * w.x + w.y * w.y + w.z * w.z + w.w * w.w;
      g.x = w.x - a.step * g.x;
      g.y = w.y - a.step * g.y;
      g.z = w.z - a.step * g.z;
      g.w = w.w - a.step * g.w;
      ss += g.x * g.x + g.y * g.y + g.z * g.z + g.w * g.w;
    }
    if (k < 4) v[k] = g;
  }
  ss = group_sum(ss, lpr);
  const float den = fmaxf(sqrtf(ss), a.norm_eps);
  const float len_new = a.norm_keep ? sqrtf(group_sum(ss_old, lpr)) : 1.f;
  if (live) {
    for (int k = 0; k < cpl; ++k) {
      const int c = c0 + lpr * k;
      const float4 g = v[k];
      const float4 x = make_float4(len_new * (g.x / den), len_new * (g.y / den), len_new * (g.z / den),
                                   len_new * (g.w / den));
      reinterpret_cast<float4*>(W + wo)[c] = x;
      if (Wb != nullptr) {
        bf16x4_t b;
        b[0] = static_cast<__bf16>(x.x);
        b[1] = static_cast<__bf16>(x.y);
        b[2] = static_cast<__bf16>(x.z);
        b[3] = static_cast<__bf16>(x.w);
        *reinterpret_cast<bf16x4_t*>(Wb + pair * hd + wb_tiled(static_cast<int>((po % hd) / len), 4 * c, len)) = b;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The bf16 weight copy of the chunk scan made from the fp32 weights (the
// update tails write the same values, in the same operand order, after every
// update): four consecutive floats of one stored row per thread, rounded to
// nearest even.  Matrix m of pair p: W1 (h x d), W2 (d x h), W3 (h x d).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_wb_copy(const float* W1, const float* W2, const float* W3,
                                                      uint16_t* wb, int P, int d, int h) {
  const int64_t hd = static_cast<int64_t>(h) * d;
  const int64_t per = hd / 4;  // float4 groups per matrix and pair
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= 3 * per * P) return;
  const int m = static_cast<int>(i / (per * P));
  const int64_t j = i % (per * P);
  const int64_t pair = j / per;
  const int64_t e = 4 * (j % per);
  const int cols = m == 1 ? h : d;
  const float* W = (m == 0 ? W1 : m == 1 ? W2 : W3) + pair * hd;
  const float4 x = *reinterpret_cast<const float4*>(W + e);
  bf16x4_t b;
  b[0] = static_cast<__bf16>(x.x);
  b[1] = static_cast<__bf16>(x.y);
  b[2] = static_cast<__bf16>(x.z);
  b[3] = static_cast<__bf16>(x.w);
  uint16_t* dst = wb + static_cast<int64_t>(m) * P * hd + pair * hd;
  *reinterpret_cast<bf16x4_t*>(dst + wb_tiled(static_cast<int>(e / cols), static_cast<int>(e % cols), cols)) = b;
}

// ---------------------------------------------------------------------------
// Query read O = W2 (silu(W1 q) * (W3 q)).  Grid (ceil(m/32), P); hidden
// units in slices of 256 staged through LDS.
// ---------------------------------------------------------------------------
constexpr int kQT = 32;
constexpr int kApplyHS = 256;

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_apply_generic(ApplyArgs a) {
  constexpr int NACC = kQT * D / kThreads;
  __shared__ float sQ[kQT][D + 1];
  __shared__ float sG[kQT][kApplyHS + 1];
  const int pair = blockIdx.y;
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * kQT;
  const int tid = threadIdx.x;
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int64_t base = static_cast<int64_t>(pair) * a.q_stride;
  const float* W1 = a.W1 + pair * hd;
  const float* W2 = a.W2 + pair * hd;
  const float* W3 = a.W3 + pair * hd;

  for (int i = tid; i < kQT * D; i += kThreads) {
    const int t = i / D, e = i % D;
    sQ[t][e] = (q0 + t < a.m) ? load_io<BF16>(a.Q, base + (q0 + t) * D + e) : 0.f;
  }
  float acc[NACC];
#pragma unroll
  for (int q = 0; q < NACC; ++q) acc[q] = 0.f;

  for (int j0 = 0; j0 < h; j0 += kApplyHS) {
    const int hs = min(kApplyHS, h - j0);
    __syncthreads();
    for (int i = tid; i < kQT * hs; i += kThreads) {
      const int t = i / hs, jj = i % hs;
      const float* w1 = W1 + static_cast<int64_t>(j0 + jj) * D;
      const float* w3 = W3 + static_cast<int64_t>(j0 + jj) * D;
      float h1 = 0.f, h3 = 0.f;
      for (int e = 0; e < D; ++e) {
        h1 += sQ[t][e] * w1[e];
        h3 += sQ[t][e] * w3[e];
      }
      sG[t][jj] = h1 * sigmoid_f(h1) * h3;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      const int idx = tid + kThreads * q;
      const int t = idx / D, e = idx % D;
      const float* w2 = W2 + static_cast<int64_t>(e) * h + j0;
      float s = 0.f;
      for (int jj = 0; jj < hs; ++jj) s += sG[t][jj] * w2[jj];
      acc[q] += s;
    }
  }
#pragma unroll
  for (int q = 0; q < NACC; ++q) {
    const int idx = tid + kThreads * q;
    const int t = idx / D, e = idx % D;
    if (q0 + t < a.m) store_io<BF16>(a.O, base + (q0 + t) * D + e, acc[q]);
  }
}

template <int D>
hipError_t grad_d(const GradArgs& a, hipStream_t s) {
  dim3 grid(a.S, a.h / kHS, a.P);
  if (a.bf16) {
    if (a.eta_mat != 0) {
      hipLaunchKernelGGL((k_grad_generic<true, D, true>), grid, dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((k_grad_generic<true, D, false>), grid, dim3(kThreads), 0, s, a);
    }
  } else {
    if (a.eta_mat != 0) {
      hipLaunchKernelGGL((k_grad_generic<false, D, true>), grid, dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((k_grad_generic<false, D, false>), grid, dim3(kThreads), 0, s, a);
    }
  }
  return hipGetLastError();
}

template <int D>
hipError_t apply_d(const ApplyArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.m + kQT - 1) / kQT), a.P);
  if (a.bf16) {
    hipLaunchKernelGGL((k_apply_generic<true, D>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_apply_generic<false, D>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

bool simple_shape_ok(int d, int h) {
  return (d == 32 || d == 64 || d == 128) && h >= kHS && h <= 64 * kMaxRowPerLane && h % kHS == 0;
}

size_t ns_simple_scratch_floats(int P, int d, int h) {
  const size_t s = d < h ? d : h, l = d < h ? h : d;
  return static_cast<size_t>(3) * P * (2 * s * l + 2 * s * s);
}

hipError_t launch_grad_simple(const GradArgs& a, hipStream_t s) {
  switch (a.d) {
    case 32: return grad_d<32>(a, s);
    case 64: return grad_d<64>(a, s);
    case 128: return grad_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_apply_simple(const ApplyArgs& a, hipStream_t s) {
  switch (a.d) {
    case 32: return apply_d<32>(a, s);
    case 64: return apply_d<64>(a, s);
    case 128: return apply_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(a.P) * 3 * a.h * a.d;
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.partials) | reinterpret_cast<uintptr_t>(a.dir) |
                         reinterpret_cast<uintptr_t>(a.M1) | reinterpret_cast<uintptr_t>(a.M2) |
                         reinterpret_cast<uintptr_t>(a.M3)) & 15) == 0;
  if (aligned && (a.h * a.d) % 4 == 0) {
    const unsigned blocks = static_cast<unsigned>((total / 4 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_reduce_v4, dim3(blocks), dim3(kThreads), 0, s, a);
  } else {
    const unsigned blocks = static_cast<unsigned>((total + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_reduce, dim3(blocks), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_ns_simple(const NSArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_ns_generic, dim3(3 * a.P), dim3(kNSThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce_step(const TailArgs& a, hipStream_t s) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.W1) | reinterpret_cast<uintptr_t>(a.W2) |
                         reinterpret_cast<uintptr_t>(a.W3) | reinterpret_cast<uintptr_t>(a.M1) |
                         reinterpret_cast<uintptr_t>(a.M2) | reinterpret_cast<uintptr_t>(a.M3)) & 15) == 0;
  // lanes per row must be a power of two (rows of d: always; rows of h:
  // h / 4 a power of two, or h a multiple of 256 up to 1024)
  auto pow2 = [](int x) { return x > 0 && (x & (x - 1)) == 0; };
  const bool shape_ok = (pow2(a.h / 4) || a.h % 256 == 0) && a.h <= 1024;
  if (aligned && shape_ok) {
    // rows per block: 4 wavefronts x (64 / lanes per row)
    auto rows_per_block = [](int len) { return 4 * (64 / (len / 4 < 64 ? len / 4 : 64)); };
    const int64_t rows_a = static_cast<int64_t>(a.P) * 2 * a.h, rows_b = static_cast<int64_t>(a.P) * a.d;
    const int64_t ba = (rows_a + rows_per_block(a.d) - 1) / rows_per_block(a.d);
    const int64_t bb = (rows_b + rows_per_block(a.h) - 1) / rows_per_block(a.h);
    hipLaunchKernelGGL(k_reduce_step_v4, dim3(static_cast<unsigned>(ba + bb)), dim3(kThreads), 0, s, a, ba);
    return hipGetLastError();
  }
  const int64_t rows = static_cast<int64_t>(a.P) * (2 * a.h + a.d);
  const unsigned blocks = static_cast<unsigned>((rows + 3) / 4);
  hipLaunchKernelGGL(k_reduce_step, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_wb_copy(const float* W1, const float* W2, const float* W3, uint16_t* wb, int P, int d, int h,
                          hipStream_t s) {
  if ((reinterpret_cast<uintptr_t>(W1) | reinterpret_cast<uintptr_t>(W2) | reinterpret_cast<uintptr_t>(W3)) & 15 ||
      d % 16 || h % 16)
    return hipErrorInvalidValue;
  const int64_t groups = 3 * static_cast<int64_t>(h) * d / 4 * P;
  hipLaunchKernelGGL(k_wb_copy, dim3(static_cast<unsigned>((groups + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     W1, W2, W3, wb, P, d, h);
  return hipGetLastError();
}

hipError_t launch_step_norm(const StepArgs& a, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.P) * (2 * a.h + a.d);
  const unsigned blocks = static_cast<unsigned>((rows + 3) / 4);
  hipLaunchKernelGGL(k_step_norm, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lact

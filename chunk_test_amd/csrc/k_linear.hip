// The linear fast net on the same chunk scan: f_W(x) = W x with one matrix
// W in R^{d x d} per (batch, head) pair, against which the pages compare the
// SwiGLU fast net ("LaCT: Large Chunk Test-Time Training" review, section
// "Large chunks alone do not explain the gains").  With the loss
// L = -sum_i eta_i <W k_i, v_i> the chunk gradient is a plain token
// contraction, dW = sum_i u_i k_i^T with u_i = -eta_i v_i; the update rules
// (GD, heavy-ball momentum, Muon) and the row normalisation are those of the
// SwiGLU layer.
//
// Every kernel here runs fp32 arithmetic (bf16 inputs are widened exactly):
//   k_lin_grad    split-K token contraction, partials [P, S, d d]
//   k_lin_reduce  fixed-order sum of the splits, momentum fused
//   k_lin_ns      Newton-Schulz on each d x d direction (global scratch)
//   k_lin_step    W <- W - step * dir, then each row to unit length, to its
//                 length before the step, or left as it is
//   k_lin_apply   O = Q W^T
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 64;  // tokens per LDS tile of the gradient and the query read

// ---------------------------------------------------------------------------
// Chunk gradient: grid (S splits, P pairs).  The d x d partial of a split is
// spread over a 16 x 16 grid of threads, each owning a (d/16) x (d/16) block
// of it: rows (u side) 16-blocks by thread row, columns (k side) by thread
// column.  Tokens past the split end load as zero.
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_lin_grad(LinGradArgs a) {
  constexpr int BS = D / 16;  // block side per thread
  __shared__ float sU[kTok][D + 1];
  __shared__ float sK[kTok][D + 1];
  const int split = blockIdx.x;
  const int pair = blockIdx.y;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  const int64_t t_begin = static_cast<int64_t>(split) * a.tps;
  const int64_t t_end = min(a.n, t_begin + a.tps);
  const int64_t kv_base = static_cast<int64_t>(pair) * a.kv_stride;
  const float* eta = a.eta + static_cast<int64_t>(pair) * a.eta_stride;

  float acc[BS][BS];
#pragma unroll
  for (int x = 0; x < BS; ++x) {
#pragma unroll
    for (int y = 0; y < BS; ++y) acc[x][y] = 0.f;
  }
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTok) {
    __syncthreads();
    for (int i = tid; i < kTok * D; i += kThreads) {
      const int t = i / D, e = i % D;
      const int64_t tok = t0 + t;
      float k = 0.f, u = 0.f;
      if (tok < t_end) {
        k = load_io<BF16>(a.K, kv_base + tok * D + e);
        u = -eta[tok] * load_io<BF16>(a.V, kv_base + tok * D + e);
      }
      sK[t][e] = k;
      sU[t][e] = u;
    }
    __syncthreads();
    for (int t = 0; t < kTok; ++t) {
      float uu[BS], kk[BS];
#pragma unroll
      for (int x = 0; x < BS; ++x) {
        uu[x] = sU[t][ti * BS + x];
        kk[x] = sK[t][tj * BS + x];
      }
#pragma unroll
      for (int x = 0; x < BS; ++x) {
#pragma unroll
        for (int y = 0; y < BS; ++y) acc[x][y] = fmaf(uu[x], kk[y], acc[x][y]);
      }
    }
  }
  float* out = a.partials + (static_cast<int64_t>(pair) * a.S + split) * D * D;
#pragma unroll
  for (int x = 0; x < BS; ++x) {
#pragma unroll
    for (int y = 0; y < BS; ++y) out[(ti * BS + x) * D + tj * BS + y] = acc[x][y];
  }
}

// ---------------------------------------------------------------------------
// Split reduction in fixed order s = 0..S-1, with M <- beta M + g fused.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_lin_reduce(LinTailArgs a) {
  const int64_t per = static_cast<int64_t>(a.d) * a.d;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= per * a.P) return;
  const int64_t pair = i / per, e = i % per;
  const float* src = a.partials + pair * a.splits * per + e;
  float g = 0.f;
  int s = 0;
  for (; s + 8 <= a.splits; s += 8) {  // eight loads in flight, summed in split order
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = src[static_cast<int64_t>(s + u) * per];
#pragma unroll
    for (int u = 0; u < 8; ++u) g += t[u];
  }
  for (; s < a.splits; ++s) g += src[static_cast<int64_t>(s) * per];
  if (a.M != nullptr) {
    g = a.beta * a.M[i] + g;
    a.M[i] = g;
  }
  a.dir[i] = g;
}

// ---------------------------------------------------------------------------
// Newton-Schulz on the d x d direction of every pair, one workgroup each,
// operands in global scratch (4 d d floats per pair):
//   X0 = G / (||G||_F + eps);  A = X X^T;  B = b A + c A A;  X <- a X + B X.
// ---------------------------------------------------------------------------
constexpr int kNSThreads = 512;

__global__ __launch_bounds__(kNSThreads) void k_lin_ns(LinTailArgs a) {
  __shared__ float red[kNSThreads];
  const int pair = blockIdx.x;
  const int d = a.d;
  const int64_t dd = static_cast<int64_t>(d) * d;
  float* G = a.dir + pair * dd;
  float* X = a.scratch + pair * 4 * dd;
  float* Xn = X + dd;
  float* A = Xn + dd;
  float* Bm = A + dd;
  const int tid = threadIdx.x;
  float part = 0.f;
  for (int64_t i = tid; i < dd; i += kNSThreads) part += G[i] * G[i];
  red[tid] = part;
  __syncthreads();
  for (int w = kNSThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float denom = sqrtf(red[0]) + a.ns_eps;
  for (int64_t i = tid; i < dd; i += kNSThreads) X[i] = G[i] / denom;
  __syncthreads();
  for (int it = 0; it < a.iters; ++it) {
    for (int64_t idx = tid; idx < dd; idx += kNSThreads) {
      const int i = static_cast<int>(idx / d), k = static_cast<int>(idx % d);
      float acc = 0.f;
      for (int j = 0; j < d; ++j) acc += X[i * d + j] * X[k * d + j];
      A[idx] = acc;
    }
    __syncthreads();
    for (int64_t idx = tid; idx < dd; idx += kNSThreads) {
      const int i = static_cast<int>(idx / d), k = static_cast<int>(idx % d);
      float acc = 0.f;
      for (int m = 0; m < d; ++m) acc += A[i * d + m] * A[m * d + k];
      Bm[idx] = a.b * A[idx] + a.c * acc;
    }
    __syncthreads();
    for (int64_t idx = tid; idx < dd; idx += kNSThreads) {
      const int i = static_cast<int>(idx / d), j = static_cast<int>(idx % d);
      float acc = 0.f;
      for (int m = 0; m < d; ++m) acc += Bm[i * d + m] * X[m * d + j];
      Xn[idx] = a.a * X[idx] + acc;
    }
    __syncthreads();
    float* t = X;
    X = Xn;
    Xn = t;
  }
  for (int64_t i = tid; i < dd; i += kNSThreads) G[i] = X[i];
}

// ---------------------------------------------------------------------------
// W <- W - step * dir, one wavefront per row (d <= 128: two entries per lane).
// norm: 0 unit rows, 1 rows back to their length before the step, 2 none.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_lin_step(LinTailArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(a.P) * a.d) return;
  float* W = a.W + row * a.d;
  const float* dr = a.dir + row * a.d;
  float v[2];
  float ss = 0.f, ss_old = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = lane + 64 * k;
    v[k] = 0.f;
    if (e < a.d) {
      const float w = W[e];
      ss_old += w * w;
      v[k] = w - a.step * dr[e];
      ss += v[k] * v[k];
    }
  }
  float scale = 1.f;
  if (a.norm != 2) {
    ss = wave_sum(ss);
    const float len = a.norm == 1 ? sqrtf(wave_sum(ss_old)) : 1.f;
    scale = len / fmaxf(sqrtf(ss), a.norm_eps);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = lane + 64 * k;
    if (e < a.d) W[e] = a.norm != 2 ? scale * v[k] : v[k];
  }
}

// ---------------------------------------------------------------------------
// Query read O = Q W^T: grid (query tiles of 64, P pairs); W of the pair and
// the tile's queries in LDS, four threads per query (outputs i = q, q + 4, ...).
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_lin_apply(LinApplyArgs a) {
  __shared__ float sW[D][D + 1];
  __shared__ float sQ[kTok][D + 1];
  const int pair = blockIdx.y;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int tid = threadIdx.x;
  const float* W = a.W + static_cast<int64_t>(pair) * D * D;
  for (int i = tid; i < D * D; i += kThreads) sW[i / D][i % D] = W[i];
  const int64_t qb = static_cast<int64_t>(pair) * a.q_stride;
  for (int i = tid; i < kTok * D; i += kThreads) {
    const int t = i / D, e = i % D;
    sQ[t][e] = (m0 + t < a.m) ? load_io<BF16>(a.Q, qb + (m0 + t) * D + e) : 0.f;
  }
  __syncthreads();
  const int t = tid / 4, q = tid % 4;
  if (m0 + t >= a.m) return;
  float acc[D / 4];
#pragma unroll
  for (int x = 0; x < D / 4; ++x) acc[x] = 0.f;
  for (int j = 0; j < D; ++j) {
    const float qj = sQ[t][j];
#pragma unroll
    for (int x = 0; x < D / 4; ++x) acc[x] = fmaf(sW[q + 4 * x][j], qj, acc[x]);
  }
#pragma unroll
  for (int x = 0; x < D / 4; ++x) store_io<BF16>(a.O, qb + (m0 + t) * D + q + 4 * x, acc[x]);
}

template <int D>
hipError_t grad_d(const LinGradArgs& a, hipStream_t s) {
  const dim3 grid(a.S, a.P);
  if (a.bf16) {
    hipLaunchKernelGGL((k_lin_grad<true, D>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_lin_grad<false, D>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t apply_d(const LinApplyArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.m + kTok - 1) / kTok), a.P);
  if (a.bf16) {
    hipLaunchKernelGGL((k_lin_apply<true, D>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_lin_apply<false, D>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

bool linear_shape_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

hipError_t launch_lin_grad(const LinGradArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return grad_d<16>(a, s);
    case 32: return grad_d<32>(a, s);
    case 64: return grad_d<64>(a, s);
    case 128: return grad_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lin_tail(const LinTailArgs& a, hipStream_t s) {
  if (!linear_shape_ok(a.d)) return hipErrorInvalidValue;
  const int64_t n = static_cast<int64_t>(a.P) * a.d * a.d;
  hipLaunchKernelGGL(k_lin_reduce, dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.muon) {
    hipLaunchKernelGGL(k_lin_ns, dim3(a.P), dim3(kNSThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t rows = static_cast<int64_t>(a.P) * a.d;
  hipLaunchKernelGGL(k_lin_step, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lin_apply(const LinApplyArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return apply_d<16>(a, s);
    case 32: return apply_d<32>(a, s);
    case 64: return apply_d<64>(a, s);
    case 128: return apply_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lact

// Causal sliding-window attention beside the TTT layer, the second half of a
// LaCT block ("LaCT: Large Chunk Test-Time Training" review, section "Local
// attention and nonlinear memory work together": window attention captures
// local order inside a chunk; the language and video variants share Q, K, V
// with the TTT layer and add the two outputs).  Query t attends keys s with
// t - window < s <= t:
//   o_t = sum_s softmax_s(scale q_t . k_s) v_s.
//
// One workgroup per (64 queries, pair); four threads per query, each owning
// d/4 features of q and of the output.  Key/value tiles of 64 tokens go
// through LDS; per tile the 64 scores of a query are formed first (partial
// dots reduced over the query's four lanes), then the running maximum and
// sum of the online softmax are updated once and the tile's values are
// accumulated (fp32 arithmetic).  With `accumulate` the result is added to
// what O holds (the block's sum with the TTT layer's output).
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

constexpr int kThreads = 256;
constexpr int kQ = 64;   // queries per workgroup
constexpr int kKT = 64;  // keys per tile

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_window_attn(WindowArgs a) {
  constexpr int DP = D / 4;  // features per lane
  __shared__ float sK[kKT][D + 1];
  __shared__ float sV[kKT][D + 1];
  const int pair = blockIdx.y;
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * kQ;
  const int tid = threadIdx.x;
  const int qi = tid >> 2;    // query of this lane group
  const int part = tid & 3;   // its quarter of the features
  const int64_t t = q0 + qi;
  const int64_t base = static_cast<int64_t>(pair) * a.stride;
  const bool valid = t < a.T;
  float q[DP], o[DP];
#pragma unroll
  for (int x = 0; x < DP; ++x) {
    q[x] = valid ? a.scale * load_io<BF16>(a.Q, base + t * D + part * DP + x) : 0.f;
    o[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  // keys any query of the tile can see
  const int64_t q_last = min(q0 + kQ, a.T) - 1;
  int64_t k_lo = q0 - a.window + 1;
  if (k_lo < 0) k_lo = 0;
  k_lo = (k_lo / kKT) * kKT;
  for (int64_t k0 = k_lo; k0 <= q_last; k0 += kKT) {
    __syncthreads();
    for (int i = tid; i < kKT * D; i += kThreads) {
      const int r = i / D, e = i % D;
      const int64_t s = k0 + r;
      const bool ok = s < a.T;
      sK[r][e] = ok ? load_io<BF16>(a.K, base + s * D + e) : 0.f;
      sV[r][e] = ok ? load_io<BF16>(a.V, base + s * D + e) : 0.f;
    }
    __syncthreads();
    float sc[kKT];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < kKT; ++r) {
      float p = 0.f;
#pragma unroll
      for (int x = 0; x < DP; ++x) p = fmaf(q[x], sK[r][part * DP + x], p);
      p += __shfl_xor(p, 1, 64);
      p += __shfl_xor(p, 2, 64);
      const int64_t s = k0 + r;
      const bool in = valid && s <= t && s > t - a.window;
      sc[r] = in ? p : -INFINITY;
      tmax = fmaxf(tmax, sc[r]);
    }
    if (tmax != -INFINITY) {  // some key of this tile is in the query's window
      const float mn = fmaxf(m, tmax);
      const float corr = __expf(m - mn);  // 0 on the first visible tile (m = -inf)
      l *= corr;
#pragma unroll
      for (int x = 0; x < DP; ++x) o[x] *= corr;
#pragma unroll
      for (int r = 0; r < kKT; ++r) {
        const float p = __expf(sc[r] - mn);
        l += p;
#pragma unroll
        for (int x = 0; x < DP; ++x) o[x] = fmaf(p, sV[r][part * DP + x], o[x]);
      }
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = 1.f / l;
#pragma unroll
  for (int x = 0; x < DP; ++x) {
    const int64_t idx = base + t * D + part * DP + x;
    float v = o[x] * inv;
    if (a.accumulate) v += load_io<BF16>(a.O, idx);
    store_io<BF16>(a.O, idx, v);
  }
}

template <int D>
hipError_t launch_d(const WindowArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.T + kQ - 1) / kQ), a.P);
  if (a.bf16) {
    hipLaunchKernelGGL((k_window_attn<true, D>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_window_attn<false, D>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

bool window_shape_ok(int d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_window_attn(const WindowArgs& a, hipStream_t s) {
  switch (a.d) {
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lact

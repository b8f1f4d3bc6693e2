// Query read O = W2 (silu(W1 q) * (W3 q)) on bf16 MFMA (gfx950), d = 64 or
// 128, h in {128, 256}: the fast weights answer the queries ("LaCT: Large
// Chunk Test-Time Training" review, sections "Local attention and nonlinear
// memory work together" and "Update order must respect the task").  The
// workgroup body is apply_body (apply_body.h); this file holds the kernel
// and its launcher.
#include "apply_body.h"

namespace lact {
namespace {

template <int D, int H, bool COPY>
__global__ __launch_bounds__(2 * H) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_apply_mfma(ApplyArgs a, int per_wg, int wg_per_pair) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[apply_detail::AGeo<D, H>::LDS];
  apply_detail::apply_body<D, H, COPY>(a, lds, blockIdx.x, gridDim.x, per_wg, wg_per_pair);
}

template <int D, int H>
hipError_t launch_dh(const ApplyArgs& a, hipStream_t s) {
  using G = apply_detail::AGeo<D, H>;
  int per = 0, gx = 0;
  apply_detail::apply_plan<D, H>(a.m, a.P, 256 * G::WG_PER_CU, &per, &gx);
  const unsigned blocks = static_cast<unsigned>((static_cast<int64_t>(gx) * a.P + 7) / 8 * 8);
  if (a.Wb1 != nullptr)
    hipLaunchKernelGGL((k_apply_mfma<D, H, true>), dim3(blocks), dim3(G::THREADS), 0, s, a, per, gx);
  else
    hipLaunchKernelGGL((k_apply_mfma<D, H, false>), dim3(blocks), dim3(G::THREADS), 0, s, a, per, gx);
  return hipGetLastError();
}

}  // namespace

bool apply_mfma_shape_ok(int d, int h) {
  return (d == 64 || d == 128) && (h == 128 || h == 256);
}

hipError_t launch_apply_mfma(const ApplyArgs& a, hipStream_t s) {
  if (a.d == 64 && a.h == 128) return launch_dh<64, 128>(a, s);
  if (a.d == 64 && a.h == 256) return launch_dh<64, 256>(a, s);
  if (a.d == 128 && a.h == 128) return launch_dh<128, 128>(a, s);
  if (a.d == 128 && a.h == 256) return launch_dh<128, 256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace lact

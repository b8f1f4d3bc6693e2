// Internal interface between the C ABI host code and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lact {

// Arguments of the chunk-gradient kernels: partial sums of
//   dW1 = dH1^T K,  dW2 = U^T G,  dW3 = dH3^T K   (U = -eta * V)
// over the tokens of one split, written to partials[pair][split][3hd] in the
// order [W1 block (h x d) | W2 block (d x h) | W3 block (h x d)].
struct GradArgs {
  const void* K;
  const void* V;
  const float* eta;
  int64_t n;           // keys in the chunk
  int64_t kv_stride;   // elements between pairs in K and V
  int64_t eta_stride;  // elements between pairs in eta
  int64_t eta_mat;     // elements between the rates of W1, W2, W3 (0: one rate per token)
  const float* W1;     // [P, h, d]
  const float* W2;     // [P, d, h]
  const float* W3;     // [P, h, d]
  float* partials;     // [P, S, 3hd]
  int P, d, h, S;
  int64_t tps;         // tokens per split (the last split may be shorter)
  int bf16;            // K, V are bfloat16
};

// Fixed-order sum of the split partials, with the momentum update fused:
//   g = sum_s partials[p][s];  if M: M <- beta M + g, g <- M;  dir[p] = g.
struct ReduceArgs {
  const float* partials;  // [P, S, 3hd]
  float* dir;             // [P, 3hd]
  float *M1, *M2, *M3;    // momentum buffers or NULL
  float beta;
  int P, d, h, S;
};

// Newton-Schulz on each of the 3P matrices held in dir (in place).
struct NSArgs {
  float* dir;      // [P, 3hd]
  float* scratch;  // simple path: 3P * (2 s l + 2 s s) floats
  int P, d, h, iters;
  float a, b, c, eps;
};

// Update tails that read the split partials directly (fixed-order sum):
//   Muon: momentum (optional), Newton-Schulz, step, unit rows (per matrix);
//   GD / momentum: momentum (optional), step, unit rows (per row).
struct TailArgs {
  const float* partials;  // [P, splits, 3hd]
  int splits;
  float *M1, *M2, *M3;    // momentum buffers or NULL
  float beta;
  float *W1, *W2, *W3;
  float step, norm_eps;
  int norm_keep;          // rows back to their length before the update (else unit)
  int P, d, h, iters;
  float a, b, c, eps;     // Newton-Schulz (Muon only)
  // when non-NULL: also store the updated W1, W2, W3 rounded to bf16 (P h d
  // values each, every matrix in the operand order of wb_tiled), the copy a
  // following query read loads directly
  uint16_t *Wb1, *Wb2, *Wb3;
};

// W <- W - step * dir, then unit L2 rows.
struct StepArgs {
  float *W1, *W2, *W3;
  const float* dir;  // [P, 3hd]
  float step, norm_eps;
  int norm_keep;     // rows back to their length before the update (else unit)
  int P, d, h;
};

// O = f_W(Q) for m queries per pair.
struct ApplyArgs {
  const void* Q;
  void* O;
  int64_t m;
  int64_t q_stride;
  const float *W1, *W2, *W3;
  int P, d, h;
  int bf16;
  int w_vec;  // W1, W2, W3 16-byte aligned
  // when non-NULL: bf16 copies of W1, W2, W3 (as stored by the update tail,
  // in the operand order of wb_tiled), read instead of converting the fp32
  // weights
  const uint16_t *Wb1, *Wb2, *Wb3;
};

// ---- generic kernels (fp32 arithmetic; any supported d, h) ----
hipError_t launch_grad_simple(const GradArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_ns_simple(const NSArgs& a, hipStream_t s);
hipError_t launch_step_norm(const StepArgs& a, hipStream_t s);
hipError_t launch_reduce_step(const TailArgs& a, hipStream_t s);  // GD / momentum tail
hipError_t launch_apply_simple(const ApplyArgs& a, hipStream_t s);
bool simple_shape_ok(int d, int h);

// ---- bf16 MFMA kernels (gfx950) ----
bool grad_d64_shape_ok(int d, int h);  // d = 64, LDS-DMA staging
hipError_t launch_grad_d64(const GradArgs& a, hipStream_t s);
bool grad_d128_shape_ok(int d, int h);  // d = 128, LDS-DMA staging, bf16 or split products
int grad_d128_stage_tokens(bool split);
hipError_t launch_grad_d128(const GradArgs& a, bool split, hipStream_t s);
bool ns_mfma_shape_ok(int d, int h);
bool apply_mfma_shape_ok(int d, int h);
hipError_t launch_apply_mfma(const ApplyArgs& a, hipStream_t s);
hipError_t launch_muon_tail(const TailArgs& a, hipStream_t s);  // bf16-mode Muon tail
size_t ns_simple_scratch_floats(int P, int d, int h);

}  // namespace lact

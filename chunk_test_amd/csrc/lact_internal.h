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

// ---- linear fast net f_W(x) = W x, W [P, d, d] (fp32 arithmetic) ----
struct LinGradArgs {
  const void* K;
  const void* V;
  const float* eta;
  int64_t n, kv_stride, eta_stride;
  float* partials;  // [P, S, d d]
  int P, d, S;
  int64_t tps;
  int bf16;
};
struct LinTailArgs {
  const float* partials;  // [P, splits, d d]
  int splits;
  float* dir;             // [P, d d]
  float* scratch;         // Newton-Schulz: 4 d d floats per pair
  float* W;               // [P, d, d]
  float* M;               // [P, d, d] or NULL
  float beta, step, norm_eps;
  int norm;               // 0 unit rows, 1 rows kept at their length, 2 no normalisation
  int muon, iters;
  float a, b, c, ns_eps;
  int P, d;
};
struct LinApplyArgs {
  const void* Q;
  void* O;
  int64_t m, q_stride;
  const float* W;
  int P, d;
  int bf16;
};
bool linear_shape_ok(int d);
hipError_t launch_lin_grad(const LinGradArgs& a, hipStream_t s);
hipError_t launch_lin_tail(const LinTailArgs& a, hipStream_t s);  // reduce (+momentum), NS, step
hipError_t launch_lin_apply(const LinApplyArgs& a, hipStream_t s);

// ---- backward pass (fp32 arithmetic) ----
struct MatRef {  // one matrix per pair: element e of pair p at p * pair_stride + e
  float* p;
  int64_t pair_stride;
};
struct BwTokArgs {  // token-local VJPs (chunk gradient: A = K, B = V; query read: A = Q, B = dO)
  const void* A;
  const void* B;
  const float* eta;  // chunk gradient only
  int64_t n, in_stride, eta_stride;
  MatRef W1, W2, W3;  // fast weights of the step
  MatRef P1, P2, P3;  // cotangents of the chunk gradient (chunk gradient only)
  float *X1, *X2, *X3;  // [P, n, h] factors of the weight cotangents
  int64_t x_stride;
  void* dA;
  void* dB;  // chunk gradient only
  int64_t out_stride;
  float* deta;  // chunk gradient only
  int64_t deta_stride;
  int P, d, h;
  int bf16;
  const uint16_t* op;  // bf16 hi | lo operands of W1, W3, W2^T ([P][3][2][h][d]) or NULL
  int64_t op_stride;   // elements per pair of op
  int split;           // matrix-core kernels: 1 hi + lo operands (~16 bits), 0 plain bf16 (hi only)
  int x_bf16;          // matrix-core kernels: factors stored as bf16 (X2 of the chunk gradient
                       // times -eta), for the plain-bf16 matrix-core contraction; else fp32
};
struct BwOpsArgs {  // matrices as bf16 hi | lo parts in [hidden][feature] order
  MatRef m[6];      // W1, W3, W2 (then P1, P3, P2): m[2], m[5] stored [d][h]
  int nm;           // 3 or 6
  uint16_t* op;     // [P][nm][2][h][d]
  int64_t op_stride;
  int P, d, h;  // d = 64 or 128
  int hi_only;  // write the hi parts only (plain bf16 products)
};
struct BwContractArgs {  // X1^T A, (b B)^T X2, X3^T A over tokens, b = -eta or 1
  const void* A;
  const void* B;
  const float* eta;  // NULL: b = 1
  int64_t n, in_stride, eta_stride;
  const float *X1, *X2, *X3;
  int64_t x_stride;
  float* partials;  // [P, S, 3hd]
  int P, d, h, S;
  int64_t tps;
  int bf16;
  int split;  // matrix-core kernel: 1 factors as hi + lo (two MFMAs per product), 0 plain bf16
  int x_bf16;  // the factors are bf16 (X2 of the chunk gradient already times -eta; needs split 0)
};
struct BwStepArgs {
  MatRef W_in[3], W_out[3];  // W1, W2, W3 before and after the update
  const float* dir;          // [P, 3hd] direction of the update (NULL: dir_m)
  MatRef dir_m[3];           // the direction as W1, W2, W3 matrices (the momentum's checkpoint)
  float* cot;                // [P, 3hd] cotangent of W_out in, of W_in (direct path) out
  // split partials [P, S, 3hd] of contractions not yet added into cot: the
  // incoming cotangent is (cot + sum pend[0]) + sum pend[1], each sum in split
  // order (NULL: none)
  const float* pend[2];
  int pend_S[2];
  float* ddir;               // [P, 3hd] cotangent of the direction
  // momentum without Newton-Schulz, when dM is set: the momentum VJP in the
  // same pass (v = cotangent of the direction + dM; pc = v; dM = beta v),
  // ddir is not written
  float* dM;
  float* pc;
  float beta;
  float step, norm_eps;
  int P, d, h;
};
struct BwNSArgs {
  const float* g;   // [P, 3hd] Newton-Schulz input
  const float* dx;  // [P, 3hd] cotangent of its output
  float* out;       // [P, 3hd] cotangent of its input
  float* scratch;   // 3P * per_mat floats
  int64_t per_mat;
  int P, d, h, iters;
  float a, b, c, eps;
  int bf16_split;   // products on bf16 matrix cores with hi + lo operands (else fp32 matrix cores)
};
bool backward_shape_ok(int d, int h);
hipError_t launch_bw_tok(const BwTokArgs& a, bool apply, hipStream_t s);
// matrix-core token kernels (bf16, d = 64 or 128, h a multiple of 32, operands from
// launch_bw_ops)
bool bw_tok_mfma_ok(const BwTokArgs& a, bool apply);
hipError_t launch_bw_tok_mfma(const BwTokArgs& a, bool apply, hipStream_t s);
hipError_t launch_bw_ops(const BwOpsArgs& a, hipStream_t s);
hipError_t launch_bw_contract(const BwContractArgs& a, hipStream_t s);
// the bf16 matrix-core contraction (d = 64 or 128, h a multiple of 128, 16-byte aligned inputs)
bool bw_contract_mfma_ok(const BwContractArgs& a);
hipError_t launch_bw_contract_mfma(const BwContractArgs& a, hipStream_t s);
hipError_t launch_bw_reduce_add(float* dst, const float* partials, int S, int64_t per, int P, hipStream_t s);
hipError_t launch_bw_step(const BwStepArgs& a, hipStream_t s);
hipError_t launch_bw_momentum(const float* t, float* dM, float* Pout, float beta, int64_t total, hipStream_t s);
int64_t bw_ns_floats_per_matrix(int d, int h, int iters);
// Newton-Schulz forward (iterates into scratch, direction into out) and its
// VJP (from the same scratch; dx the direction's cotangent, out the input's)
hipError_t launch_bw_ns_fwd(const BwNSArgs& a, hipStream_t s);
hipError_t launch_bw_ns(const BwNSArgs& a, hipStream_t s);
hipError_t launch_bw_copy(float* blocks, const MatRef& m1, const MatRef& m2, const MatRef& m3, int P, int d, int h,
                          bool to_blocks, hipStream_t s);

// ---- causal sliding-window attention (the LaCT block's local half) ----
struct WindowArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int64_t T, stride, window;  // stride: elements between pairs
  float scale;
  int accumulate;  // O += attention (else O = attention)
  int P, d;
  int bf16;
};
bool window_shape_ok(int d);
hipError_t launch_window_attn(const WindowArgs& a, hipStream_t s);

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
hipError_t launch_grad_d64(const GradArgs& a, bool split, hipStream_t s);
bool d128_mfma_shape_ok(int d, int h);  // d = 128 shapes of the matrix-core path (h a multiple of 128)
bool grad_d128w_shape_ok(int d, int h);  // d = 128, bf16 or split products, 16x16x32 tiles, two waves per SIMD
int grad_d128w_stage_tokens(bool split);
int grad_d128w_hidden_per_workgroup();
int grad_d128w_workgroups_per_cu();
hipError_t launch_grad_d128w(const GradArgs& a, bool split, hipStream_t s);
bool ns_mfma_shape_ok(int d, int h);
// Muon update tail of one chunk and the query read of the same chunk (from
// the bf16 copy of its weights) in one launch, where h > d, both have
// matrix-core kernels and 3P <= 192 (the tail leaves CUs for the read).
bool muon_tail_apply_ok(int d, int h, int P);
hipError_t launch_muon_tail_apply(const TailArgs& ta, const ApplyArgs& aa, hipStream_t s);
// The bf16 weight copy (P h d values per matrix, W1 | W2 | W3, each matrix in
// the operand order of wb_tiled) from 16-byte aligned fp32 weights.
hipError_t launch_wb_copy(const float* W1, const float* W2, const float* W3, uint16_t* wb, int P, int d, int h,
                          hipStream_t s);
bool apply_mfma_shape_ok(int d, int h);
hipError_t launch_apply_mfma(const ApplyArgs& a, hipStream_t s);
hipError_t launch_muon_tail(const TailArgs& a, hipStream_t s);  // bf16-mode Muon tail
size_t ns_simple_scratch_floats(int P, int d, int h);

}  // namespace lact

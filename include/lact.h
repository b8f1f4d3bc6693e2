/*
 * lact.h - C ABI of the LaCT large-chunk test-time-training layer on gfx950.
 *
 * What the layer computes (the text of "LaCT: Large Chunk Test-Time
 * Training", iplexlaw.co.kr review, sections "Local attention and nonlinear
 * memory work together" and "Update order must respect the task"; "Test-Time
 * Training Done Right", Abstract and project page Figure 2):
 *
 *   per (batch, head) pair the fast weights are a SwiGLU MLP
 *       f_W(x) = W2 (silu(W1 x) * (W3 x)),  W1, W3: [h x d],  W2: [d x h];
 *   for every chunk of keys/values (2K .. ~1M tokens) the layer
 *     (1) reads f_W(q) for the chunk's queries,
 *     (2) takes the gradient of L = - sum_i eta_i <f_W(k_i), v_i> over the
 *         whole chunk (eta_i: a per-token learning rate),
 *     (3) applies plain GD, heavy-ball momentum, or Muon (Newton-Schulz
 *         orthogonalisation of each matrix gradient),
 *     (4) L2-normalises every row of the updated W1, W3 (length d) and W2
 *         (length h);
 *   (1) runs before (2)-(4) for causal text/video (apply-then-update) and
 *   after them for posed image sets (update-then-apply).  W is carried from
 *   chunk to chunk.
 *
 * Conventions shared by every entry point
 *   - All buffers are DEVICE memory owned by the caller.  The library never
 *     allocates device memory and never synchronises the host: every call
 *     validates its arguments on the host, then enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and returns.  Errors of the
 *     kernels themselves surface at the caller's next synchronisation.
 *   - Layouts (row-major, elements, not bytes):
 *       Q, O: [B, H, T_q, d];  K, V: [B, H, T_kv, d];  eta: [B, H, T_kv];
 *       W1, W3, M1, M3: [B, H, h, d];  W2, M2: [B, H, d, h].
 *     Rows of one pair are contiguous; consecutive pairs are `*_stride_bh`
 *     elements apart (so chunk views of a longer sequence can be passed).
 *   - io_dtype LACT_F32: Q, K, V, O are float.  LACT_BF16: they are
 *     bfloat16 (raw 16-bit words); products use bf16 operands with fp32
 *     accumulation.  eta, W and M are always float.
 *   - The state is updated in place.  M1..M3 must be non-NULL (and are
 *     read and written) exactly when the optimizer keeps a momentum buffer:
 *     opt == LACT_OPT_MOMENTUM, or opt == LACT_OPT_MUON with beta > 0.
 *     Zero them before the first chunk.
 *   - Scratch: `ws` (device, 256-byte aligned) of at least
 *     lact_workspace_bytes(...) bytes; its contents need no initialisation
 *     and are not meaningful after the call.  Two calls in flight at once
 *     must not share a workspace.
 *   - Results are deterministic: a fixed launch plan derived from the
 *     shapes, the options and the alignment of the buffers (16-byte aligned
 *     Q, K, V, O, W and M, and strides of whole 16-byte rows, select the
 *     matrix-core kernels; other buffers run fp32-arithmetic kernels whose
 *     results agree within the stated tolerances but not bit for bit), and
 *     fixed-order reductions.  The same call on the same buffers gives the
 *     same bits.
 *   - Return value: LACT_OK or a negative lact_status.  Nothing is enqueued
 *     when validation fails.  lact_last_error() gives a thread-local text.
 *   - NaN / Inf inputs propagate; there is no device-side check.
 */
#ifndef LACT_H
#define LACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LACT_OK = 0,
  LACT_ERR_INVALID_ARG = -1, /* NULL pointer, non-positive size, chunks that do not divide T, ... */
  LACT_ERR_UNSUPPORTED = -2, /* a shape / dtype / optimizer combination that is not built      */
  LACT_ERR_WORKSPACE = -3,   /* ws too small or misaligned                                       */
  LACT_ERR_HIP = -4          /* a HIP launch error (text in lact_last_error())                  */
} lact_status;

typedef enum { LACT_F32 = 0, LACT_BF16 = 1 } lact_dtype;

/* Read/update order ("Update order must respect the task"). */
typedef enum { LACT_APPLY_THEN_UPDATE = 0, LACT_UPDATE_THEN_APPLY = 1 } lact_order;

/* Update rule ("Local attention and nonlinear memory work together"). */
typedef enum { LACT_OPT_GD = 0, LACT_OPT_MOMENTUM = 1, LACT_OPT_MUON = 2 } lact_opt;

/* bf16 I/O mode only.  LACT_PRODUCTS_BF16: every product operand is rounded
 * to bf16 (the inputs already are; the W copies and the SwiGLU values, which
 * carry the -eta factor, are rounded), fp32 accumulation.
 * LACT_PRODUCTS_SPLIT: only the inputs Q, K, V are bf16; every derived
 * operand keeps ~16 significant bits (computed in fp32, or as a hi + lo pair
 * of bf16 values on the matrix cores).
 * Muon maps every singular value of the gradient towards one, so it lifts the
 * rounding of bf16 operands in the weak directions of short chunks (~7e-2 on
 * 100-key chunks) and compounds it over a scan (~1.4x per chunk: 3e-3 after
 * one 4096-key chunk, 0.25 after fourteen).  Under Muon, LACT_PRODUCTS_BF16
 * is therefore accepted only for chunks of >= 1024 keys and runs of at most
 * 4 chunks (one lact_update call counts as one chunk); otherwise the call
 * returns LACT_ERR_UNSUPPORTED.  LACT_PRODUCTS_AUTO (the default) takes
 * LACT_PRODUCTS_BF16 where it is accepted and LACT_PRODUCTS_SPLIT elsewhere.
 * Callers that drive a long Muon scan through lact_update should ask for
 * LACT_PRODUCTS_SPLIT themselves.  Ignored in fp32 I/O mode. */
typedef enum { LACT_PRODUCTS_BF16 = 0, LACT_PRODUCTS_SPLIT = 1, LACT_PRODUCTS_AUTO = 2 } lact_products;

/* Length of the updated rows (step (4)).  LACT_NORM_UNIT: every stored row r
 * of W1, W3 (length d) and W2 (length h) becomes r / max(||r||_2, norm_eps).
 * LACT_NORM_KEEP: the stepped row u is rescaled to the length the row had
 * before the update, u * ||r_old||_2 / max(||u||_2, norm_eps), so the update
 * turns the rows and every row keeps its initial length through the scan (the
 * direction / length split of weight normalisation, with the length held;
 * "Weight Normalization: A Simple Reparameterization to Accelerate Training
 * of Deep Neural Networks" is in the reference list of the "Test-Time
 * Training Done Right" arXiv page).  Identical to LACT_NORM_UNIT for rows of
 * unit length. */
typedef enum { LACT_NORM_UNIT = 0, LACT_NORM_KEEP = 1, LACT_NORM_NONE = 2 } lact_norm_mode;
/* (LACT_NORM_NONE: rows are left as the step leaves them; linear fast net
 * only, where it gives the chunk-causal linear-attention closed form.) */

/* The fast net.  LACT_NET_SWIGLU: the layer's f_W above.  LACT_NET_LINEAR:
 * f_W(x) = W x with one matrix W [d x d] per pair, the linear state the
 * pages compare the SwiGLU fast net against ("LaCT: Large Chunk Test-Time
 * Training" review, section "Large chunks alone do not explain the gains"):
 * the same scan, loss, update rules and row normalisation; the chunk
 * gradient is dW = -sum_i eta_i v_i k_i^T.  The state is W1 = W
 * [B, H, d, d] (M1 for momentum); W2, W3 (M2, M3) are not used and may be
 * NULL; h is ignored; d in {16, 32, 64, 128}; one rate per token; fp32
 * arithmetic throughout (bf16 inputs and outputs where io_dtype says so). */
typedef enum { LACT_NET_SWIGLU = 0, LACT_NET_LINEAR = 1 } lact_net;

/* Learning rates.  LACT_ETA_SHARED: one rate eta_i per token, shared by W1,
 * W2 and W3 (the loss of step (2)).  LACT_ETA_PER_MATRIX: three rates per
 * token, and each matrix follows the gradient of the loss written with its
 * own rates: dW_m = d/dW_m (-sum_i eta_{i,m} <f_W(k_i), v_i>), m = W1, W2,
 * W3.  The rates are then three blocks laid out like the shared ones, W1's
 * first: the rate of matrix m, pair p, token t sits at
 * eta[m * P * eta_stride_bh + p * eta_stride_bh + t] (P = B*H), i.e. a
 * [3, B, H, T] array for lact_chunked_forward.  Three equal blocks give the
 * shared-rate result. */
typedef enum { LACT_ETA_SHARED = 0, LACT_ETA_PER_MATRIX = 1 } lact_eta_mode;

typedef struct {
  int32_t B, H;      /* batch and heads: P = B*H independent pairs                        */
  int32_t d, h;      /* head dim and SwiGLU hidden dim                                    */
  int32_t io_dtype;  /* lact_dtype of Q, K, V, O                                          */
  int32_t opt;       /* lact_opt                                                          */
  float beta;        /* momentum coefficient in [0, 1): M <- beta M + grad               */
  int32_t ns_iters;  /* Newton-Schulz iterations (Muon), 0..32                            */
  float ns_a, ns_b, ns_c; /* X <- a X + (b A + c A A) X, A = X X^T                        */
  float ns_eps;      /* X0 = G / (||G||_F + ns_eps)                                       */
  float step;        /* W <- W - step * direction                                         */
  float norm_eps;    /* row r <- r / max(||r||_2, norm_eps)                               */
  int32_t products;  /* lact_products: how bf16-mode products treat derived operands      */
  int32_t norm_mode; /* lact_norm_mode: rows to unit length, or kept at their length      */
  int32_t eta_mode;  /* lact_eta_mode: one rate per token, or one per token and matrix    */
  int32_t net;       /* lact_net: SwiGLU fast weights (the layer) or a linear one         */
} lact_config;

typedef struct {
  float *W1, *W2, *W3; /* fast weights (in/out)                                           */
  float *M1, *M2, *M3; /* momentum buffers (in/out) or NULL, see above                    */
} lact_state;

/* Defaults: opt GD, beta 0, ns_iters 5, (a,b,c) = (3.4445, -4.7750, 2.0315)
 * (the quintic published with the Muon optimizer; the pages only name
 * Newton-Schulz), ns_eps 1e-7, step 1, norm_eps 1e-12, io_dtype LACT_BF16,
 * products LACT_PRODUCTS_AUTO, norm_mode LACT_NORM_UNIT, eta_mode LACT_ETA_SHARED,
 * net LACT_NET_SWIGLU.
 * B, H, d, h are set to 0 and must be filled in. */
void lact_config_default(lact_config* cfg);

/* Bytes of scratch that lact_update / lact_apply / lact_chunked_forward
 * need for chunks of at most `max_chunk_kv` keys and `max_chunk_q`
 * queries.  Pure host function.  Returns 0 for an invalid or unsupported
 * configuration. */
size_t lact_workspace_bytes(const lact_config* cfg, int64_t max_chunk_kv, int64_t max_chunk_q);

/* One large-chunk update of every pair: steps (2)-(4) above on n keys.
 * K, V: pair p's rows start at K + p*kv_stride_bh (elements); eta: pair p
 * starts at eta + p*eta_stride_bh (per matrix: see lact_eta_mode).  n >= 1
 * (any n: ragged tails are handled).  The state is read and written. */
int lact_update(const lact_config* cfg, const lact_state* st,
                const void* K, const void* V, const float* eta,
                int64_t n, int64_t kv_stride_bh, int64_t eta_stride_bh,
                void* ws, size_t ws_bytes, void* stream);

/* Query read, step (1) above: O = f_W(Q) row by row for m queries of every
 * pair.  Q and O rows of pair p start at p*q_stride_bh.  The state is only
 * read.  m >= 1. */
int lact_apply(const lact_config* cfg, const lact_state* st,
               const void* Q, void* O, int64_t m, int64_t q_stride_bh,
               void* ws, size_t ws_bytes, void* stream);

/* The whole layer: a sequential scan over N = T_kv / chunk_kv chunks
 * (T_q / chunk_q must equal N).  Chunk c updates with keys
 * [c*chunk_kv, (c+1)*chunk_kv) and reads for queries
 * [c*chunk_q, (c+1)*chunk_q), in `order` (lact_order).  The last update
 * always runs, so the state on return is W after all chunks.  Inputs are
 * contiguous [B, H, T, d] (eta [B, H, T_kv]). */
int lact_chunked_forward(const lact_config* cfg, const lact_state* st,
                         const void* Q, const void* K, const void* V, const float* eta,
                         void* O, int64_t T_kv, int64_t T_q, int64_t chunk_kv,
                         int64_t chunk_q, int32_t order, void* ws, size_t ws_bytes,
                         void* stream);

/* lact_chunked_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace.  Its scratch is a
 * fixed array of lact_noalloc_scratch_bytes() bytes (64 MiB) that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * nothing.  The device is the current one (the stream must belong to it).
 * Chunks whose workspace (lact_workspace_bytes) exceeds the array are
 * refused with LACT_ERR_WORKSPACE.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (several streams or threads) race,
 * and must be ordered by the caller.  Nothing in the array needs clearing
 * between calls.  Results are the same bits as lact_chunked_forward's. */
int lact_chunked_forward_noalloc(const lact_config* cfg, const lact_state* st,
                                 const void* Q, const void* K, const void* V, const float* eta,
                                 void* O, int64_t T_kv, int64_t T_q, int64_t chunk_kv,
                                 int64_t chunk_q, int32_t order, void* stream);

/* Size of the allocation-free entry point's scratch array. */
size_t lact_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------- the block
 * The LaCT block ("LaCT: Large Chunk Test-Time Training" review, section
 * "Local attention and nonlinear memory work together"; project page,
 * Figure 2): causal sliding-window attention handles the structure inside a
 * chunk, the TTT layer the history across chunks; the language and video
 * variants share Q, K, V between the two and add their outputs.
 *
 * lact_window_attention: O = attention(Q, K, V) (accumulate = 0) or
 * O += attention(Q, K, V) (accumulate = 1) for Q, K, V, O [B, H, T, d] of
 * cfg's io_dtype (pairs T d elements apart), where query t attends the
 * keys s with t - window < s <= t:
 *   o_t = sum_s softmax_s(scale q_t . k_s) v_s,  scale <= 0 means 1/sqrt(d).
 * d in {32, 64, 128}; window >= 1; fp32 arithmetic.  Only B, H, d and
 * io_dtype of cfg are used.
 *
 * lact_block_forward: O = attention(Q, K, V) + TTT(Q, K, V) with one shared
 * Q, K, V [B, H, T, d]: lact_chunked_forward with T_q = T_kv = T and
 * chunk_q = chunk_kv = chunk (state updated in place, workspace as for it),
 * then the window attention added into O, on one stream. */
int lact_window_attention(const lact_config* cfg, const void* Q, const void* K, const void* V,
                          void* O, int64_t T, int64_t window, float scale, int32_t accumulate,
                          void* stream);
int lact_block_forward(const lact_config* cfg, const lact_state* st, const void* Q, const void* K,
                       const void* V, const float* eta, void* O, int64_t T, int64_t chunk,
                       int64_t window, float scale, int32_t order, void* ws, size_t ws_bytes,
                       void* stream);

/* ------------------------------------------------------------------ backward
 * Training through the layer: the pages' throughput figures are training
 * throughput ("LaCT: Large Chunk Test-Time Training" review, section
 * "Language modelling: quality and throughput differ").  Given the cotangent
 * dO of lact_chunked_forward's outputs (and, optionally, of the final fast
 * weights), lact_chunked_backward returns the cotangents of its inputs: dQ,
 * dK, dV, deta and the initial fast weights dW1, dW2, dW3.  It first reruns
 * the forward updates from the initial weights (with zero momentum), keeping
 * the weights entering every chunk in the workspace, then takes every chunk
 * back in reverse order: the query read, the step and row normalisation,
 * the optimizer (momentum's buffer cotangent carried back over the chunks,
 * Newton-Schulz differentiated through every iteration and its pre-scaling)
 * and the chunk gradient itself (a gradient: its VJP carries the second
 * derivative of silu).  The forward updates run on the same kernels as
 * lact_chunked_forward; every VJP runs fp32 arithmetic.
 * Scope: the SwiGLU fast net with unit rows (norm_mode LACT_NORM_UNIT), one
 * rate per token, d in {32, 64, 128}, h a multiple of 32 up to 1024; any
 * order and optimizer.  Others return LACT_ERR_UNSUPPORTED. */
typedef struct {
  void *dQ, *dK, *dV;      /* like Q, K, V (io_dtype), written                         */
  float* deta;             /* [B, H, T_kv], written                                     */
  float *dW1, *dW2, *dW3;  /* like W1, W2, W3: cotangents of the initial weights, written */
} lact_grads;

/* Scratch for lact_chunked_backward on sequences of T_kv keys in chunks of
 * chunk_kv keys and chunk_q queries: the forward's workspace, N + 1 copies
 * of the fast weights (and momentum), per-token factors of the weight
 * cotangents (3 h floats per token and pair) and small per-pair buffers.
 * 0 for an invalid or unsupported configuration. */
size_t lact_backward_workspace_bytes(const lact_config* cfg, int64_t T_kv, int64_t chunk_kv,
                                     int64_t chunk_q);

/* st: the initial fast weights (read only; M is taken as zero).  Q, K, V,
 * eta, T_kv, T_q, chunk sizes and order as for lact_chunked_forward.  dO:
 * cotangent of O, like Q.  dW_final: NULL, or a state whose W1, W2, W3 hold
 * the cotangents of the final fast weights (its M fields are ignored).
 * Every output of `out` is written (not accumulated). */
int lact_chunked_backward(const lact_config* cfg, const lact_state* st, const void* Q,
                          const void* K, const void* V, const float* eta, const void* dO,
                          const lact_state* dW_final, const lact_grads* out, int64_t T_kv,
                          int64_t T_q, int64_t chunk_kv, int64_t chunk_q, int32_t order,
                          void* ws, size_t ws_bytes, void* stream);

/* Static text of a status code. */
const char* lact_status_string(int status);

/* Thread-local text of the last failure on this thread ("" if none). */
const char* lact_last_error(void);

/* 1 when the bf16 MFMA kernels serve (d, h); 0 when the generic fp32-math
 * kernels do; -1 when (d, h) is not supported at all. */
int lact_mfma_path(int32_t d, int32_t h, int32_t io_dtype);

/* Kernel timing for measurement tools (not thread-safe; off by default).
 * While enabled, every entry point records HIP events on its stream around
 * each phase; lact_profile_read() waits for the recorded events, adds their
 * durations into ms[phase] / launches[phase] (arrays of LACT_PROFILE_PHASES)
 * and clears the record.  Phases: 0 chunk gradient; 1 update tail (the
 * fixed-order sum of the token splits and the momentum update, with the
 * step and row normalisation, and for bf16-mode Muon with Newton-Schulz
 * too: one or two kernels); 2 Newton-Schulz and 3 step + row normalisation
 * when they run as kernels of their own (fp32-arithmetic Muon); 4 query
 * read; in lact_chunked_backward (whose forward rerun also records phases
 * 0-4): 5 the key-side token kernel (VJP of the chunk gradient), 6 the
 * query-side token kernel (VJP of the query read), 7 the weight-cotangent
 * contractions with their fixed-order sum, 8 Newton-Schulz forward and VJP;
 * 9 window attention (lact_window_attention, lact_block_forward). */
#define LACT_PROFILE_PHASES 10
int lact_profile_enable(int on);
int lact_profile_read(double* ms, int64_t* launches);

int lact_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LACT_H */

// Query read O = W2 (silu(W1 q) * (W3 q)) on bf16 MFMA (gfx950), d = 64 or
// 128, h in {128, 256}, as a device function: the body of the query-read
// kernel, also run by the workgroups of a fused launch beside the Muon
// update tail ("LaCT: Large Chunk Test-Time Training" review, sections
// "Local attention and nonlinear memory work together" and "Update order
// must respect the task").
//
// A workgroup of h / 32 wavefronts owns one pair and a contiguous run of
// queries.  Wavefront w keeps, as bf16 MFMA operands in registers, the W1
// and W3 rows of hidden units 32 w .. 32 w + 31 and the 32 rows of W2 of
// its phase-2 tile.  Per step of TQ = 32 (h / 32) / (d / 32) queries:
//   1. wave w computes H1^T, H3^T = W1 Q^T, W3 Q^T for its 32 hidden units
//      (A = W rows in registers, B = query rows from LDS), gates them,
//      G = silu(H1) * H3, and writes G (bf16) to LDS as [token][hidden];
//   2. wave w computes one 32 x 32 tile of O^T = W2 G^T (A = its W2 rows,
//      B = G rows from LDS) and stores it.
// Two wavefronts share each SIMD (two workgroups per CU for h = 128, one
// of eight wavefronts for h = 256).  All LDS tiles are XOR-swizzled in
// 16-byte chunks (see swz) so the operand reads and writes are free of bank
// conflicts.
#ifndef LACT_APPLY_BODY_H
#define LACT_APPLY_BODY_H

#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {
namespace apply_detail {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

template <int D, int H>
struct AGeo {
  static constexpr int NW = H / 32;            // wavefronts (one per 32 hidden units)
  static constexpr int THREADS = 64 * NW;
  static constexpr int NTT = NW / (D / 32);    // 32-token tiles per step
  static constexpr int TQ = 32 * NTT;          // queries per step
  static constexpr int WROW = 2 * D;           // bytes per row of Q
  static constexpr int GROW = 2 * H;           // bytes per row of G
  static constexpr int QBUF = TQ * WROW;       // one query tile
  static constexpr int GBUF = TQ * GROW;       // one gated-hidden tile
  static constexpr int OFF_Q = 0;              // two query buffers
  static constexpr int OFF_G = 2 * QBUF;       // two G buffers
  static constexpr int LDS = OFF_G + 2 * GBUF;
  static constexpr int WG_PER_CU = NW == 4 ? 2 : 1;
};

// eight consecutive floats as a bf16 operand: two 16-byte loads when the
// weights are 16-byte aligned, else eight 4-byte loads
__device__ __forceinline__ bf16x8_t load8_bf16(const float* p, bool vec) {
  bf16x8_t v;
  if (vec) {
    const float4 x = reinterpret_cast<const float4*>(p)[0];
    const float4 y = reinterpret_cast<const float4*>(p)[1];
    v[0] = static_cast<__bf16>(x.x);
    v[1] = static_cast<__bf16>(x.y);
    v[2] = static_cast<__bf16>(x.z);
    v[3] = static_cast<__bf16>(x.w);
    v[4] = static_cast<__bf16>(y.x);
    v[5] = static_cast<__bf16>(y.y);
    v[6] = static_cast<__bf16>(y.z);
    v[7] = static_cast<__bf16>(y.w);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = static_cast<__bf16>(p[k]);
  }
  return v;
}

// operand of eight consecutive weights: with COPY from the bf16 copy
// (element offset `toff` in its operand order, 16 consecutive bytes per
// lane), else converted from the fp32 weights at element offset `off`
template <bool COPY>
__device__ __forceinline__ bf16x8_t weight_op(const uint16_t* wb, int64_t toff, const float* wf, int64_t off,
                                              bool vec) {
  // (without COPY the choice stays a runtime branch per operand: the
  // conversions then run one operand at a time, where hoisting all of the
  // fp32 loads ahead would run out of registers)
  if (COPY || wb != nullptr) return *reinterpret_cast<const bf16x8_t*>(wb + toff);
  return load8_bf16(wf + off, vec);
}

// byte offset of 16-byte chunk `c` of row `r` (rows of `rowbytes`: 128,
// 256 or 512), XOR-swizzled so that 16 consecutive rows put a given chunk
// in 16 different 16-byte slots of the 256-byte bank window (LDS serves
// these accesses 16 lanes at a time, one row each): c ^ (r & 15) for rows
// of 16 or more chunks, c ^ ((r >> 1) & 7) for 128-byte rows (two per
// window).
__device__ __forceinline__ int swz(int r, int c, int rowbytes) {
  const int x = rowbytes >= 256 ? (r & 15) : ((r >> 1) & 7);
  return r * rowbytes + ((c ^ x) << 4);
}

// One workgroup's share of the query read: virtual block vb of nvb (nvb a
// multiple of 8, and vb congruent mod 8 to the hardware block id, so that
// block ids congruent mod 8 still share an XCD); LDS of AGeo<D, H>::LDS bytes.
// XCD-aware order: the workgroups of a pair take consecutive slots of one
// XCD's share, so its W reads after the first hit that XCD's L2.
template <int D, int H, bool COPY>
__device__ __forceinline__ void apply_body(const ApplyArgs& a, unsigned char* lds, int vb, int nvb, int per_wg,
                                           int wg_per_pair) {
  using G = AGeo<D, H>;
  constexpr int kThreads = G::THREADS;  // = 2 H (the launch bound)
  static_assert(kThreads == 2 * H, "threads");
  // XCD-aware order: block ids congruent mod 8 run on one XCD, and the
  // workgroups of a pair take consecutive slots of one XCD's share, so
  // its W reads after the first hit that XCD's L2.
  const int o = (vb & 7) * (nvb >> 3) + (vb >> 3);
  if (o >= wg_per_pair * a.P) return;
  const int pair = o / wg_per_pair;
  const int64_t q_begin = static_cast<int64_t>(o % wg_per_pair) * per_wg;
  const int64_t q_end = min(a.m, q_begin + per_wg);
  if (q_begin >= q_end) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, ln = lane & 31;
  const int64_t hd = static_cast<int64_t>(H) * D;

  // ---- W1, W3 operands (A side: hidden row 32 w + ln, features 16 ks + 8 g .. +7)
  constexpr int KS1 = D / 16;
  bf16x8_t w1a[KS1], w3a[KS1];
  {
    const int64_t row = pair * hd + static_cast<int64_t>(32 * w + ln) * D;
    // (the copy's block (w, ks), lane slice = wb_tiled(32 w + ln, 16 ks + 8 g, D))
    const int64_t tb = pair * hd + static_cast<int64_t>(w) * (D / 16) * 512 + 8 * lane;
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks) {
      w1a[ks] = weight_op<COPY>(a.Wb1, tb + 512 * ks, a.W1, row + 16 * ks + 8 * g, a.w_vec);
      w3a[ks] = weight_op<COPY>(a.Wb3, tb + 512 * ks, a.W3, row + 16 * ks + 8 * g, a.w_vec);
    }
  }
  // ---- this wave's phase-2 tile: rows 32 dt .. of O^T, tokens 32 tt ..
  const int dt = w % (D / 32);
  const int tt = w / (D / 32);
  constexpr int KS2 = H / 16;
  bf16x8_t w2b[KS2];
  {
    const int64_t row = pair * hd + static_cast<int64_t>(32 * dt + ln) * H;
    const int64_t tb = pair * hd + static_cast<int64_t>(dt) * (H / 16) * 512 + 8 * lane;
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks)
      w2b[ks] = weight_op<COPY>(a.Wb2, tb + 512 * ks, a.W2, row + 16 * ks + 8 * g, a.w_vec);
  }

  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + static_cast<int64_t>(pair) * a.q_stride;
  uint16_t* Og = static_cast<uint16_t*>(a.O) + static_cast<int64_t>(pair) * a.q_stride;

  // query staging: TQ rows x D bf16 = TQ * D / 8 chunks of 16 bytes
  constexpr int QCH = G::TQ * D / 8;
  constexpr int QPT = QCH / kThreads;  // chunks per thread (= 2)
  static_assert(QPT * kThreads == QCH, "query staging");
  u32x4_t qr[QPT];
  auto load_q = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = tid + kThreads * k;
      const int r = i / (D / 8), c = i % (D / 8);
      const int64_t tok = t0 + r;
      qr[k] = (tok < q_end) ? *reinterpret_cast<const u32x4_t*>(Qg + tok * D + 8 * c)
                            : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_q = [&](int b) {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = tid + kThreads * k;
      const int r = i / (D / 8), c = i % (D / 8);
      *reinterpret_cast<u32x4_t*>(lds + G::OFF_Q + b * G::QBUF + swz(r, c, G::WROW)) = qr[k];
    }
  };

  constexpr float kLog2e = 1.4426950408889634f;
  // phase 1 of one step: H^T for hidden units [32 w, 32 w + 32) x TQ
  // tokens from query buffer b, gated, into G buffer b
  auto phase1 = [&](int b) {
#pragma unroll
    for (int t = 0; t < G::NTT; ++t) {
      bf16x8_t bq[KS1];
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks)
        bq[ks] = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_Q + b * G::QBUF + swz(32 * t + ln, 2 * ks + g, G::WROW));
      f32x16_t c1, c3;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c1[r] = 0.f;
        c3[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks) {
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1a[ks], bq[ks], c1, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w3a[ks], bq[ks], c3, 0, 0, 0);
      }
      // c[r] = H^T[hidden 32 w + 8 (r/4) + 4 g + r%4][token 32 t + ln]
      const int tok = 32 * t + ln;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4_t gv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float h1 = c1[4 * rg + i], h3 = c3[4 * rg + i];
          const float s = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * h1));
          gv[i] = static_cast<__bf16>(h1 * s * h3);
        }
        const int hid = 32 * w + 8 * rg + 4 * g;
        *reinterpret_cast<bf16x4_t*>(lds + G::OFF_G + b * G::GBUF + swz(tok, hid >> 3, G::GROW) + 2 * (hid & 7)) = gv;
      }
    }
  };
  // phase 2 of the step starting at query t0: O^T tile (d rows 32 dt..,
  // tokens 32 tt..) = W2 G^T from G buffer b
  auto phase2 = [&](int b, int64_t t0) {
    f32x16_t acc0, acc1;  // two accumulator chains over alternate k-steps
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[r] = 0.f;
      acc1[r] = 0.f;
    }
    // G operands in groups of eight k-steps, each group read before its MFMAs
#pragma unroll
    for (int k0 = 0; k0 < KS2; k0 += 8) {
      bf16x8_t bg[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bg[j] = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_G + b * G::GBUF + swz(32 * tt + ln, 2 * (k0 + j) + g, G::GROW));
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2b[k0 + j], bg[j], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2b[k0 + j + 1], bg[j + 1], acc1, 0, 0, 0);
      }
    }
    const int64_t tok = t0 + 32 * tt + ln;
    if (tok < q_end) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4_t ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(acc0[4 * rg + i] + acc1[4 * rg + i]);
        const int dd = 32 * dt + 8 * rg + 4 * g;
        *reinterpret_cast<bf16x4_t*>(Og + tok * D + dd) = ov;
      }
    }
  };

  // Software pipeline, one barrier per step: between two barriers a wave
  // runs phase 2 of step j (G buffer j % 2) and phase 1 of step j + 1
  // (query and G buffers (j + 1) % 2), and stages the queries of step j + 2
  // into query buffer j % 2, whose last readers (phase 1 of step j) ran
  // before the previous barrier.
  const int nsteps = static_cast<int>((q_end - q_begin + G::TQ - 1) / G::TQ);
  load_q(q_begin);
  store_q(0);
  if (nsteps > 1) load_q(q_begin + G::TQ);
  __syncthreads();
  phase1(0);
  if (nsteps > 1) store_q(1);
  if (nsteps > 2) load_q(q_begin + 2 * G::TQ);
  __syncthreads();
#pragma unroll 1
  for (int j = 0; j + 1 < nsteps; ++j) {
    const int b = j & 1;
    phase2(b, q_begin + static_cast<int64_t>(j) * G::TQ);
    phase1(b ^ 1);
    if (j + 2 < nsteps) store_q(b);
    if (j + 3 < nsteps) load_q(q_begin + static_cast<int64_t>(j + 3) * G::TQ);
    __syncthreads();
  }
  phase2((nsteps - 1) & 1, q_begin + static_cast<int64_t>(nsteps - 1) * G::TQ);
}

// Workgroup plan of the query read over at most `slots` workgroups: queries
// per workgroup (a multiple of the step, at least two steps) and workgroups
// per pair; each workgroup loads its pair's W once, so the workgroups of all
// pairs should fill the slots about once.
template <int D, int H>
inline void apply_plan(int64_t m, int P, int64_t slots, int* per_wg, int* wg_per_pair) {
  constexpr int TQ = AGeo<D, H>::TQ;
  const int64_t per_pair = P >= slots ? 1 : slots / P;
  int64_t per = (m + per_pair - 1) / per_pair;
  per = (per + TQ - 1) / TQ * TQ;
  if (per < 2 * TQ) per = 2 * TQ;  // at least one pipelined step pair
  *per_wg = static_cast<int>(per);
  *wg_per_pair = static_cast<int>((m + per - 1) / per);
}

}  // namespace apply_detail
}  // namespace
}  // namespace lact

#endif  // LACT_APPLY_BODY_H

// Chunk gradient of the LaCT layer for d = 128 on bf16 MFMA (gfx950), with
// plain bf16 products or with near-fp32 "split" products.
//
// For one (pair, token split, 128-unit hidden slice) a workgroup of four
// wavefronts (32 hidden units each) sums, over the split's tokens i,
//   dW1 += dh1_i k_i^T,  dW3 += dh3_i k_i^T,  dW2 += v_i (-eta_i g_i)^T
// with h1 = W1 k, h3 = W3 k, a = silu(h1), g = a * h3, dg = -eta_i W2^T v_i,
// dh3 = dg * a, dh1 = dg * h3 * silu'(h1): the gradient of
// -sum_i eta_i <f_W(k_i), v_i> for f_W(x) = W2 (silu(W1 x) * (W3 x))
// ("LaCT: Large Chunk Test-Time Training" review, section "Local attention
// and nonlinear memory work together").  The chunk is a set, so the sum is
// split over tokens across workgroups and reduced afterwards in fixed order.
//
// Same dataflow as the d = 64 kernel: keys, values and eta move from HBM
// straight into double-buffered, chunk-swizzled LDS tiles (global_load_lds)
// one stage ahead; -eta enters in the SwiGLU step; projections and
// contractions are 32x32x16 MFMAs; the token-side operands come from LDS
// transpose reads.  The dW tiles (192 fp32 per lane) need one wavefront
// per SIMD.
//
// Split products: keys and values are exact bf16 inputs, so only the other
// operand of every product is split, x = x_hi + x_lo (both bf16), and each
// product is two MFMAs, K W^T ~ K W_hi^T + K W_lo^T, P K ~ P_hi K + P_lo K:
// ~16 significant bits per operand.  W_lo of W1 and W3 sits in LDS (read
// per k-step), W_lo of W2 in registers.
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_t;

constexpr int D = 128;
constexpr int kThreads = 256;
constexpr int kHidPerWave = 32;
constexpr int kHidPerWG = 128;
constexpr int KS = D / 16;    // k-steps of the projections
constexpr int NT = D / 32;    // 32-wide d tiles of the contractions
constexpr int ROW = 2 * D;    // bytes per token row (sixteen 16-byte chunks)

constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

template <bool SPLIT, bool PM>
struct Geo {
  static constexpr int TT = SPLIT ? 64 : 128;  // tokens per LDS stage
  static constexpr int SUB = TT / 32;
  static constexpr int TILE = TT * ROW;
  static constexpr int NE = PM ? 3 : 1;        // rows of rates per stage (W1, W2, W3 with PM)
  static constexpr int OFF_K = 0;              // K[2]
  static constexpr int OFF_V = 2 * TILE;       // V[2]
  static constexpr int OFF_E = 4 * TILE;       // eta[2][NE][TT]
  static constexpr int OFF_WLO = 4 * TILE + 2 * NE * TT * 4;  // W1_lo, W3_lo operands (split)
  static constexpr int WLO_BYTES = SPLIT ? 2 * 4 * KS * 64 * 16 : 0;
  static constexpr int LDS = OFF_WLO + WLO_BYTES;
};

// XOR swizzle of the 16-byte chunks of token row r (r_i: bit i of r),
//     swz(r) = 8 r1 + 4 (r0 ^ r3) + 2 r0 + r2.
// A row is one 256-byte bank window (64 four-byte banks).  The projections'
// 16-byte row reads are served 16 lanes (16 consecutive rows, one chunk) at
// a time: swz is one-to-one on the low four row bits, so each lane gets its
// own 16-byte slot.  The contractions' 8-byte transpose reads are checked
// 32 lanes at a time: four rows 4m .. 4m + 3 and an aligned quad of chunks;
// bits 2, 3 of swz take four different values on those rows (r0, r1), so
// the four quads fill the window.  Bits 0, 1 of swz depend on lane bits of
// the transpose-read row only, which keeps those addresses a lane constant
// per (nt & 1) ^ hh and nt >> 1 plus immediates.
__device__ __forceinline__ int swz(int r) {
  return 8 * ((r >> 1) & 1) + 4 * ((r ^ (r >> 3)) & 1) + 2 * (r & 1) + ((r >> 2) & 1);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// lo bf16 part of a float given its hi part (the rounded remainder)
__device__ __forceinline__ __bf16 lo_bf16(float x, __bf16 hi) {
  return static_cast<__bf16>(x - static_cast<float>(hi));
}

// PM: a learning rate per token and matrix (rows of rates for W1, W2, W3,
// a.eta_mat elements apart); otherwise one rate per token.
template <bool SPLIT, bool PM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_grad_d128(GradArgs a, int hsl, int nbase) {
  using G = Geo<SPLIT, PM>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS];

  // XCD-aware block order: the hidden slices of one (pair, split) land on
  // the same XCD (block ids congruent mod 8) so their key/value reads share L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int rest = bid >> 3;
  const int hs = rest % hsl;
  const int base = (rest / hsl) * 8 + xcd;
  if (base >= nbase) return;
  const int pair = base / a.S;
  const int split = base % a.S;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int ln = lane & 31;
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int n0 = hs * kHidPerWG + wave * kHidPerWave;

  // ---- W^T operands of the projections: lane holds hidden unit n0 + ln,
  // features 16 ks + 8 g .. +7 (hi parts in registers; for split products
  // the lo parts of W1 and W3 go to LDS, slot [matrix][wave][ks][lane], and
  // W2's to registers)
  bf16x8_t w1b[KS], w3b[KS], w2b[KS];
  bf16x8_t w2l[SPLIT ? KS : 1];
  {
    const float* W1 = a.W1 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W3 = a.W3 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W2 = a.W2 + pair * hd + n0 + ln;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t l1, l3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dd = 16 * ks + 8 * g + i;
        const float x1 = kNegLog2e * W1[dd], x3 = W3[dd];
        w1b[ks][i] = static_cast<__bf16>(x1);
        w3b[ks][i] = static_cast<__bf16>(x3);
        l1[i] = lo_bf16(x1, w1b[ks][i]);
        l3[i] = lo_bf16(x3, w3b[ks][i]);
        if constexpr (SPLIT) {
          const float x2 = W2[static_cast<int64_t>(dd) * h];
          w2b[ks][i] = static_cast<__bf16>(x2);
          w2l[ks][i] = lo_bf16(x2, w2b[ks][i]);
        } else {
          w2b[ks][i] = static_cast<__bf16>(W2[static_cast<int64_t>(dd) * h]);
        }
      }
      if constexpr (SPLIT) {
        *reinterpret_cast<bf16x8_t*>(lds + G::OFF_WLO + (((0 * 4 + wave) * KS + ks) * 64 + lane) * 16) = l1;
        *reinterpret_cast<bf16x8_t*>(lds + G::OFF_WLO + (((1 * 4 + wave) * KS + ks) * 64 + lane) * 16) = l3;
      }
    }
  }

  f32x16_t aW1[NT], aW3[NT], aW2[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      aW1[t][r] = 0.f;
      aW3[t][r] = 0.f;
      aW2[t][r] = 0.f;
    }
  }

  const int64_t t_begin = static_cast<int64_t>(split) * a.tps;
  const int64_t t_end = min(a.n, t_begin + a.tps);
  const int64_t kv_base = static_cast<int64_t>(pair) * a.kv_stride;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + kv_base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + kv_base;
  const float* etag = a.eta + static_cast<int64_t>(pair) * a.eta_stride;
  // (token offsets inside one pair's rows fit 32 bits: the host routes
  // longer sequences elsewhere)
  const int t_last = static_cast<int>(t_end - 1);

  // DMA of one stage into buffer b: 1 KiB pieces (4 rows each), wave wv
  // moving pieces wv, wv + 4, ...; lane l of a piece lands at its byte 16 l:
  // row 4 piece + l / 16, physical chunk l % 16.  Rows past the end re-read
  // the split's last token (finite values); their eta is written as 0.
  auto dma_stage = [&](int64_t t0, int b) {
    // (the lane-derived offsets are recomputed per stage: a few
    // instructions, where keeping them live would spill registers)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int k = 0; k < G::TT / 16; ++k) {
      const int piece = 4 * k + wv;
      const int r = 4 * piece + (lane >> 4);
      const int cl = (lane & 15) ^ swz(r);
      const int tok = static_cast<int>(t0) + r;
      const int tc = tok < t_last ? tok : t_last;
      const unsigned off = static_cast<unsigned>(tc) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Kg + off), (lds_ptr_t)(lds + G::OFF_K + b * G::TILE + 1024 * piece), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Vg + off), (lds_ptr_t)(lds + G::OFF_V + b * G::TILE + 1024 * piece), 16, 0, 0);
    }
    // rates: pieces of 64 (matrix piece / (TT / 64), tokens 64 (piece % (TT / 64)) ..),
    // wave wv moving pieces wv and wv + 4
    constexpr int HPM = G::TT / 64;  // pieces per row of rates
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
      const int piece = wv + 4 * pc;
      if (piece < G::NE * HPM) {
        const int tok = static_cast<int>(t0) + 64 * (piece % HPM) + lane;
        const float* src = etag + (PM ? (piece / HPM) * a.eta_mat : 0);
        unsigned char* dst = lds + G::OFF_E + b * G::NE * G::TT * 4 + 256 * piece;
        if (tok <= t_last) {
          __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src + static_cast<unsigned>(tok)), (lds_ptr_t)dst, 4, 0, 0);
        } else {
          *reinterpret_cast<float*>(dst + 4 * lane) = 0.f;
        }
      }
    }
  };

  // transpose-read addressing (see the d = 64 kernel): within each 16-lane
  // row Q, lane 16 Q + 4 k' + a addresses token 4 (Q >> 1) + k' (+ 8 hh) of
  // a 16-token half, features 32 nt + 16 (Q & 1) + 4 a .. +3.
  const int tq = lane >> 4, tk = (lane >> 2) & 3, ta = lane & 3;
  // Operand addresses as lane constants plus immediates (the XOR swizzle
  // reduces to additions here):
  //  row reads, token 32 st + ln, chunk 2 ks + g:  ak_off[ks] + 8192 st;
  //  transpose reads, token 32 st + 16 s + 8 hh + L (L = 4 (tq >> 1) + tk),
  //  features from 32 nt + 16 (tq & 1) + 4 ta:
  //      tr_off[(nt & 1) ^ hh][nt >> 1] + 8192 st + 4096 s + 2048 hh.
  int ak_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ak_off[ks] = ln * ROW + 16 * ((2 * ks + g) ^ swz(ln));
  int tr_off[2][2];
  {
    const int tl = 4 * (tq >> 1) + tk;
    const int r0 = tl & 1, r1 = (tl >> 1) & 1, r2 = (tl >> 2) & 1;
    const int low = (2 * (tq & 1) + (ta >> 1)) ^ (2 * r0 + r2);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int n1 = 0; n1 < 2; ++n1)
        tr_off[x][n1] = tl * ROW + 16 * (8 * (n1 ^ r1) + 4 * (x ^ r0) + low) + 8 * (ta & 1);
    }
  }

  if (t_begin < t_end) dma_stage(t_begin, 0);
  int b = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += G::TT, b ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this stage has landed
    __syncthreads();
    if (t0 + G::TT < t_end) dma_stage(t0 + G::TT, b ^ 1);

    const unsigned char* kb = lds + G::OFF_K + b * G::TILE;
    const unsigned char* vb = lds + G::OFF_V + b * G::TILE;
    // rates of this stage (with PM rows for W1, W2, W3)
    const float* eb = reinterpret_cast<const float*>(lds + G::OFF_E + b * G::NE * G::TT * 4);

#pragma unroll 1
    for (int st = 0; st < G::SUB; ++st) {
      f32x16_t c1, c3, cg;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c1[r] = 0.f;
        c3[r] = 0.f;
        cg[r] = 0.f;
      }
      // With bf16 products every group of operand reads is issued before its
      // first use, so one wait covers the group instead of one exposed
      // latency per read (one wavefront per SIMD: nothing else hides it);
      // the split variant has no registers to spare for that.
      auto kv_row = [&](int ks, bool v) {
        return *reinterpret_cast<const bf16x8_t*>((v ? vb : kb) + ak_off[ks] + 8192 * st);
      };
      constexpr int PRE = SPLIT ? 1 : KS;
      bf16x8_t akv[PRE], avv[PRE];
      if constexpr (!SPLIT) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          akv[ks] = kv_row(ks, false);
          avv[ks] = kv_row(ks, true);
        }
      }
      // eta of this lane's 16 tokens (operand slot i of half s <-> token
      // 16 s + 8 (i / 4) + 4 g + i % 4); with PM the rates of W2 (read per
      // half below, with those of W1 and W3)
      f32x4_t eta4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        eta4[q] = *reinterpret_cast<const f32x4_t*>(eb + (PM ? G::TT : 0) + 32 * st + 8 * q + 4 * g);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ak = SPLIT ? kv_row(ks, false) : akv[SPLIT ? 0 : ks];
        const bf16x8_t av = SPLIT ? kv_row(ks, true) : avv[SPLIT ? 0 : ks];
        c1 = mfma32(ak, w1b[ks], c1);
        c3 = mfma32(ak, w3b[ks], c3);
        cg = mfma32(av, w2b[ks], cg);
        if constexpr (SPLIT) {
          const bf16x8_t l1 = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_WLO + (((0 * 4 + wave) * KS + ks) * 64 + lane) * 16);
          const bf16x8_t l3 = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_WLO + (((1 * 4 + wave) * KS + ks) * 64 + lane) * 16);
          c1 = mfma32(ak, l1, c1);
          c3 = mfma32(ak, l3, c3);
          cg = mfma32(av, w2l[ks], cg);
        }
      }
      // SwiGLU forward and backward, one 16-token half at a time (operand
      // slot i <-> token 16 s + 8 (i / 4) + 4 g + i % 4 of the sub-tile); see
      // the d = 64 kernel for the algebra.
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4_t e0 = eta4[2 * s], e1 = eta4[2 * s + 1];
        // with PM: rates of W1 (x1) and W3 (x3) for the same slots
        f32x4_t x10, x11, x30, x31;
        if constexpr (PM) {
          x10 = *reinterpret_cast<const f32x4_t*>(eb + 32 * st + 16 * s + 4 * g);
          x11 = *reinterpret_cast<const f32x4_t*>(eb + 32 * st + 16 * s + 8 + 4 * g);
          x30 = *reinterpret_cast<const f32x4_t*>(eb + 2 * G::TT + 32 * st + 16 * s + 4 * g);
          x31 = *reinterpret_cast<const f32x4_t*>(eb + 2 * G::TT + 32 * st + 16 * s + 8 + 4 * g);
        }
        // token-side operands: slots 0-3 <-> tokens 16 s + 4 g + k',
        // slots 4-7 <-> tokens 16 s + 8 + 4 g + k' (bf16 products: read
        // before the elementwise step, which hides their latency)
        auto tr_op = [&](int nt, bool v) {
          s16x4_t t[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int off = tr_off[(nt & 1) ^ hh][nt >> 1] + 8192 * st + 4096 * s + 2048 * hh;
            t[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)((v ? vb : kb) + off));
          }
          return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
        };
        constexpr int PRT = SPLIT ? 1 : NT;
        bf16x8_t bkv[PRT], bvv[PRT];
        if constexpr (!SPLIT) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            bkv[nt] = tr_op(nt, false);
            bvv[nt] = tr_op(nt, true);
          }
        }
        bf16x8_t pg, pd1, pd3, lg, l1, l3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * s + i;
          const float ne = -((i < 4) ? e0[i & 3] : e1[i & 3]);
          const float z = c1[r], h3 = c3[r];
          // dG of the losses W1 and W3 follow (the same one without PM)
          const float dg = ne * cg[r];
          const float dg1 = PM ? -((i < 4) ? x10[i & 3] : x11[i & 3]) * cg[r] : dg;
          const float dg3 = PM ? -((i < 4) ? x30[i & 3] : x31[i & 3]) * cg[r] : dg;
          const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z));
          const float act = z * sg;
          const float gs = act * h3;
          const float t = fmaf(h3, kNegLog2e, -gs);
          const float vg = ne * gs, v3 = dg3 * act, v1 = dg1 * fmaf(sg, t, gs);
          pg[i] = static_cast<__bf16>(vg);
          pd3[i] = static_cast<__bf16>(v3);
          pd1[i] = static_cast<__bf16>(v1);
          if constexpr (SPLIT) {
            lg[i] = lo_bf16(vg, pg[i]);
            l3[i] = lo_bf16(v3, pd3[i]);
            l1[i] = lo_bf16(v1, pd1[i]);
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8_t bk = SPLIT ? tr_op(nt, false) : bkv[SPLIT ? 0 : nt];
          const bf16x8_t bv = SPLIT ? tr_op(nt, true) : bvv[SPLIT ? 0 : nt];
          aW1[nt] = mfma32(pd1, bk, aW1[nt]);
          aW3[nt] = mfma32(pd3, bk, aW3[nt]);
          aW2[nt] = mfma32(bv, pg, aW2[nt]);
          if constexpr (SPLIT) {
            aW1[nt] = mfma32(l1, bk, aW1[nt]);
            aW3[nt] = mfma32(l3, bk, aW3[nt]);
            aW2[nt] = mfma32(bv, lg, aW2[nt]);
          }
        }
      }
    }
  }

  // ---- partial sums of this split: [W1 block h x D | W2 block D x h | W3 block h x D]
  float* out = a.partials + (static_cast<int64_t>(pair) * a.S + split) * 3 * hd;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * g + (r & 3);
      out[static_cast<int64_t>(n0 + row) * D + 32 * nt + ln] = kNegLn2 * aW1[nt][r];
      out[2 * hd + static_cast<int64_t>(n0 + row) * D + 32 * nt + ln] = kNegLn2 * aW3[nt][r];
      out[hd + static_cast<int64_t>(32 * nt + row) * h + n0 + ln] = kNegLn2 * aW2[nt][r];
    }
  }
}

}  // namespace

bool grad_d128_shape_ok(int d, int h) {
  return d == D && h % kHidPerWG == 0 && h >= kHidPerWG && h <= 1024;
}

int grad_d128_stage_tokens(bool split) { return split ? Geo<true, false>::TT : Geo<false, false>::TT; }

hipError_t launch_grad_d128(const GradArgs& a, bool split, hipStream_t s) {
  if (a.d != D) return hipErrorInvalidValue;
  const int hsl = a.h / kHidPerWG;
  const int nbase = a.S * a.P;
  const int blocks = ((nbase + 7) / 8) * 8 * hsl;
  const bool pm = a.eta_mat != 0;
  if (split && pm) {
    hipLaunchKernelGGL((k_grad_d128<true, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else if (split) {
    hipLaunchKernelGGL((k_grad_d128<true, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else if (pm) {
    hipLaunchKernelGGL((k_grad_d128<false, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else {
    hipLaunchKernelGGL((k_grad_d128<false, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  }
  return hipGetLastError();
}

}  // namespace lact

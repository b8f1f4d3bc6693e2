// Chunk gradient of the LaCT layer for d = 64 on bf16 MFMA (gfx950), with
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
// Staging: keys, values and eta of the next 128-token stage move from HBM
// straight into LDS (global_load_lds, no registers, double-buffered) while
// the current stage computes; one barrier per stage.  Rows are 128 bytes
// with their 16-byte chunks XOR-swizzled per row.  The per-token factor
// -eta enters in the SwiGLU step (on dG' = W2^T v and on g), so the values
// need no conversion pass.
//
// Per 32-token sub-tile and wavefront, all on 32x32x16 MFMAs:
//   H1, H3 = K W^T and dG' = V W2 (A = key / value rows from LDS, B = W in
//   registers); the SwiGLU forward/backward runs on the fp32 outputs in the
//   MFMA output layout (lane = hidden unit, 16 tokens per lane) and is packed
//   to bf16, which is directly the hidden-side operand of the contractions
//   (token order inside an operand is the same permutation on both sides).
//   The token-side operands (K, V with tokens along k) come from the
//   row-major tiles through LDS transpose reads.
//
// Split products: keys and values are exact bf16 inputs, so only the other
// operand of every product is split, x = x_hi + x_lo (both bf16), and each
// product is two MFMAs (~16 significant bits per operand, twice the matrix
// work): K W^T = K W_hi^T + K W_lo^T with both parts of W in registers, and
// the contractions take the SwiGLU outputs as hi and lo parts.  That needs
// more registers than two wavefronts per SIMD leave, so the split kernel
// runs one workgroup per CU.
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(8))) short s16x8_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_t;

constexpr int D = 64;
constexpr int kThreads = 256;
constexpr int kHidPerWave = 32;
constexpr int kHidPerWG = 128;
constexpr int TT = 128;              // tokens per LDS stage
constexpr int SUB = TT / 32;         // 32-token sub-tiles per stage
constexpr int KS = D / 16;           // k-steps of the projections
constexpr int NT = D / 32;           // 32-wide d tiles of the contractions
constexpr int ROW = 2 * D;           // bytes per token row (eight 16-byte chunks)
constexpr int TILE = TT * ROW;       // one stage of K (or V)
// one stage buffer: K tile, V tile, eta; two buffers as separate LDS arrays
// (so the compiler sees that reads of one never alias the DMA into the other
// and puts no wait for the in-flight loads before them)
constexpr int OFF_K = 0;
constexpr int OFF_V = TILE;
constexpr int OFF_E = 2 * TILE;  // eta: one row of TT rates, or three (W1, W2, W3)
template <bool PM>
constexpr int buf_bytes() { return 2 * TILE + (PM ? 3 : 1) * TT * 4; }

// W1 enters pre-scaled by -log2(e) (sigmoid(h1) = 1 / (1 + 2^z), z = -log2(e) h1);
// G, dH3 and dH1 then carry that factor, removed at the end (times -ln 2).
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

// XOR swizzle of the 16-byte chunks of token row r (r_i: bit i of r),
//     swz(r) = 4 (r1 ^ r3) + 2 r2 + r1.
// LDS has 64 four-byte banks (256 bytes: two 128-byte rows).  A 16-byte
// read is served 16 lanes at a time: the projections' row reads (16
// consecutive rows, one chunk) find, among the eight rows of each parity,
// eight different chunk positions (swz is one-to-one on r1, r2, r3).  The
// contractions' 8-byte transpose reads are checked 32 lanes at a time: four
// rows 4m .. 4m + 3 and an aligned quad of chunks; rows 4m and 4m + 2 (and
// 4m + 1, 4m + 3) differ in r1, so bit 2 of swz puts their quads in the two
// different halves of the row.  Both read kinds are free of bank conflicts.
__device__ __forceinline__ int swz(int r) { return 4 * (((r >> 1) ^ (r >> 3)) & 1) + 2 * ((r >> 2) & 1) + ((r >> 1) & 1); }

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// lo bf16 part of a float given its hi part (the rounded remainder)
__device__ __forceinline__ __bf16 lo_bf16(float x, __bf16 hi) {
  return static_cast<__bf16>(x - static_cast<float>(hi));
}

// PM: a learning rate per token and matrix (rows of rates for W1, W2, W3,
// a.eta_mat elements apart); otherwise one rate per token.  SPLIT: split
// products (one wavefront per SIMD).
template <bool PM, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SPLIT ? 1 : 2, SPLIT ? 1 : 2)))
void k_grad_d64(GradArgs a, int hsl, int nbase) {
  __shared__ __attribute__((aligned(16))) unsigned char buf0[buf_bytes<PM>()];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[buf_bytes<PM>()];

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
  const int g = lane >> 5;   // operands: k-slots 8g..8g+7; outputs: rows 4g + ..
  const int ln = lane & 31;  // operands: row / column
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int n0 = hs * kHidPerWG + wave * kHidPerWave;  // this wave's hidden units

  // ---- W^T operands of the projections: lane holds hidden unit n0 + ln,
  // features 16 ks + 8 g .. +7 (with split products also the lo parts)
  bf16x8_t w1b[KS], w3b[KS], w2b[KS];
  bf16x8_t w1l[SPLIT ? KS : 1], w3l[SPLIT ? KS : 1], w2l[SPLIT ? KS : 1];
  {
    const float* W1 = a.W1 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W3 = a.W3 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W2 = a.W2 + pair * hd + n0 + ln;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dd = 16 * ks + 8 * g + i;
        const float x1 = kNegLog2e * W1[dd], x3 = W3[dd], x2 = W2[static_cast<int64_t>(dd) * h];
        w1b[ks][i] = static_cast<__bf16>(x1);
        w3b[ks][i] = static_cast<__bf16>(x3);
        w2b[ks][i] = static_cast<__bf16>(x2);
        if constexpr (SPLIT) {
          w1l[ks][i] = lo_bf16(x1, w1b[ks][i]);
          w3l[ks][i] = lo_bf16(x3, w3b[ks][i]);
          w2l[ks][i] = lo_bf16(x2, w2b[ks][i]);
        }
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

  // DMA of one stage into buffer b: wave wv moves rows 32 wv .. 32 wv + 31
  // of K and V (four 1 KiB pieces each; lane l of piece k lands at byte 16 l
  // of it: row 8 (4 wv + k) + l / 8, physical chunk l % 8) and waves 0, 1
  // move 64 eta values each (with PM waves wv and wv + 4 < 6 move rates
  // 64 (wv % 2) .. of matrix wv / 2).  Rows past the end re-read the split's last
  // token (finite values); their eta is written as 0 instead of loaded, so
  // they add nothing to the sums.
  auto dma_stage = [&](int64_t t0, unsigned char* dst) {
    // (the lane-derived offsets are recomputed per stage: a few
    // instructions, where keeping them live would spill registers)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int piece = 4 * wv + k;
      const int r = 8 * piece + (lane >> 3);
      const int cl = (lane & 7) ^ swz(r);  // logical chunk stored at this lane's slot
      const int tok = static_cast<int>(t0) + r;
      const int tc = tok < t_last ? tok : t_last;
      const unsigned off = static_cast<unsigned>(tc) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Kg + off), (lds_ptr_t)(dst + OFF_K + 1024 * piece), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Vg + off), (lds_ptr_t)(dst + OFF_V + 1024 * piece), 16, 0, 0);
    }
#pragma unroll
    for (int pc = 0; pc < (PM ? 2 : 1); ++pc) {
      const int piece = wv + 4 * pc;  // 64 rates: matrix piece / 2, tokens 64 (piece % 2) ..
      if (piece < (PM ? 6 : 2)) {
        const int tok = static_cast<int>(t0) + 64 * (piece & 1) + lane;
        const float* src = etag + (PM ? (piece >> 1) * a.eta_mat : 0);
        if (tok <= t_last) {
          __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src + static_cast<unsigned>(tok)),
                                           (lds_ptr_t)(dst + OFF_E + 256 * piece), 4, 0, 0);
        } else {
          *reinterpret_cast<float*>(dst + OFF_E + 256 * piece + 4 * lane) = 0.f;
        }
      }
    }
  };

  // transpose-read addressing: within each 16-lane row Q of the wave, lane
  // 16 Q + 4 k' + a addresses token 4 (Q >> 1) + k' (+ 8 hh) of a 16-token
  // half, features 32 nt + 16 (Q & 1) + 4 a .. +3; lane 16 Q + 4 a + b' then
  // holds feature 32 nt + 16 (Q & 1) + 4 a + b' of those four tokens.
  const int tq = lane >> 4, tk = (lane >> 2) & 3, ta = lane & 3;

  // Operand addresses as lane constants plus immediates (the XOR swizzle
  // reduces to additions here):
  //  row reads, token 32 st + ln, chunk 2 ks + g:  ak_off[ks] + 4096 st;
  //  transpose reads, token 32 st + 16 s + 8 hh + L (L = 4 (tq >> 1) + tk),
  //  features from 32 nt + 16 (tq & 1) + 4 ta:
  //      tr_off[nt ^ hh] + 4096 st + 2048 s + 1024 hh.
  int ak_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ak_off[ks] = ln * ROW + 16 * ((2 * ks + g) ^ swz(ln));
  int tr_off[2];
  {
    const int tl = 4 * (tq >> 1) + tk;
    const int t1 = (tl >> 1) & 1, t2 = (tl >> 2) & 1;
    const int low = (2 * (tq & 1) + (ta >> 1)) ^ (2 * t2 + t1);
#pragma unroll
    for (int x = 0; x < 2; ++x) tr_off[x] = tl * ROW + 16 * (4 * (x ^ t1) + low) + 8 * (ta & 1);
  }

  // one stage: compute on buffer cur while the next stage loads into nxt
  auto stage = [&](int64_t t0, const unsigned char* cur, unsigned char* nxt) {
    // this stage has landed (each wave waits for its own loads, the barrier
    // for everyone's, and makes the eta zeros visible); every wave is past
    // the previous stage, so its buffer can take the next one
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (t0 + TT < t_end) dma_stage(t0 + TT, nxt);

    const unsigned char* kb = cur + OFF_K;
    const unsigned char* vb = cur + OFF_V;
    const float* eb = reinterpret_cast<const float*>(cur + OFF_E);

#pragma unroll 1
    for (int st = 0; st < SUB; ++st) {
      // projections of 32 tokens x this wave's 32 hidden units; output
      // lane = hidden unit, register r = token 8 (r / 4) + 4 g + r % 4
      f32x16_t c1, c3, cg;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c1[r] = 0.f;
        c3[r] = 0.f;
        cg[r] = 0.f;
      }
      // (every LDS read of a phase is issued before its first use, so one
      // wait covers the group instead of one exposed latency per read)
      bf16x8_t ak[KS], av[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = ak_off[ks] + 4096 * st;
        ak[ks] = *reinterpret_cast<const bf16x8_t*>(kb + off);
        av[ks] = *reinterpret_cast<const bf16x8_t*>(vb + off);
      }
      // eta of this lane's 16 tokens (operand slot i of half s <-> token
      // 16 s + 8 (i / 4) + 4 g + i % 4); with PM all rates are read per half
      // below
      f32x4_t eta4[PM ? 1 : 4];
      if constexpr (!PM) {
#pragma unroll
        for (int q = 0; q < 4; ++q) eta4[q] = *reinterpret_cast<const f32x4_t*>(eb + 32 * st + 8 * q + 4 * g);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        c1 = mfma32(ak[ks], w1b[ks], c1);
        c3 = mfma32(ak[ks], w3b[ks], c3);
        cg = mfma32(av[ks], w2b[ks], cg);
        if constexpr (SPLIT) {
          c1 = mfma32(ak[ks], w1l[ks], c1);
          c3 = mfma32(ak[ks], w3l[ks], c3);
          cg = mfma32(av[ks], w2l[ks], cg);
        }
      }
      // SwiGLU forward and backward, one 16-token half at a time (operand
      // slot i <-> token 16 s + 8 (i / 4) + 4 g + i % 4 of the sub-tile).
      // With z = -log2(e) h1, s = sigmoid(h1) = 1 / (1 + 2^z), a = silu(h1),
      // g = a h3, e = -eta and dg = e dG':
      //   a' = z s = -log2(e) a,  g' = a' h3,  dh3' = dg a',
      //   dh1' = dg (g' + s t'),  t' = -log2(e) h3 - g'  (= -log2(e) dh1, since
      //   dh1 = dg h3 s (1 + h1 (1 - s)) = dg (g + s (h3 - g))),
      // and the contraction with v takes e g'.
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // with PM: rates of W2 (e), W1 (x1) and W3 (x3) for the half's slots,
        // read here (registers are short before the projections)
        f32x4_t e0, e1, x10, x11, x30, x31;
        if constexpr (!PM) {
          e0 = eta4[2 * s];
          e1 = eta4[2 * s + 1];
        } else {
          e0 = *reinterpret_cast<const f32x4_t*>(eb + TT + 32 * st + 16 * s + 4 * g);
          e1 = *reinterpret_cast<const f32x4_t*>(eb + TT + 32 * st + 16 * s + 8 + 4 * g);
          x10 = *reinterpret_cast<const f32x4_t*>(eb + 32 * st + 16 * s + 4 * g);
          x11 = *reinterpret_cast<const f32x4_t*>(eb + 32 * st + 16 * s + 8 + 4 * g);
          x30 = *reinterpret_cast<const f32x4_t*>(eb + 2 * TT + 32 * st + 16 * s + 4 * g);
          x31 = *reinterpret_cast<const f32x4_t*>(eb + 2 * TT + 32 * st + 16 * s + 8 + 4 * g);
        }
        // token-side operands: slots 0-3 <-> tokens 16 s + 4 g + k',
        // slots 4-7 <-> tokens 16 s + 8 + 4 g + k' (read before the
        // elementwise step, which hides their latency)
        bf16x8_t bk[NT], bv[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          s16x4_t kt[2], vt[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int off = tr_off[nt ^ hh] + 4096 * st + 2048 * s + 1024 * hh;
            kt[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(kb + off));
            vt[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(vb + off));
          }
          bk[nt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(kt[0], kt[1], 0, 1, 2, 3, 4, 5, 6, 7));
          bv[nt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vt[0], vt[1], 0, 1, 2, 3, 4, 5, 6, 7));
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
          aW1[nt] = mfma32(pd1, bk[nt], aW1[nt]);
          aW3[nt] = mfma32(pd3, bk[nt], aW3[nt]);
          aW2[nt] = mfma32(bv[nt], pg, aW2[nt]);
          if constexpr (SPLIT) {
            aW1[nt] = mfma32(l1, bk[nt], aW1[nt]);
            aW3[nt] = mfma32(l3, bk[nt], aW3[nt]);
            aW2[nt] = mfma32(bv[nt], lg, aW2[nt]);
          }
        }
      }
    }
  };

  // stages alternate between the two buffers (unrolled by two, so every
  // access names its buffer statically)
  if (t_begin < t_end) dma_stage(t_begin, buf0);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * TT) {
    stage(t0, buf0, buf1);
    if (t0 + TT < t_end) stage(t0 + TT, buf1, buf0);
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

bool grad_d64_shape_ok(int d, int h) {
  return d == D && h % kHidPerWG == 0 && h >= kHidPerWG && h <= 1024;
}

hipError_t launch_grad_d64(const GradArgs& a, bool split, hipStream_t s) {
  if (a.d != D) return hipErrorInvalidValue;
  const int hsl = a.h / kHidPerWG;
  const int nbase = a.S * a.P;
  const int blocks = ((nbase + 7) / 8) * 8 * hsl;
  const bool pm = a.eta_mat != 0;
  if (split && pm) {
    hipLaunchKernelGGL((k_grad_d64<true, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else if (split) {
    hipLaunchKernelGGL((k_grad_d64<false, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else if (pm) {
    hipLaunchKernelGGL((k_grad_d64<true, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else {
    hipLaunchKernelGGL((k_grad_d64<false, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  }
  return hipGetLastError();
}

}  // namespace lact

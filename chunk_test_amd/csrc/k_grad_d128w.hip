// Chunk gradient of the LaCT layer for d = 128 on bf16 MFMA (gfx950), bf16
// or near-fp32 "split" products, two wavefronts per SIMD.
//
// For one (pair, token split, 128-unit hidden slice) a workgroup of eight
// wavefronts (16 hidden units each) sums, over the split's tokens i,
//   dW1 += dh1_i k_i^T,  dW3 += dh3_i k_i^T,  dW2 += v_i (-eta_i g_i)^T
// with h1 = W1 k, h3 = W3 k, a = silu(h1), g = a * h3, dg = -eta_i W2^T v_i,
// dh3 = dg * a, dh1 = dg * h3 * silu'(h1): the gradient of
// -sum_i eta_i <f_W(k_i), v_i> for f_W(x) = W2 (silu(W1 x) * (W3 x))
// ("LaCT: Large Chunk Test-Time Training" review, section "Local attention
// and nonlinear memory work together").  The chunk is a set, so the sum is
// split over tokens across workgroups and reduced afterwards in fixed order.
//
// Why 16 hidden units per wavefront: with 32 (the d = 64 geometry) the dW
// tiles take 192 fp32 per lane and the kernel runs one wavefront per SIMD,
// which leaves nothing to issue while a wavefront waits on its own LDS reads
// and product chains.  Here every product is a 16x16x32 MFMA and a wavefront
// owns 16 hidden units: 96 fp32 of dW tiles per lane, about 250 registers in
// all, so two wavefronts share each SIMD.  A workgroup of eight wavefronts
// (128 hidden units, one per CU) shares each key / value stage among all
// eight: half the LDS-DMA writes and L2 reads of two four-wavefront
// workgroups, and 1-1.5 % faster in the LM and video scans.
//
// Staging as in the other gradient kernels: keys, values and eta of the next
// 64-token stage move from HBM straight into LDS (global_load_lds, no
// registers, double-buffered) while the current stage computes; one barrier
// per stage; rows of 256 bytes with their 16-byte chunks XOR-swizzled.
//
// Per 32-token sub-tile and wavefront (16x16x32 MFMA layouts: A lane l =
// row l % 16 with k = 8 (l / 16) .. + 7; B lane l = column l % 16, same k;
// D lane l = column l % 16, rows 4 (l / 16) .. + 3):
//   H1, H3 = K W^T and dG' = V W2 for two 16-token tiles (A = key / value
//   rows from LDS, B = W in registers): lane l then holds hidden unit
//   n0 + l % 16 for tokens 4 q + r and 16 + 4 q + r (q = l / 16, r < 4);
//   the SwiGLU step turns these eight values into eight bf16 operand slots,
//   slot 4 t + r <-> token 16 t + 4 q + r, which is directly the hidden-side
//   operand of the contractions; the token-side operands (K, V with tokens
//   along k in the same slot order) come from LDS transpose reads.
//
// Split products: keys and values are exact bf16 inputs, so only the other
// operand of every product is split, x = x_hi + x_lo (both bf16), and each
// product is two MFMAs (~16 significant bits per operand).  The lo parts of
// W1 and W3 sit in LDS (read per k-step), W2's in registers, and the stages
// shrink to 32 tokens (96.25 KiB of LDS per workgroup).
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_t;

constexpr int D = 128;
constexpr int kWaves = 8;                      // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kHidPerWave = 16;
constexpr int kHidPerWG = 16 * kWaves;
constexpr int KS = D / 32;         // k-steps of the projections
constexpr int NT = D / 16;         // 16-wide d tiles of the contractions
constexpr int ROW = 2 * D;         // bytes per token row (sixteen 16-byte chunks)

template <bool SPLIT, bool PM>
struct Geo {
  static constexpr int TT = SPLIT ? 32 : 64;   // tokens per LDS stage
  static constexpr int SUB = TT / 32;          // 32-token sub-tiles per stage
  static constexpr int TILE = TT * ROW;        // one stage of K (or V)
  static constexpr int OFF_K = 0;              // K[2]
  static constexpr int OFF_V = 2 * TILE;       // V[2]
  static constexpr int NE = PM ? 3 : 1;        // rows of rates per stage (W1, W2, W3 with PM)
  static constexpr int OFF_E = 4 * TILE;       // eta[2][NE][TT]
  static constexpr int OFF_WLO = OFF_E + 2 * NE * TT * 4;  // W1_lo, W3_lo operands [matrix][wave][ks][lane]
  static constexpr int WLO_BYTES = SPLIT ? 2 * kWaves * KS * 64 * 16 : 0;
  static constexpr int LDS = OFF_WLO + WLO_BYTES;
};

// W1 enters pre-scaled by -log2(e) (sigmoid(h1) = 1 / (1 + 2^z), z = -log2(e) h1);
// G, dH3 and dH1 then carry that factor, removed at the end (times -ln 2).
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

// XOR swizzle of the 16-byte chunks of token row r (r_i: bit i of r),
//     swz(r) = 2 (r mod 8) + r3.
// A row is one 256-byte bank window (64 four-byte banks).  The projections'
// 16-byte row reads are served 16 lanes (16 consecutive rows, one logical
// chunk) at a time: swz is one-to-one on the low four row bits, so the 16
// rows land in 16 different chunk positions.  The contractions' 8-byte
// transpose reads are checked 32 lanes at a time: eight consecutive rows
// (an aligned group, r3 fixed) and an aligned pair of chunks 2 nt, 2 nt + 1;
// bits 1..3 of swz take eight different values on those rows and bit 0
// keeps the pair's two chunks apart, so the 16 pieces fill the window.
__device__ __forceinline__ int swz(int r) { return 2 * (r & 7) + ((r >> 3) & 1); }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// lo bf16 part of a float given its hi part (the rounded remainder)
__device__ __forceinline__ __bf16 lo_bf16(float x, __bf16 hi) {
  return static_cast<__bf16>(x - static_cast<float>(hi));
}

// PM: a learning rate per token and matrix (rows of rates for W1, W2, W3,
// a.eta_mat elements apart); otherwise one rate per token.
template <bool SPLIT, bool PM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_grad_d128w(GradArgs a, int hsl, int nbase) {
  using G = Geo<SPLIT, PM>;
  constexpr int TT = G::TT, TILE = G::TILE, OFF_K = G::OFF_K, OFF_V = G::OFF_V, OFF_E = G::OFF_E;
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
  const int q = lane >> 4;    // operands: k-slots 8 q .. 8 q + 7; outputs: rows 4 q ..
  const int l16 = lane & 15;  // operands: row / column
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int n0 = hs * kHidPerWG + wave * kHidPerWave;  // this wave's hidden units

  // ---- B operands of the projections: lane holds hidden unit n0 + l16,
  // features 32 ks + 8 q .. +7 (with split products the lo parts of W1 and
  // W3 go to LDS, slot [matrix][wave][ks][lane], and W2's to registers)
  bf16x8_t w1b[KS], w3b[KS], w2b[KS];
  bf16x8_t w2l[SPLIT ? KS : 1];
  {
    const float* W1 = a.W1 + pair * hd + static_cast<int64_t>(n0 + l16) * D;
    const float* W3 = a.W3 + pair * hd + static_cast<int64_t>(n0 + l16) * D;
    const float* W2 = a.W2 + pair * hd + n0 + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t l1, l3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dd = 32 * ks + 8 * q + i;
        const float x1 = kNegLog2e * W1[dd], x3 = W3[dd], x2 = W2[static_cast<int64_t>(dd) * h];
        w1b[ks][i] = static_cast<__bf16>(x1);
        w3b[ks][i] = static_cast<__bf16>(x3);
        w2b[ks][i] = static_cast<__bf16>(x2);
        if constexpr (SPLIT) {
          l1[i] = lo_bf16(x1, w1b[ks][i]);
          l3[i] = lo_bf16(x3, w3b[ks][i]);
          w2l[ks][i] = lo_bf16(x2, w2b[ks][i]);
        }
      }
      if constexpr (SPLIT) {
        *reinterpret_cast<bf16x8_t*>(lds + G::OFF_WLO + (((0 * kWaves + wave) * KS + ks) * 64 + lane) * 16) = l1;
        *reinterpret_cast<bf16x8_t*>(lds + G::OFF_WLO + (((1 * kWaves + wave) * KS + ks) * 64 + lane) * 16) = l3;
      }
    }
  }

  // dW tiles: aW1[nt], aW3[nt] = hidden rows n0 + 4 q .. +3, feature column
  // 16 nt + l16; aW2[nt] = feature rows 16 nt + 4 q .. +3, hidden column n0 + l16
  f32x4_t aW1[NT], aW3[NT], aW2[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
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
  // moving pieces wv, wv + kWaves, ...; lane l of a piece lands at its byte
  // 16 l: row 4 piece + l / 16, physical chunk l % 16.  Lanes 0 .. TT - 1 of
  // wave m move the stage's row m of rates (one row, or three with PM).  Rows
  // past the end re-read the split's last token (finite values); their eta is
  // written as 0, so they add nothing.
  auto dma_stage = [&](int64_t t0, int b) {
    // (the lane-derived offsets are recomputed per stage: a few
    // instructions, where keeping them live would take registers)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int k = 0; k < TT / (4 * kWaves); ++k) {
      const int piece = kWaves * k + wv;
      const int r = 4 * piece + (lane >> 4);
      const int cl = (lane & 15) ^ swz(r);
      const int tok = static_cast<int>(t0) + r;
      const int tc = tok < t_last ? tok : t_last;
      const unsigned off = static_cast<unsigned>(tc) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Kg + off), (lds_ptr_t)(lds + OFF_K + b * TILE + 1024 * piece), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Vg + off), (lds_ptr_t)(lds + OFF_V + b * TILE + 1024 * piece), 16, 0, 0);
    }
    if (wv < G::NE && lane < TT) {
      const int tok = static_cast<int>(t0) + lane;
      unsigned char* dst = lds + OFF_E + (b * G::NE + wv) * TT * 4;
      if (tok <= t_last) {
        const float* src = etag + (PM ? wv * a.eta_mat : 0) + static_cast<unsigned>(tok);
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)dst, 4, 0, 0);
      } else {
        *reinterpret_cast<float*>(dst + 4 * lane) = 0.f;
      }
    }
  };

  // Operand addresses inside a stage tile, as lane constants plus immediates:
  //  row reads (projections), token 32 st + 16 t + l16, logical chunk
  //  4 ks + q:  ak_off[ks] + 8192 st + 4096 t  (swz of the row is swz(l16));
  //  transpose reads (contractions): within each 16-lane group q, lane
  //  16 q + 4 k' + a' addresses token 32 st + 16 hh + 4 q + k' and features
  //  16 nt + 4 a' .. +3 (logical chunk 2 nt + a' / 2, half a' % 2); after the
  //  read lane 16 q + j holds feature 16 nt + j of the four tokens
  //  32 st + 16 hh + 4 q .. +3, i.e. operand slots 4 hh .. 4 hh + 3:
  //      tr_off[nt] + 8192 st + 4096 hh.
  int ak_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ak_off[ks] = l16 * ROW + 16 * ((4 * ks + q) ^ swz(l16));
  int tr_off[NT];
  {
    const int kp = (lane >> 2) & 3, ap = lane & 3;
    const int tl = 4 * q + kp;  // row inside the 16-token tile
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      tr_off[nt] = tl * ROW + 16 * ((2 * nt + (ap >> 1)) ^ swz(tl)) + 8 * (ap & 1);
  }

  if (t_begin < t_end) dma_stage(t_begin, 0);
  int b = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TT, b ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this stage has landed
    __syncthreads();                      // every wave's loads (and eta zeros) visible
    if (t0 + TT < t_end) dma_stage(t0 + TT, b ^ 1);

    const unsigned char* kb = lds + OFF_K + b * TILE;
    const unsigned char* vb = lds + OFF_V + b * TILE;
    // rates of this stage (with PM rows for W1, W2, W3)
    const float* eb = reinterpret_cast<const float*>(lds + OFF_E + b * G::NE * TT * 4);

#pragma unroll
    for (int st = 0; st < G::SUB; ++st) {
      // projections of 32 tokens (two 16-token tiles) x this wave's 16 hidden units
      f32x4_t c1[2], c3[2], cg[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          c1[t][r] = 0.f;
          c3[t][r] = 0.f;
          cg[t][r] = 0.f;
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8_t ak[2], av[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int off = ak_off[ks] + 8192 * st + 4096 * t;
          ak[t] = *reinterpret_cast<const bf16x8_t*>(kb + off);
          av[t] = *reinterpret_cast<const bf16x8_t*>(vb + off);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          c1[t] = mfma16(ak[t], w1b[ks], c1[t]);
          c3[t] = mfma16(ak[t], w3b[ks], c3[t]);
          cg[t] = mfma16(av[t], w2b[ks], cg[t]);
        }
        if constexpr (SPLIT) {
          const bf16x8_t l1 = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_WLO + (((0 * kWaves + wave) * KS + ks) * 64 + lane) * 16);
          const bf16x8_t l3 = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_WLO + (((1 * kWaves + wave) * KS + ks) * 64 + lane) * 16);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            c1[t] = mfma16(ak[t], l1, c1[t]);
            c3[t] = mfma16(ak[t], l3, c3[t]);
            cg[t] = mfma16(av[t], w2l[ks], cg[t]);
          }
        }
      }
      // rates of this lane's eight tokens 32 st + 16 t + 4 q + r: the one of W2
      // (g), and with PM those of W1 (x1) and W3 (x3)
      const float* e2b = eb + (PM ? TT : 0);
      const f32x4_t e0 = *reinterpret_cast<const f32x4_t*>(e2b + 32 * st + 4 * q);
      const f32x4_t e1 = *reinterpret_cast<const f32x4_t*>(e2b + 32 * st + 16 + 4 * q);
      f32x4_t x10, x11, x30, x31;
      if constexpr (PM) {
        x10 = *reinterpret_cast<const f32x4_t*>(eb + 32 * st + 4 * q);
        x11 = *reinterpret_cast<const f32x4_t*>(eb + 32 * st + 16 + 4 * q);
        x30 = *reinterpret_cast<const f32x4_t*>(eb + 2 * TT + 32 * st + 4 * q);
        x31 = *reinterpret_cast<const f32x4_t*>(eb + 2 * TT + 32 * st + 16 + 4 * q);
      }
      // SwiGLU forward and backward on the eight values.  With
      // z = -log2(e) h1, s = sigmoid(h1) = 1 / (1 + 2^z), a = silu(h1),
      // g = a h3, e = -eta and dg = e dG':
      //   a' = z s = -log2(e) a,  g' = a' h3,  dh3' = dg a',
      //   dh1' = dg (g' + s t'),  t' = -log2(e) h3 - g'  (= -log2(e) dh1, since
      //   dh1 = dg h3 s (1 + h1 (1 - s)) = dg (g + s (h3 - g))),
      // and the contraction with v takes e g'.
      bf16x8_t pg, pd1, pd3, lg, ld1, ld3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = i >> 2, r = i & 3;
        const float ne = -((t == 0) ? e0[r] : e1[r]);
        const float z = c1[t][r], h3 = c3[t][r];
        // dG of the losses W1 and W3 follow (the same one without PM)
        const float dg = ne * cg[t][r];
        const float dg1 = PM ? -((t == 0) ? x10[r] : x11[r]) * cg[t][r] : dg;
        const float dg3 = PM ? -((t == 0) ? x30[r] : x31[r]) * cg[t][r] : dg;
        const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z));
        const float act = z * sg;
        const float gs = act * h3;
        const float tt = fmaf(h3, kNegLog2e, -gs);
        const float vg = ne * gs, v3 = dg3 * act, v1 = dg1 * fmaf(sg, tt, gs);
        pg[i] = static_cast<__bf16>(vg);
        pd3[i] = static_cast<__bf16>(v3);
        pd1[i] = static_cast<__bf16>(v1);
        if constexpr (SPLIT) {
          lg[i] = lo_bf16(vg, pg[i]);
          ld3[i] = lo_bf16(v3, pd3[i]);
          ld1[i] = lo_bf16(v1, pd1[i]);
        }
      }
      // contractions over the 32 tokens (k), one 16-feature tile at a time
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s16x4_t kt[2], vt[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int off = tr_off[nt] + 8192 * st + 4096 * hh;
          kt[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(kb + off));
          vt[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(vb + off));
        }
        const bf16x8_t bk = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(kt[0], kt[1], 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vt[0], vt[1], 0, 1, 2, 3, 4, 5, 6, 7));
        aW1[nt] = mfma16(pd1, bk, aW1[nt]);
        aW3[nt] = mfma16(pd3, bk, aW3[nt]);
        aW2[nt] = mfma16(bv, pg, aW2[nt]);
        if constexpr (SPLIT) {
          aW1[nt] = mfma16(ld1, bk, aW1[nt]);
          aW3[nt] = mfma16(ld3, bk, aW3[nt]);
          aW2[nt] = mfma16(bv, lg, aW2[nt]);
        }
      }
    }
  }

  // ---- partial sums of this split: [W1 block h x D | W2 block D x h | W3 block h x D]
  float* out = a.partials + (static_cast<int64_t>(pair) * a.S + split) * 3 * hd;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q + r;
      out[static_cast<int64_t>(n0 + row) * D + 16 * nt + l16] = kNegLn2 * aW1[nt][r];
      out[2 * hd + static_cast<int64_t>(n0 + row) * D + 16 * nt + l16] = kNegLn2 * aW3[nt][r];
      out[hd + static_cast<int64_t>(16 * nt + row) * h + n0 + l16] = kNegLn2 * aW2[nt][r];
    }
  }
}

}  // namespace

bool d128_mfma_shape_ok(int d, int h) { return d == D && h % 128 == 0 && h >= 128 && h <= 1024; }

bool grad_d128w_shape_ok(int d, int h) {
  return d == D && h % kHidPerWG == 0 && h >= kHidPerWG && h <= 1024;
}

int grad_d128w_stage_tokens(bool split) { return split ? Geo<true, false>::TT : Geo<false, false>::TT; }

int grad_d128w_hidden_per_workgroup() { return kHidPerWG; }

int grad_d128w_workgroups_per_cu() { return 8 / kWaves; }

hipError_t launch_grad_d128w(const GradArgs& a, bool split, hipStream_t s) {
  if (a.d != D) return hipErrorInvalidValue;
  const int hsl = a.h / kHidPerWG;
  const int nbase = a.S * a.P;
  const int blocks = ((nbase + 7) / 8) * 8 * hsl;
  const bool pm = a.eta_mat != 0;
  if (split && pm) {
    hipLaunchKernelGGL((k_grad_d128w<true, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else if (split) {
    hipLaunchKernelGGL((k_grad_d128w<true, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else if (pm) {
    hipLaunchKernelGGL((k_grad_d128w<false, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else {
    hipLaunchKernelGGL((k_grad_d128w<false, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  }
  return hipGetLastError();
}

}  // namespace lact

// Chunk gradient of the LaCT layer on bf16 MFMA (gfx950), d = 64 or 128.
//
// For one (pair, token split, 128-unit hidden slice) a workgroup of four
// wavefronts sums, over the split's tokens i,
//   dW1 += dh1_i k_i^T,  dW3 += dh3_i k_i^T,  dW2 += u_i g_i^T,   u_i = -eta_i v_i
// with h1 = W1 k, h3 = W3 k, a = silu(h1), g = a * h3, dg = W2^T u,
// dh3 = dg * a, dh1 = dg * h3 * silu'(h1): the gradient of
// -sum_i eta_i <f_W(k_i), v_i> for f_W(x) = W2 (silu(W1 x) * (W3 x))
// ("LaCT: Large Chunk Test-Time Training" review, section "Local attention
// and nonlinear memory work together").  The chunk is a set, so the sum is
// split over tokens across workgroups and reduced afterwards in fixed order.
//
// Dataflow per 32-token sub-tile and wavefront (32 hidden units each):
//   MFMA 32x32x16 bf16:  H1, H3 = K W^T (A = key rows from LDS, B = W in
//   registers), dG = U W2 (A = u rows from LDS).  The fp32 results stay in
//   registers in the MFMA output layout (lane = hidden unit, 16 tokens per
//   lane); the SwiGLU forward/backward runs there and is packed to bf16,
//   which is directly the hidden-side operand of the token contractions.
//   The token-side operands (K and U with tokens along the reduction axis)
//   are written once per stage into a transposed, bank-swizzled LDS layout.
//   The three dW tiles (96 fp32 per lane at d=64) stay in registers for
//   the whole split.
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

constexpr int kThreads = 256;
constexpr int kHidPerWave = 32;
// The key projection through W1 is computed pre-scaled by -log2(e), so the
// sigmoid needs no extra multiply: sigmoid(h1) = 1 / (1 + 2^(-log2(e) h1)).
// G, dH3 and dH1 then carry the same factor, removed once from the three
// sums at the end (times -ln 2).
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;
constexpr int kHidPerWG = 128;

template <int D>
struct Geo {
  static constexpr int TT = 8192 / D;         // tokens per LDS stage
  static constexpr int NS16 = TT / 16;        // 16-token groups per stage
  static constexpr int SUB = TT / 32;         // 32-token sub-tiles per stage
  static constexpr int KS = D / 16;           // k-steps over d (K = 16 per MFMA)
  static constexpr int NT = D / 32;           // 32-wide tiles over d
  static constexpr int NAT_ROW = 2 * D + 16;  // bytes per token row, padded
  static constexpr int NAT_BYTES = TT * NAT_ROW;
  static constexpr int TR_GROUP = 34 * D;     // bytes per 16-token group, transposed
  static constexpr int TR_BYTES = NS16 * TR_GROUP;
  static constexpr int OFF_KN = 0;
  static constexpr int OFF_UN = NAT_BYTES;
  static constexpr int OFF_KT = 2 * NAT_BYTES;
  static constexpr int OFF_UT = 2 * NAT_BYTES + TR_BYTES;
  static constexpr int LDS = 2 * NAT_BYTES + 2 * TR_BYTES;
  // d = 64: two workgroups per CU (two wavefronts per SIMD, at most 256
  // registers each, so the MFMAs write VGPRs and one wave's SwiGLU math
  // overlaps the other's MFMAs).  d = 128 needs more accumulator registers:
  // one wavefront per SIMD, with the next stage prefetched into registers.
  static constexpr int WAVES_PER_SIMD = (D == 64) ? 2 : 1;
  static constexpr bool PREFETCH = (D != 64);
};

// Byte offset of the 16-byte half `half` of row (s16, d) in a transposed
// tile: 16 tokens of one feature d, in the order the MFMA k-slots use.
// Every 8 rows are shifted by 16 bytes and the halves swap on bit 2 of d,
// which keeps both the 8-byte writes and the 16-byte reads free of bank
// conflicts.
template <int D>
__device__ __forceinline__ int tr_off(int s16, int d, int half) {
  return s16 * Geo<D>::TR_GROUP + d * 32 + (d >> 3) * 16 + 16 * (half ^ ((d >> 2) & 1));
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(unsigned, v);
}

template <int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Geo<D>::WAVES_PER_SIMD, Geo<D>::WAVES_PER_SIMD)))
void k_grad_mfma(GradArgs a, int hsl, int nbase) {
  using G = Geo<D>;
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
  const int g = lane >> 5;   // lane group: k-slots 8g..8g+7 of an MFMA operand
  const int ln = lane & 31;  // row / column index inside a 32x32 tile
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int n0 = hs * kHidPerWG + wave * kHidPerWave;  // this wave's hidden units

  // ---- fast-weight operands (bf16, registers) for the key/value products
  bf16x8_t w1b[G::KS], w3b[G::KS], w2b[G::KS];
  {
    const float* W1 = a.W1 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W3 = a.W3 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W2 = a.W2 + pair * hd + n0 + ln;
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dd = 16 * ks + 8 * g + i;
        w1b[ks][i] = static_cast<__bf16>(kNegLog2e * W1[dd]);
        w3b[ks][i] = static_cast<__bf16>(W3[dd]);
        w2b[ks][i] = static_cast<__bf16>(W2[static_cast<int64_t>(dd) * h]);
      }
    }
  }

  f32x16_t aW1[G::NT], aW3[G::NT], aW2[G::NT];
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      aW1[t][r] = 0.f;
      aW3[t][r] = 0.f;
      aW2[t][r] = 0.f;
    }
  }

  // ---- loader mapping: each thread moves 4 consecutive tokens x 8 features
  const int c_lo = tid & 7;
  const int sub = (tid >> 3) & 1;
  int hf, s16, c;
  if constexpr (D == 64) {
    hf = (tid >> 4) & 1;
    s16 = tid >> 5;
    c = c_lo;
  } else {
    hf = (tid >> 5) & 1;
    s16 = tid >> 6;
    c = c_lo + 8 * ((tid >> 4) & 1);
  }
  const int qd = 2 * sub + hf;
  const int t_first = 16 * s16 + 4 * qd;  // first of this thread's tokens in a stage

  const int64_t t_begin = static_cast<int64_t>(split) * a.tps;
  const int64_t t_end = min(a.n, t_begin + a.tps);
  const int64_t kv_base = static_cast<int64_t>(pair) * a.kv_stride;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + kv_base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + kv_base;
  const float* etag = a.eta + static_cast<int64_t>(pair) * a.eta_stride;

  u32x4_t kr[4], vr[4];
  float er[4];
  // Tokens past the end of the split re-read the split's last token with
  // eta = 0: u = 0 and dg = 0 then, so they add nothing to any of the three
  // sums (finite inputs), and the loads need no branches.
  // (token offsets inside one pair's rows fit 32 bits: the host routes
  // longer sequences elsewhere)
  const int t_last = static_cast<int>(t_end - 1);
  auto load_stage = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tok = static_cast<int>(t0) + t_first + k;
      const int tc = tok < t_last ? tok : t_last;
      const unsigned off = static_cast<unsigned>(tc) * D + 8 * c;
      kr[k] = *reinterpret_cast<const u32x4_t*>(Kg + off);
      vr[k] = *reinterpret_cast<const u32x4_t*>(Vg + off);
      const float ev = etag[static_cast<unsigned>(tc)];
      er[k] = tok <= t_last ? ev : 0.f;
    }
  };

  auto store_stage = [&]() {
    u32x4_t ur[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float ne = -er[k];
#pragma unroll
      for (int w = 0; w < 4; ++w) ur[k][w] = pack_bf16x2(ne * bf_lo(vr[k][w]), ne * bf_hi(vr[k][w]));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = (t_first + k) * G::NAT_ROW + c * 16;
      *reinterpret_cast<u32x4_t*>(lds + G::OFF_KN + row) = kr[k];
      *reinterpret_cast<u32x4_t*>(lds + G::OFF_UN + row) = ur[k];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int dd = 8 * c + j;
      const int w = j >> 1;
      // (low halves of tokens 0,1 | high halves) -> one byte permute each
      const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x2_t pk, pu;
      pk[0] = __builtin_amdgcn_perm(kr[1][w], kr[0][w], sel);
      pk[1] = __builtin_amdgcn_perm(kr[3][w], kr[2][w], sel);
      pu[0] = __builtin_amdgcn_perm(ur[1][w], ur[0][w], sel);
      pu[1] = __builtin_amdgcn_perm(ur[3][w], ur[2][w], sel);
      const int off = tr_off<D>(s16, dd, hf) + 8 * sub;
      *reinterpret_cast<u32x2_t*>(lds + G::OFF_KT + off) = pk;
      *reinterpret_cast<u32x2_t*>(lds + G::OFF_UT + off) = pu;
    }
  };

  if (G::PREFETCH && t_begin < t_end) load_stage(t_begin);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += G::TT) {
    if (!G::PREFETCH) load_stage(t0);
    __syncthreads();
    store_stage();
    __syncthreads();
    if (G::PREFETCH && t0 + G::TT < t_end) load_stage(t0 + G::TT);

#pragma unroll 1
    for (int st = 0; st < G::SUB; ++st) {
      // key / value products for 32 tokens x this wave's 32 hidden units
      f32x16_t c1, c3, cg;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c1[r] = 0.f;
        c3[r] = 0.f;
        cg[r] = 0.f;
      }
      const unsigned char* krow = lds + G::OFF_KN + (32 * st + ln) * G::NAT_ROW + 16 * g;
      const unsigned char* urow = lds + G::OFF_UN + (32 * st + ln) * G::NAT_ROW + 16 * g;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(krow + 32 * ks);
        const bf16x8_t au = *reinterpret_cast<const bf16x8_t*>(urow + 32 * ks);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, w1b[ks], c1, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, w3b[ks], c3, 0, 0, 0);
        cg = __builtin_amdgcn_mfma_f32_32x32x16_bf16(au, w2b[ks], cg, 0, 0, 0);
      }
      // SwiGLU forward and backward, then the token contractions, one k-step
      // (16 tokens) at a time.  With z = -log2(e) h1 (from the scaled W1),
      // s = sigmoid(h1) = 1 / (1 + 2^z) and a = silu(h1), g = a h3:
      //   a' = z s = -log2(e) a,   g' = a' h3 = -log2(e) g,   dh3' = dg a',
      //   dh1 = dg h3 s (1 + h1 (1 - s)) = dg (g + s (h3 - g)),
      //   dh1' = dg (g' + s t'),  t' = -log2(e) h3 - g'   (= -log2(e) dh1),
      // so all three carry -log2(e), removed once at the end (times -ln 2).
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t pg, pd1, pd3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * s + i;
          const float z = c1[r], h3 = c3[r], dg = cg[r];
          const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z));
          const float act = z * sg;
          const float gs = act * h3;
          pg[i] = static_cast<__bf16>(gs);
          pd3[i] = static_cast<__bf16>(dg * act);
          const float t = fmaf(h3, kNegLog2e, -gs);
          pd1[i] = static_cast<__bf16>(dg * fmaf(sg, t, gs));
        }
        const int grp = 2 * st + s;
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt) {
          const int dd = 32 * nt + ln;
          const int off = tr_off<D>(grp, dd, g);
          const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_KT + off);
          const bf16x8_t bu = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_UT + off);
          aW1[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pd1, bk, aW1[nt], 0, 0, 0);
          aW3[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pd3, bk, aW3[nt], 0, 0, 0);
          aW2[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bu, pg, aW2[nt], 0, 0, 0);
        }
      }
    }
  }

  // ---- partial sums of this split: [W1 block h x D | W2 block D x h | W3 block h x D]
  float* out = a.partials + (static_cast<int64_t>(pair) * a.S + split) * 3 * hd;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * g + (r & 3);
      out[static_cast<int64_t>(n0 + row) * D + 32 * nt + ln] = kNegLn2 * aW1[nt][r];
      out[2 * hd + static_cast<int64_t>(n0 + row) * D + 32 * nt + ln] = kNegLn2 * aW3[nt][r];
      out[hd + static_cast<int64_t>(32 * nt + row) * h + n0 + ln] = kNegLn2 * aW2[nt][r];
    }
  }
}

template <int D>
hipError_t launch_d(const GradArgs& a, hipStream_t s) {
  const int hsl = a.h / kHidPerWG;
  const int nbase = a.S * a.P;
  const int blocks = ((nbase + 7) / 8) * 8 * hsl;
  hipLaunchKernelGGL((k_grad_mfma<D>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  return hipGetLastError();
}

}  // namespace

bool grad_mfma_shape_ok(int d, int h) {
  return (d == 64 || d == 128) && h % kHidPerWG == 0 && h >= kHidPerWG && h <= 1024;
}

int grad_mfma_stage_tokens(int d) { return 8192 / d; }

int grad_mfma_wgs_per_cu(int d) { return d == 64 ? Geo<64>::WAVES_PER_SIMD : Geo<128>::WAVES_PER_SIMD; }

hipError_t launch_grad_mfma(const GradArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lact

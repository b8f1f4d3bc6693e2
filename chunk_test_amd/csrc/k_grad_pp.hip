// Chunk gradient of the LaCT layer on bf16 MFMA (gfx950), d = 64:
// "ping-pong" variant with two wavefront groups per workgroup.
//
// Same arithmetic and LDS operand layouts as k_grad_mfma.hip (see there for
// the dataflow of one 32-token sub-tile): per token split and 128-unit hidden
// slice it sums dW1 += dh1 k^T, dW3 += dh3 k^T, dW2 += u g^T over the tokens,
// the gradient of -sum_i eta_i <f_W(k_i), v_i> ("LaCT: Large Chunk
// Test-Time Training" review, section "Local attention and nonlinear memory
// work together").
//
// Scheduling: a workgroup has 8 wavefronts, two per SIMD.  Wavefronts 0-3
// (group A) and 4-7 (group B) each own 32 hidden units apiece and split every
// 128-token stage's four sub-tiles between the groups (A: 0, 2; B: 1, 3).
// A sub-tile is four phases separated by workgroup barriers:
//     M1  key / value products (12 MFMA)
//     V1  SwiGLU forward/backward of 16 tokens (VALU), plus staging work
//     M2  token contractions of those 16 tokens (6 MFMA)
//     V2  SwiGLU of the other 16 tokens (VALU) and their contractions (6 MFMA)
// Group B runs one phase behind group A, so on every SIMD one wavefront is in
// an MFMA phase while the other is in a VALU phase.  Stages are double
// buffered in LDS; each thread keeps the next stage's 2 tokens x 8 features
// of K and V in registers and writes them (with u = -eta v and the
// transposed copies) during a V1 phase.
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr int D = 64;
constexpr int kThreads = 512;
constexpr int TT = 128;              // tokens per stage
constexpr int KS = D / 16;           // k-steps of the key / value products
constexpr int NT = D / 32;           // 32-wide tiles over d
constexpr int NAT_ROW = 2 * D + 16;  // padded natural row (bytes)
constexpr int NAT_BYTES = TT * NAT_ROW;
constexpr int TR_GROUP = 34 * D;     // transposed 16-token group (bytes)
constexpr int TR_BYTES = (TT / 16) * TR_GROUP;
constexpr int OFF_KN = 0;
constexpr int OFF_UN = NAT_BYTES;
constexpr int OFF_KT = 2 * NAT_BYTES;
constexpr int OFF_UT = 2 * NAT_BYTES + TR_BYTES;
constexpr int STAGE_BYTES = 2 * NAT_BYTES + 2 * TR_BYTES;  // 71680
constexpr int LDS_BYTES = 2 * STAGE_BYTES;                 // 143360

constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

// transposed row (s16, d): 16 tokens of feature d in MFMA k-slot order; the
// 16-byte halves swap on bit 2 of d and every 8 rows shift by 16 bytes
__device__ __forceinline__ int tr_off(int s16, int d, int half) {
  return s16 * TR_GROUP + d * 32 + (d >> 3) * 16 + 16 * (half ^ ((d >> 2) & 1));
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

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads) void k_grad_pp(GradArgs a, int hsl, int nbase) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  // XCD-aware order (hidden slices of one (pair, split) share an XCD's L2)
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
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int g = lane >> 5, ln = lane & 31;
  const int h = a.h;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int n0 = hs * 128 + (wave & 3) * 32;

  // ---- W operands (bf16, registers); W1 pre-scaled by -log2(e)
  bf16x8_t w1b[KS], w3b[KS], w2b[KS];
  {
    const float* W1 = a.W1 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W3 = a.W3 + pair * hd + static_cast<int64_t>(n0 + ln) * D;
    const float* W2 = a.W2 + pair * hd + n0 + ln;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dd = 16 * ks + 8 * g + i;
        w1b[ks][i] = static_cast<__bf16>(kNegLog2e * W1[dd]);
        w3b[ks][i] = static_cast<__bf16>(W3[dd]);
        w2b[ks][i] = static_cast<__bf16>(W2[static_cast<int64_t>(dd) * h]);
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

  // ---- loader: thread = (16-token group s16, quad (sub, half), token pair pr, chunk c)
  const int c = tid & 7;
  const int pr = (tid >> 3) & 1;
  const int sub = (tid >> 4) & 1;
  const int half = (tid >> 5) & 1;
  const int s16 = tid >> 6;
  const int t_first = 16 * s16 + 4 * (2 * sub + half) + 2 * pr;

  const int64_t t_begin = static_cast<int64_t>(split) * a.tps;
  const int64_t t_end = min(a.n, t_begin + a.tps);
  const int nstage = static_cast<int>((t_end - t_begin + TT - 1) / TT);
  const int64_t kv_base = static_cast<int64_t>(pair) * a.kv_stride;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + kv_base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + kv_base;
  const float* etag = a.eta + static_cast<int64_t>(pair) * a.eta_stride;

  u32x4_t kr[2], vr[2];
  float er[2];
  auto load_stage = [&](int64_t t0) {
    if (t0 + TT <= t_end) {  // full stage: no masking
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int64_t tok = t0 + t_first + k;
        kr[k] = *reinterpret_cast<const u32x4_t*>(Kg + tok * D + 8 * c);
        vr[k] = *reinterpret_cast<const u32x4_t*>(Vg + tok * D + 8 * c);
        er[k] = etag[tok];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int64_t tok = t0 + t_first + k;
        const bool ok = tok < t_end;
        kr[k] = ok ? *reinterpret_cast<const u32x4_t*>(Kg + tok * D + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
        vr[k] = ok ? *reinterpret_cast<const u32x4_t*>(Vg + tok * D + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
        er[k] = ok ? etag[tok] : 0.f;
      }
    }
  };
  auto store_stage = [&](unsigned char* buf) {
    // u = -eta v, formed in place of v
    u32x4_t* ur = vr;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float ne = -er[k];
#pragma unroll
      for (int w = 0; w < 4; ++w) ur[k][w] = pack_bf16x2(ne * bf_lo(vr[k][w]), ne * bf_hi(vr[k][w]));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int row = (t_first + k) * NAT_ROW + c * 16;
      *reinterpret_cast<u32x4_t*>(buf + OFF_KN + row) = kr[k];
      *reinterpret_cast<u32x4_t*>(buf + OFF_UN + row) = ur[k];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int dd = 8 * c + j;
      const int w = j >> 1;
      unsigned pk, pu;
      if (j & 1) {
        pk = __builtin_amdgcn_perm(kr[1][w], kr[0][w], 0x07060302u);
        pu = __builtin_amdgcn_perm(ur[1][w], ur[0][w], 0x07060302u);
      } else {
        pk = __builtin_amdgcn_perm(kr[1][w], kr[0][w], 0x05040100u);
        pu = __builtin_amdgcn_perm(ur[1][w], ur[0][w], 0x05040100u);
      }
      const int off = tr_off(s16, dd, half) + 8 * sub + 4 * pr;
      *reinterpret_cast<unsigned*>(buf + OFF_KT + off) = pk;
      *reinterpret_cast<unsigned*>(buf + OFF_UT + off) = pu;
    }
  };

  // ---- prologue: stage 0 into buffer 0, stage 1 into registers
  load_stage(t_begin);
  store_stage(lds);
  if (nstage > 1) load_stage(t_begin + TT);
  __syncthreads();
  if (grp == 1) __syncthreads();  // group B runs one phase behind

  for (int s = 0; s < nstage; ++s) {
    unsigned char* buf = lds + (s & 1) * STAGE_BYTES;
#pragma unroll 1
    for (int q = 0; q < 2; ++q) {
      const int st = 2 * q + grp;  // sub-tile of this stage
      // -- M1: H1' (= -log2e H1), H3, dG for 32 tokens x 32 hidden units
      f32x16_t c1, c3, cg;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c1[r] = 0.f;
        c3[r] = 0.f;
        cg[r] = 0.f;
      }
      {
        const unsigned char* krow = buf + OFF_KN + (32 * st + ln) * NAT_ROW + 16 * g;
        const unsigned char* urow = buf + OFF_UN + (32 * st + ln) * NAT_ROW + 16 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(krow + 32 * ks);
          const bf16x8_t au = *reinterpret_cast<const bf16x8_t*>(urow + 32 * ks);
          c1 = mfma(ak, w1b[ks], c1);
          c3 = mfma(ak, w3b[ks], c3);
          cg = mfma(au, w2b[ks], cg);
        }
      }
      __syncthreads();

      // -- V1 / M2 / V2
      bf16x8_t pg, pd1, pd3;
      auto epilogue = [&](int ss) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * ss + i;
          const float z = c1[r], h3 = c3[r], dg = cg[r];
          const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z));
          const float act = z * sg;
          pg[i] = static_cast<__bf16>(act * h3);
          pd3[i] = static_cast<__bf16>(dg * act);
          const float u = fmaf(-act, sg, act);
          pd1[i] = static_cast<__bf16>((dg * h3) * fmaf(kNegLn2, u, sg));
        }
      };
      auto contract = [&](int ss) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int off = tr_off(2 * st + ss, 32 * nt + ln, g);
          const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(buf + OFF_KT + off);
          const bf16x8_t bu = *reinterpret_cast<const bf16x8_t*>(buf + OFF_UT + off);
          aW1[nt] = mfma(pd1, bk, aW1[nt]);
          aW3[nt] = mfma(pd3, bk, aW3[nt]);
          aW2[nt] = mfma(bu, pg, aW2[nt]);
        }
      };
      epilogue(0);
      if (q == 0 && s + 1 < nstage) {
        // next stage into the other buffer (its last readers finished
        // before this stage began), then fetch the stage after it
        store_stage(lds + ((s + 1) & 1) * STAGE_BYTES);
        if (s + 2 < nstage) load_stage(t_begin + static_cast<int64_t>(s + 2) * TT);
      }
      __syncthreads();
      contract(0);
      __syncthreads();
      epilogue(1);
      contract(1);
      __syncthreads();
    }
  }
  if (grp == 0) __syncthreads();  // same barrier count as group B

  // ---- combine the two groups' sums through LDS, then write the split's partials
  float* red = reinterpret_cast<float*>(lds);  // 4 waves x 6 tiles x 16 x 64 floats = 96 KiB
  const int slot0 = (wave & 3) * 3 * NT;
  if (grp == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[((slot0 + nt) * 16 + r) * 64 + lane] = aW1[nt][r];
        red[((slot0 + NT + nt) * 16 + r) * 64 + lane] = aW3[nt][r];
        red[((slot0 + 2 * NT + nt) * 16 + r) * 64 + lane] = aW2[nt][r];
      }
    }
  }
  __syncthreads();
  if (grp == 0) {
    float* out = a.partials + (static_cast<int64_t>(pair) * a.S + split) * 3 * hd;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * g + (r & 3);
        const float v1 = aW1[nt][r] + red[((slot0 + nt) * 16 + r) * 64 + lane];
        const float v3 = aW3[nt][r] + red[((slot0 + NT + nt) * 16 + r) * 64 + lane];
        const float v2 = aW2[nt][r] + red[((slot0 + 2 * NT + nt) * 16 + r) * 64 + lane];
        out[static_cast<int64_t>(n0 + row) * D + 32 * nt + ln] = v1;
        out[2 * hd + static_cast<int64_t>(n0 + row) * D + 32 * nt + ln] = kNegLn2 * v3;
        out[hd + static_cast<int64_t>(32 * nt + row) * h + n0 + ln] = kNegLn2 * v2;
      }
    }
  }
}

}  // namespace

hipError_t launch_grad_pp(const GradArgs& a, hipStream_t s) {
  if (a.d != D || a.h % 128 != 0) return hipErrorInvalidValue;
  const int hsl = a.h / 128;
  const int nbase = a.S * a.P;
  const int blocks = ((nbase + 7) / 8) * 8 * hsl;
  hipLaunchKernelGGL(k_grad_pp, dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  return hipGetLastError();
}

}  // namespace lact

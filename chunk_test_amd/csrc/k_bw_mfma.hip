// Backward pass of the LaCT layer on bf16 MFMA (gfx950): the weight
// cotangents as token contractions,
//   dW1 += X1^T A,   dW3 += X3^T A,   dW2 += (b B)^T X2      (b = -eta or 1),
// where A, B are the chunk's keys and values (or queries and output
// cotangents) and X1, X2, X3 the per-(token, hidden unit) factors the token
// kernels computed in fp32.  These are the cotangents of the chunk gradient
// and of the query read with respect to the fast weights ("LaCT: Large Chunk
// Test-Time Training" review, sections "Local attention and nonlinear memory
// work together" and "Language modelling: quality and throughput differ",
// where the layer is trained through its outputs).
//
// A and B arrive in bf16 and enter the products exactly; the fp32 factors are
// split, x = x_hi + x_lo (both bf16), so every product is two MFMAs with fp32
// accumulation (~16 significant bits per factor, products of A and B exact).
// One workgroup per (pair, token split, 128-unit hidden slice); wave w owns
// hidden units 32 w .. 32 w + 31 of the slice and every 32-wide feature tile,
// twelve 32 x 32 accumulator tiles per wave at d = 128.  Each stage of 32
// tokens (A, B, the rates and the three factor rows of the slice) moves from
// HBM into double-buffered LDS with global_load_lds one stage ahead; A and B
// enter the products through LDS transpose reads (tokens as the k index).
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
constexpr int NT = D / 32;         // 32-wide feature tiles
constexpr int ROW = 2 * D;         // bytes per token row of A or B (sixteen 16-byte chunks)
constexpr int HS = 128;            // hidden units per workgroup
constexpr int XROW = 4 * HS;       // bytes per token row of one factor slice (32 chunks)
constexpr int TT = 32;             // tokens per stage (two k-steps of 16)
constexpr int TILE = TT * ROW;     // A or B stage
constexpr int XTILE = TT * XROW;   // one factor stage
constexpr int OFF_A = 0;                    // A[2]
constexpr int OFF_B = 2 * TILE;             // B[2]
constexpr int OFF_X = 4 * TILE;             // [2][3] factor stages
constexpr int OFF_E = OFF_X + 6 * XTILE;    // rates [2][TT]
constexpr int LDS_BYTES = OFF_E + 2 * TT * 4;

// XOR swizzle of the 16-byte chunks of a 256-byte token row of A or B (the
// layout of the d = 128 chunk-gradient kernel's key tiles): conflict-free
// 8-byte transpose reads over four rows 4m .. 4m + 3.
__device__ __forceinline__ int swz(int r) {
  return 8 * ((r >> 1) & 1) + 4 * ((r ^ (r >> 3)) & 1) + 2 * (r & 1) + ((r >> 2) & 1);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_bw_contract_mfma(BwContractArgs a, int hsl, int nbase) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  // XCD-aware block order: the hidden slices of one (pair, split) land on the
  // same XCD (block ids congruent mod 8), so their A and B reads share L2.
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
  const int j0 = hs * HS;  // first hidden unit of the slice

  const int64_t t_begin = static_cast<int64_t>(split) * a.tps;
  const int64_t t_end = min(a.n, t_begin + a.tps);
  const int t_last = static_cast<int>(t_end - 1);  // (offsets inside one pair fit 32 bits: host check)
  const uint16_t* Ag = static_cast<const uint16_t*>(a.A) + static_cast<int64_t>(pair) * a.in_stride;
  const uint16_t* Bg = static_cast<const uint16_t*>(a.B) + static_cast<int64_t>(pair) * a.in_stride;
  const float* etag = a.eta ? a.eta + static_cast<int64_t>(pair) * a.eta_stride : nullptr;
  const float* Xg[3] = {a.X1 + static_cast<int64_t>(pair) * a.x_stride + j0,
                        a.X3 + static_cast<int64_t>(pair) * a.x_stride + j0,
                        a.X2 + static_cast<int64_t>(pair) * a.x_stride + j0};

  // DMA of one stage into buffer b.  A, B: 1 KiB pieces of four rows, lane l
  // of a piece landing at byte 16 l (row 4 piece + l / 16, physical chunk
  // l % 16 holding logical chunk (l % 16) ^ swz(row)).  Factors: 1 KiB pieces
  // of two 512-byte rows, physical chunk p of row t holding logical chunk
  // p ^ (8 ((t >> 2) & 1)), so the two half-waves of a factor read (tokens
  // four apart) use different banks.  Rows past the split's end re-read its
  // last token; their factors are masked to zero where they are used.
  auto dma_stage = [&](int64_t t0, int b) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int k = 0; k < TT / 16; ++k) {
      const int piece = 4 * k + wv;
      const int r = 4 * piece + (lane >> 4);
      const int cl = (lane & 15) ^ swz(r);
      const int tok = static_cast<int>(t0) + r;
      const int tc = tok < t_last ? tok : t_last;
      const unsigned off = static_cast<unsigned>(tc) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Ag + off), (lds_ptr_t)(lds + OFF_A + b * TILE + 1024 * piece), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Bg + off), (lds_ptr_t)(lds + OFF_B + b * TILE + 1024 * piece), 16, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
#pragma unroll
      for (int k = 0; k < TT / 8; ++k) {
        const int piece = 4 * k + wv;  // rows 2 piece, 2 piece + 1
        const int r = 2 * piece + (lane >> 5);
        const int cl = (lane & 31) ^ (8 * ((r >> 2) & 1));
        const int tok = static_cast<int>(t0) + r;
        const int tc = tok < t_last ? tok : t_last;
        const float* src = Xg[x] + static_cast<int64_t>(tc) * h + 4 * cl;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(lds + OFF_X + (b * 3 + x) * XTILE + 1024 * piece),
                                         16, 0, 0);
      }
    }
    if (etag != nullptr && wv == 0 && lane < TT) {
      const int tok = static_cast<int>(t0) + lane;
      unsigned char* dst = lds + OFF_E + b * TT * 4;
      if (tok <= t_last) {
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(etag + static_cast<unsigned>(tok)), (lds_ptr_t)dst, 4, 0, 0);
      } else {
        *reinterpret_cast<float*>(dst + 4 * lane) = 0.f;
      }
    }
  };

  // transpose reads of A and B (as in the d = 128 chunk-gradient kernel):
  // lane 16 Q + 4 k' + a of each 16-lane row Q addresses token
  // 4 (Q >> 1) + k' (+ 8 hh) of a 16-token half, features
  // 32 nt + 16 (Q & 1) + 4 a .. +3; the pair (hh = 0, 1) gives the operand
  // whose slot i holds token 8 (i / 4) + 4 g + i % 4 of the half.
  const int tq = lane >> 4, tk = (lane >> 2) & 3, ta = lane & 3;
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
  // factor reads: slot i of lane (g, ln) is token 8 (i / 4) + 4 g + i % 4 of
  // the 16-token half, hidden unit 32 wave + ln of the slice; bit 2 of those
  // tokens is g, so the swizzled chunk is a lane constant.
  const int x_off = 16 * ((8 * wave + (ln >> 2)) ^ (8 * g)) + 4 * (ln & 3);

  f32x16_t acc1[NT], acc3[NT], acc2[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc1[t][r] = 0.f;
      acc3[t][r] = 0.f;
      acc2[t][r] = 0.f;
    }
  }

  if (t_begin < t_end) dma_stage(t_begin, 0);
  int b = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TT, b ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this stage has landed
    __syncthreads();
    if (t0 + TT < t_end) dma_stage(t0 + TT, b ^ 1);
    const unsigned char* ab = lds + OFF_A + b * TILE;
    const unsigned char* bb = lds + OFF_B + b * TILE;
    const unsigned char* xb = lds + OFF_X + b * 3 * XTILE;
    const float* eb = reinterpret_cast<const float*>(lds + OFF_E + b * TT * 4);
    const int valid = static_cast<int>(t_end - t0);  // tokens of this stage that exist (may exceed TT)
#pragma unroll
    for (int s = 0; s < TT / 16; ++s) {
      // factors of this lane's eight tokens, zero past the end; the rate
      // (for the contraction with B) multiplies X2
      float xv[3][8];
#pragma unroll
      for (int x = 0; x < 3; ++x) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = 16 * s + 8 * (i >> 2) + 4 * g + (i & 3);
          const float v = *reinterpret_cast<const float*>(xb + x * XTILE + t * XROW + x_off);
          xv[x][i] = t < valid ? v : 0.f;
        }
      }
      if (etag != nullptr) {
        const f32x4_t e0 = *reinterpret_cast<const f32x4_t*>(eb + 16 * s + 4 * g);
        const f32x4_t e1 = *reinterpret_cast<const f32x4_t*>(eb + 16 * s + 8 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[2][i] *= -e0[i];
          xv[2][4 + i] *= -e1[i];
        }
      }
      bf16x8_t xh[3], xl[3];
#pragma unroll
      for (int x = 0; x < 3; ++x) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xh[x][i] = static_cast<__bf16>(xv[x][i]);
          xl[x][i] = static_cast<__bf16>(xv[x][i] - static_cast<float>(xh[x][i]));
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s16x4_t ta2[2], tb2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int off = tr_off[(nt & 1) ^ hh][nt >> 1] + 4096 * s + 2048 * hh;
          ta2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(ab + off));
          tb2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(bb + off));
        }
        const bf16x8_t opA = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ta2[0], ta2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8_t opB = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(tb2[0], tb2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc1[nt] = mfma32(xh[0], opA, acc1[nt]);
        acc3[nt] = mfma32(xh[1], opA, acc3[nt]);
        acc2[nt] = mfma32(opB, xh[2], acc2[nt]);
        acc1[nt] = mfma32(xl[0], opA, acc1[nt]);
        acc3[nt] = mfma32(xl[1], opA, acc3[nt]);
        acc2[nt] = mfma32(opB, xl[2], acc2[nt]);
      }
    }
  }

  // ---- partial sums of this split: [W1 block h x D | W2 block D x h | W3 block h x D]
  float* out = a.partials + (static_cast<int64_t>(pair) * a.S + split) * 3 * hd;
  const int jw = j0 + 32 * wave;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * g + (r & 3);
      out[static_cast<int64_t>(jw + row) * D + 32 * nt + ln] = acc1[nt][r];
      out[2 * hd + static_cast<int64_t>(jw + row) * D + 32 * nt + ln] = acc3[nt][r];
      out[hd + static_cast<int64_t>(32 * nt + row) * h + jw + ln] = acc2[nt][r];
    }
  }
}

}  // namespace

bool bw_contract_mfma_ok(const BwContractArgs& a) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.B) |
                       reinterpret_cast<uintptr_t>(a.X1) | reinterpret_cast<uintptr_t>(a.X2) |
                       reinterpret_cast<uintptr_t>(a.X3);
  return a.bf16 && a.d == D && a.h % HS == 0 && (al & 15) == 0 && (a.in_stride % 8) == 0 && (a.x_stride % 4) == 0 &&
         a.n * D < (int64_t(1) << 31);
}

hipError_t launch_bw_contract_mfma(const BwContractArgs& a, hipStream_t s) {
  const int hsl = a.h / HS;
  const int nbase = a.S * a.P;
  const int blocks = ((nbase + 7) / 8) * 8 * hsl;
  hipLaunchKernelGGL(k_bw_contract_mfma, dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  return hipGetLastError();
}

}  // namespace lact

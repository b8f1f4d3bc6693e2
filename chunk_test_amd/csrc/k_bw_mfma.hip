// Backward pass of the LaCT layer on bf16 MFMA (gfx950), d = 64 or 128: the
// weight cotangents as token contractions,
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
// accumulation (~16 significant bits per factor, products of A and B exact)
// -- or, where the layer runs with plain bf16 operand products (the
// forward's products setting), rounded to bf16, one MFMA per product.
// One workgroup per (pair, token split, 128-unit hidden slice); wave w owns
// hidden units 32 w .. 32 w + 31 of the slice and every 32-wide feature tile,
// twelve 32 x 32 accumulator tiles per wave at d = 128 (six at d = 64).  Each stage of 32
// tokens (A, B, the rates and the three factor rows of the slice) moves from
// HBM into double-buffered LDS with global_load_lds one stage ahead; A and B
// enter the products through LDS transpose reads (tokens as the k index).
//
// The query read's token-local VJP runs here too (k_bw_apply_mfma): per query
// q and hidden unit j, with h1 = W1 q, h3 = W3 q, ob = (dO W2)_j,
//   X1 = ob h3 silu'(h1),  X2 = silu(h1) h3,  X3 = ob silu(h1),
//   dq = W1^T X1 + W3^T X3,
// the three projections and dq as split-operand MFMAs (the weights enter as
// bf16 hi + lo operands prepared once per call by k_bw_ops, the queries and
// output cotangents exactly), the element math in fp32.  With plain bf16
// products (SPLIT false) every operand is its bf16 rounding (the hi part
// alone) and every product one MFMA, as in the forward pass.
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_t;

constexpr int kThreads = 256;
constexpr int HS = 128;            // hidden units per contraction workgroup
constexpr int XROW = 4 * HS;       // bytes per token row of one factor slice (32 chunks)
constexpr int TT = 32;             // tokens per contraction stage (two k-steps of 16)
constexpr int XTILE = TT * XROW;   // one factor stage

// bf16 rows of D features (keys, values, queries, or the weight operands) in
// LDS: rows of 2 D bytes in 16-byte chunks, chunk c of row r stored at chunk
// c ^ swz(r), the layouts of the d = 128 and d = 64 chunk-gradient kernels'
// key tiles: 16-byte row reads (16 consecutive rows, one chunk) and 8-byte
// transpose reads (four rows 4m .. 4m + 3, lanes 16 Q + 4 k' + a addressing
// row 4 (Q >> 1) + k' (+ 8 hh) of a 16-row half, features
// 32 nt + 16 (Q & 1) + 4 a .. +3) are both free of bank conflicts.  A pair of
// transpose reads (hh = 0, 1) gives an MFMA operand whose slot i holds row
// 8 (i / 4) + 4 g + i % 4 of the half; 1 KiB DMA pieces hold 1024 / ROW rows,
// lane l landing in row l / LPR, physical chunk l % LPR.
template <int D>
struct Rows;
template <>
struct Rows<128> {
  static constexpr int ROW = 256, LPR = 16;
  __device__ static int swz(int r) {
    return 8 * ((r >> 1) & 1) + 4 * ((r ^ (r >> 3)) & 1) + 2 * (r & 1) + ((r >> 2) & 1);
  }
  __device__ static void tr_init(int lane, int (&o)[4]) {
    const int tq = lane >> 4, tk = (lane >> 2) & 3, ta = lane & 3;
    const int tl = 4 * (tq >> 1) + tk;
    const int r0 = tl & 1, r1 = (tl >> 1) & 1, r2 = (tl >> 2) & 1;
    const int low = (2 * (tq & 1) + (ta >> 1)) ^ (2 * r0 + r2);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int n1 = 0; n1 < 2; ++n1) o[2 * x + n1] = tl * ROW + 16 * (8 * (n1 ^ r1) + 4 * (x ^ r0) + low) + 8 * (ta & 1);
    }
  }
  __device__ static int tr(const int (&o)[4], int nt, int hh) { return o[2 * ((nt & 1) ^ hh) + (nt >> 1)]; }
};
template <>
struct Rows<64> {
  static constexpr int ROW = 128, LPR = 8;
  __device__ static int swz(int r) { return 4 * (((r >> 1) ^ (r >> 3)) & 1) + 2 * ((r >> 2) & 1) + ((r >> 1) & 1); }
  __device__ static void tr_init(int lane, int (&o)[4]) {
    const int tq = lane >> 4, tk = (lane >> 2) & 3, ta = lane & 3;
    const int tl = 4 * (tq >> 1) + tk;
    const int t1 = (tl >> 1) & 1, t2 = (tl >> 2) & 1;
    const int low = (2 * (tq & 1) + (ta >> 1)) ^ (2 * t2 + t1);
#pragma unroll
    for (int x = 0; x < 2; ++x) o[x] = tl * ROW + 16 * (4 * (x ^ t1) + low) + 8 * (ta & 1);
    o[2] = o[3] = 0;
  }
  __device__ static int tr(const int (&o)[4], int nt, int hh) { return o[nt ^ hh]; }
};

// the contraction kernel's LDS: A[2], B[2] stages, [2][3] factor stages, rates [2][TT]
// (bf16 factors, XB: rows of the 128-unit slice in the Rows<128> layout)
template <int D, bool XB = false>
struct CGeo {
  static constexpr int NT = D / 32;
  static constexpr int TILE = TT * Rows<D>::ROW;
  static constexpr int XT = XB ? TT * Rows<128>::ROW : XTILE;  // one factor stage
  static constexpr int OFF_A = 0;
  static constexpr int OFF_B = 2 * TILE;
  static constexpr int OFF_X = 4 * TILE;
  static constexpr int OFF_E = OFF_X + 6 * XT;
  static constexpr int LDS_BYTES = OFF_E + 2 * TT * 4;
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool SPLIT, bool XB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_bw_contract_mfma(BwContractArgs a, int hsl, int nbase) {
  static_assert(!(SPLIT && XB), "bf16 factors come with plain products");
  using R = Rows<D>;
  using C = CGeo<D, XB>;
  constexpr int XT = C::XT;
  constexpr int NT = C::NT, ROW = R::ROW, TILE = C::TILE;
  constexpr int OFF_A = C::OFF_A, OFF_B = C::OFF_B, OFF_X = C::OFF_X, OFF_E = C::OFF_E;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];

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
  // (bf16 factors: the same element offsets in arrays of 2-byte elements)
  const uint16_t* Xh[3] = {reinterpret_cast<const uint16_t*>(a.X1) + static_cast<int64_t>(pair) * a.x_stride + j0,
                           reinterpret_cast<const uint16_t*>(a.X3) + static_cast<int64_t>(pair) * a.x_stride + j0,
                           reinterpret_cast<const uint16_t*>(a.X2) + static_cast<int64_t>(pair) * a.x_stride + j0};

  // DMA of one stage into buffer b.  A, B: 1 KiB pieces in the Rows<D>
  // layout (one piece per wave at d = 64, two at d = 128).  Factors: 1 KiB pieces
  // of two 512-byte rows, physical chunk p of row t holding logical chunk
  // p ^ (8 ((t >> 2) & 1)), so the two half-waves of a factor read (tokens
  // four apart) use different banks.  Rows past the split's end re-read its
  // last token; their factors are masked to zero where they are used.
  auto dma_stage = [&](int64_t t0, int b) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int k = 0; k < TILE / 4096; ++k) {
      const int piece = 4 * k + wv;
      const int r = (1024 / ROW) * piece + lane / R::LPR;
      const int cl = (lane % R::LPR) ^ R::swz(r);
      const int tok = static_cast<int>(t0) + r;
      const int tc = tok < t_last ? tok : t_last;
      const unsigned off = static_cast<unsigned>(tc) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Ag + off), (lds_ptr_t)(lds + OFF_A + b * TILE + 1024 * piece), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Bg + off), (lds_ptr_t)(lds + OFF_B + b * TILE + 1024 * piece), 16, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      if constexpr (XB) {
        // bf16 factor rows of 256 bytes in the Rows<128> layout: 1 KiB pieces of four rows
#pragma unroll
        for (int k = 0; k < TT / 16; ++k) {
          const int piece = 4 * k + wv;
          const int r = 4 * piece + (lane >> 4);
          const int cl = (lane & 15) ^ Rows<128>::swz(r);
          const int tok = static_cast<int>(t0) + r;
          const int tc = tok < t_last ? tok : t_last;
          const uint16_t* src = Xh[x] + static_cast<int64_t>(tc) * h + 8 * cl;
          __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(lds + OFF_X + (b * 3 + x) * XT + 1024 * piece),
                                           16, 0, 0);
        }
      } else {
#pragma unroll
        for (int k = 0; k < TT / 8; ++k) {
          const int piece = 4 * k + wv;  // rows 2 piece, 2 piece + 1
          const int r = 2 * piece + (lane >> 5);
          const int cl = (lane & 31) ^ (8 * ((r >> 2) & 1));
          const int tok = static_cast<int>(t0) + r;
          const int tc = tok < t_last ? tok : t_last;
          const float* src = Xg[x] + static_cast<int64_t>(tc) * h + 4 * cl;
          __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(lds + OFF_X + (b * 3 + x) * XT + 1024 * piece),
                                           16, 0, 0);
        }
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

  // transpose reads of A and B (tokens as the k index, Rows<D>), and of the
  // bf16 factors (Rows<128>: lane = hidden unit 32 wave + ln of the slice)
  int tro[4], trx[4];
  R::tr_init(lane, tro);
  Rows<128>::tr_init(lane, trx);
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
    const unsigned char* xb = lds + OFF_X + b * 3 * XT;
    const float* eb = reinterpret_cast<const float*>(lds + OFF_E + b * TT * 4);
    const int valid = static_cast<int>(t_end - t0);  // tokens of this stage that exist (may exceed TT)
#pragma unroll
    for (int s = 0; s < TT / 16; ++s) {
      bf16x8_t xh[3], xl[3];
      if constexpr (XB) {
        // bf16 factors (X2 already carries the rate) by transpose reads: slot
        // i = token 16 s + 8 (i / 4) + 4 g + i % 4; zero past the end
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          s16x4_t t2[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            t2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t)(xb + x * XT + Rows<128>::tr(trx, wave, hh) + 16 * Rows<128>::ROW * s +
                              8 * Rows<128>::ROW * hh));
          xh[x] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t2[0], t2[1], 0, 1, 2, 3, 4, 5, 6, 7));
          if (valid < TT) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int t = 16 * s + 8 * (i >> 2) + 4 * g + (i & 3);
              if (t >= valid) xh[x][i] = static_cast<__bf16>(0.f);
            }
          }
        }
      } else {
        // factors of this lane's eight tokens, zero past the end; the rate
        // (for the contraction with B) multiplies X2
        float xv[3][8];
#pragma unroll
        for (int x = 0; x < 3; ++x) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int t = 16 * s + 8 * (i >> 2) + 4 * g + (i & 3);
            const float v = *reinterpret_cast<const float*>(xb + x * XT + t * XROW + x_off);
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
#pragma unroll
        for (int x = 0; x < 3; ++x) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            xh[x][i] = static_cast<__bf16>(xv[x][i]);
            if constexpr (SPLIT) xl[x][i] = static_cast<__bf16>(xv[x][i] - static_cast<float>(xh[x][i]));
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s16x4_t ta2[2], tb2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int off = R::tr(tro, nt, hh) + 16 * ROW * s + 8 * ROW * hh;
          ta2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(ab + off));
          tb2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(bb + off));
        }
        const bf16x8_t opA = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ta2[0], ta2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8_t opB = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(tb2[0], tb2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc1[nt] = mfma32(xh[0], opA, acc1[nt]);
        acc3[nt] = mfma32(xh[1], opA, acc3[nt]);
        acc2[nt] = mfma32(opB, xh[2], acc2[nt]);
        if constexpr (SPLIT) {
          acc1[nt] = mfma32(xl[0], opA, acc1[nt]);
          acc3[nt] = mfma32(xl[1], opA, acc3[nt]);
          acc2[nt] = mfma32(opB, xl[2], acc2[nt]);
        }
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


// Operands of the token kernels: every matrix as bf16 hi and lo parts in
// [hidden unit][feature] order (W2 and P2, stored [feature][hidden unit], are
// transposed): op[pair][m][hl][j][e], m over W1, W3, W2 (and P1, P3, P2).
// the matrices stored [hidden][feature] (W1, W3, P1, P3): element by element
// (four consecutive elements per thread: hd is a multiple of 64)
template <int D>
__global__ __launch_bounds__(kThreads) void k_bw_ops(BwOpsArgs a) {
  const int64_t hd = static_cast<int64_t>(a.h) * D;
  const int64_t idx = 4 * (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x);
  const int nd = a.nm == 6 ? 4 : 2;  // direct matrices: m = 0, 1 (and 3, 4)
  const int64_t total = static_cast<int64_t>(a.P) * nd * hd;
  if (idx >= total) return;
  const int64_t pm = idx / hd, e_idx = idx % hd;
  const int pair = static_cast<int>(pm / nd), k = static_cast<int>(pm % nd);
  const int m = k < 2 ? k : k + 1;
  const MatRef& r = a.m[m];
  const float* src = r.p + pair * r.pair_stride + e_idx;
  f32x4_t x;
  if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    x = *reinterpret_cast<const f32x4_t*>(src);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = src[i];
  }
  bf16x4_t hi, lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = static_cast<__bf16>(x[i]);
    lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(hi[i]));
  }
  __bf16* o = reinterpret_cast<__bf16*>(a.op) + pair * a.op_stride + static_cast<int64_t>(m) * 2 * hd;
  *reinterpret_cast<bf16x4_t*>(o + e_idx) = hi;
  if (!a.hi_only) *reinterpret_cast<bf16x4_t*>(o + hd + e_idx) = lo;
}

// W2 and P2 (stored [feature][hidden]) transposed into [hidden][feature]:
// one 64 x 64 tile per workgroup through LDS, so both the fp32 reads (64
// hidden units of a feature row) and the bf16 writes (64 features of a
// hidden row) are contiguous
template <int D>
__global__ __launch_bounds__(kThreads) void k_bw_ops_tr(BwOpsArgs a) {
  __shared__ float tile[64][65];
  const int jt = blockIdx.x;           // 64-unit hidden tile
  const int et = blockIdx.y;           // 64-feature tile
  const int pair = blockIdx.z / (a.nm == 6 ? 2 : 1);
  const int m = (a.nm == 6 && (blockIdx.z & 1)) ? 5 : 2;
  const MatRef& r = a.m[m];
  const int64_t hd = static_cast<int64_t>(a.h) * D;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const float* src = r.p + pair * r.pair_stride;
  for (int i = ty; i < 64; i += kThreads / 64) {
    const int e = 64 * et + i, j = 64 * jt + tx;
    tile[i][tx] = (e < D && j < a.h) ? src[static_cast<int64_t>(e) * a.h + j] : 0.f;
  }
  __syncthreads();
  __bf16* o = reinterpret_cast<__bf16*>(a.op) + pair * a.op_stride + static_cast<int64_t>(m) * 2 * hd;
  for (int i = ty; i < 64; i += kThreads / 64) {
    const int j = 64 * jt + i, e = 64 * et + tx;
    if (j < a.h && e < D) {
      const float x = tile[tx][i];
      const __bf16 hi = static_cast<__bf16>(x);
      o[static_cast<int64_t>(j) * D + e] = hi;
      if (!a.hi_only) o[hd + static_cast<int64_t>(j) * D + e] = static_cast<__bf16>(x - static_cast<float>(hi));
    }
  }
}

// four factors at hidden units j .. j + 3 of a token's bf16 factor row Xb,
// times f, rounded to bf16
__device__ __forceinline__ void store_bf16x4(uint16_t* Xb, int j, const float* v, float f) {
  bf16x4_t b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = static_cast<__bf16>(f * v[i]);
  *reinterpret_cast<bf16x4_t*>(Xb + j) = b;
}

constexpr int QWG = 128;             // tokens per token-kernel workgroup (32 per wave)
constexpr int JT = 32;               // hidden units per weight tile

__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_bw_apply_mfma(BwTokArgs a) {
  using R = Rows<D>;
  constexpr int NT = D / 32, KS = D / 16, ROW = R::ROW;
  constexpr int WHALF = JT * ROW;     // one matrix part (hi or lo) of a weight tile
  constexpr int NPART = SPLIT ? 6 : 3;
  constexpr int WTILE3 = NPART * WHALF;  // W1, W3, W2^T: hi and lo parts (hi only without SPLIT)
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * WTILE3];
  // XCD-aware order: block ids congruent mod 8 run on one XCD, and the
  // token tiles of a pair take consecutive slots of one XCD's share, so the
  // pair's weight tiles come from HBM once and then from that XCD's L2
  const int nblk = gridDim.x;  // a multiple of 8
  const int ntiles = static_cast<int>((a.n + QWG - 1) / QWG);
  const int o = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  if (o >= ntiles * a.P) return;
  const int pair = o / ntiles;
  const int64_t tb = static_cast<int64_t>(o % ntiles) * QWG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int ln = lane & 31;
  const int h = a.h;
  const int ntile = h / JT;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const uint16_t* opg = a.op + pair * a.op_stride;

  // this lane's query (past the end: the last one, outputs dropped) as the
  // B operand of the projections: features 16 ks + 8 g .. +7
  const int64_t t = tb + 32 * wave + ln;
  const int64_t tcl = t < a.n ? t : a.n - 1;
  bf16x8_t qop[KS], oop[KS];
  {
    const uint16_t* Qg = static_cast<const uint16_t*>(a.A) + pair * a.in_stride + tcl * D;
    const uint16_t* Og = static_cast<const uint16_t*>(a.B) + pair * a.in_stride + tcl * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qop[ks] = *reinterpret_cast<const bf16x8_t*>(Qg + 16 * ks + 8 * g);
      oop[ks] = *reinterpret_cast<const bf16x8_t*>(Og + 16 * ks + 8 * g);
    }
  }

  // DMA of weight tile jt (rows 32 jt .. +31 of the six parts) into buffer b,
  // 1 KiB pieces in the Rows<D> layout (PP pieces per part)
  constexpr int PP = WHALF / 1024;
  auto dma_w = [&](int jt, int b) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int k = 0; k < NPART * PP / 4; ++k) {
      const int piece = 4 * k + wv;
      const int part = piece / PP;
      const int r = (1024 / ROW) * (piece % PP) + lane / R::LPR;
      const int cl = (lane % R::LPR) ^ R::swz(r);
      const int src_part = SPLIT ? part : 2 * part;  // (the hi parts only)
      const uint16_t* src = opg + src_part * hd + static_cast<int64_t>(JT * jt + r) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(lds + b * WTILE3 + part * WHALF + 1024 * (piece % PP)),
                                       16, 0, 0);
    }
  };

  // row reads of a part (lane = hidden unit ln of the tile, features
  // 16 ks + 8 g .. +7) and transpose reads (lane = feature 32 nt + ln, slot i
  // = hidden unit 16 s + 8 (i / 4) + 4 g + i % 4 of the tile), Rows<D>
  int ak_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ak_off[ks] = ln * ROW + 16 * ((2 * ks + g) ^ R::swz(ln));
  int tro[4];
  R::tr_init(lane, tro);
  auto tr_read = [&](const unsigned char* base, int nt, int s) {
    s16x4_t t2[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      t2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t)(base + R::tr(tro, nt, hh) + 16 * ROW * s + 8 * ROW * hh));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t2[0], t2[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t dq[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[nt][r] = 0.f;
  }
  float* X1 = a.X1 + pair * a.x_stride + t * h;
  float* X2 = a.X2 + pair * a.x_stride + t * h;
  float* X3 = a.X3 + pair * a.x_stride + t * h;
  // (bf16 factors: the same element offsets in arrays of 2-byte elements)
  uint16_t* Xb1 = reinterpret_cast<uint16_t*>(a.X1) + pair * a.x_stride + t * h;
  uint16_t* Xb2 = reinterpret_cast<uint16_t*>(a.X2) + pair * a.x_stride + t * h;
  uint16_t* Xb3 = reinterpret_cast<uint16_t*>(a.X3) + pair * a.x_stride + t * h;
  const bool live = t < a.n;

  dma_w(0, 0);
  for (int jt = 0; jt < ntile; ++jt) {
    const int b = jt & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile jt has landed
    __syncthreads();
    if (jt + 1 < ntile) dma_w(jt + 1, b ^ 1);
    constexpr int HL = SPLIT ? 2 : 1;  // parts per matrix
    const unsigned char* w1h = lds + b * WTILE3;
    const unsigned char* w1l = w1h + WHALF;
    const unsigned char* w3h = w1h + HL * WHALF;
    const unsigned char* w3l = w3h + WHALF;
    const unsigned char* w2h = w1h + 2 * HL * WHALF;
    const unsigned char* w2l = w2h + WHALF;
    // projections, transposed: c[j][query] (lane = query, register r =
    // hidden unit 8 (r / 4) + 4 g + r % 4 of the tile)
    f32x16_t c1, c3, cb;
#pragma unroll
    for (int r = 0; r < 16; ++r) c1[r] = c3[r] = cb[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(w1h + ak_off[ks]);
      const bf16x8_t a3 = *reinterpret_cast<const bf16x8_t*>(w3h + ak_off[ks]);
      const bf16x8_t a2 = *reinterpret_cast<const bf16x8_t*>(w2h + ak_off[ks]);
      c1 = mfma32(a1, qop[ks], c1);
      c3 = mfma32(a3, qop[ks], c3);
      cb = mfma32(a2, oop[ks], cb);
      if constexpr (SPLIT) {
        const bf16x8_t l1 = *reinterpret_cast<const bf16x8_t*>(w1l + ak_off[ks]);
        const bf16x8_t l3 = *reinterpret_cast<const bf16x8_t*>(w3l + ak_off[ks]);
        const bf16x8_t l2 = *reinterpret_cast<const bf16x8_t*>(w2l + ak_off[ks]);
        c1 = mfma32(l1, qop[ks], c1);
        c3 = mfma32(l3, qop[ks], c3);
        cb = mfma32(l2, oop[ks], cb);
      }
    }
    // element math; x1 = X1, x3 = X3 (the operands of dq), G
    float x1[16], x3[16], gg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float h1 = c1[r], h3 = c3[r], ob = cb[r];
      const float sg = sigmoid_fast(h1);
      const float act = h1 * sg;
      x3[r] = ob * act;
      x1[r] = ob * h3 * (sg * (1.f + h1 * (1.f - sg)));
      gg[r] = act * h3;
    }
    if (live) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int j = JT * jt + 8 * rg + 4 * g;
        if (a.x_bf16) {
          store_bf16x4(Xb1, j, x1 + 4 * rg, 1.f);
          store_bf16x4(Xb2, j, gg + 4 * rg, 1.f);
          store_bf16x4(Xb3, j, x3 + 4 * rg, 1.f);
        } else {
          *reinterpret_cast<f32x4_t*>(X1 + j) = f32x4_t{x1[4 * rg], x1[4 * rg + 1], x1[4 * rg + 2], x1[4 * rg + 3]};
          *reinterpret_cast<f32x4_t*>(X2 + j) = f32x4_t{gg[4 * rg], gg[4 * rg + 1], gg[4 * rg + 2], gg[4 * rg + 3]};
          *reinterpret_cast<f32x4_t*>(X3 + j) = f32x4_t{x3[4 * rg], x3[4 * rg + 1], x3[4 * rg + 2], x3[4 * rg + 3]};
        }
      }
    }
    // dq[e][query] += sum over the tile's hidden units of W1[j][e] X1 + W3[j][e] X3
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8_t b1h, b1l, b3h, b3l;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        b1h[i] = static_cast<__bf16>(x1[8 * s + i]);
        b3h[i] = static_cast<__bf16>(x3[8 * s + i]);
        if constexpr (SPLIT) {
          b1l[i] = static_cast<__bf16>(x1[8 * s + i] - static_cast<float>(b1h[i]));
          b3l[i] = static_cast<__bf16>(x3[8 * s + i] - static_cast<float>(b3h[i]));
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8_t o1h = tr_read(w1h, nt, s);
        const bf16x8_t o3h = tr_read(w3h, nt, s);
        dq[nt] = mfma32(o1h, b1h, dq[nt]);
        dq[nt] = mfma32(o3h, b3h, dq[nt]);
        if constexpr (SPLIT) {
          const bf16x8_t o1l = tr_read(w1l, nt, s), o3l = tr_read(w3l, nt, s);
          dq[nt] = mfma32(o1h, b1l, dq[nt]);
          dq[nt] = mfma32(o3h, b3l, dq[nt]);
          dq[nt] = mfma32(o1l, b1h, dq[nt]);
          dq[nt] = mfma32(o3l, b3h, dq[nt]);
        }
      }
    }
  }
  // dq (lane = query, register r = feature 32 nt + 8 (r / 4) + 4 g + r % 4)
  if (live) {
    uint16_t* dQ = static_cast<uint16_t*>(a.dA) + pair * a.out_stride + t * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4_t v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = static_cast<__bf16>(dq[nt][4 * rg + i]);
        *reinterpret_cast<bf16x4_t*>(dQ + 32 * nt + 8 * rg + 4 * g) = v4;
      }
    }
  }
}


// Token-local VJP of the chunk gradient on MFMA: per key k (value v, rate
// eta) and hidden unit j, with u = -eta v,
//   h1 = W1 k, h3 = W3 k, dg = (u W2)_j, p1 = P1 k, p3 = P3 k, gb = (u P2)_j
// (P: the cotangents reaching the chunk gradient), the factors
//   X2 = p3 a + p1 h3 s1,  X3 = p1 dg s1 + gb a,
//   X1 = p1 dg h3 s2 + (p3 dg + gb h3) s1
// (a = silu(h1), s1 = silu'(h1), s2 = silu''(h1)) and the per-token sums
//   ubar = P2 G + W2 X2  (G = a h3),
//   kbar = P1^T dH1 + P3^T dH3 + W1^T X1 + W3^T X3  (dH1 = dg h3 s1, dH3 = dg a),
// giving dk = kbar, dv = -eta ubar, deta = -ubar . v.  Six projections and
// six token-side products per weight tile, all split-operand MFMAs; the
// weight tile (twelve bf16 parts) is one LDS buffer, refilled after every
// wave has finished with it.
template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_bw_grad_mfma(BwTokArgs a) {
  using R = Rows<D>;
  constexpr int NT = D / 32, KS = D / 16, ROW = R::ROW;
  constexpr int WHALF = JT * ROW;     // one matrix part (hi or lo) of a weight tile
  constexpr int NPART = SPLIT ? 12 : 6;
  constexpr int WTILE6 = NPART * WHALF;  // W1, W3, W2^T, P1, P3, P2^T: hi and lo (hi only without SPLIT)
  __shared__ __attribute__((aligned(16))) unsigned char lds[WTILE6];
  // the token-side products' LDS operand reads grouped ahead of their
  // products too (not in the split d = 128 kernel, which has no registers
  // left for them)
  constexpr bool GROUP = !(SPLIT && D == 128);
  // XCD-aware order: block ids congruent mod 8 run on one XCD, and the
  // token tiles of a pair take consecutive slots of one XCD's share, so the
  // pair's weight tiles come from HBM once and then from that XCD's L2
  const int nblk = gridDim.x;  // a multiple of 8
  const int ntiles = static_cast<int>((a.n + QWG - 1) / QWG);
  const int o = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  if (o >= ntiles * a.P) return;
  const int pair = o / ntiles;
  const int64_t tb = static_cast<int64_t>(o % ntiles) * QWG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int ln = lane & 31;
  const int h = a.h;
  const int ntile = h / JT;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const uint16_t* opg = a.op + pair * a.op_stride;

  const int64_t t = tb + 32 * wave + ln;
  const bool live = t < a.n;
  const int64_t tcl = live ? t : a.n - 1;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.A) + pair * a.in_stride + tcl * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.B) + pair * a.in_stride + tcl * D;
  bf16x8_t kop[KS], vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kop[ks] = *reinterpret_cast<const bf16x8_t*>(Kg + 16 * ks + 8 * g);
    vop[ks] = *reinterpret_cast<const bf16x8_t*>(Vg + 16 * ks + 8 * g);
  }
  const float ne = live ? -a.eta[pair * a.eta_stride + t] : 0.f;

  constexpr int PP = WHALF / 1024;  // 1 KiB pieces per part
  auto dma_w = [&](int jt) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int k = 0; k < NPART * PP / 4; ++k) {
      const int piece = 4 * k + wv;
      const int part = piece / PP;
      const int r = (1024 / ROW) * (piece % PP) + lane / R::LPR;
      const int cl = (lane % R::LPR) ^ R::swz(r);
      const int src_part = SPLIT ? part : 2 * part;  // (the hi parts only)
      const uint16_t* src = opg + src_part * hd + static_cast<int64_t>(JT * jt + r) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(lds + part * WHALF + 1024 * (piece % PP)), 16, 0, 0);
    }
  };

  int ak_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ak_off[ks] = ln * ROW + 16 * ((2 * ks + g) ^ R::swz(ln));
  int tro[4];
  R::tr_init(lane, tro);
  auto tr_read = [&](const unsigned char* base, int nt, int s) {
    s16x4_t t2[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      t2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t)(base + R::tr(tro, nt, hh) + 16 * ROW * s + 8 * ROW * hh));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t2[0], t2[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto part = [&](int m, int hl) {
    return static_cast<const unsigned char*>(lds + (SPLIT ? 2 * m + hl : m) * WHALF);
  };

  f32x16_t ub[NT], kb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) ub[nt][r] = kb[nt][r] = 0.f;
  }
  float* X1 = a.X1 + pair * a.x_stride + t * h;
  float* X2 = a.X2 + pair * a.x_stride + t * h;
  float* X3 = a.X3 + pair * a.x_stride + t * h;
  // (bf16 factors: the same element offsets in arrays of 2-byte elements)
  uint16_t* Xb1 = reinterpret_cast<uint16_t*>(a.X1) + pair * a.x_stride + t * h;
  uint16_t* Xb2 = reinterpret_cast<uint16_t*>(a.X2) + pair * a.x_stride + t * h;
  uint16_t* Xb3 = reinterpret_cast<uint16_t*>(a.X3) + pair * a.x_stride + t * h;

  dma_w(0);
  for (int jt = 0; jt < ntile; ++jt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile jt has landed
    __syncthreads();
    // the six projections, transposed (lane = key, register r = hidden unit
    // 8 (r / 4) + 4 g + r % 4 of the tile); m: W1, W3, W2^T, P1, P3, P2^T
    f32x16_t c[6];
#pragma unroll
    for (int m = 0; m < 6; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) c[m][r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // (a k-step's weight reads are issued together, ahead of its products:
      // with one wavefront per SIMD nothing else hides their latency)
      bf16x8_t wh[6], wl[6];
#pragma unroll
      for (int m = 0; m < 6; ++m) {
        wh[m] = *reinterpret_cast<const bf16x8_t*>(part(m, 0) + ak_off[ks]);
        if constexpr (SPLIT) wl[m] = *reinterpret_cast<const bf16x8_t*>(part(m, 1) + ak_off[ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < 6; ++m) {
        const bf16x8_t bo = (m == 2 || m == 5) ? vop[ks] : kop[ks];
        c[m] = mfma32(wh[m], bo, c[m]);
        if constexpr (SPLIT) c[m] = mfma32(wl[m], bo, c[m]);
      }
    }
    // element math (fp32)
    float x1[16], x2[16], x3[16], dh1[16], dh3[16], gg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float h1 = c[0][r], h3 = c[1][r], dg = ne * c[2][r];
      const float p1 = c[3][r], p3 = c[4][r], gb = ne * c[5][r];
      const float sg = sigmoid_fast(h1);
      const float act = h1 * sg;
      const float s1 = sg * (1.f + h1 * (1.f - sg));
      const float s2 = sg * (1.f - sg) * (2.f + h1 * (1.f - 2.f * sg));
      x2[r] = p3 * act + p1 * h3 * s1;
      const float ab = p3 * dg + gb * h3;
      x3[r] = p1 * dg * s1 + gb * act;
      x1[r] = p1 * dg * h3 * s2 + ab * s1;
      dh1[r] = dg * h3 * s1;
      dh3[r] = dg * act;
      gg[r] = act * h3;
    }
    if (live) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int j = JT * jt + 8 * rg + 4 * g;
        if (a.x_bf16) {
          store_bf16x4(Xb1, j, x1 + 4 * rg, 1.f);
          store_bf16x4(Xb2, j, x2 + 4 * rg, ne);  // (the rate of the contraction with V)
          store_bf16x4(Xb3, j, x3 + 4 * rg, 1.f);
        } else {
          *reinterpret_cast<f32x4_t*>(X1 + j) = f32x4_t{x1[4 * rg], x1[4 * rg + 1], x1[4 * rg + 2], x1[4 * rg + 3]};
          *reinterpret_cast<f32x4_t*>(X2 + j) = f32x4_t{x2[4 * rg], x2[4 * rg + 1], x2[4 * rg + 2], x2[4 * rg + 3]};
          *reinterpret_cast<f32x4_t*>(X3 + j) = f32x4_t{x3[4 * rg], x3[4 * rg + 1], x3[4 * rg + 2], x3[4 * rg + 3]};
        }
      }
    }
    // token-side sums over the tile's hidden units
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // B operands (lane = key, slot i = hidden unit 16 s + 8 (i / 4) + 4 g + i % 4)
      bf16x8_t bh[6], bl[6];  // G, X2 (for ubar); dH1, dH3, X1, X3 (for kbar)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v6[6] = {gg[8 * s + i], x2[8 * s + i], dh1[8 * s + i], dh3[8 * s + i], x1[8 * s + i], x3[8 * s + i]};
#pragma unroll
        for (int q = 0; q < 6; ++q) {
          bh[q][i] = static_cast<__bf16>(v6[q]);
          if constexpr (SPLIT) bl[q][i] = static_cast<__bf16>(v6[q] - static_cast<float>(bh[q][i]));
        }
      }
      // matrix of each B operand: P2^T, W2^T (ubar); P1, P3, W1, W3 (kbar)
      constexpr int mat[6] = {5, 2, 3, 4, 0, 1};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (GROUP) {
          bf16x8_t oh[6], ol[6];
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            oh[q] = tr_read(part(mat[q], 0), nt, s);
            if constexpr (SPLIT) ol[q] = tr_read(part(mat[q], 1), nt, s);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            f32x16_t& acc = q < 2 ? ub[nt] : kb[nt];
            acc = mfma32(oh[q], bh[q], acc);
            if constexpr (SPLIT) {
              acc = mfma32(oh[q], bl[q], acc);
              acc = mfma32(ol[q], bh[q], acc);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            const bf16x8_t oh = tr_read(part(mat[q], 0), nt, s);
            f32x16_t& acc = q < 2 ? ub[nt] : kb[nt];
            acc = mfma32(oh, bh[q], acc);
            if constexpr (SPLIT) {
              const bf16x8_t ol = tr_read(part(mat[q], 1), nt, s);
              acc = mfma32(oh, bl[q], acc);
              acc = mfma32(ol, bh[q], acc);
            }
          }
        }
      }
    }
    __syncthreads();  // every wave is done with tile jt
    if (jt + 1 < ntile) dma_w(jt + 1);
  }
  // outputs (lane = key, register r = feature 32 nt + 8 (r / 4) + 4 g + r % 4)
  if (live) {
    uint16_t* dK = static_cast<uint16_t*>(a.dA) + pair * a.out_stride + t * D;
    uint16_t* dV = static_cast<uint16_t*>(a.dB) + pair * a.out_stride + t * D;
    const uint16_t* Vr = static_cast<const uint16_t*>(a.B) + pair * a.in_stride + t * D;
    float de = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int f = 32 * nt + 8 * rg + 4 * g;
        const bf16x4_t v4 = *reinterpret_cast<const bf16x4_t*>(Vr + f);
        bf16x4_t k4, w4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u = ub[nt][4 * rg + i];
          k4[i] = static_cast<__bf16>(kb[nt][4 * rg + i]);
          w4[i] = static_cast<__bf16>(ne * u);
          de -= u * static_cast<float>(v4[i]);
        }
        *reinterpret_cast<bf16x4_t*>(dK + f) = k4;
        *reinterpret_cast<bf16x4_t*>(dV + f) = w4;
      }
    }
    de += __shfl_xor(de, 32, 64);
    if (g == 0) a.deta[pair * a.deta_stride + t] = de;  // (both halves of a key are live or not)
  }
}

}  // namespace

bool bw_contract_mfma_ok(const BwContractArgs& a) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.B) |
                       reinterpret_cast<uintptr_t>(a.X1) | reinterpret_cast<uintptr_t>(a.X2) |
                       reinterpret_cast<uintptr_t>(a.X3);
  return a.bf16 && (a.d == 64 || a.d == 128) && a.h % HS == 0 && (al & 15) == 0 && (a.in_stride % 8) == 0 &&
         (a.x_stride % 4) == 0 && a.n * a.d < (int64_t(1) << 31);
}

hipError_t launch_bw_contract_mfma(const BwContractArgs& a, hipStream_t s) {
  const int hsl = a.h / HS;
  const int nbase = a.S * a.P;
  const int blocks = ((nbase + 7) / 8) * 8 * hsl;
  if (a.d == 128) {
    if (a.split)
      hipLaunchKernelGGL((k_bw_contract_mfma<128, true, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
    else if (a.x_bf16)
      hipLaunchKernelGGL((k_bw_contract_mfma<128, false, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
    else
      hipLaunchKernelGGL((k_bw_contract_mfma<128, false, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else if (a.d == 64) {
    if (a.split)
      hipLaunchKernelGGL((k_bw_contract_mfma<64, true, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
    else if (a.x_bf16)
      hipLaunchKernelGGL((k_bw_contract_mfma<64, false, true>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
    else
      hipLaunchKernelGGL((k_bw_contract_mfma<64, false, false>), dim3(blocks), dim3(kThreads), 0, s, a, hsl, nbase);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lact

namespace lact {

bool bw_tok_mfma_ok(const BwTokArgs& a, bool apply) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.B) |
                       reinterpret_cast<uintptr_t>(a.X1) | reinterpret_cast<uintptr_t>(a.X2) |
                       reinterpret_cast<uintptr_t>(a.X3) | reinterpret_cast<uintptr_t>(a.dA) |
                       reinterpret_cast<uintptr_t>(a.op);
  const uintptr_t al2 = apply ? 0 : reinterpret_cast<uintptr_t>(a.dB);
  return a.op != nullptr && a.bf16 && (a.d == 64 || a.d == 128) && a.h % JT == 0 && ((al | al2) & 15) == 0 &&
         (a.in_stride % 8) == 0 && (a.out_stride % 8) == 0 && (a.x_stride % 4) == 0 && (apply || a.eta != nullptr);
}

hipError_t launch_bw_ops(const BwOpsArgs& a, hipStream_t s) {
  if ((a.d != 64 && a.d != 128) || (a.nm != 3 && a.nm != 6) ||
      a.op_stride < static_cast<int64_t>(2) * a.nm * a.h * a.d || static_cast<int64_t>(a.P) * (a.nm / 3) > 65535)
    return hipErrorInvalidValue;
  const int64_t total = static_cast<int64_t>(a.P) * (a.nm == 6 ? 4 : 2) * a.h * a.d / 4;
  const dim3 grid(static_cast<unsigned>((total + kThreads - 1) / kThreads));
  const dim3 grid_tr(static_cast<unsigned>((a.h + 63) / 64), static_cast<unsigned>((a.d + 63) / 64),
                     static_cast<unsigned>(a.P * (a.nm / 3)));
  if (a.d == 128) {
    hipLaunchKernelGGL(k_bw_ops<128>, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(k_bw_ops_tr<128>, grid_tr, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_bw_ops<64>, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(k_bw_ops_tr<64>, grid_tr, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bw_tok_mfma(const BwTokArgs& a, bool apply, hipStream_t s) {
  const int64_t total = (a.n + QWG - 1) / QWG * a.P;
  const dim3 grid(static_cast<unsigned>((total + 7) / 8 * 8));
  if (a.d == 128 && a.split) {
    if (apply) hipLaunchKernelGGL((k_bw_apply_mfma<128, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_bw_grad_mfma<128, true>), grid, dim3(kThreads), 0, s, a);
  } else if (a.d == 128) {
    if (apply) hipLaunchKernelGGL((k_bw_apply_mfma<128, false>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_bw_grad_mfma<128, false>), grid, dim3(kThreads), 0, s, a);
  } else if (a.d == 64 && a.split) {
    if (apply) hipLaunchKernelGGL((k_bw_apply_mfma<64, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_bw_grad_mfma<64, true>), grid, dim3(kThreads), 0, s, a);
  } else if (a.d == 64) {
    if (apply) hipLaunchKernelGGL((k_bw_apply_mfma<64, false>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_bw_grad_mfma<64, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lact

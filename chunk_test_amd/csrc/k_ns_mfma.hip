// The update tail of a Muon step, one workgroup per fast-weight matrix
// (W1, W2 or W3 of one pair): fixed-order sum of the token-split partial
// gradients, the momentum update when one is kept, Newton-Schulz
// orthogonalisation (Muon's transform, "LaCT: Large Chunk Test-Time
// Training" review, section "Local attention and nonlinear memory work
// together"; coefficients as given in the layer configuration) on bf16 MFMA
// with split operands, then W <- W - step X and the row normalisation (unit
// rows, or with norm_keep every row back to its length before the step) and,
// when asked, a bf16 copy of the new W for the next query read (in the
// operand order of wb_tiled).
//
// X is the s x l orientation of the gradient (s = min(d, h), l = max(d, h)),
// X0 = G / (||G||_F + eps), then `iters` times
//     A = X X^T,  B = b A + c A A,  X <- a X + B X.
// Every product uses the three-term split x = x_hi + x_lo (both bf16):
//     P Q ~ P_hi Q_hi + P_hi Q_lo + P_lo Q_hi   (fp32 accumulation),
// which keeps ~16 significant bits per operand.  Plain bf16 operands move
// the orthogonalised result by ~3e-2 (relative) and the updated weights by
// ~2e-2, which the split avoids.
//
// Work split: wave w owns CT tiles of 32 columns of X, in registers in the
// MFMA output layout (fp32 between steps; during a step only as packed
// hi / lo bf16 pairs, and X <- a X + B X takes X as hi + lo, which is as
// precise as the products; at s = 64, l = 128 the fp32 X stays live, see
// NSGeo::PRE).  That layout is directly the B operand of B X
// (16 rows of X per k-step), so only two LDS layouts are needed: X
// row-major (for X X^T, written once per iteration) and the symmetric s x s
// matrices A and then B (written as the transpose of their own output
// tiles, which for a symmetric matrix is the matrix itself).
#include "lact_device.h"
#include "lact_internal.h"
#include "apply_body.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// the same split for two values, as packed bf16 pairs (element 0 in the low half)
__device__ __forceinline__ void split2(float x0, float x1, unsigned& hi, unsigned& lo) {
  bf16x2_t h, l;
  h[0] = static_cast<__bf16>(x0);
  h[1] = static_cast<__bf16>(x1);
  l[0] = static_cast<__bf16>(x0 - static_cast<float>(h[0]));
  l[1] = static_cast<__bf16>(x1 - static_cast<float>(h[1]));
  hi = __builtin_bit_cast(unsigned, h);
  lo = __builtin_bit_cast(unsigned, l);
}

// element k (0 or 1) of a packed bf16 pair, as a float
__device__ __forceinline__ float bf16_half(unsigned w, int k) {
  return __uint_as_float(k ? (w & 0xffff0000u) : (w << 16));
}

// Split-operand products of NQ 32 x 32 tiles, all over the same KSTEPS
// k-steps: for tile q, hh[q] += P_hi Q_hi^T and cross[q] += P_hi Q_lo^T +
// P_lo Q_hi^T, with P rows at pa[q] and Q rows at pb[q] (row-major bf16 in
// LDS, the 16-byte operand slice of k-step ks at byte koff(ks) of the row;
// the lo block `half` bytes after the hi block).  With PRE every operand of the phase is read before the first
// product (one wave per SIMD has no other wave to hide the read latency);
// otherwise the k loop is unrolled and the tiles interleaved inside it, so
// the reads of one k-step overlap the products of the previous ones.
template <int NQ, int KSTEPS, bool PRE, bool SWZ>
__device__ __forceinline__ void split_tiles(const unsigned char* const (&pa)[NQ],
                                            const unsigned char* const (&pb)[NQ], int yx, int half,
                                            f32x16_t (&hh)[NQ], f32x16_t (&cross)[NQ]) {
  // byte offset of k-step ks in a row: 16-byte chunk 2 ks + g, in swizzled
  // rows chunk (2 ks + g) ^ xsw(row) with yx = 16 (g ^ xsw(row)) (xsw < 16
  // leaves bit 4 of the chunk index, 256-byte steps, alone); otherwise yx = 16 g
  auto koff = [&](int ks) { return SWZ ? (((32 * ks) & 255) ^ yx) + 256 * (ks >> 3) : yx + 32 * ks; };
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      hh[q][r] = 0.f;
      cross[q][r] = 0.f;
    }
  }
  if constexpr (PRE) {
    bf16x8_t ah[KSTEPS][NQ], al[KSTEPS][NQ], bh[KSTEPS][NQ], bl[KSTEPS][NQ];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        ah[ks][q] = *reinterpret_cast<const bf16x8_t*>(pa[q] + koff(ks));
        bh[ks][q] = *reinterpret_cast<const bf16x8_t*>(pb[q] + koff(ks));
        al[ks][q] = *reinterpret_cast<const bf16x8_t*>(pa[q] + half + koff(ks));
        bl[ks][q] = *reinterpret_cast<const bf16x8_t*>(pb[q] + half + koff(ks));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        hh[q] = mfma(ah[ks][q], bh[ks][q], hh[q]);
        cross[q] = mfma(ah[ks][q], bl[ks][q], cross[q]);
        cross[q] = mfma(al[ks][q], bh[ks][q], cross[q]);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      bf16x8_t ah[NQ], al[NQ], bh[NQ], bl[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        ah[q] = *reinterpret_cast<const bf16x8_t*>(pa[q] + koff(ks));
        al[q] = *reinterpret_cast<const bf16x8_t*>(pa[q] + half + koff(ks));
        bh[q] = *reinterpret_cast<const bf16x8_t*>(pb[q] + koff(ks));
        bl[q] = *reinterpret_cast<const bf16x8_t*>(pb[q] + half + koff(ks));
      }
      // the two cross products of a tile are NQ products apart
#pragma unroll
      for (int q = 0; q < NQ; ++q) hh[q] = mfma(ah[q], bh[q], hh[q]);
#pragma unroll
      for (int q = 0; q < NQ; ++q) cross[q] = mfma(ah[q], bl[q], cross[q]);
#pragma unroll
      for (int q = 0; q < NQ; ++q) cross[q] = mfma(al[q], bh[q], cross[q]);
    }
  }
}

// Row-major X in LDS: 16-byte chunk c of row r sits at chunk c ^ xsw(r),
// xsw(r) = 4 (r % 4) + (r / 4) % 4.  The operand reads of X X^T (16 rows in a
// row, one chunk: xsw is one-to-one on r % 16) and the 8-byte stores of
// quad_tr's output (rows 4m .. 4m + 3, eight 8-byte column groups: the rows
// differ in bits 2, 3 of xsw, the groups in bits 0, 1 and in the half
// chunk) are both free of bank conflicts.
__device__ __forceinline__ int xsw(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

__device__ __forceinline__ unsigned dpp_u32_xor1(unsigned v) {
  return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ unsigned dpp_u32_xor2(unsigned v) {
  return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));
}

// 4 x 4 transpose of bf16 values across the four lanes of a quad: on entry
// lane p holds column p, rows 0-3 as w0 = (row 0, row 1), w1 = (row 2, row 3)
// (element 0 in the low half); on exit it holds row p, columns 0-3 as
// w0 = (column 0, column 1), w1 = (column 2, column 3).  Two butterfly
// exchanges: 16-bit halves with lane p ^ 1, then words with lane p ^ 2.
__device__ __forceinline__ void quad_tr(unsigned& w0, unsigned& w1, int p) {
  const unsigned r0 = dpp_u32_xor1(w0), r1 = dpp_u32_xor1(w1);
  // even lanes: (own low, partner's low); odd lanes: (partner's high, own high)
  const unsigned sel = (p & 1) ? 0x03020706u : 0x05040100u;
  const unsigned n0 = __builtin_amdgcn_perm(r0, w0, sel);
  const unsigned n1 = __builtin_amdgcn_perm(r1, w1, sel);
  const unsigned send = (p & 2) ? n0 : n1;
  const unsigned recv = dpp_u32_xor2(send);
  w0 = (p & 2) ? recv : n0;
  w1 = (p & 2) ? n1 : recv;
}

// Tile u of the tiles on and above the diagonal of an MT x MT tile grid, row
// by row: (0, 0), (0, 1), .., (0, MT - 1), (1, 1), ...
template <int MT>
__device__ __forceinline__ void upper_tile(int u, int& ti, int& tj) {
  ti = 0;
#pragma unroll
  for (int r = 0; r < MT - 1; ++r) {
    if (u >= MT - ti) {
      u -= MT - ti;
      ++ti;
    }
  }
  tj = ti + u;
}

// Column order of the stored s x s matrices A and B: inside every 16 columns
// the two groups {0-3, 8-11} and {4-7, 12-15} are stored as contiguous runs of
// eight, so the B X step (whose k order follows the MFMA output rows of X)
// reads its operand as one 16-byte slice per lane.  Products over A's columns
// read both operands in the same stored order, which leaves them unchanged.
// Column 32 ti + 8 rg + 4 g + i (i < 4) is stored at the returned column.
__device__ __forceinline__ int stored_col(int ti, int rg, int g) {
  return 32 * ti + 16 * (rg >> 1) + 8 * g + 4 * (rg & 1);
}

template <int S, int L>
struct NSGeo {
  static constexpr int NW = L / 32;          // waves
  static constexpr int CT = L / (32 * NW);   // 32-column tiles of X per wave (1)
  static constexpr int MT = S / 32;          // 32-row tiles of X (and of A)
  static constexpr int XRS = 2 * L;          // bytes per row of X (bf16; 16-byte chunks swizzled, see xsw)
  static constexpr int X_HALF = S * XRS;     // hi block, then lo block
  static constexpr int ARS = 2 * S + 16;     // bytes per row of A / B
  static constexpr int A_HALF = S * ARS;
  // fp32 staging of G and of the final X in the stored matrix's own
  // orientation: rows of rowlen floats (S for the tall W1, W3, L for W2)
  // padded by 16 bytes
  static constexpr int STG_TALL = L * (4 * S + 16);
  static constexpr int STG_WIDE = S * (4 * L + 16);
  static constexpr int STG = STG_TALL > STG_WIDE ? STG_TALL : STG_WIDE;
  static constexpr int R1 = (2 * X_HALF > 2 * A_HALF) ? 2 * X_HALF : 2 * A_HALF;
  static constexpr int REGION = (R1 > STG) ? R1 : STG;  // the staging shares the region
  static constexpr int ATILES = MT * MT;
  // with two wavefronts per SIMD (eight in all) only the tiles on and above
  // the diagonal of the symmetric A and B are computed (NU of them, at most
  // UTW per wave: three per SIMD instead of four at s = 128) and each is
  // stored in both places
  static constexpr bool SYM = (NW == 8);
  static constexpr int NU = MT * (MT + 1) / 2;
  static constexpr int UTW = (NU + NW - 1) / NW;
  static constexpr int ATW0 = (ATILES + NW - 1) / NW;
  static constexpr int ATW = SYM ? UTW : ATW0;  // A tiles per wave
  // one wave per SIMD with registers to spare: read each phase's operands
  // ahead, keep X in fp32 across the iteration, load W at the start
  static constexpr bool PRE = (S == 64 && L == 128);
};

// The tail of one matrix; TR: G is tall (stored l x s), X = G^T.  (One body
// per orientation, so that each is straight-line code for the register
// allocator.)
template <int S, int L, bool TR>
__device__ __forceinline__ void muon_tail_body(const TailArgs& a, unsigned char* lds, float* red, int pair,
                                               int which) {
  using G = NSGeo<S, L>;
  const int64_t hd = static_cast<int64_t>(a.h) * a.d;
  constexpr bool tr = TR;
  float* Wm = (which == 0 ? a.W1 : which == 1 ? a.W2 : a.W3) + pair * hd;
  float* Mm = (a.M1 == nullptr) ? nullptr : (which == 0 ? a.M1 : which == 1 ? a.M2 : a.M3) + pair * hd;
  uint16_t* Wbm = (a.Wb1 == nullptr) ? nullptr : (which == 0 ? a.Wb1 : which == 1 ? a.Wb2 : a.Wb3) + pair * hd;
  const float* part = a.partials + static_cast<int64_t>(pair) * a.splits * 3 * hd + which * hd;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, ln = lane & 31;
  // column tile ct of this wave holds columns 32 (NW ct + w) .. +31
  auto colof = [&](int ct) { return 32 * (G::NW * ct + w) + ln; };

  // ---- G = sum of the split partials in fixed order (then the momentum
  // update M <- beta M + G, G <- M), staged through LDS in G's own row-major
  // order (rows of rowlen floats, padded to grs bytes) so the global reads
  // and the staging stores move 16-byte groups.  X0 = G / (||G||_F + eps) in
  // registers, MFMA output layout:
  // x[ct][mt][r] = X[32 mt + 8 (r/4) + 4 g + r%4][colof(ct)].  When G is tall
  // (X = G^T), the four X rows of a register group are four consecutive
  // floats of one staged row (one 16-byte read); otherwise they are four
  // staged rows (lanes read consecutive words of each).
  const int rowlen = tr ? S : L;  // (S and L are powers of two)
  const int lg_rowlen = tr ? __builtin_ctz(S) : __builtin_ctz(L);
  const int grs = 4 * rowlen + 16;
  constexpr int NV = S * L / 4;  // float4 groups per matrix
  constexpr int GPT = NV / (2 * L);
  float4* W4 = reinterpret_cast<float4*>(Wm);
  float4 wv[GPT];
  const float4* part4 = reinterpret_cast<const float4*>(part);
  const int64_t sstride4 = 3 * hd / 4;
  // every thread sums CPT float4 groups (tid + 2 L k) over the splits, with
  // UD splits x CPT groups of loads in flight, in split order
  constexpr int CPT = NV / (2 * L);
  constexpr int UD = CPT >= 32 ? 1 : 32 / CPT;
  float4 acc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  int sp = 0;
  for (; sp + UD <= a.splits; sp += UD) {
    float4 t[UD][CPT];
#pragma unroll
    for (int u = 0; u < UD; ++u) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) t[u][k] = part4[(sp + u) * sstride4 + tid + 2 * L * k];
    }
#pragma unroll
    for (int u = 0; u < UD; ++u) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        acc[k].x += t[u][k].x;
        acc[k].y += t[u][k].y;
        acc[k].z += t[u][k].z;
        acc[k].w += t[u][k].w;
      }
    }
  }
  for (; sp < a.splits; ++sp) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const float4 t = part4[sp * sstride4 + tid + 2 * L * k];
      acc[k].x += t.x;
      acc[k].y += t.y;
      acc[k].z += t.z;
      acc[k].w += t.w;
    }
  }
  if constexpr (G::PRE) {
#pragma unroll
    for (int k = 0; k < GPT; ++k) wv[k] = W4[tid + 2 * L * k];
  }
  if (Mm != nullptr) {
    // M <- beta M + G, G <- M (all loads issued before the first store)
    float4* M4 = reinterpret_cast<float4*>(Mm);
    float4 mv[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) mv[k] = M4[tid + 2 * L * k];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      acc[k].x = a.beta * mv[k].x + acc[k].x;
      acc[k].y = a.beta * mv[k].y + acc[k].y;
      acc[k].z = a.beta * mv[k].z + acc[k].z;
      acc[k].w = a.beta * mv[k].w + acc[k].w;
      M4[tid + 2 * L * k] = acc[k];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int e = 4 * (tid + 2 * L * k);
    ss += acc[k].x * acc[k].x + acc[k].y * acc[k].y + acc[k].z * acc[k].z + acc[k].w * acc[k].w;
    *reinterpret_cast<float4*>(lds + (e >> lg_rowlen) * grs + 4 * (e & (rowlen - 1))) = acc[k];
  }
  {
    float t[1] = {ss};
    group_sums<64>(t);
    ss = t[0];
  }
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < G::NW; ++i) tot += red[i];
  const float inv_denom = 1.f / (sqrtf(tot) + a.eps);
  f32x16_t x[G::CT][G::MT];
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) {
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      if (tr) {
        const unsigned char* xb = lds + colof(ct) * grs + 4 * (32 * mt + 4 * g);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float4 v = *reinterpret_cast<const float4*>(xb + 32 * rg);
          x[ct][mt][4 * rg] = v.x * inv_denom;
          x[ct][mt][4 * rg + 1] = v.y * inv_denom;
          x[ct][mt][4 * rg + 2] = v.z * inv_denom;
          x[ct][mt][4 * rg + 3] = v.w * inv_denom;
        }
      } else {
        const unsigned char* xb = lds + (32 * mt + 4 * g) * grs + 4 * colof(ct);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          x[ct][mt][r] = *reinterpret_cast<const float*>(xb + (8 * (r >> 2) + (r & 3)) * grs) * inv_denom;
      }
    }
  }

  unsigned char* xhi = lds;
  unsigned char* ahi = lds;
  unsigned char* alo = lds + G::A_HALF;

  // Stores tile (ti, tj) of a symmetric s x s matrix (A or B) as hi / lo
  // bf16: transposed, at rows 32 tj + ln, columns 32 ti + 8 (r/4) + 4 g .. +3
  // (four consecutive bf16 per store, at their stored columns), which for a
  // symmetric matrix is tile (tj, ti); off the diagonal, with only the tiles
  // on and above it computed, also in place, through a quad transpose
  // (lane p of quad m then holds row 32 ti + 8 rg + 4 g + p, columns
  // 32 tj + 4 m .. +3).
  auto store_sym = [&](const f32x16_t& v, int ti, int tj) {
    const int p = ln & 3, m = ln >> 2;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      bf16x4_t h4, l4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __bf16 hi, lo;
        split(v[4 * rg + i], hi, lo);
        h4[i] = hi;
        l4[i] = lo;
      }
      const int off = (32 * tj + ln) * G::ARS + 2 * stored_col(ti, rg, g);
      *reinterpret_cast<bf16x4_t*>(ahi + off) = h4;
      *reinterpret_cast<bf16x4_t*>(alo + off) = l4;
      if (G::SYM && ti != tj) {
        unsigned hw0 = __builtin_bit_cast(unsigned, bf16x2_t{h4[0], h4[1]});
        unsigned hw1 = __builtin_bit_cast(unsigned, bf16x2_t{h4[2], h4[3]});
        unsigned lw0 = __builtin_bit_cast(unsigned, bf16x2_t{l4[0], l4[1]});
        unsigned lw1 = __builtin_bit_cast(unsigned, bf16x2_t{l4[2], l4[3]});
        quad_tr(hw0, hw1, p);
        quad_tr(lw0, lw1, p);
        const int off2 = (32 * ti + 8 * rg + 4 * g + p) * G::ARS + 2 * stored_col(tj, m >> 1, m & 1);
        *reinterpret_cast<uint2*>(ahi + off2) = make_uint2(hw0, hw1);
        *reinterpret_cast<uint2*>(alo + off2) = make_uint2(lw0, lw1);
      }
    }
  };

  for (int it = 0; it < a.iters; ++it) {
    // ---- X split once into hi / lo bf16 operands, kept in registers as
    // packed pairs in the B-operand order of B X (k-step s, slot i <->
    // x[ct][s / 2][8 (s % 2) + i]), and written row-major into LDS for X X^T
    u32x4_t xh[G::CT][S / 16], xl[G::CT][S / 16];
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
#pragma unroll
      for (int ks = 0; ks < S / 16; ++ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 8 * (ks & 1) + 2 * j;
          unsigned wh, wl;
          split2(x[ct][ks >> 1][r], x[ct][ks >> 1][r + 1], wh, wl);
          xh[ct][ks][j] = wh;
          xl[ct][ks][j] = wl;
        }
      }
    }
    __syncthreads();
    // row-major stores: every group of four rows of a lane quad is
    // transposed across the quad (lane p then holds row 4 m' + p, four
    // consecutive columns) and stored as 8 bytes
    {
      const int p = ln & 3;
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        // logical chunk and half of the quad's four columns
        const int lc = 4 * (G::NW * ct + w) + (ln >> 3), hf = (ln >> 2) & 1;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int ks = 2 * mt + (rg >> 1), j = 2 * (rg & 1);
            unsigned h0 = xh[ct][ks][j], h1 = xh[ct][ks][j + 1];
            unsigned l0 = xl[ct][ks][j], l1 = xl[ct][ks][j + 1];
            quad_tr(h0, h1, p);
            quad_tr(l0, l1, p);
            const int row = 32 * mt + 8 * rg + 4 * g + p;
            const int off = row * G::XRS + 16 * (lc ^ (4 * p + ((2 * rg + g) & 3))) + 8 * hf;
            *reinterpret_cast<uint2*>(xhi + off) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(xhi + G::X_HALF + off) = make_uint2(l0, l1);
          }
        }
      }
    }
    __syncthreads();

    // ---- A = X X^T: this wave's tiles (ti, tj) = (t / MT, t % MT),
    // t = w + NW q; K = l
    f32x16_t at[G::ATW];
    // chunk 2 ks + g of row 32 t + ln, swizzled (xsw depends on ln % 16 only)
    const int yx = 16 * (g ^ xsw(ln));
    if constexpr (G::SYM) {
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
        const int u = w + G::NW * q;
#pragma unroll
        for (int r = 0; r < 16; ++r) at[q][r] = 0.f;
        if (u < G::NU) {
          int ti, tj;
          upper_tile<G::MT>(u, ti, tj);
          const unsigned char* pa[1] = {xhi + (32 * ti + ln) * G::XRS};
          const unsigned char* pb[1] = {xhi + (32 * tj + ln) * G::XRS};
          f32x16_t hh[1], a2[1];
          split_tiles<1, L / 16, false, true>(pa, pb, yx, G::X_HALF, hh, a2);
#pragma unroll
          for (int r = 0; r < 16; ++r) at[q][r] = hh[0][r] + a2[0][r];
        }
      }
    } else if constexpr (G::ATILES % G::NW == 0) {
      const unsigned char* pa[G::ATW];
      const unsigned char* pb[G::ATW];
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
        const int t = w + G::NW * q;
        pa[q] = xhi + (32 * (t / G::MT) + ln) * G::XRS;
        pb[q] = xhi + (32 * (t % G::MT) + ln) * G::XRS;
      }
      f32x16_t a2[G::ATW];
      split_tiles<G::ATW, L / 16, G::PRE, true>(pa, pb, yx, G::X_HALF, at, a2);
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
#pragma unroll
        for (int r = 0; r < 16; ++r) at[q][r] += a2[q][r];
      }
    } else {
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
        const int t = w + G::NW * q;
#pragma unroll
        for (int r = 0; r < 16; ++r) at[q][r] = 0.f;
        if (t < G::ATILES) {
          const unsigned char* pa[1] = {xhi + (32 * (t / G::MT) + ln) * G::XRS};
          const unsigned char* pb[1] = {xhi + (32 * (t % G::MT) + ln) * G::XRS};
          f32x16_t hh[1], a2[1];
          split_tiles<1, L / 16, false, true>(pa, pb, yx, G::X_HALF, hh, a2);
#pragma unroll
          for (int r = 0; r < 16; ++r) at[q][r] = hh[0][r] + a2[0][r];
        }
      }
    }
    __syncthreads();  // X row-major no longer needed: the region becomes A

    // A is symmetric: tile (ti, tj) transposed lands at rows 32 tj + ln,
    // columns 32 ti + 8 (r/4) + 4 g .. +3 (four consecutive bf16 per store,
    // at their stored columns)
#pragma unroll
    for (int q = 0; q < G::ATW; ++q) {
      const int t = w + G::NW * q;
      if (t < (G::SYM ? G::NU : G::ATILES)) {
        int ti, tj;
        if constexpr (G::SYM) {
          upper_tile<G::MT>(t, ti, tj);
        } else {
          ti = t / G::MT;
          tj = t % G::MT;
        }
        store_sym(at[q], ti, tj);
      }
    }
    __syncthreads();

    // ---- B = b A + c A A on the same tiles (A symmetric: both operands are rows of A)
    if constexpr (G::SYM) {
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
        const int u = w + G::NW * q;
        if (u < G::NU) {
          int ti, tj;
          upper_tile<G::MT>(u, ti, tj);
          const unsigned char* pa[1] = {ahi + (32 * ti + ln) * G::ARS};
          const unsigned char* pb[1] = {ahi + (32 * tj + ln) * G::ARS};
          f32x16_t acc[1], a2[1];
          split_tiles<1, S / 16, false, false>(pa, pb, 16 * g, G::A_HALF, acc, a2);
#pragma unroll
          for (int r = 0; r < 16; ++r) at[q][r] = a.b * at[q][r] + a.c * (acc[0][r] + a2[0][r]);  // now B
        }
      }
    } else if constexpr (G::ATILES % G::NW == 0) {
      const unsigned char* pa[G::ATW];
      const unsigned char* pb[G::ATW];
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
        const int t = w + G::NW * q;
        pa[q] = ahi + (32 * (t / G::MT) + ln) * G::ARS;
        pb[q] = ahi + (32 * (t % G::MT) + ln) * G::ARS;
      }
      f32x16_t acc[G::ATW], a2[G::ATW];
      split_tiles<G::ATW, S / 16, G::PRE, false>(pa, pb, 16 * g, G::A_HALF, acc, a2);
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
#pragma unroll
        for (int r = 0; r < 16; ++r) at[q][r] = a.b * at[q][r] + a.c * (acc[q][r] + a2[q][r]);  // now B
      }
    } else {
#pragma unroll
      for (int q = 0; q < G::ATW; ++q) {
        const int t = w + G::NW * q;
        if (t < G::ATILES) {
          const unsigned char* pa[1] = {ahi + (32 * (t / G::MT) + ln) * G::ARS};
          const unsigned char* pb[1] = {ahi + (32 * (t % G::MT) + ln) * G::ARS};
          f32x16_t acc[1], a2[1];
          split_tiles<1, S / 16, false, false>(pa, pb, 16 * g, G::A_HALF, acc, a2);
#pragma unroll
          for (int r = 0; r < 16; ++r) at[q][r] = a.b * at[q][r] + a.c * (acc[0][r] + a2[0][r]);  // now B
        }
      }
    }
    __syncthreads();  // all reads of A done: the region becomes B
    // B is symmetric too: same store
#pragma unroll
    for (int q = 0; q < G::ATW; ++q) {
      const int t = w + G::NW * q;
      if (t < (G::SYM ? G::NU : G::ATILES)) {
        int ti, tj;
        if constexpr (G::SYM) {
          upper_tile<G::MT>(t, ti, tj);
        } else {
          ti = t / G::MT;
          tj = t % G::MT;
        }
        store_sym(at[q], ti, tj);
      }
    }
    __syncthreads();

    // ---- X <- a X + B X for this wave's 32 columns.  The B operand (X,
    // 16 rows per k-step) comes from this lane's own registers; the A
    // operand (rows of B) uses the matching row order:
    // slot 8g + i of k-step s <-> row 16 s + 8 (i/4) + 4 g + i%4, which is
    // stored column 16 s + 8 g + i (one 16-byte read per lane and half).
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      f32x16_t accs[G::MT];
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) accs[mt][r] = 0.f;
      }
      bf16x8_t bh[G::PRE ? S / 16 : 1][G::MT], bl[G::PRE ? S / 16 : 1][G::MT];
      if constexpr (G::PRE) {
#pragma unroll
        for (int s = 0; s < S / 16; ++s) {
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt) {
            const unsigned char* rb = ahi + (32 * mt + ln) * G::ARS + 16 * g + 32 * s;
            bh[s][mt] = *reinterpret_cast<const bf16x8_t*>(rb);
            bl[s][mt] = *reinterpret_cast<const bf16x8_t*>(rb + G::A_HALF);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // products of one k-step, the MT tiles interleaved (a tile's three
      // products are MT apart)
#pragma unroll
      for (int s = 0; s < S / 16; ++s) {
        const int sp = G::PRE ? s : 0;
        if constexpr (!G::PRE) {
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt) {
            const unsigned char* rb = ahi + (32 * mt + ln) * G::ARS + 16 * g + 32 * s;
            bh[0][mt] = *reinterpret_cast<const bf16x8_t*>(rb);
            bl[0][mt] = *reinterpret_cast<const bf16x8_t*>(rb + G::A_HALF);
          }
        }
        const bf16x8_t oh = __builtin_bit_cast(bf16x8_t, xh[ct][s]);
        const bf16x8_t ol = __builtin_bit_cast(bf16x8_t, xl[ct][s]);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) accs[mt] = mfma(bh[sp][mt], oh, accs[mt]);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) accs[mt] = mfma(bh[sp][mt], ol, accs[mt]);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) accs[mt] = mfma(bl[sp][mt], oh, accs[mt]);
      }
      // X <- a X + B X.  With PRE the fp32 X stays live across the
      // iteration; otherwise X is taken as hi + lo (~16 significant bits,
      // the precision of every product here), which frees its registers.
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (G::PRE) {
            x[ct][mt][r] = a.a * x[ct][mt][r] + accs[mt][r];
          } else {
            const int ks = 2 * mt + (r >> 3), j = (r & 7) >> 1, k = r & 1;
            const float xv = bf16_half(xh[ct][ks][j], k) + bf16_half(xl[ct][ks][j], k);
            x[ct][mt][r] = a.a * xv + accs[mt][r];
          }
        }
      }
    }
  }

  // ---- W <- W - step X, then unit L2 rows.  Every thread takes GPT float4
  // groups of the stored matrix (rows of `rowlen`, rowlen / 4 lanes per row,
  // so a row's lanes are an aligned lane group); all W loads are issued
  // together (with PRE at the start of the kernel, otherwise here, once X
  // is in LDS), so their latency is paid once.  X goes back to the staging
  // layout (W1, W3 rows are columns of X, W2 rows are rows of X).
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) {
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      if (tr) {
        unsigned char* xb = lds + colof(ct) * grs + 4 * (32 * mt + 4 * g);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<float4*>(xb + 32 * rg) =
              make_float4(x[ct][mt][4 * rg], x[ct][mt][4 * rg + 1], x[ct][mt][4 * rg + 2], x[ct][mt][4 * rg + 3]);
      } else {
        unsigned char* xb = lds + (32 * mt + 4 * g) * grs + 4 * colof(ct);
#pragma unroll
        for (int r = 0; r < 16; ++r) *reinterpret_cast<float*>(xb + (8 * (r >> 2) + (r & 3)) * grs) = x[ct][mt][r];
      }
    }
  }
  if constexpr (!G::PRE) {
#pragma unroll
    for (int k = 0; k < GPT; ++k) wv[k] = W4[tid + 2 * L * k];
  }
  __syncthreads();
  // (every row's squared norm first, then all GPT group reductions together,
  // so their shuffle latencies overlap)
  float v[GPT][4], sq[GPT], sq_old[GPT];
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int e = 4 * (tid + 2 * L * k);
    const float4 xs = *reinterpret_cast<const float4*>(lds + (e >> lg_rowlen) * grs + 4 * (e & (rowlen - 1)));
    const float xq[4] = {xs.x, xs.y, xs.z, xs.w};
    v[k][0] = wv[k].x;
    v[k][1] = wv[k].y;
    v[k][2] = wv[k].z;
    v[k][3] = wv[k].w;
    sq_old[k] = v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
    sq[k] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[k][q] -= a.step * xq[q];
      sq[k] += v[k][q] * v[k][q];
    }
  }
  const float inv_eps = 1.f / a.norm_eps;
  if (tr) {
    group_sums<S / 4>(sq);
    if (a.norm_keep) group_sums<S / 4>(sq_old);
  } else {
    group_sums<L / 4>(sq);
    if (a.norm_keep) group_sums<L / 4>(sq_old);
  }
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    // 1 / max(||r||, eps) as min(1 / sqrt(||r||^2), 1 / eps), the
    // reciprocal square root from the hardware approximation (~1 ulp)
    float inv = fminf(__builtin_amdgcn_rsqf(sq[k]), inv_eps);
    if (a.norm_keep) inv *= sqrtf(sq_old[k]);  // back to the length before the step
    const float4 xw = make_float4(v[k][0] * inv, v[k][1] * inv, v[k][2] * inv, v[k][3] * inv);
    W4[tid + 2 * L * k] = xw;
    if (Wbm != nullptr) {
      bf16x4_t b4;
      b4[0] = static_cast<__bf16>(xw.x);
      b4[1] = static_cast<__bf16>(xw.y);
      b4[2] = static_cast<__bf16>(xw.z);
      b4[3] = static_cast<__bf16>(xw.w);
      const int e = 4 * (tid + 2 * L * k);
      *reinterpret_cast<bf16x4_t*>(Wbm + wb_tiled(e >> lg_rowlen, e & (rowlen - 1), rowlen)) = b4;
    }
  }
}

template <int S, int L>
__global__ __launch_bounds__(2 * L) void k_muon_tail(TailArgs a) {
  using G = NSGeo<S, L>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::REGION];
  __shared__ float red[G::NW];
  const int mat = blockIdx.x;
  const int pair = mat / 3, which = mat % 3;  // 0: W1 (h x d), 1: W2 (d x h), 2: W3 (h x d)
  const int cols = (which == 1) ? a.h : a.d;
  if (((which == 1) ? a.d : a.h) > cols) {
    muon_tail_body<S, L, true>(a, lds, red, pair, which);
  } else {
    muon_tail_body<S, L, false>(a, lds, red, pair, which);
  }
}

// One launch for two independent jobs of the chunk scan (apply-then-update,
// chunk c >= 1): blocks [0, nt) run the Muon update tail of chunk c (one
// matrix each; nt is 3P rounded up to a multiple of 8, the blocks past 3P
// idle), blocks [nt, nt + na) the query read of chunk c, which reads the
// bf16 copy of W_c that the previous tail wrote while this tail writes W_c+1
// and the other copy.  The tail fills only 3P CUs; the query read takes the
// rest of the chip in the same launch (one workgroup per CU for both parts),
// where two launches would run one after the other.
template <int S, int L>
__global__ __launch_bounds__(2 * L) void k_muon_tail_apply(TailArgs ta, ApplyArgs aa, int nt, int na, int per_wg,
                                                          int wg_per_pair) {
  using G = NSGeo<S, L>;
  using AG = apply_detail::AGeo<S, L>;
  static_assert(AG::THREADS == 2 * L, "one block size for both parts");
  // (the tail's partial sums sit after its region, inside the one array)
  constexpr int kRed = (G::REGION + 15) / 16 * 16;
  constexpr int kTail = kRed + 4 * G::NW;
  constexpr int kLds = kTail > AG::LDS ? kTail : AG::LDS;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  float* red = reinterpret_cast<float*>(lds + kRed);
  if (static_cast<int>(blockIdx.x) >= nt) {
    apply_detail::apply_body<S, L, true>(aa, lds, static_cast<int>(blockIdx.x) - nt, na, per_wg, wg_per_pair);
    return;
  }
  const int mat = blockIdx.x;
  if (mat >= 3 * ta.P) return;
  const int pair = mat / 3, which = mat % 3;
  const int cols = (which == 1) ? ta.h : ta.d;
  if (((which == 1) ? ta.d : ta.h) > cols) {
    muon_tail_body<S, L, true>(ta, lds, red, pair, which);
  } else {
    muon_tail_body<S, L, false>(ta, lds, red, pair, which);
  }
}

template <int S, int L>
hipError_t launch_fused(const TailArgs& ta, const ApplyArgs& aa, hipStream_t st) {
  const int nt = (3 * ta.P + 7) / 8 * 8;
  const int slots = (256 - nt) / 8 * 8;
  int per = 0, gx = 0;
  apply_detail::apply_plan<S, L>(aa.m, aa.P, slots, &per, &gx);
  const int na = (gx * aa.P + 7) / 8 * 8;
  hipLaunchKernelGGL((k_muon_tail_apply<S, L>), dim3(nt + na), dim3(2 * L), 0, st, ta, aa, nt, na, per, gx);
  return hipGetLastError();
}

}  // namespace

bool muon_tail_apply_ok(int d, int h, int P) {
  return h > d && ns_mfma_shape_ok(d, h) && apply_mfma_shape_ok(d, h) && 3 * P <= 192;
}

hipError_t launch_muon_tail_apply(const TailArgs& ta, const ApplyArgs& aa, hipStream_t st) {
  if (!muon_tail_apply_ok(ta.d, ta.h, ta.P) || aa.d != ta.d || aa.h != ta.h || aa.P != ta.P ||
      aa.Wb1 == nullptr || aa.Wb2 == nullptr || aa.Wb3 == nullptr)
    return hipErrorInvalidValue;
  if (ta.d == 64 && ta.h == 128) return launch_fused<64, 128>(ta, aa, st);
  if (ta.d == 128 && ta.h == 256) return launch_fused<128, 256>(ta, aa, st);
  if (ta.d == 64 && ta.h == 256) return launch_fused<64, 256>(ta, aa, st);
  return hipErrorInvalidValue;
}

bool ns_mfma_shape_ok(int d, int h) {
  const int s = d < h ? d : h, l = d < h ? h : d;
  return (s == 64 && l == 128) || (s == 128 && l == 256) || (s == 64 && l == 256);
}

hipError_t launch_muon_tail(const TailArgs& a, hipStream_t st) {
  const int s = a.d < a.h ? a.d : a.h, l = a.d < a.h ? a.h : a.d;
  const dim3 grid(3 * a.P);
  if (s == 64 && l == 128) {
    hipLaunchKernelGGL((k_muon_tail<64, 128>), grid, dim3(2 * 128), 0, st, a);
  } else if (s == 128 && l == 256) {
    hipLaunchKernelGGL((k_muon_tail<128, 256>), grid, dim3(2 * 256), 0, st, a);
  } else if (s == 64 && l == 256) {
    hipLaunchKernelGGL((k_muon_tail<64, 256>), grid, dim3(2 * 256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lact

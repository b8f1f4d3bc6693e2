// Causal sliding-window attention beside the TTT layer, the second half of a
// LaCT block ("LaCT: Large Chunk Test-Time Training" review, section "Local
// attention and nonlinear memory work together": window attention captures
// local order inside a chunk; the language and video variants share Q, K, V
// with the TTT layer and add the two outputs).  Query t attends keys s with
// t - window < s <= t:
//   o_t = sum_s softmax_s(scale q_t . k_s) v_s.
//
// bf16 at d = 128 runs on the matrix cores (k_window_attn_mfma below); the
// general kernel (fp32 arithmetic, any supported d and I/O type): one
// workgroup per (64 queries, pair); four threads per query, each owning
// d/4 features of q and of the output.  Key/value tiles of 64 tokens go
// through LDS; per tile the 64 scores of a query are formed first (partial
// dots reduced over the query's four lanes), then the running maximum and
// sum of the online softmax are updated once and the tile's values are
// accumulated (fp32 arithmetic).  With `accumulate` the result is added to
// what O holds (the block's sum with the TTT layer's output).
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

constexpr int kThreads = 256;
constexpr int kQ = 64;   // queries per workgroup
constexpr int kKT = 64;  // keys per tile

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_window_attn(WindowArgs a) {
  constexpr int DP = D / 4;  // features per lane
  __shared__ float sK[kKT][D + 1];
  __shared__ float sV[kKT][D + 1];
  const int pair = blockIdx.y;
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * kQ;
  const int tid = threadIdx.x;
  const int qi = tid >> 2;    // query of this lane group
  const int part = tid & 3;   // its quarter of the features
  const int64_t t = q0 + qi;
  const int64_t base = static_cast<int64_t>(pair) * a.stride;
  const bool valid = t < a.T;
  float q[DP], o[DP];
#pragma unroll
  for (int x = 0; x < DP; ++x) {
    q[x] = valid ? a.scale * load_io<BF16>(a.Q, base + t * D + part * DP + x) : 0.f;
    o[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  // keys any query of the tile can see
  const int64_t q_last = min(q0 + kQ, a.T) - 1;
  int64_t k_lo = q0 - a.window + 1;
  if (k_lo < 0) k_lo = 0;
  k_lo = (k_lo / kKT) * kKT;
  for (int64_t k0 = k_lo; k0 <= q_last; k0 += kKT) {
    __syncthreads();
    for (int i = tid; i < kKT * D; i += kThreads) {
      const int r = i / D, e = i % D;
      const int64_t s = k0 + r;
      const bool ok = s < a.T;
      sK[r][e] = ok ? load_io<BF16>(a.K, base + s * D + e) : 0.f;
      sV[r][e] = ok ? load_io<BF16>(a.V, base + s * D + e) : 0.f;
    }
    __syncthreads();
    float sc[kKT];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < kKT; ++r) {
      float p = 0.f;
#pragma unroll
      for (int x = 0; x < DP; ++x) p = fmaf(q[x], sK[r][part * DP + x], p);
      p += __shfl_xor(p, 1, 64);
      p += __shfl_xor(p, 2, 64);
      const int64_t s = k0 + r;
      const bool in = valid && s <= t && s > t - a.window;
      sc[r] = in ? p : -INFINITY;
      tmax = fmaxf(tmax, sc[r]);
    }
    if (tmax != -INFINITY) {  // some key of this tile is in the query's window
      const float mn = fmaxf(m, tmax);
      const float corr = __expf(m - mn);  // 0 on the first visible tile (m = -inf)
      l *= corr;
#pragma unroll
      for (int x = 0; x < DP; ++x) o[x] *= corr;
#pragma unroll
      for (int r = 0; r < kKT; ++r) {
        const float p = __expf(sc[r] - mn);
        l += p;
#pragma unroll
        for (int x = 0; x < DP; ++x) o[x] = fmaf(p, sV[r][part * DP + x], o[x]);
      }
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = 1.f / l;
#pragma unroll
  for (int x = 0; x < DP; ++x) {
    const int64_t idx = base + t * D + part * DP + x;
    float v = o[x] * inv;
    if (a.accumulate) v += load_io<BF16>(a.O, idx);
    store_io<BF16>(a.O, idx, v);
  }
}

// ---------------------------------------------------------------------------
// bf16 matrix-core variant for d = 128.  A workgroup of four wavefronts owns
// 128 QT consecutive queries of a pair, QT tiles of 32 per wavefront (the
// launch uses QT = 1: two tiles share each key and value read from LDS, but
// need one wavefront per SIMD, which measured 1.5x slower); keys and values of
// 64-token stages move from HBM straight into double-buffered LDS tiles
// (global_load_lds, rows of 256 bytes with their 16-byte chunks XOR-swizzled
// per row).  Per wavefront and 32-key sub-tile, on 32x32x16 MFMAs:
//   S^T = K Q^T   (A = key rows from LDS, B = the wave's queries, held in
//                  registers): lane = query, 16 registers = 16 keys;
//   online softmax in that layout: the maximum of a query is shared with the
//   lane holding its other 16 keys (lane ^ 32); p = 2^(s c - m), c = scale
//   log2(e), where the reference m moves only when a sub-tile's maximum
//   exceeds it by more than 8 (so p <= 2^8), and the output is rarely rescaled;
//   O^T += V^T P^T  (A = value columns from LDS transpose reads, B = p as
//                  bf16 in the same key order): lane = query, registers =
//                  features, so the rescale is per lane.
// Masks are applied only on sub-tiles that cross the diagonal or the
// window's lower edge; sub-tiles outside every query's window are skipped.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_t;

namespace mf {
constexpr int D = 128;
constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
constexpr int NT = D / 32;   // 32-feature tiles of the output
constexpr int ROW = 2 * D;   // bytes per token row
constexpr int TT = 64;       // keys per stage
constexpr int TILE = TT * ROW;
constexpr float kLazy = 8.f;  // largest exponent of an unnormalised probability (base 2)

// XOR swizzle of the sixteen 16-byte chunks of row r (r_i: bit i of r):
// conflict-free 16-byte row reads over 16 consecutive rows and 8-byte
// transpose reads over four rows 4m .. 4m + 3 (see the d = 128 chunk-gradient
// kernel, which uses the same tile layout).
__device__ __forceinline__ int swz(int r) {
  return 8 * ((r >> 1) & 1) + 4 * ((r ^ (r >> 3)) & 1) + 2 * (r & 1) + ((r >> 2) & 1);
}
}  // namespace mf

template <int QT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 2 : 1, QT == 1 ? 2 : 1)))
void k_window_attn_mfma(WindowArgs a, int nq) {
  using namespace mf;
  constexpr int QWV = 32 * QT;     // queries per wavefront
  constexpr int QWG = 4 * QWV;     // queries per workgroup
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * TILE];  // K[2], V[2]
  // XCD-aware order: block ids congruent mod 8 run on one XCD, and each
  // XCD takes a contiguous run of (pair, query block)s in order, so the
  // neighbouring query blocks that read the same keys and values share its L2
  const int nblk = gridDim.x;  // a multiple of 8
  const int ob = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  if (ob >= nq * a.P) return;
  const int pair = ob / nq;
  const int64_t q0 = static_cast<int64_t>(ob % nq) * QWG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int ln = lane & 31;
  const int64_t base = static_cast<int64_t>(pair) * a.stride;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + base;
  const int T = static_cast<int>(a.T);
  const int W = static_cast<int>(a.window < a.T ? a.window : a.T);
  const int qw0 = static_cast<int>(q0) + QWV * wv;  // this wave's first query
  const float c = a.scale * 1.4426950408889634f;   // scores to base-2 exponents

  // this wave's queries as B operands: query tile qt, lane holds query
  // qw0 + 32 qt + ln, features 16 ks + 8 g .. +7 (queries past the end
  // re-read the last one)
  bf16x8_t qb[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int myq = qw0 + 32 * qt + ln;
    const int qr = myq < T ? myq : T - 1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[qt][ks] = *reinterpret_cast<const bf16x8_t*>(Qg + static_cast<int64_t>(qr) * D + 16 * ks + 8 * g);
  }

  f32x16_t o[QT][NT];
  float m[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qt][t][r] = 0.f;
    }
  }

  // stage range: keys any query of the workgroup can see
  const int q_hi = static_cast<int>(q0) + QWG - 1 < T - 1 ? static_cast<int>(q0) + QWG - 1 : T - 1;
  int k_begin = static_cast<int>(q0) - W + 1;
  if (k_begin < 0) k_begin = 0;
  k_begin = (k_begin / TT) * TT;
  const int k_end = q_hi + 1;  // exclusive

  // (element offset of this lane's 16 bytes inside a stage, per piece: a
  // lane constant, so a whole stage needs only the stage's base address)
  int dofs[TT / 16];
#pragma unroll
  for (int k = 0; k < TT / 16; ++k) {
    const int r = 4 * (4 * k + wv) + (lane >> 4);
    dofs[k] = r * D + 8 * ((lane & 15) ^ swz(r));
  }
  auto dma_stage = [&](int k0, int b) {
    if (k0 + TT <= T) {
      const uint16_t* kst = Kg + static_cast<int64_t>(k0) * D;
      const uint16_t* vst = Vg + static_cast<int64_t>(k0) * D;
#pragma unroll
      for (int k = 0; k < TT / 16; ++k) {
        const int piece = 4 * k + wv;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(kst + dofs[k]), (lds_ptr_t)(lds + b * TILE + 1024 * piece), 16, 0,
                                         0);
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)(vst + dofs[k]), (lds_ptr_t)(lds + (2 + b) * TILE + 1024 * piece),
                                         16, 0, 0);
      }
      return;
    }
    // the last stage: rows past the end re-read the last token
#pragma unroll
    for (int k = 0; k < TT / 16; ++k) {
      const int piece = 4 * k + wv;
      const int r = 4 * piece + (lane >> 4);
      const int cl = (lane & 15) ^ swz(r);
      const int tok = k0 + r < T ? k0 + r : T - 1;
      const unsigned off = static_cast<unsigned>(tok) * D + 8 * cl;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Kg + off), (lds_ptr_t)(lds + b * TILE + 1024 * piece), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Vg + off), (lds_ptr_t)(lds + (2 + b) * TILE + 1024 * piece), 16, 0,
                                       0);
    }
  };

  // operand addresses (lane constants plus immediates)
  int ak_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ak_off[ks] = ln * ROW + 16 * ((2 * ks + g) ^ swz(ln));
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

  if (k_begin < k_end) dma_stage(k_begin, 0);
  int b = 0;
  for (int k0 = k_begin; k0 < k_end; k0 += TT, b ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this stage has landed
    __syncthreads();
    if (k0 + TT < k_end) dma_stage(k0 + TT, b ^ 1);
    const unsigned char* kb = lds + b * TILE;
    const unsigned char* vb = lds + (2 + b) * TILE;
#pragma unroll 1
    for (int st = 0; st < TT / 32; ++st) {
      const int kb0 = k0 + 32 * st;  // first key of the sub-tile
      // skipped when outside every window of this wave's queries
      if (kb0 > qw0 + QWV - 1 || kb0 + 31 < qw0 - W + 1 || kb0 >= T) continue;
      // key rows of the sub-tile, shared by the wave's query tiles
      bf16x8_t ak[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ak[ks] = *reinterpret_cast<const bf16x8_t*>(kb + ak_off[ks] + 8192 * st);
      f32x16_t s[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qt][r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[ks], qb[qt][ks], s[qt], 0, 0, 0);
      }
      // value operands of this sub-tile (read while the scores complete)
      bf16x8_t vt[2][NT];
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          s16x4_t t2[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int off = tr_off[(nt & 1) ^ hh][nt >> 1] + 8192 * st + 4096 * hs + 2048 * hh;
            t2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(vb + off));
          }
          vt[hs][nt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t2[0], t2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        // register r holds key kb0 + 8 (r / 4) + 4 g + r % 4 of query myq
        const int qq = qw0 + 32 * qt, myq = qq + ln;
        const bool edge = (kb0 + 31 > qq) || (kb0 < qq + 31 - W + 1);
        if (edge) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb0 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (!(key <= myq && key > myq - W)) s[qt][r] = -INFINITY;
          }
        }
        float mx = s[qt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // The reference maximum m (base-2 units, -inf: nothing seen yet)
        // moves only when the sub-tile's maximum exceeds it by more than
        // kLazy, so every p = 2^(s c - m) stays below 2^kLazy and the rescale
        // of l and O (which both carry the same factor 2^-m) is rare.
        const float mxc = mx * c;
        const bool grow = mxc > m[qt] + kLazy;
        if (__any(grow)) {
          const float corr = grow ? exp2f(m[qt] - mxc) : 1.f;  // 0 on the first visible sub-tile
          l[qt] *= corr;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qt][t][r] *= corr;
          }
          if (grow) m[qt] = mxc;
        }
        bf16x8_t p[2];
        const float mm = (m[qt] == -INFINITY) ? 0.f : m[qt];  // (then every score of the lane is -inf: p = 0)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[qt][r], c, -mm));
          l[qt] += e;
          p[r >> 3][r & 7] = static_cast<__bf16>(e);
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            o[qt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt[hs][nt], p[hs], o[qt][nt], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
    const int myq = qw0 + 32 * qt + ln;
    if (myq >= T) continue;
    const float inv = 1.f / lt;
    uint16_t* Og = static_cast<uint16_t*>(a.O) + base + static_cast<int64_t>(myq) * D;
    // register r of tile nt: feature 32 nt + 8 (r / 4) + 4 g + r % 4 (four consecutive per group)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int f = 32 * nt + 8 * rg + 4 * g;
        bf16x4_t v4;
        if (a.accumulate) v4 = *reinterpret_cast<const bf16x4_t*>(Og + f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = o[qt][nt][4 * rg + i] * inv;
          if (a.accumulate) v += static_cast<float>(v4[i]);
          v4[i] = static_cast<__bf16>(v);
        }
        *reinterpret_cast<bf16x4_t*>(Og + f) = v4;
      }
    }
  }
}

template <int D>
hipError_t launch_d(const WindowArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.T + kQ - 1) / kQ), a.P);
  if (a.bf16) {
    hipLaunchKernelGGL((k_window_attn<true, D>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_window_attn<false, D>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

bool window_shape_ok(int d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_window_attn(const WindowArgs& a, hipStream_t s) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.Q) | reinterpret_cast<uintptr_t>(a.K) |
                         reinterpret_cast<uintptr_t>(a.V) | reinterpret_cast<uintptr_t>(a.O)) & 15) == 0;
  if (a.bf16 && a.d == mf::D && aligned && a.T * a.d < (int64_t(1) << 31)) {
    constexpr int QT = 1;  // query tiles per wavefront
    const int64_t nq = (a.T + 128 * QT - 1) / (128 * QT);
    const int64_t blocks = (nq * a.P + 7) / 8 * 8;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_window_attn_mfma<QT>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a,
                       static_cast<int>(nq));
    return hipGetLastError();
  }
  switch (a.d) {
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lact

// Query read O = W2 (silu(W1 q) * (W3 q)) on bf16 MFMA (gfx950), d = 64 or
// 128, h in {128, 256}: the fast weights answer the queries ("LaCT: Large
// Chunk Test-Time Training" review, sections "Local attention and nonlinear
// memory work together" and "Update order must respect the task").
//
// A workgroup (4 wavefronts) owns one pair and a contiguous run of queries.
// Each wavefront keeps its 32 rows of W2 and, where they fit (h = 128), the
// W1 and W3 rows of its quarter of the hidden units as bf16 MFMA operands in
// registers; otherwise W1 and W3 are staged once into LDS.  Per step
// of 64 (d = 64) or 32 (d = 128) queries:
//   1. wave w computes H1^T, H3^T = W1 Q^T, W3 Q^T for its quarter of the
//      hidden units (A = W rows, B = query rows from LDS),
//      gates them, G = silu(H1) * H3, and writes G (bf16) to LDS as
//      [token][hidden];
//   2. wave w computes one 32 x 32 tile of O^T = W2 G^T (A = its W2 rows,
//      B = G rows from LDS) and stores it.
// All LDS tiles are XOR-swizzled in 16-byte chunks (chunk c of row r sits
// at c ^ (r & 7)) so the 16-byte operand reads are conflict-free.
#include "lact_device.h"
#include "lact_internal.h"

namespace lact {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr int kThreads = 256;

template <int D, int H>
struct AGeo {
  static constexpr int NTT = 128 / D;          // 32-token tiles per step
  static constexpr int TQ = 32 * NTT;          // queries per step
  static constexpr int HQ = H / 4;             // hidden units per wave in phase 1
  static constexpr int HM = HQ / 32;           // 32-row tiles of them
  static constexpr int WROW = 2 * D;           // bytes per row of W1 / W3 / Q
  static constexpr int GROW = 2 * H;           // bytes per row of G
  // W1, W3 operands take 2 HM D / 4 registers per lane, W2's H / 4: when
  // that stays under 128 they live in registers (two wavefronts per SIMD);
  // otherwise W1 and W3 are staged in LDS (one wavefront per SIMD)
  static constexpr bool WREG = 2 * HM * D / 4 + H / 4 < 128;
  static constexpr int WAVES_PER_SIMD = WREG ? 2 : 1;
  static constexpr int OFF_W1 = 0;
  static constexpr int OFF_W3 = WREG ? 0 : H * WROW;
  static constexpr int OFF_Q = WREG ? 0 : 2 * H * WROW;
  static constexpr int OFF_G = OFF_Q + TQ * WROW;
  static constexpr int LDS = OFF_G + TQ * GROW;
};

// byte offset of 16-byte chunk `c` of row `r` (rows of `rowbytes`), swizzled
__device__ __forceinline__ int swz(int r, int c, int rowbytes) {
  return r * rowbytes + ((c ^ (r & 7)) << 4);
}

template <int D, int H>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(AGeo<D, H>::WAVES_PER_SIMD, AGeo<D, H>::WAVES_PER_SIMD)))
void k_apply_mfma(ApplyArgs a, int per_wg) {
  using G = AGeo<D, H>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS];

  const int pair = blockIdx.y;
  const int64_t q_begin = static_cast<int64_t>(blockIdx.x) * per_wg;
  const int64_t q_end = min(a.m, q_begin + per_wg);
  if (q_begin >= q_end) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, ln = lane & 31;
  const int64_t hd = static_cast<int64_t>(H) * D;

  // ---- W1, W3 operands (A side: hidden row w HQ + 32 m + ln, features
  // 16 ks + 8 g .. +7), in registers or staged in LDS
  bf16x8_t w1a[G::WREG ? G::HM : 1][G::WREG ? D / 16 : 1], w3a[G::WREG ? G::HM : 1][G::WREG ? D / 16 : 1];
  if constexpr (!G::WREG) {
    const float* W1 = a.W1 + pair * hd;
    const float* W3 = a.W3 + pair * hd;
    for (int i = tid; i < H * D / 8; i += kThreads) {
      const int r = i / (D / 8), c = i % (D / 8);
      bf16x8_t v1, v3;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v1[k] = static_cast<__bf16>(W1[static_cast<int64_t>(r) * D + 8 * c + k]);
        v3[k] = static_cast<__bf16>(W3[static_cast<int64_t>(r) * D + 8 * c + k]);
      }
      *reinterpret_cast<bf16x8_t*>(lds + G::OFF_W1 + swz(r, c, G::WROW)) = v1;
      *reinterpret_cast<bf16x8_t*>(lds + G::OFF_W3 + swz(r, c, G::WROW)) = v3;
    }
  } else {
    const float* W1 = a.W1 + pair * hd;
    const float* W3 = a.W3 + pair * hd;
#pragma unroll
    for (int m = 0; m < G::HM; ++m) {
      const int64_t hrow = w * G::HQ + 32 * m + ln;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          w1a[m][ks][k] = static_cast<__bf16>(W1[hrow * D + 16 * ks + 8 * g + k]);
          w3a[m][ks][k] = static_cast<__bf16>(W3[hrow * D + 16 * ks + 8 * g + k]);
        }
      }
    }
  }
  // ---- this wave's phase-2 tile: rows dt*32.. of O^T, tokens tt*32..
  const int dt = w % (D / 32);
  const int tt = w / (D / 32);
  bf16x8_t w2b[H / 16];
  {
    const float* W2 = a.W2 + pair * hd + static_cast<int64_t>(32 * dt + ln) * H;
#pragma unroll
    for (int ks = 0; ks < H / 16; ++ks) {
#pragma unroll
      for (int k = 0; k < 8; ++k) w2b[ks][k] = static_cast<__bf16>(W2[16 * ks + 8 * g + k]);
    }
  }

  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + static_cast<int64_t>(pair) * a.q_stride;
  uint16_t* Og = static_cast<uint16_t*>(a.O) + static_cast<int64_t>(pair) * a.q_stride;

  // query staging: TQ rows x D bf16 = TQ * D / 8 chunks of 16 bytes
  constexpr int QCH = G::TQ * D / 8;
  constexpr int QPT = QCH / kThreads;  // chunks per thread (= 2)
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
  auto store_q = [&]() {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = tid + kThreads * k;
      const int r = i / (D / 8), c = i % (D / 8);
      *reinterpret_cast<u32x4_t*>(lds + G::OFF_Q + swz(r, c, G::WROW)) = qr[k];
    }
  };

  constexpr float kLog2e = 1.4426950408889634f;
  load_q(q_begin);
  for (int64_t t0 = q_begin; t0 < q_end; t0 += G::TQ) {
    __syncthreads();  // previous step's readers of Q and G are done
    store_q();
    __syncthreads();
    if (t0 + G::TQ < q_end) load_q(t0 + G::TQ);

    // ---- phase 1: H^T for hidden units [w HQ, (w+1) HQ) x TQ tokens
#pragma unroll
    for (int t = 0; t < G::NTT; ++t) {
#pragma unroll
      for (int m = 0; m < G::HM; ++m) {
        const int hrow = w * G::HQ + 32 * m + ln;
        f32x16_t c1, c3;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          c1[r] = 0.f;
          c3[r] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int ch = 2 * ks + g;
          const bf16x8_t bq = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_Q + swz(32 * t + ln, ch, G::WROW));
          if constexpr (G::WREG) {
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1a[m][ks], bq, c1, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w3a[m][ks], bq, c3, 0, 0, 0);
          } else {
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_W1 + swz(hrow, ch, G::WROW));
            const bf16x8_t a3 = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_W3 + swz(hrow, ch, G::WROW));
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bq, c1, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, bq, c3, 0, 0, 0);
          }
        }
        // c[r] = H^T[hidden w HQ + 32 m + 8 (r/4) + 4 g + r%4][token 32 t + ln]
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
          const int hid = w * G::HQ + 32 * m + 8 * rg + 4 * g;
          *reinterpret_cast<bf16x4_t*>(lds + G::OFF_G + swz(tok, hid >> 3, G::GROW) + 2 * (hid & 7)) = gv;
        }
      }
    }
    __syncthreads();

    // ---- phase 2: O^T tile (d rows 32 dt.., tokens 32 tt..) = W2 G^T
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < H / 16; ++ks) {
      const bf16x8_t bg = *reinterpret_cast<const bf16x8_t*>(lds + G::OFF_G + swz(32 * tt + ln, 2 * ks + g, G::GROW));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2b[ks], bg, acc, 0, 0, 0);
    }
    const int64_t tok = t0 + 32 * tt + ln;
    if (tok < q_end) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4_t ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(acc[4 * rg + i]);
        const int dd = 32 * dt + 8 * rg + 4 * g;
        *reinterpret_cast<bf16x4_t*>(Og + tok * D + dd) = ov;
      }
    }
  }
}

template <int D, int H>
hipError_t launch_dh(const ApplyArgs& a, hipStream_t s) {
  // queries per workgroup: enough workgroups to cover 256 CUs about twice,
  // and a multiple of the step
  constexpr int TQ = AGeo<D, H>::TQ;
  int64_t per = (a.m * a.P + 511) / 512;
  per = (per + TQ - 1) / TQ * TQ;
  if (per < 4 * TQ) per = 4 * TQ;
  const unsigned gx = static_cast<unsigned>((a.m + per - 1) / per);
  hipLaunchKernelGGL((k_apply_mfma<D, H>), dim3(gx, a.P), dim3(kThreads), 0, s, a, static_cast<int>(per));
  return hipGetLastError();
}

}  // namespace

bool apply_mfma_shape_ok(int d, int h) {
  return (d == 64 || d == 128) && (h == 128 || h == 256);
}

hipError_t launch_apply_mfma(const ApplyArgs& a, hipStream_t s) {
  if (a.d == 64 && a.h == 128) return launch_dh<64, 128>(a, s);
  if (a.d == 64 && a.h == 256) return launch_dh<64, 256>(a, s);
  if (a.d == 128 && a.h == 128) return launch_dh<128, 128>(a, s);
  if (a.d == 128 && a.h == 256) return launch_dh<128, 256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace lact

// Host-side exercise of the C ABI for the address and undefined-behaviour
// sanitizers: defaults, workspace sizing over many shapes, every validation
// failure, status texts, and calls that pass validation (which, with no GPU
// visible, end in the first launch with LACT_ERR_HIP).  Stand-in device
// addresses are used throughout, so this program must only run where no GPU
// is visible; it refuses to run otherwise.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <hip/hip_runtime.h>

#include "lact.h"

static int g_fail = 0;
#define EXPECT(cond)                                               \
  do {                                                             \
    if (!(cond)) {                                                 \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                    \
    }                                                              \
  } while (0)

static lact_config cfg(int B, int H, int d, int h, int io, int opt, float beta) {
  lact_config c;
  lact_config_default(&c);
  c.B = B;
  c.H = H;
  c.d = d;
  c.h = h;
  c.io_dtype = io;
  c.opt = opt;
  c.beta = beta;
  return c;
}

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::fprintf(stderr, "a GPU is visible: this check hands the library stand-in addresses\n");
    return 2;
  }
  void* const fake = reinterpret_cast<void*>(256);
  float* const ffake = reinterpret_cast<float*>(256);
  lact_state st{ffake, ffake, ffake, ffake, ffake, ffake};
  lact_state st_nom{ffake, ffake, ffake, nullptr, nullptr, nullptr};

  // defaults and texts
  lact_config c = cfg(1, 1, 64, 128, LACT_BF16, LACT_OPT_GD, 0.f);
  EXPECT(c.products == LACT_PRODUCTS_AUTO && c.ns_iters == 5);
  for (int s = -6; s <= 1; ++s) EXPECT(lact_status_string(s) != nullptr);
  EXPECT(std::strlen(lact_last_error()) < 4096);
  EXPECT(lact_version() >= 1);

  // workspace sizing over shapes, options and lengths
  const int ds[] = {16, 32, 64, 100, 128, 256};
  const int hs[] = {32, 64, 96, 128, 256, 1024, 2048};
  const long long ns[] = {1, 7, 128, 1000, 196608, 1029120, 1LL << 33};
  for (int d : ds)
    for (int h : hs)
      for (int io = 0; io < 2; ++io)
        for (int opt = 0; opt < 3; ++opt)
          for (int prod = 0; prod < 3; ++prod)
            for (long long n : ns) {
              lact_config x = cfg(2, 3, d, h, io, opt, opt == LACT_OPT_MOMENTUM ? 0.9f : 0.f);
              x.products = prod;
              const size_t b = lact_workspace_bytes(&x, n, 64);
              EXPECT(b % 256 == 0);
              EXPECT((b == 0) == (lact_mfma_path(d, h, io) < 0));
            }
  EXPECT(lact_workspace_bytes(nullptr, 10, 10) == 0);

  // validation failures of every entry point
  EXPECT(lact_update(nullptr, &st, fake, fake, ffake, 16, 1024, 16, fake, 1 << 30, nullptr) ==
         LACT_ERR_INVALID_ARG);
  EXPECT(lact_update(&c, nullptr, fake, fake, ffake, 16, 1024, 16, fake, 1 << 30, nullptr) ==
         LACT_ERR_INVALID_ARG);
  EXPECT(lact_update(&c, &st, nullptr, fake, ffake, 16, 1024, 16, fake, 1 << 30, nullptr) ==
         LACT_ERR_INVALID_ARG);
  EXPECT(lact_update(&c, &st, fake, fake, ffake, 0, 1024, 16, fake, 1 << 30, nullptr) ==
         LACT_ERR_INVALID_ARG);
  EXPECT(lact_update(&c, &st, fake, fake, ffake, 16, 10, 16, fake, 1 << 30, nullptr) ==
         LACT_ERR_INVALID_ARG);
  EXPECT(lact_update(&c, &st, fake, fake, ffake, 16, 1024, 16, fake, 16, nullptr) == LACT_ERR_WORKSPACE);
  EXPECT(lact_update(&c, &st, fake, fake, ffake, 16, 1024, 16, reinterpret_cast<void*>(257), 1 << 30,
                     nullptr) == LACT_ERR_WORKSPACE);
  lact_config m = cfg(1, 1, 64, 128, LACT_BF16, LACT_OPT_MOMENTUM, 0.9f);
  EXPECT(lact_update(&m, &st_nom, fake, fake, ffake, 16, 1024, 16, fake, 1 << 30, nullptr) ==
         LACT_ERR_INVALID_ARG);
  lact_config bad = c;
  bad.beta = 1.5f;
  EXPECT(lact_update(&bad, &st, fake, fake, ffake, 16, 1024, 16, fake, 1 << 30, nullptr) ==
         LACT_ERR_INVALID_ARG);
  bad = c;
  bad.norm_eps = 0.f;
  EXPECT(lact_apply(&bad, &st, fake, fake, 4, 256, nullptr, 0, nullptr) == LACT_ERR_INVALID_ARG);
  bad = c;
  bad.d = 60;
  EXPECT(lact_apply(&bad, &st, fake, fake, 4, 256, nullptr, 0, nullptr) == LACT_ERR_UNSUPPORTED);
  EXPECT(lact_apply(&c, &st, fake, nullptr, 4, 256, nullptr, 0, nullptr) == LACT_ERR_INVALID_ARG);
  EXPECT(lact_apply(&c, &st, fake, fake, 8, 100, nullptr, 0, nullptr) == LACT_ERR_INVALID_ARG);
  EXPECT(lact_chunked_forward(&c, &st, fake, fake, fake, ffake, fake, 1024, 1024, 300, 256, 0, fake,
                              1 << 30, nullptr) == LACT_ERR_INVALID_ARG);
  EXPECT(lact_chunked_forward(&c, &st, fake, fake, fake, ffake, fake, 1024, 512, 256, 256, 0, fake,
                              1 << 30, nullptr) == LACT_ERR_INVALID_ARG);
  EXPECT(lact_chunked_forward(&c, &st, fake, fake, fake, ffake, fake, 1024, 1024, 256, 256, 7, fake,
                              1 << 30, nullptr) == LACT_ERR_INVALID_ARG);
  lact_config mu = cfg(1, 2, 128, 256, LACT_BF16, LACT_OPT_MUON, 0.f);
  mu.products = LACT_PRODUCTS_BF16;
  EXPECT(lact_chunked_forward(&mu, &st, fake, fake, fake, ffake, fake, 14 * 4096, 14 * 4096, 4096, 4096,
                              0, fake, 1 << 30, nullptr) == LACT_ERR_UNSUPPORTED);
  EXPECT(std::strstr(lact_last_error(), "1024 keys") != nullptr);

  // calls that pass validation: with no device the first launch fails
  const int opts[] = {LACT_OPT_GD, LACT_OPT_MOMENTUM, LACT_OPT_MUON};
  for (int io = 0; io < 2; ++io)
    for (int opt : opts)
      for (int order = 0; order < 2; ++order) {
        lact_config x = cfg(1, 2, 64, 128, io, opt, opt == LACT_OPT_GD ? 0.f : 0.5f);
        const int rc = lact_chunked_forward(&x, &st, fake, fake, fake, ffake, fake, 2048, 512, 1024, 256,
                                            order, fake, size_t(1) << 40, nullptr);
        EXPECT(rc == LACT_ERR_HIP);
        EXPECT(std::strlen(lact_last_error()) > 0);
      }
  EXPECT(lact_profile_enable(1) == LACT_OK);
  double ms[LACT_PROFILE_PHASES] = {0};
  int64_t launches[LACT_PROFILE_PHASES] = {0};
  EXPECT(lact_profile_read(ms, launches) == LACT_OK);
  EXPECT(lact_profile_enable(0) == LACT_OK);

  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("abi host check: ok\n");
  return 0;
}

// Host-only exercise of libcgtp's plan construction and argument checks, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
// Every call here runs on the host: plans are created with CGTP_PLAN_HOST_ONLY, and the
// device entry points are called only with arguments they refuse before any launch.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/cgtp.h"

static int g_fail = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static void check_plan(const char* in, const char* sh, int lmax, int rule) {
  cgtp_plan_t p = nullptr;
  const int rc = cgtp_plan_create(in, sh, lmax, rule, CGTP_PLAN_HOST_ONLY, &p);
  EXPECT(rc == CGTP_OK && p);
  if (!p) return;
  int64_t f_in = 0, f_out = 0, w = 0;
  int n_paths = 0, l_sh = 0;
  char out[4096];
  EXPECT(cgtp_plan_info(p, &f_in, &f_out, &w, &n_paths, &l_sh, out, sizeof(out)) == CGTP_OK);
  EXPECT(f_in > 0 && f_out > 0 && w > 0 && n_paths > 0 && std::strlen(out) > 0);
  char tiny[4];
  EXPECT(cgtp_plan_info(p, nullptr, nullptr, nullptr, nullptr, nullptr, tiny, sizeof(tiny)) == CGTP_OK);
  EXPECT(std::strlen(tiny) == 3);   // truncated, NUL-terminated
  std::vector<int32_t> rows(size_t(n_paths) * 10);
  EXPECT(cgtp_plan_paths(p, rows.data()) == CGTP_OK);
  int64_t w_sum = 0;
  for (int k = 0; k < n_paths; ++k) {
    const int l1 = rows[10 * k], l2 = rows[10 * k + 2], l3 = rows[10 * k + 4], mul = rows[10 * k + 6];
    w_sum += mul;
    std::vector<float> cg(size_t(2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1));
    EXPECT(cgtp_plan_cg(p, k, cg.data()) == CGTP_OK);
    // real CG columns are orthonormal: sum over m1, m2 of C^2 is 1 for every m3
    for (int c = 0; c < 2 * l3 + 1; ++c) {
      double s = 0.0;
      for (int a = 0; a < 2 * l1 + 1; ++a)
        for (int b = 0; b < 2 * l2 + 1; ++b) {
          const double v = cg[(size_t(a) * (2 * l2 + 1) + b) * (2 * l3 + 1) + c];
          s += v * v;
        }
      EXPECT(std::fabs(s - 1.0) < 1e-5);
    }
  }
  EXPECT(w_sum == w);
  EXPECT(cgtp_plan_cg(p, -1, nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_plan_cg(p, n_paths, nullptr) == CGTP_ERR_INVALID_ARG);
  int n_jobs = 0, n_var = 0;
  EXPECT(cgtp_plan_schedule(p, &n_jobs, &n_var) == CGTP_OK && n_jobs >= n_paths && n_var > 0);
  size_t b0 = 0, b1 = 0, bb = 0;
  EXPECT(cgtp_workspace_size(p, 0, 0, 0, &b0) == CGTP_OK);
  EXPECT(cgtp_workspace_size(p, 4096, 114688, 1, &b1) == CGTP_OK && b1 > b0);
  EXPECT(cgtp_workspace_size(p, -1, 0, 0, &b0) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_backward_workspace_size(p, 4096, 114688, &bb) == CGTP_OK && bb > b1);
  // device entry points refuse a host-only plan before touching the device
  float dummy[16] = {};
  int32_t rp[2] = {0, 0};
  EXPECT(cgtp_conv_forward(p, dummy, 1, nullptr, rp, rp, nullptr, 0, dummy, dummy, nullptr, dummy, dummy, 256,
                           nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_conv_forward_noalloc(p, dummy, 1, nullptr, rp, rp, nullptr, 0, dummy, dummy, nullptr, nullptr, dummy,
                                   nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_conv_backward(p, dummy, 1, nullptr, rp, rp, nullptr, 0, dummy, dummy, nullptr, nullptr, dummy, dummy,
                            dummy, dummy, dummy, 256, nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_conv_prepare(p, rp, nullptr, 1, 0, rp, rp, rp, dummy, 256, nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_edge_sh(p, dummy, 1, nullptr, rp, rp, nullptr, 0, dummy, nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(std::strlen(cgtp_last_error()) > 0);
  cgtp_plan_destroy(p);
}

int main() {
  // the workloads' plans, LunaTP Table 1 cases 4-6, and multiplicities past one channel block
  check_plan("8x0e+8x1o", "1x0e+1x1o", 1, CGTP_PATHS_ALL);
  check_plan("128x0e+64x1e+32x2e", "1x0e+1x1e+1x2e", 2, CGTP_PATHS_ALL);
  check_plan("128x0e+128x1o+128x2e", "1x0e+1x1o+1x2e+1x3o", 3, CGTP_PATHS_PARITY);
  check_plan("64x0e+64x1o+64x2e+64x3o+64x4e+64x5o+64x6e", "0e+1o+2e+3o+4e+5o+6e", 6, CGTP_PATHS_PARITY);
  check_plan("128x0e+64x1o+32x2e+32x3o", "1x0e+1x1o+1x2e+1x3o", 3, CGTP_PATHS_PARITY);
  check_plan("256x0e+256x1o+256x2e+256x3o", "1x0e+1x1o+1x2e+1x3o", 3, CGTP_PATHS_PARITY);
  check_plan("320x0e+96x1o+64x2e+32x3o+32x4e", "1x0e+1x1o+1x2e+1x3o+1x4e", 4, CGTP_PATHS_PARITY);
  check_plan("1000x0e+999x1o+3x2e", "1x0e+1x1o", 2, CGTP_PATHS_ALL);
  check_plan(" 3x1o + 5x0e ", "1x1o", 2, CGTP_PATHS_ALL);
  // parse and support errors, each with a message
  const char* bad_in[] = {"", "128x", "x0e", "12x0q", "1x", "+", "1x0e+", "abc", "1x-1e", "1234567890x0e", "1x99999e"};
  for (const char* s : bad_in) {
    cgtp_plan_t p = reinterpret_cast<cgtp_plan_t>(1);
    const int rc = cgtp_plan_create(s, "1x0e", 1, CGTP_PATHS_ALL, CGTP_PLAN_HOST_ONLY, &p);
    EXPECT((rc == CGTP_ERR_PARSE || rc == CGTP_ERR_UNSUPPORTED) && p == nullptr);
    EXPECT(std::strlen(cgtp_last_error()) > 0);
  }
  cgtp_plan_t p = nullptr;
  EXPECT(cgtp_plan_create("0x0e", "1x0e", 0, 0, CGTP_PLAN_HOST_ONLY, &p) == CGTP_ERR_UNSUPPORTED);
  EXPECT(cgtp_plan_create("1x7e", "1x0e", 7, 0, CGTP_PLAN_HOST_ONLY, &p) == CGTP_ERR_UNSUPPORTED);
  EXPECT(cgtp_plan_create("1x0e", "2x1o", 1, 0, CGTP_PLAN_HOST_ONLY, &p) == CGTP_ERR_UNSUPPORTED);
  EXPECT(cgtp_plan_create("1x0e", "1x1e", 1, CGTP_PATHS_PARITY, CGTP_PLAN_HOST_ONLY, &p) == CGTP_ERR_UNSUPPORTED);
  EXPECT(cgtp_plan_create("1x0e", "1x0e", -1, 0, CGTP_PLAN_HOST_ONLY, &p) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_plan_create("1x0e", "1x0e", 0, 7, CGTP_PLAN_HOST_ONLY, &p) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_plan_create("1x0e", "1x0e", 0, 0, 0x80u, &p) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_plan_create("1x0e", "1x0e", 0, 0, CGTP_PLAN_HOST_ONLY, nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_plan_create("1x5e", "1x0e", 5, 0, CGTP_PLAN_HOST_ONLY | CGTP_PLAN_FP64, &p) == CGTP_ERR_UNSUPPORTED);
  // NULL handles and arguments
  EXPECT(cgtp_plan_info(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_plan_paths(nullptr, nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_plan_schedule(nullptr, nullptr, nullptr) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_workspace_size(nullptr, 1, 1, 0, nullptr) == CGTP_ERR_INVALID_ARG);
  size_t b = 0;
  const float box[3] = {10.f, 10.f, 10.f}, bad_box[3] = {10.f, 0.f, 10.f};
  EXPECT(cgtp_neighbors_workspace_size(100, box, 2.5f, &b) == CGTP_OK && b > 0);
  EXPECT(cgtp_neighbors_workspace_size(100, bad_box, 2.5f, &b) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_neighbors_workspace_size(-1, box, 2.5f, &b) == CGTP_ERR_INVALID_ARG);
  EXPECT(cgtp_neighbors_workspace_size(100, box, -1.f, &b) == CGTP_ERR_INVALID_ARG);
  int64_t ne = 0;
  EXPECT(cgtp_neighbors_build(nullptr, 1, box, 2.5f, nullptr, nullptr, nullptr, 0, &ne, nullptr, 0, nullptr) ==
         CGTP_ERR_INVALID_ARG);
  cgtp_plan_destroy(nullptr);
  EXPECT(std::strncmp(cgtp_version(), "cgtp", 4) == 0);
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("plan driver: all checks passed\n");
  return 0;
}

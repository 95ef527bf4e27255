// Host-side checks of the C ABI, built together with the library's sources
// under AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
// tests/test_host_sanitizers.py.  Nothing here launches a kernel or touches
// device memory: every call either answers a size query or fails argument
// validation before its first HIP call.  Pointers passed to failing calls
// are never dereferenced.
//
// Checked:
//  * workspace queries over a grid of shapes from empty to the largest
//    representable batch: no overflow (UBSan), 0 for invalid shapes, never
//    smaller for a larger batch (a size_t wrap would show as a drop);
//  * every entry point's validation codes for bad shapes, NULL buffers,
//    misaligned workspaces and short workspaces;
//  * the status and stage-name strings for every small integer, and the
//    stage-timing calls with NULL, zero and negative arguments.
#include <climits>
#include <limits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "moe_mi355x.h"

static int g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t(1) << 20) + off); }

static moe_shape_t shape(int32_t T, int32_t d = 512, int32_t L = 256, int32_t n = 40,
                         int32_t k = 6, int32_t m = 192, int32_t ms = 320,
                         int32_t act = MOE_BF16, int32_t routed = MOE_BF16) {
  moe_shape_t s;
  std::memset(&s, 0, sizeof s);
  s.T = T;
  s.d = d;
  s.latent = L;
  s.n_experts = n;
  s.top_k = k;
  s.inter = m;
  s.shared_inter = ms;
  s.act_dtype = act;
  s.routed_dtype = routed;
  s.rms_eps = 1e-6f;
  s.qb_mode = MOE_QB_BATCH;
  s.qb_max_rounds = 0;
  return s;
}

static void route_queries() {
  const int32_t Ts[] = {-1, 0, 1, 3, 64, 65, 4096, 57344, MOE_MAX_TOKENS, MOE_MAX_TOKENS + 1,
                        INT_MAX / 64, INT_MAX};
  const int32_t ns[] = {-1, 0, 1, 2, 7, 64, 896, 1024, 1025, INT_MAX};
  const int32_t ks[] = {-1, 0, 1, 2, 16, 64, 65, INT_MAX};
  for (int32_t n : ns)
    for (int32_t k : ks) {
      size_t prev = 0;
      for (int32_t T : Ts) {
        const size_t b = moe_route_workspace_bytes(T, n, k);
        const bool valid = T >= 0 && T <= MOE_MAX_TOKENS && n >= 1 && n <= 1024 && k >= 1 &&
                           k <= n && k <= 64;
        if (!valid) {
          CHECK(b == 0);
          continue;
        }
        if (b == 0) continue;  // a batch too large to describe is refused
        CHECK(b >= prev);
        prev = b;
      }
    }
}

static void layer_queries() {
  const int32_t Ts[] = {-1, 0, 1, 64, 200, 4096, 16384, MOE_MAX_TOKENS, MOE_MAX_TOKENS + 1,
                        INT_MAX / 64, INT_MAX};
  const int32_t widths[] = {-64, 0, 32, 64, 192, 256, 2048, 3584, 7168, 1 << 20};
  const int32_t dts[] = {-1, MOE_F32, MOE_BF16, MOE_MXFP4, MOE_MXFP4_A8, MOE_MXFP4_A4, 5};
  for (int32_t act : dts)
    for (int32_t routed : dts)
      for (int32_t w : widths) {
        size_t pf = 0, pb = 0;
        for (int32_t T : Ts) {
          moe_shape_t s = shape(T, w, w / 2 > 0 ? (w / 2 + 63) / 64 * 64 : w / 2, 896, 16, 2048,
                                6144, act, routed);
          const size_t f = moe_forward_workspace_bytes(&s);
          const size_t b = moe_backward_workspace_bytes(&s);
          if (T < 0 || T > MOE_MAX_TOKENS) {
            CHECK(f == 0 && b == 0);
            continue;
          }
          if (f) {
            CHECK(f >= pf);
            pf = f;
          }
          if (b) {
            CHECK(b >= pb);
            pb = b;
            CHECK(act == MOE_BF16 && routed == MOE_BF16);
          }
        }
      }
  // odd shape fields one at a time
  for (int field = 0; field < 7; ++field)
    for (int32_t v : {-1, 0, 1, 63, 65, 1025, INT_MAX}) {
      moe_shape_t s = shape(100);
      int32_t* f[] = {&s.T, &s.d, &s.latent, &s.n_experts, &s.top_k, &s.inter, &s.shared_inter};
      *f[field] = v;
      (void)moe_forward_workspace_bytes(&s);
      (void)moe_backward_workspace_bytes(&s);
    }
  moe_shape_t s = shape(100);
  s.rms_eps = -1.f;
  (void)moe_forward_workspace_bytes(&s);
  s = shape(100);
  s.qb_mode = 7;
  (void)moe_forward_workspace_bytes(&s);
  CHECK(moe_forward_workspace_bytes(nullptr) == 0);
  CHECK(moe_backward_workspace_bytes(nullptr) == 0);
}

static void route_validation() {
  const size_t need = moe_route_workspace_bytes(100, 64, 4);
  CHECK(need > 0);
  auto qb = [&](int32_t T, int32_t n, int32_t k, int32_t mode, void* ws, size_t wsb) {
    return moe_route_qb(static_cast<const float*>(fake()), T, n, k, mode, 64,
                        static_cast<double*>(fake()), static_cast<int32_t*>(fake()),
                        static_cast<float*>(fake()), static_cast<int32_t*>(fake()),
                        static_cast<int32_t*>(fake()), ws, wsb, nullptr);
  };
  CHECK(qb(100, 64, 65, 1, fake(), need) == MOE_EINVAL);
  CHECK(qb(100, 64, 0, 1, fake(), need) == MOE_EINVAL);
  CHECK(qb(-1, 64, 4, 1, fake(), need) == MOE_EINVAL);
  CHECK(qb(100, 2048, 4, 1, fake(), need) == MOE_EUNSUPPORTED);
  CHECK(qb(100, 128, 100, 1, fake(), need) == MOE_EUNSUPPORTED);
  CHECK(qb(100, 64, 4, 7, fake(), need) == MOE_EINVAL);
  CHECK(qb(100, 64, 4, 1, nullptr, need) == MOE_EINVAL);
  CHECK(qb(100, 64, 4, 1, fake(8), need) == MOE_EINVAL);
  CHECK(qb(100, 64, 4, 1, fake(), need - 1) == MOE_EWORKSPACE);
  CHECK(qb(MOE_MAX_TOKENS + 1, 64, 4, 1, fake(), need) == MOE_EUNSUPPORTED);
  CHECK(moe_route_qb(nullptr, 100, 64, 4, 1, 64, static_cast<double*>(fake()), nullptr, nullptr,
                     nullptr, nullptr, fake(), need, nullptr) == MOE_EINVAL);

  auto na = [&](int32_t T, int32_t n, int32_t k, int32_t mode) {
    return moe_route_qb_noalloc(static_cast<const float*>(fake()), T, n, k, mode, 64,
                                static_cast<double*>(fake()), static_cast<int32_t*>(fake()),
                                static_cast<float*>(fake()), static_cast<int32_t*>(fake()),
                                static_cast<int32_t*>(fake()), nullptr);
  };
  CHECK(na(100, 64, 65, 1) == MOE_EINVAL);
  CHECK(na(100, 2048, 4, 1) == MOE_EUNSUPPORTED);
  CHECK(na(100, 64, 4, 7) == MOE_EINVAL);
  CHECK(na(8192, 896, 16, 1) == MOE_EWORKSPACE);
  CHECK(na(INT_MAX, 896, 16, 1) == MOE_EUNSUPPORTED);

  auto sg = [&](int32_t T, int32_t n, int32_t k, double step, int32_t rounds) {
    return moe_route_sign(static_cast<const float*>(fake()), T, n, k, step, rounds,
                          static_cast<double*>(fake()), static_cast<int32_t*>(fake()),
                          static_cast<float*>(fake()), static_cast<int32_t*>(fake()),
                          static_cast<int32_t*>(fake()), fake(), need, nullptr);
  };
  CHECK(sg(100, 64, 65, 1.0 / 1024, 8) == MOE_EINVAL);
  CHECK(sg(100, 2048, 4, 1.0 / 1024, 8) == MOE_EUNSUPPORTED);
  CHECK(sg(100, 64, 4, 0.0, 8) == MOE_EINVAL);
  CHECK(sg(100, 64, 4, -1.0, 8) == MOE_EINVAL);
  CHECK(sg(100, 64, 4, 1e300, 8) == MOE_EINVAL);
  CHECK(sg(100, 64, 4, 1e-300, 8) == MOE_EINVAL);
  CHECK(sg(100, 64, 4, 0.0 / 0.0, 8) == MOE_EINVAL);
  CHECK(sg(100, 64, 4, 1.0 / 1024, -1) == MOE_EINVAL);
}

static moe_weights_t weights() {
  moe_weights_t w;
  void** p = reinterpret_cast<void**>(&w);
  for (size_t i = 0; i < sizeof w / sizeof(void*); ++i) p[i] = fake();
  return w;
}

static void layer_validation() {
  moe_shape_t s = shape(64);
  const size_t need = moe_forward_workspace_bytes(&s);
  CHECK(need > 0);
  moe_weights_t w = weights();
  auto fwd = [&](const moe_shape_t* sh, const moe_weights_t* wt, void* ws, size_t wsb) {
    return moe_latent_forward(sh, wt, fake(), fake(), static_cast<double*>(fake()), nullptr,
                              nullptr, static_cast<int32_t*>(fake()), static_cast<float*>(fake()),
                              static_cast<int32_t*>(fake()), static_cast<int32_t*>(fake()), ws,
                              wsb, nullptr);
  };
  CHECK(fwd(nullptr, &w, fake(), need) == MOE_EINVAL);
  CHECK(fwd(&s, nullptr, fake(), need) == MOE_EINVAL);
  CHECK(fwd(&s, &w, fake(), need - 1) == MOE_EWORKSPACE);
  CHECK(fwd(&s, &w, fake(8), need) == MOE_EINVAL);
  moe_shape_t bad = shape(64, 500);
  CHECK(fwd(&bad, &w, fake(), need) != MOE_OK);
  bad = shape(64, 512, 256, 40, 41);
  CHECK(fwd(&bad, &w, fake(), need) == MOE_EINVAL);

  const size_t bneed = moe_backward_workspace_bytes(&s);
  CHECK(bneed > 0);
  moe_grads_t g;
  void** gp = reinterpret_cast<void**>(&g);
  for (size_t i = 0; i < sizeof g / sizeof(void*); ++i) gp[i] = fake();
  auto bwd = [&](const moe_shape_t* sh, const moe_grads_t* gr, void* ws, size_t wsb) {
    return moe_latent_backward(sh, &w, fake(), static_cast<const float*>(fake()),
                               static_cast<const int32_t*>(fake()),
                               static_cast<const float*>(fake()), fake(), gr, ws, wsb, nullptr);
  };
  CHECK(bwd(&s, &g, fake(), bneed - 1) == MOE_EWORKSPACE);
  CHECK(bwd(&s, &g, fake(8), bneed) == MOE_EINVAL);
  CHECK(bwd(&s, nullptr, fake(), bneed) == MOE_EINVAL);
  moe_grads_t g2 = g;
  g2.d_router_logit_offset = nullptr;
  CHECK(bwd(&s, &g2, fake(), bneed) == MOE_EINVAL);
  g2 = g;
  g2.dx = nullptr;
  CHECK(bwd(&s, &g2, fake(), bneed) == MOE_EINVAL);
  moe_shape_t mx = shape(64, 512, 256, 40, 6, 192, 320, MOE_BF16, MOE_MXFP4);
  CHECK(bwd(&mx, &g, fake(), bneed) == MOE_EUNSUPPORTED);

  CHECK(moe_sgd_step(nullptr, &w, &g, 0.1f, nullptr) == MOE_EINVAL);
  CHECK(moe_sgd_step(&s, nullptr, &g, 0.1f, nullptr) == MOE_EINVAL);
  CHECK(moe_sgd_step(&s, &w, nullptr, 0.1f, nullptr) == MOE_EINVAL);
  CHECK(moe_sgd_step(&s, &w, &g, std::numeric_limits<float>::quiet_NaN(), nullptr) == MOE_EINVAL);
  CHECK(moe_sgd_step(&s, &w, &g, std::numeric_limits<float>::infinity(), nullptr) == MOE_EINVAL);
  g2 = g;
  g2.d_router_logit_offset = nullptr;
  CHECK(moe_sgd_step(&s, &w, &g2, 0.1f, nullptr) == MOE_EINVAL);
  CHECK(moe_sgd_step(&mx, &w, &g, 0.1f, nullptr) == MOE_EUNSUPPORTED);

  auto fused = [&](const moe_shape_t* sh, const moe_grads_t* gr, float lr, void* ws, size_t wsb) {
    return moe_latent_backward_sgd(sh, &w, fake(), static_cast<const float*>(fake()),
                                   static_cast<const int32_t*>(fake()),
                                   static_cast<const float*>(fake()), fake(), gr, lr, ws, wsb,
                                   nullptr);
  };
  CHECK(fused(&s, &g, std::numeric_limits<float>::quiet_NaN(), fake(), bneed) == MOE_EINVAL);
  CHECK(fused(&s, &g, 0.1f, fake(), bneed - 1) == MOE_EWORKSPACE);
  CHECK(fused(&s, &g, 0.1f, fake(8), bneed) == MOE_EINVAL);
  CHECK(fused(&s, nullptr, 0.1f, fake(), bneed) == MOE_EINVAL);
  CHECK(fused(&mx, &g, 0.1f, fake(), bneed) == MOE_EUNSUPPORTED);
  CHECK(fused(nullptr, &g, 0.1f, fake(), bneed) == MOE_EINVAL);

  const size_t sneed = moe_saved_activations_bytes(&s);
  CHECK(sneed > 0 && moe_saved_activations_bytes(&mx) == 0 &&
        moe_saved_activations_bytes(nullptr) == 0);
  auto ftrain = [&](void* saved, size_t nsaved) {
    return moe_latent_forward_train(&s, &w, fake(), fake(), static_cast<double*>(fake()), nullptr,
                                    nullptr, static_cast<int32_t*>(fake()),
                                    static_cast<float*>(fake()), static_cast<int32_t*>(fake()),
                                    static_cast<int32_t*>(fake()), saved, nsaved, fake(), need,
                                    nullptr);
  };
  CHECK(ftrain(nullptr, sneed) == MOE_EINVAL);
  CHECK(ftrain(fake(8), sneed) == MOE_EINVAL);
  CHECK(ftrain(fake(), sneed - 1) == MOE_EWORKSPACE);
  auto btrain = [&](void* saved, size_t nsaved, int sgd, float lr) {
    return moe_latent_backward_train(&s, &w, fake(), static_cast<const float*>(fake()),
                                     static_cast<const int32_t*>(fake()),
                                     static_cast<const float*>(fake()), fake(), saved, nsaved, &g,
                                     sgd, lr, fake(), bneed, nullptr);
  };
  CHECK(btrain(nullptr, sneed, 0, 0.f) == MOE_EINVAL);
  CHECK(btrain(fake(), sneed - 1, 0, 0.f) == MOE_EWORKSPACE);
  CHECK(btrain(fake(), sneed, 2, 0.1f) == MOE_EINVAL);
  CHECK(btrain(fake(), sneed, 1, std::numeric_limits<float>::infinity()) == MOE_EINVAL);

  for (auto q : {moe_mxfp8_quantize, moe_mxfp4_quantize}) {
    uint8_t* c = static_cast<uint8_t*>(fake());
    CHECK(q(fake(), 4, 48, c, c, nullptr) == MOE_EINVAL);
    CHECK(q(fake(), -1, 64, c, c, nullptr) == MOE_EINVAL);
    CHECK(q(nullptr, 4, 64, c, c, nullptr) == MOE_EINVAL);
    CHECK(q(fake(8), 4, 64, c, c, nullptr) == MOE_EINVAL);
    CHECK(q(fake(), INT64_MAX, 64, c, c, nullptr) != MOE_OK);
    CHECK(q(fake(), 4, INT64_MAX - 31, c, c, nullptr) != MOE_OK);
    CHECK(q(nullptr, 0, 64, nullptr, nullptr, nullptr) == MOE_OK);
  }
}

static void strings_and_timing() {
  for (int i = -1000; i <= 1000; ++i) {
    const char* a = moe_status_str(i);
    const char* b = moe_stage_name(i);
    CHECK(a && std::strlen(a) > 0 && b && std::strlen(b) > 0);
  }
  CHECK(std::strcmp(moe_status_str(INT_MIN), "unknown status") == 0);
  CHECK(std::strcmp(moe_stage_name(INT_MAX), "unknown") == 0);
  CHECK(moe_stage_timing(0) == MOE_OK);
  CHECK(moe_stage_timing(1) == MOE_OK);
  const int nst = moe_stage_times(nullptr, nullptr, 0);
  CHECK(nst > 0);
  std::vector<double> t(nst + 4, -1.0);
  std::vector<int32_t> c(nst + 4, -1);
  CHECK(moe_stage_times(t.data(), c.data(), nst + 4) == nst);
  for (int i = 0; i < nst; ++i) CHECK(t[i] == 0.0 && c[i] == 0);
  CHECK(t[nst] == -1.0 && c[nst] == -1);  // nothing written past the stages
  CHECK(moe_stage_times(t.data(), c.data(), -5) == nst);
  CHECK(moe_stage_timing(0) == MOE_OK);
}

int main() {
  // The failing calls below are given placeholder pointers; they must never
  // reach a device, so the checks run only where no GPU is visible.
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::printf("skipped: a GPU is visible\n");
    return 0;
  }
  route_queries();
  layer_queries();
  route_validation();
  layer_validation();
  strings_and_timing();
  if (g_fail) {
    std::fprintf(stderr, "%d host checks failed\n", g_fail);
    return 1;
  }
  std::printf("all host checks passed\n");
  return 0;
}

// Routing driver shared by moe_route_qb and moe_latent_forward.
#pragma once

#include "common.hpp"

namespace moe {

// A token's k-th and (k+1)-th largest packed keys, read together as one
// 16-byte load.
struct alignas(16) KeyPair {
  int64_t k, k1;
};

// Device scratch of the routing driver, carved from the caller's workspace.
struct RouteWorkspace {
  float* scoresT;       // [n][T] transposed scores (per-expert margin passes)
  int64_t* bfx;         // [2][n] fixed-point biases (live half chosen on the device)
  KeyPair* th;          // [T] k-th and (k+1)-th largest keys per token
  int32_t* loads;       // [n]
  int32_t* acc;         // [copies][n] load accumulators of the top-k pass (cleared by the status pass)
  int64_t* ctrl;        // control words (phase, counters)
  int32_t* cnt;         // edge count and error flags
  uint64_t* edges;      // sparse edge list of the augmenting-path phase
  int32_t edge_cap;
};

size_t route_workspace_layout(int32_t T, int32_t n, RouteWorkspace* ws, void* base);
int route_validate(int32_t T, int32_t n, int32_t k);
int route_run(const float* scores, int32_t T, int32_t n, int32_t k, int32_t mode,
              int32_t max_rounds, double* bias, int32_t* idx, float* w, int32_t* loads_out,
              int32_t* info, const RouteWorkspace& ws, hipStream_t stream);

}  // namespace moe

// Routing driver shared by moe_route_qb and moe_latent_forward.
#pragma once

#include "common.hpp"

namespace moe {

// Device scratch of the routing driver, carved from the caller's workspace.
struct RouteWorkspace {
  float* scoresT;       // [n][T] transposed scores (per-expert margin passes)
  int64_t* bfx;         // [2][n] fixed-point biases (live half chosen on the device)
  int64_t* th_k;        // [T] k-th largest key per token
  int64_t* th_k1;       // [T] (k+1)-th largest key per token
  int32_t* loads;       // [n]
  int32_t* acc;         // [n] load accumulator of the top-k pass (cleared by the status pass)
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

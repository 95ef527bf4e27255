// Routing driver shared by moe_route_qb, moe_route_sign and moe_latent_forward.
#pragma once

#include "common.hpp"

namespace moe {

// A token's k-th and (k+1)-th largest packed keys.
struct alignas(16) KeyPair {
  int64_t k, k1;
};

// Device scratch of the routing loop, carved from the caller's workspace.
struct RouteWorkspace {
  float* scoresT;       // [n][T] transposed scores (per-expert margin passes)
  int64_t* bfx;         // [2][n] fixed-point biases (live and next)
  KeyPair* th;          // [T] k-th and (k+1)-th largest keys per token
  int32_t* loads;       // [n] loads under the final bias
  int32_t* acc;         // [2][copies][n] load accumulators, one set per step parity
  uint32_t* bar;        // grid-barrier counters (one 256-byte line each) and the abort word
  int64_t* ctrl;        // outcome words of an augmenting-path move, status at entry
  int32_t* cnt;         // edge-segment counters and error flags
  uint64_t* edges;      // sparse edge list of the augmenting-path phase
  int32_t edge_cap;
};

size_t route_workspace_layout(int32_t T, int32_t n, RouteWorkspace* ws, void* base);
int route_validate(int32_t T, int32_t n, int32_t k);
int route_run(const float* scores, int32_t T, int32_t n, int32_t k, int32_t mode,
              int32_t max_rounds, double* bias, int32_t* idx, float* w, int32_t* loads_out,
              int32_t* info, const RouteWorkspace& ws, hipStream_t stream, int cu_share);

}  // namespace moe

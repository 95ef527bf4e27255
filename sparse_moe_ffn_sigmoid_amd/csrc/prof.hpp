// Optional per-stage timing with HIP events on the caller's stream.
#pragma once

#include "common.hpp"

namespace moe {
namespace prof {

enum Stage {
  ST_ROUTER = 0,
  ST_LATENT_DOWN,
  ST_SHARED_GATE_UP,
  ST_ROUTING,
  ST_PERMUTE,
  ST_ROUTED_GATE_UP,
  ST_ROUTED_DOWN,
  ST_COMBINE_RMSNORM,
  ST_UP_SHARED_DOWN,
  ST_COUNT
};

bool enabled();
void record(int stage, bool start, hipStream_t s);

// Records a start event on construction and an end event on destruction.
struct Scope {
  int stage;
  hipStream_t s;
  bool on;
  Scope(int st, hipStream_t str) : stage(st), s(str), on(enabled()) {
    if (on) record(stage, true, s);
  }
  ~Scope() {
    if (on) record(stage, false, s);
  }
};

}  // namespace prof
}  // namespace moe

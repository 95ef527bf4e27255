// Kernels and helpers of the forward layer that the backward pass reuses
// (defined in layer.hip).
#pragma once

#include "common.hpp"
#include "gemm.hpp"

namespace moe {
namespace layer {

__global__ void fill_u32(uint32_t* p, uint32_t v, int64_t count);

// offs = exclusive scan of loads; grouped tile list for tile height bm.
__global__ void scan_and_tiles(const int32_t* loads, int n, int bm, int32_t* offs, int32_t* tiles,
                               int32_t* ntiles);

// sel[e][t] = j + 1 when token t chose expert e as its j-th expert.
__global__ void scatter_sel(const int32_t* idx, int T, int k, uint8_t* sel);

// The tokens that chose e, in increasing token order, take the slots
// offs[e], offs[e]+1, ...: perm[slot] = token, inv[t][j] = slot.
__global__ void expert_slots(const uint8_t* sel, int T, int k, const int32_t* offs, int32_t* perm,
                             int32_t* inv);

// Tile height of the grouped expert GEMMs for this shape.
int grouped_bm(const moe_shape_t& s);

// Activations a training forward keeps for the backward pass (bf16 layers):
// z [T][latent], the experts' pre-activations g and u (fp32) and h (bf16) per
// slot [T*k][inter], the experts' fp32 outputs per slot [T*k][latent], and
// the shared branch's pre-activations gs, us (fp32) and hs (bf16) [T][shared].
// Slots are in the forward's permutation order (experts ascending, tokens
// ascending within an expert).
struct SavedActivations {
  bf16_t* z;
  float* g;
  float* u;
  bf16_t* h;
  float* yp;
  float* gs;
  float* us;
  bf16_t* hs;
};

// Carves the saved activations from base (null: sizes only); returns bytes.
size_t saved_layout(const moe_shape_t& s, SavedActivations* out, void* base);

// One K segment of a GEMM: A [rows][K] (leading dimension lda), B [N][K].
inline gemm::Seg seg(const void* A, int64_t lda, const void* B, int64_t ldb, int K) {
  gemm::Seg g{};
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.K = K;
  return g;
}

}  // namespace layer
}  // namespace moe

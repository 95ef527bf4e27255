// GEMM interfaces of the latent MoE layer: C = epilogue(sum_s A_s B_s^T).
#pragma once

#include "common.hpp"

namespace moe {
namespace gemm {

enum Epilogue : int {
  EPI_BF16 = 0,     // C (bf16) = acc
  EPI_F32 = 1,      // C (f32)  = acc
  EPI_SIGMOID = 2,  // C (f32)  = sigmoid(acc + col_add[col])
  EPI_SITU = 3,     // C (act)  = SiTU-GLU(acc_gate, acc_up); B rows come in gate/up pairs
  EPI_SGD = 4,      // C (bf16, in place) = C - sgd_lr * acc (K-grouped weight gradients only)
};

// B_MXFP4_A8: MXFP4 B with MXFP8 (E4M3) A codes and E8M0 A scales (W4A8);
// B_MXFP4_A4: MXFP4 B with MXFP4 (E2M1, two per byte) A codes (W4A4);
// B_DENSE_KN: bf16 B stored [K][N] (N contiguous, ldb = elements per k-row),
// grouped problems with fp32 outputs only.
enum BFormat : int { B_DENSE = 0, B_MXFP4 = 1, B_MXFP4_A8 = 2, B_MXFP4_A4 = 3, B_DENSE_KN = 4 };

// One K segment: A [rows][K] (K contiguous, leading dim lda), B [N][K] (ldb).
struct Seg {
  const void* A;
  int64_t lda;
  const void* B;   // dense: element type of the GEMM; MXFP4: codes [N][K/2]
  const void* B2;  // EPI_SITU: the "up" matrix paired with B (the gate matrix)
  const uint8_t* Bs;   // MXFP4 scales [N][K/32] for B
  const uint8_t* Bs2;  // MXFP4 scales for B2
  const uint8_t* As;   // B_MXFP4_A8 / _A4: E8M0 scales of A [rows][K/32] (A holds E4M3 or
                       // E2M1 codes, lda in bytes)
  int64_t ldb;         // elements (dense) or bytes (MXFP4 codes)
  int K;
};

struct Params {
  int M;             // rows (dense problems)
  int N;             // output columns
  int nseg;
  Seg seg[4];
  // Grouped problems: per-expert base offsets of B and its scales, the tile
  // list and the gather map from output slot to A row.
  int64_t b_expert_stride;   // elements / code bytes between experts
  int64_t bs_expert_stride;  // scale bytes between experts
  const int32_t* tiles;      // [max_tiles][4] = (expert, row0, rows, -) or null (dense)
  const int32_t* ntiles;     // device count of tiles
  int max_mtiles;            // grid bound on M tiles
  const int32_t* a_rows;     // slot -> A row (null: identity)
  // K-grouped problems (weight gradients of the routed experts): group g
  // multiplies A[:, kofs[g], kofs[g+1]) by B[:, the same range]^T into
  // C + g * c_group_stride, kgroups groups of M x N each.  The K offsets are
  // multiples of 64 (zero-padded ranges); kgroups = 0: off.
  const int32_t* kofs;
  int kgroups;
  int64_t c_group_stride;
  void* C;
  void* C2;                  // bf16 outputs of dense problems: the rounding residue
                             // bf16(v - bf16(v)) of each value, or null
  int64_t ldc;
  const float* col_add;      // EPI_SIGMOID: per-column logit offset or null
  // EPI_SITU with bf16 dense B: also store the pre-activations (fp32, the
  // output's row stride ldc), gate to save_g and up to save_u, or null
  float* save_g;
  float* save_u;
  // Split-K for dense problems with few output tiles: fp32 partial sums
  // [ksplit][M][tiles_n * BN] (set by launch(), room given by partial_bytes),
  // reduced with the epilogue by a second kernel.  Null: no split.
  float sgd_lr;              // EPI_SGD: step size
  float* partial;
  size_t partial_bytes;
  int ksplit;
  // Set by launch() for grouped problems whose output rows can be written
  // 16 bytes per lane (fp32 or SiTU-GLU outputs, no residue or pre-activation
  // stores, N and ldc multiples of 8, C 16-byte aligned): the kernel stages
  // each tile through LDS and writes whole rows with non-temporal stores.
  int stage_out;
};

// Bytes of fp32 partials launch() uses for a bf16 dense problem (0: no split).
size_t splitk_bytes(int M, int N, int K, int epi);

// Whether the pipelined MXFP4 kernel takes 160-row tiles for this K.
size_t fp4_tall_tile_fits(int K);

// Whether the 320-row MXFP4 kernel (scales through the ring) takes this K.
bool fp4_tile320_fits(int K);

// Launch helpers (defined in gemm.hip).  `act_bf16` selects the bf16 MFMA
// kernels, otherwise the fp32 kernels run.
int launch(const Params& p, int epi, int bfmt, bool act_bf16, int bm_hint, hipStream_t stream);

}  // namespace gemm
}  // namespace moe

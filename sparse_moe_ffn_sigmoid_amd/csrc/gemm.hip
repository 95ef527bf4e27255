// MFMA (gfx950) and fp32 GEMM kernels for the latent MoE layer.
//
// Every product of the layer has the form C = epilogue(sum_s A_s B_s^T) with
// both operands K-contiguous ("NT"): the router (three K segments holding
// the exact bf16 split hi/mid/lo of the fp32 router weights against the same
// bf16 tokens), the latent down-projection, the shared gate/up pair, the
// routed gate/up pair per expert (rows gathered by the token permutation),
// the routed down-projection per expert, and the up-projection concatenated
// along K with the shared down-projection (so the shared-expert add is free).
//
// Kernels:
// * gemm_pipe: the main bf16 kernel.  Waves in a WM x WN grid,
//   v_mfma_f32_32x32x16_bf16 on 32x32 blocks; tiles go from HBM straight into
//   LDS (global_load_lds_dwordx4) through a ring of 2 - 3 stages with
//   XOR-swizzled 16-byte chunks; dense, grouped (experts, gathered rows) and
//   K-grouped (expert weight gradients) problems; B stored [N][K] or [K][N]
//   (ds_read_b64_tr_b16).  Dense products store straight from the
//   accumulators; grouped and K-grouped ones stage each fragment pass through
//   the ring and write whole rows, 16 bytes per lane, non-temporally; the
//   in-place SGD update is staged the same way.
// * gemm_pipe_fp4: MXFP4 routed experts.  E2M1 codes go to LDS as they are
//   and are decoded per fragment (E8M0 scales from a per-block panel or the
//   ring), or, with quantised activations (W4A8 / W4A4), multiplied as codes
//   by the scaled MFMA; grouped outputs staged like gemm_pipe's.
// * gemm_bf16: register-staged kernel for shapes outside the pipelined
//   kernels' limits (LDS rows padded by 16 bytes, MXFP4 decoded while
//   written to LDS, epilogue through LDS).
// * gemm_f32: the fp32 layer (FMA), and splitk_reduce: the fixed-order sum
//   of split-K partials with the epilogue.
#include "gemm.hpp"

#include <atomic>

namespace moe {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)
constexpr int NTHREADS = 256;
constexpr int DENSE_GROUP_M = 4;

struct Tile {
  int expert, row0, rows, n0;
};

// Block -> tile, with consecutive tiles kept on one XCD (blocks are dealt to
// the 8 XCDs round robin), M-tile-major so one XCD's L2 reuses the A rows.
// Grouped problems launch for an upper bound on the tile count; the mapping
// spreads only the tiles that exist (the device count) over the XCDs and the
// surplus blocks exit.  Grouped tiles are ordered in pairs of row tiles per
// column tile.
template <int BM>
__device__ __forceinline__ bool locate_tile(const Params& p, int ntn, int bn_out, Tile& t) {
  const int b = blockIdx.x;
  if (p.kgroups > 0) {  // one M x N problem per group, tiles column by column
    const int G = gridDim.x;
    const int tau = (b & 7) * (G >> 3) + (b >> 3);
    const int ntm = (p.M + BM - 1) / BM;
    const int per = ntm * ntn;
    if (tau >= p.kgroups * per) return false;
    const int grp = tau / per, r = tau - grp * per;
    const int mt = r % ntm, nt = r / ntm;
    t.expert = grp;
    t.row0 = mt * BM;
    t.rows = min(BM, p.M - t.row0);
    t.n0 = nt * bn_out;
    return true;
  }
  if (p.tiles) {
    const int nt_m = *p.ntiles;
    const int gv = nt_m * ntn;
    const int gv8 = (gv + 7) & ~7;
    if (b >= gv8) return false;
    const int tau = (b & 7) * (gv8 >> 3) + (b >> 3);
    if (tau >= gv) return false;
    // pairs of row tiles per column tile: the two row tiles of a tall expert
    // read the same weight rows side by side (one XCD's L2)
    int mt, nt;
    const int pair = tau / (2 * ntn);
    if (2 * pair + 1 < nt_m) {
      const int r = tau - pair * 2 * ntn;
      nt = r >> 1;
      mt = 2 * pair + (r & 1);
    } else {  // an odd last row tile
      mt = 2 * pair;
      nt = tau - pair * 2 * ntn;
    }
    const int32_t* q = p.tiles + 4 * mt;
    t.expert = q[0];
    t.row0 = q[1];
    t.rows = q[2];
    t.n0 = nt * bn_out;
    return true;
  }
  const int G = gridDim.x;
  const int tau = (b & 7) * (G >> 3) + (b >> 3);
  const int ntm = (p.M + BM - 1) / BM;
  if (tau >= ntm * ntn) return false;
  // groups of DENSE_GROUP_M row tiles walked column by column: the blocks an
  // XCD runs side by side share a few A and B panels in its L2
  const int grp = tau / (DENSE_GROUP_M * ntn);
  const int gm = min(DENSE_GROUP_M, ntm - grp * DENSE_GROUP_M);
  const int r = tau - grp * DENSE_GROUP_M * ntn;
  const int mt = grp * DENSE_GROUP_M + r % gm, nt = r / gm;
  t.expert = 0;
  t.row0 = mt * BM;
  t.rows = min(BM, p.M - t.row0);
  t.n0 = nt * bn_out;
  return true;
}

// bf16 bit pattern of an E2M1 magnitude code m (values 0, .5, 1, 1.5, 2, 3, 4, 6):
// 0.5 is special, otherwise exponent 126 + m/2 and mantissa bit (m & 1).
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t m) {
  if (m == 0u) return 0u;
  if (m == 1u) return 0x3F00u;
  return ((126u + (m >> 1)) << 7) | ((m & 1u) << 6);
}

// 8 MXFP4 codes (one 32-bit word, element 0 in the low nibble) times the
// E8M0 scale 2^(sbyte-127) -> 8 bf16.  For scale bytes 2..252 every product
// is a normal bf16, and the scale is added to the exponent field; outside
// that range the products are formed in fp32 (exact: an E2M1 value has two
// significant bits, so 2^-128 and up are representable, and products above
// the bf16 range become infinities); byte 255, NaN in the format, gives NaN.
__device__ __forceinline__ u32x4_t decode8(uint32_t q, int32_t sbyte) {
  u32x4_t out;
  if (sbyte >= 2 && sbyte <= 252) {
    const int32_t exp_add = (sbyte - 127) << 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t nib = (q >> (8 * i + 4 * h)) & 15u;
        const uint32_t mag = nib & 7u;
        uint32_t bits = e2m1_bits(mag);
        bits = mag ? static_cast<uint32_t>(static_cast<int32_t>(bits) + exp_add) : 0u;
        bits |= (nib & 8u) << 12;
        pair |= bits << (16 * h);
      }
      out[i] = pair;
    }
    return out;
  }
  // 2^(sbyte-127) in fp32: 2^-127 is a subnormal
  const float sc = sbyte == 255 ? __uint_as_float(0x7FC00000u)
                                : __uint_as_float(sbyte ? (static_cast<uint32_t>(sbyte) << 23)
                                                        : 0x00400000u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t pair = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t nib = (q >> (8 * i + 4 * h)) & 15u;
      const float v = __uint_as_float(e2m1_bits(nib & 7u) << 16) * sc;
      // v has at most two significant bits: dropping the low half is exact
      const uint32_t bits = (__float_as_uint(v) >> 16) | ((nib & 8u) << 12);
      pair |= bits << (16 * h);
    }
    out[i] = pair;
  }
  return out;
}

// A bf16 output value and, where a second output is given, the bf16 of
// what the first one rounded away: hi + lo holds v to about 16 bits.
__device__ __forceinline__ void store_bf16(void* C, void* C2, int64_t off, float v) {
  const bf16_t hi = f32_to_bf16(v);
  static_cast<bf16_t*>(C)[off] = hi;
  if (C2) static_cast<bf16_t*>(C2)[off] = f32_to_bf16(v - bf16_to_f32(hi));
}
__device__ __forceinline__ void store_bf16(const Params& p, int64_t off, float v) {
  store_bf16(p.C, p.C2, off, v);
}

template <int BM, int BN, int WM, int EPI, int BFMT>
__global__ __launch_bounds__(NTHREADS) void gemm_bf16(Params p) {
  constexpr int WN = 4 / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold 32x32 blocks");
  constexpr int BN_OUT = (EPI == EPI_SITU) ? BN / 2 : BN;
  constexpr int A_CH = BM * (BK / 8) / NTHREADS;  // 16-byte chunks per thread
  constexpr int B_CH = (BFMT == B_DENSE) ? BN * (BK / 8) / NTHREADS : BN * 2 / NTHREADS;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for 256 threads");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* As = reinterpret_cast<bf16_t*>(smem);            // [2][BM][LDK]
  bf16_t* Bs = As + 2 * BM * LDK;                          // [2][BN][LDK]

  const int ntn = (EPI == EPI_SITU) ? (p.N + BN_OUT - 1) / BN_OUT : (p.N + BN - 1) / BN;
  Tile tile;
  if (!locate_tile<BM>(p, ntn, BN_OUT, tile)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // per-thread A row pointers (gather) for its chunks
  int a_row[A_CH];
  bool a_ok[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + NTHREADS * i;
    const int r = c >> 3;
    a_ok[i] = r < tile.rows;
    const int slot = tile.row0 + r;
    a_row[i] = a_ok[i] ? (p.a_rows ? p.a_rows[slot] : slot) : 0;
  }
  // per-thread B row of its chunks
  int b_row[B_CH];
  bool b_ok[B_CH];
  bool b_up[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + NTHREADS * i;
    const int r = (BFMT == B_DENSE) ? (c >> 3) : (c >> 1);
    if (EPI == EPI_SITU) {
      b_up[i] = r >= BN / 2;
      b_row[i] = tile.n0 + (r % (BN / 2));
    } else {
      b_up[i] = false;
      b_row[i] = tile.n0 + r;
    }
    b_ok[i] = b_row[i] < p.N;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int ktot = 0;
  for (int s = 0; s < p.nseg; ++s) ktot += p.seg[s].K / BK;

  u32x4_t ra[A_CH];
  u32x4_t rb[B_CH];
  int32_t rsc[B_CH];

  auto load_tile = [&](int kt) {
    int s = 0, kk = kt;
    while (s < p.nseg - 1 && kk >= p.seg[s].K / BK) {
      kk -= p.seg[s].K / BK;
      ++s;
    }
    const Seg& g = p.seg[s];
    const int k0 = kk * BK;
    const bf16_t* A = static_cast<const bf16_t*>(g.A);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + NTHREADS * i;
      const int kc = c & 7;
      if (a_ok[i])
        ra[i] = *reinterpret_cast<const u32x4_t*>(A + static_cast<int64_t>(a_row[i]) * g.lda + k0 + kc * 8);
      else
        ra[i] = u32x4_t{0, 0, 0, 0};
    }
    if (BFMT == B_DENSE) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + NTHREADS * i;
        const int kc = c & 7;
        const bf16_t* B = static_cast<const bf16_t*>(b_up[i] ? g.B2 : g.B) +
                          static_cast<int64_t>(tile.expert) * p.b_expert_stride;
        if (b_ok[i])
          rb[i] = *reinterpret_cast<const u32x4_t*>(B + static_cast<int64_t>(b_row[i]) * g.ldb + k0 + kc * 8);
        else
          rb[i] = u32x4_t{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + NTHREADS * i;
        const int half = c & 1;
        const uint8_t* Bq = static_cast<const uint8_t*>(b_up[i] ? g.B2 : g.B) +
                            static_cast<int64_t>(tile.expert) * p.b_expert_stride;
        const uint8_t* Bsc = (b_up[i] ? g.Bs2 : g.Bs) +
                             static_cast<int64_t>(tile.expert) * p.bs_expert_stride;
        if (b_ok[i]) {
          rb[i] = *reinterpret_cast<const u32x4_t*>(Bq + static_cast<int64_t>(b_row[i]) * g.ldb +
                                                    (k0 >> 1) + half * 16);
          rsc[i] = Bsc[static_cast<int64_t>(b_row[i]) * (g.ldb >> 4) + (k0 >> 5) + half];
        } else {
          rb[i] = u32x4_t{0, 0, 0, 0};
          rsc[i] = 127;
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    bf16_t* a_s = As + buf * BM * LDK;
    bf16_t* b_s = Bs + buf * BN * LDK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + NTHREADS * i;
      *reinterpret_cast<u32x4_t*>(a_s + (c >> 3) * LDK + (c & 7) * 8) = ra[i];
    }
    if (BFMT == B_DENSE) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + NTHREADS * i;
        *reinterpret_cast<u32x4_t*>(b_s + (c >> 3) * LDK + (c & 7) * 8) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + NTHREADS * i;
        const int r = c >> 1, half = c & 1;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<u32x4_t*>(b_s + r * LDK + half * 32 + w * 8) = decode8(rb[i][w], rsc[i]);
      }
    }
  };

  if (ktot > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = 0; kt < ktot; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktot) load_tile(kt + 1);
    const bf16_t* a_s = As + buf * BM * LDK;
    const bf16_t* b_s = Bs + buf * BN * LDK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[FM], bfr[FN];
      const int koff = kk * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(a_s + (wm * WTM + i * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(b_s + (wn * WTN + j * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < ktot) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue through LDS ----
  constexpr int LDC = BN + 4;
  float* Ct = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * WTN + j * 32 + (lane & 31);
        Ct[row * LDC + col] = acc[i][j][r];
      }
  __syncthreads();
  constexpr int CH = BN_OUT / 8;
  for (int idx = tid; idx < BM * CH; idx += NTHREADS) {
    const int r = idx / CH, c = (idx % CH) * 8;
    if (r >= tile.rows) continue;
    const int col = tile.n0 + c;
    if (col >= p.N) continue;
    const int64_t orow = tile.row0 + r;
    float v[8];
    if (EPI == EPI_SITU) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = situ_glu(Ct[r * LDC + c + e], Ct[r * LDC + c + e + BN / 2]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Ct[r * LDC + c + e];
    }
    const int nval = min(8, p.N - col);
    if (EPI == EPI_BF16 || EPI == EPI_SITU) {
      bf16_t* C = static_cast<bf16_t*>(p.C) + orow * p.ldc + col;
      if (nval == 8) {
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = static_cast<uint32_t>(f32_to_bf16(v[2 * e])) |
                 (static_cast<uint32_t>(f32_to_bf16(v[2 * e + 1])) << 16);
        *reinterpret_cast<u32x4_t*>(C) = o;
      } else {
        for (int e = 0; e < nval; ++e) C[e] = f32_to_bf16(v[e]);
      }
    } else {
      float* C = static_cast<float*>(p.C) + orow * p.ldc + col;
      for (int e = 0; e < nval; ++e) {
        float x = v[e];
        if (EPI == EPI_SIGMOID) {
          if (p.col_add) x += p.col_add[col + e];
          x = 1.0f / (1.0f + expf(-x));
        }
        C[e] = x;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined bf16 kernel for dense B operands.
//
// Tiles move from HBM straight into LDS with global_load_lds_dwordx4 (each
// lane supplies its own global address -- row gathers included -- and the 64
// lanes of an instruction fill 1 KB of LDS in lane order), through a ring of
// three stages so that two tiles are in flight while the MFMAs consume the
// third.  A stage holds BK = 64 or 32 K-elements per row (128- or 64-byte
// rows); the 16-byte chunk index is XORed with a function of the row so that
// both the lane-ordered fills and the 32-row fragment reads are free of bank
// conflicts.  Each stage lives in its own __shared__ array, the waits count
// only this wave's own loads (s_waitcnt vmcnt) and the barrier is fenced for
// the compiler only, so loads stay in flight across barriers.  For SiTU-GLU
// the gate and up rows of B alternate in groups of 32, so every wave holds
// both halves of its outputs in registers; results are stored straight from
// the accumulators.
// ---------------------------------------------------------------------------
constexpr int STAGES = 3;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte global -> LDS copy per lane (lane i fills bytes [16i, 16i+16) after
// the wave-uniform LDS base in M0).  Issued as inline assembly so that the
// compiler does not track these LDS writes: it would otherwise wait for every
// load in flight (vmcnt(0)) before the LDS reads of another stage, which
// drains the ring.  The kernels order them explicitly (vmcnt waits, then a
// barrier) and no other instruction in them uses M0.
__device__ __forceinline__ void load_lds16_asm(const void* g, void* lds, bool nt = false) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if (nt)  // read once: non-temporal cache policy
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(m)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m)
                 : "memory", "m0");
#pragma clang diagnostic pop
#endif
}

// 4-byte global -> LDS copy per lane (lane i fills bytes [4i, 4i+4) after the
// M0 base); same ordering rules as load_lds16_asm.
__device__ __forceinline__ void load_lds4_asm(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m) : "memory", "m0");
#pragma clang diagnostic pop
#endif
}

__device__ __forceinline__ void load_lds16(const bf16_t* g, bf16_t* lds, bool nt = false) {
  load_lds16_asm(g, lds, nt);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `ahead` stages of PER load instructions each are still
// in flight (ahead is uniform across the block and at most MAXA).
template <int MAXA, int PER>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (MAXA <= 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= MAXA)
      wait_vmcnt<MAXA * PER>();
    else
      wait_stages<MAXA - 1, PER>(ahead);
  }
}

// chunk swizzle of a row: 128-byte rows XOR with r mod 8, 64-byte rows with
// (r / 2) mod 4 (two rows share a 128-byte bank window)
template <int BKP>
__device__ __forceinline__ int swz(int r) {
  return BKP == 64 ? (r & 7) : ((r >> 1) & 3);
}

// B stored [K][N] (BKN): a stage holds BKP k-rows of BN columns (N
// contiguous), 16-byte chunks swizzled by kn_swz(row) = 0, 6, 12, 10 for
// row mod 4.  The B operand of an MFMA comes from two ds_read_b64_tr_b16
// reads: within each 16-lane group, lane 4j + q addresses the 4 columns
// n0 + 4q .. n0 + 4q + 3 of k-row k0 + j, and lane i receives column n0 + i
// of k-rows k0 .. k0 + 3.  The swizzle keeps the 4 rows x 32 bytes of one
// group, and the 4 rows x 64 bytes of two groups, on distinct LDS banks.
__device__ __forceinline__ int kn_swz(int row) { return (6 * (row & 1)) ^ (12 * ((row >> 1) & 1)); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t read_b_kn(const bf16_t* lo, const bf16_t* hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lo));
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(hi));
  const s16x8_t v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
#else
  (void)lo;
  (void)hi;
  return bf16x8_t{};
#endif
}

// BKN: B is stored [K][N] (see kn_swz); EPI_F32 / EPI_BF16 only.
template <int BM, int BN, int WM, int EPI, int BKP, int NST, bool BNT, int NW, bool BKN = false>
__global__ __launch_bounds__(64 * NW, (NW == 4 && BKP == 32 && BM * BN <= 128 * 256) ? 2 : 1) void gemm_pipe(Params p) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per block");
  constexpr int WN = NW / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold 32x32 blocks");
  static_assert(EPI != EPI_SITU || FN % 2 == 0, "SiTU needs gate/up fragment pairs");
  static_assert(BKP == 64 || BKP == 32, "stage depth");
  static_assert(!BKN || (EPI != EPI_SITU && EPI != EPI_SIGMOID && BN % 128 == 0),
                "[K][N] B operands: plain epilogues, 16 or more chunks per k-row");
  constexpr int BN_OUT = (EPI == EPI_SITU) ? BN / 2 : BN;
  constexpr int CH = BKP / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / CH;       // rows per load instruction
  constexpr int NA = BM / RPI, NB = BN / RPI;
  static_assert(NA * RPI == BM && NB * RPI == BN, "tile rows per instruction");
  constexpr int MA = (NA + NW - 1) / NW, MB = (NB + NW - 1) / NW;
  static_assert(NA >= NW && NB >= NW, "every wave loads A and B rows");
  // Every wave issues MA (MB) load instructions per stage; when NW does not
  // divide NA (NB) the surplus ones repeat the wave's own instruction i-1
  // (same source, same LDS bytes), so the per-wave count of outstanding loads
  // is uniform and known at compile time.
  auto a_ins = [](int w, int i) { const int x = w + NW * i; return x < NA ? x : x - NW; };
  auto b_ins = [](int w, int i) { const int x = w + NW * i; return x < NB ? x : x - NW; };

  static_assert(NST >= 2 && NST <= 6, "ring depth");
  static_assert((NST - 2) * (MA + MB) < 64, "loads in flight exceed the vmcnt range");
  // One LDS variable per stage (A rows, then B rows): the compiler tracks
  // direct-to-LDS loads per variable, so reads of one stage do not wait for
  // loads still in flight into another.
  constexpr int SW = (BM + BN) * BKP;
  __shared__ __attribute__((aligned(1024))) bf16_t st0[SW];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[SW];
  // (unused stages are 16-byte stubs, so a 160 KB ring is not pushed over
  // the limit by alignment padding)
  __shared__ __attribute__((aligned(NST >= 3 ? 1024 : 16))) bf16_t st2[NST >= 3 ? SW : 8];
  __shared__ __attribute__((aligned(NST >= 4 ? 1024 : 16))) bf16_t st3[NST >= 4 ? SW : 8];
  __shared__ __attribute__((aligned(NST >= 5 ? 1024 : 16))) bf16_t st4[NST >= 5 ? SW : 8];
  __shared__ __attribute__((aligned(NST >= 6 ? 1024 : 16))) bf16_t st5[NST >= 6 ? SW : 8];
  bf16_t* const stg[6] = {st0, st1, st2, st3, st4, st5};

  const int ntn = (p.N + BN_OUT - 1) / BN_OUT;
  Tile tile;
  int ks = 0;  // K split of this block (dense problems with few tiles)
  const int kn = p.ksplit > 1 ? p.ksplit : 1;
  if (kn > 1) {
    const int G = gridDim.x, b = blockIdx.x;
    int tau = (b & 7) * (G >> 3) + (b >> 3);
    ks = tau % kn;
    tau /= kn;
    const int mt = tau / ntn;
    tile.expert = 0;
    tile.row0 = mt * BM;
    if (tile.row0 >= p.M) return;
    tile.rows = min(BM, p.M - tile.row0);
    tile.n0 = (tau - mt * ntn) * BN_OUT;
  } else if (!locate_tile<BM>(p, ntn, BN_OUT, tile)) {
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // rows this lane fills in each of its load instructions (clamped to valid
  // rows; rows past the tile only feed outputs that are never stored)
  const int lrow = lane / CH;
  int64_t a_off[MA];  // row * lda + chunk * 8 is set per segment; here row and chunk
  int a_chunk[MA];
#pragma unroll
  for (int i = 0; i < MA; ++i) {
    const int ins = a_ins(wave, i);
    int r = ins * RPI + lrow;
    a_chunk[i] = (lane % CH) ^ swz<BKP>(r);
    r = r < tile.rows ? r : 0;
    const int slot = tile.row0 + r;
    a_off[i] = p.a_rows ? p.a_rows[slot] : slot;
  }
  int64_t b_off[MB];
  int b_chunk[MB];
  bool b_up[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if constexpr (BKN) {  // k-row of the stage and the first column of this lane's chunk
      constexpr int CPR = BN / 8;
      const int slot = b_ins(wave, i) * 64 + lane;
      const int kr = slot / CPR;
      int col = tile.n0 + ((slot % CPR) ^ kn_swz(kr)) * 8;
      col = col + 8 <= p.N ? col : p.N - 8;  // past N: a valid chunk, never stored
      b_up[i] = false;
      b_off[i] = kr;
      b_chunk[i] = col;
      continue;
    }
    const int r = b_ins(wave, i) * RPI + lrow;
    b_chunk[i] = (lane % CH) ^ swz<BKP>(r);
    int row;
    if (EPI == EPI_SITU) {
      const int g = r >> 5;
      b_up[i] = g & 1;
      row = tile.n0 + (g >> 1) * 32 + (r & 31);
    } else {
      b_up[i] = false;
      row = tile.n0 + r;
    }
    b_off[i] = row < p.N ? row : p.N - 1;
  }

  int kall = 0;
  for (int sg = 0; sg < p.nseg; ++sg) kall += p.seg[sg].K / BKP;
  // K-grouped problems: this group's K range of the single segment
  const int64_t kbase = p.kgroups > 0 ? p.kofs[tile.expert] : 0;
  if (p.kgroups > 0) kall = (p.kofs[tile.expert + 1] - p.kofs[tile.expert]) / BKP;
  // stages of segment sg (a K-grouped problem's one segment spans its range)
  auto seg_stages = [&](int sg) { return p.kgroups > 0 ? kall : p.seg[sg].K / BKP; };
  // this block's K stages [k_begin, k_begin + ktot) of the concatenated segments
  const int k_begin = (ks * kall) / kn;
  const int ktot = ((ks + 1) * kall) / kn - k_begin;

  // Per-lane source pointers of the next tile to issue; tiles are issued in
  // order, so the pointers advance by one stage of K and are reset at
  // segment starts.
  const bf16_t* pa[MA];
  const bf16_t* pb[MB];
  int64_t bstep = BKP;  // elements a B pointer advances per stage
  int seg_i = -1, seg_end = 0, next_kt = k_begin;
  auto start_segment = [&](int sg, int skip) {
    const Seg& g = p.seg[sg];
    const bf16_t* A = static_cast<const bf16_t*>(g.A) + kbase + skip;
    const bf16_t* B = static_cast<const bf16_t*>(g.B) +
                      static_cast<int64_t>(tile.expert) * p.b_expert_stride + kbase + skip;
    const bf16_t* B2 = static_cast<const bf16_t*>(g.B2) +
                       static_cast<int64_t>(tile.expert) * p.b_expert_stride + kbase + skip;
#pragma unroll
    for (int i = 0; i < MA; ++i)
      pa[i] = A + a_off[i] * g.lda + a_chunk[i] * 8;
    if constexpr (BKN) {
      // B [K][N]: k advances by rows
      const bf16_t* Bk = static_cast<const bf16_t*>(g.B) +
                         static_cast<int64_t>(tile.expert) * p.b_expert_stride +
                         (kbase + skip) * g.ldb;
#pragma unroll
      for (int i = 0; i < MB; ++i) pb[i] = Bk + b_off[i] * g.ldb + b_chunk[i];
      bstep = static_cast<int64_t>(BKP) * g.ldb;
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i) pb[i] = (b_up[i] ? B2 : B) + b_off[i] * g.ldb + b_chunk[i] * 8;
    }
  };
  if (ktot > 0) {  // position the walk at k_begin
    int seg_start = 0;
    do {
      ++seg_i;
      seg_start = seg_end;
      seg_end += seg_stages(seg_i);
    } while (seg_end <= k_begin);
    start_segment(seg_i, (k_begin - seg_start) * BKP);
  }
  auto issue = [&](bf16_t* As, bf16_t* Bs) {
    if (next_kt == seg_end) {
      ++seg_i;
      start_segment(seg_i, 0);
      seg_end += seg_stages(seg_i);
    }
    ++next_kt;
#pragma unroll
    for (int i = 0; i < MA; ++i) {
      load_lds16(pa[i], As + a_ins(wave, i) * 512);
      pa[i] += BKP;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      load_lds16(pb[i], Bs + b_ins(wave, i) * 512, BNT);
      pb[i] += bstep;
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](const bf16_t* As, const bf16_t* Bs) {
    const int hi = lane >> 5, sw = swz<BKP>(lane & 31);
#pragma unroll
    for (int kk = 0; kk < BKP / 16; ++kk) {
      const int ch = ((kk * 2 + hi) ^ sw) * 8;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * WTM + i * 32 + (lane & 31)) * BKP + ch);
      if constexpr (BKN) {
        // lane (group g, 4j + q): k-rows kk*16 + (g/2)*8 + j (+4), columns
        // (g%2)*16 + 4q of the fragment
        const int grp = lane >> 4, jq = lane & 15;
        const int r0 = kk * 16 + (grp >> 1) * 8 + (jq >> 2);
        const int sw = kn_swz(r0);  // r0 + 4 has the same swizzle
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = wn * WTN + j * 32 + (grp & 1) * 16 + (jq & 3) * 4;
          const int off = ((col >> 3) ^ sw) * 8 + (col & 7);
          bfr[j] = read_b_kn(Bs + r0 * BN + off, Bs + (r0 + 4) * BN + off);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * WTN + j * 32 + (lane & 31)) * BKP + ch);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // prologue: tiles 0 .. NST-2 in flight
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < ktot) issue(stg[s], stg[s] + BM * BKP);
  // one ring step: wait for tile kt (tiles kt+1 .. kt+NST-2 may stay in
  // flight), refill the stage freed by tile kt-1 with tile kt+NST-1, multiply
  // tile kt
  auto ring = [&](int kt, bf16_t* Ac, bf16_t* Bc, bf16_t* An, bf16_t* Bn) {
    if (kt < ktot) {  // uniform across the block
      const int ahead = min(NST - 2, ktot - 1 - kt);  // tiles issued after tile kt
      wait_stages<NST - 2, MA + MB>(ahead);
      lds_barrier();
      if (kt + NST - 1 < ktot) issue(An, Bn);
      compute(Ac, Bc);
    }
  };
  for (int kt = 0; kt < ktot; kt += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      bf16_t* cur = stg[s];
      bf16_t* nxt = stg[(s + NST - 1) % NST];
      ring(kt + s, cur, cur + BM * BKP, nxt, nxt + BM * BKP);
    }
  }

  // ---- epilogue straight from the accumulators ----
  const int64_t cgrp = p.kgroups > 0 ? tile.expert * p.c_group_stride : 0;
  if constexpr (EPI == EPI_SGD) {
    // The fp32 tile passes through the ring's two stages (128 rows x BN
    // floats) in two halves, so that every lane updates eight consecutive
    // weights with one 16-byte load and one 16-byte store.
    static_assert(WM == 2 && WTM == 128 && NST == 2 && BN == 256 &&
                      SW * sizeof(bf16_t) == 64 * BN * sizeof(float),
                  "the staged update needs 256 x 256 tiles on two 64-element stages");
    constexpr int CPW = BN / 8;  // 8-column chunks per row
    constexpr int PER = 128 * CPW / (64 * NW);
    float* const hb0 = reinterpret_cast<float*>(stg[0]);
    float* const hb1 = reinterpret_cast<float*>(stg[1]);
    lds_barrier();  // every wave is done with the ring
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            float* dst = ((lr >> 6) ? hb1 : hb0) + (lr & 63) * BN + wn * WTN + (lane & 31);
#pragma unroll
            for (int j = 0; j < FN; ++j) dst[j * 32] = acc[i][j][r];
          }
      }
      lds_barrier();
      uint4 wv[PER];
      bf16_t* wp[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int c = tid + q * 64 * NW, lr = c / CPW, col = tile.n0 + (c % CPW) * 8;
        const bool ok = h * 128 + lr < tile.rows && col < p.N;
        wp[q] = ok ? static_cast<bf16_t*>(p.C) + cgrp + (tile.row0 + h * 128 + lr) * p.ldc + col
                   : nullptr;
        if (ok) wv[q] = *reinterpret_cast<const uint4*>(wp[q]);
      }
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        if (!wp[q]) continue;
        const int c = tid + q * 64 * NW, lr = c / CPW;
        const float* src = ((lr >> 6) ? hb1 : hb0) + (lr & 63) * BN + (c % CPW) * 8;
        const float4 g0 = *reinterpret_cast<const float4*>(src);
        const float4 g1 = *reinterpret_cast<const float4*>(src + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        uint32_t words[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = sgd_value(bf16_to_f32(static_cast<bf16_t>(words[e] & 0xFFFFu)),
                                     gv[2 * e], p.sgd_lr);
          const float hi = sgd_value(bf16_to_f32(static_cast<bf16_t>(words[e] >> 16)),
                                     gv[2 * e + 1], p.sgd_lr);
          words[e] = static_cast<uint32_t>(f32_to_bf16(lo)) |
                     (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
        }
        *reinterpret_cast<uint4*>(wp[q]) = make_uint4(words[0], words[1], words[2], words[3]);
      }
      lds_barrier();
    }
    return;
  }
  // Staged output (grouped and K-grouped problems, see Params::stage_out):
  // per pass, every wave of the pass's row groups writes one 32-row fragment
  // of its results (fp32, or SiTU-GLU as bf16) into stage 0 of the ring
  // (all row groups at once when they fit, else one at a time), rows padded
  // by 32 bytes so that the two row halves of one store land on different
  // banks; then each lane copies 16 bytes, a wave's store covering whole
  // output rows, with the non-temporal policy (the outputs are read once, by
  // the next kernel).  Bit-identical to the direct epilogue below; writing
  // rows instead of 2- and 4-byte pieces, and keeping them out of L2, costs
  // less of the weight stream's bandwidth.
  constexpr int ST_ESZ = (EPI == EPI_SITU) ? 2 : 4;
  constexpr int ST_RB = BN_OUT * ST_ESZ, ST_RBP = ST_RB + 32;
  if constexpr ((EPI == EPI_F32 || EPI == EPI_SITU) && 32 * ST_RBP <= SW * 2 &&
                ST_RB % 16 == 0) {
    if (p.stage_out && kn == 1) {
      typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
      constexpr int GP = WM * 32 * ST_RBP <= SW * 2 ? WM : 1;  // row groups per pass
      constexpr int CPR = ST_RB / 16;  // 16-byte chunks per output row
      char* const sb = reinterpret_cast<char*>(stg[0]);
      char* const cbase = static_cast<char*>(p.C) + cgrp * ST_ESZ;
      lds_barrier();  // every wave is done with the ring
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int h0 = 0; h0 < WM; h0 += GP) {
          if (h0 * WTM + i * 32 < tile.rows) {  // uniform: the pass holds valid rows
            if (wm >= h0 && wm < h0 + GP) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int lr = (wm - h0) * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if constexpr (EPI == EPI_SITU) {
#pragma unroll
                  for (int j = 0; j < FN; j += 2) {
                    const int oc = ((wn * FN + j) >> 1) * 32 + (lane & 31);
                    *reinterpret_cast<bf16_t*>(sb + lr * ST_RBP + oc * 2) =
                        f32_to_bf16(situ_glu(acc[i][j][r], acc[i][j + 1][r]));
                  }
                } else {
#pragma unroll
                  for (int j = 0; j < FN; ++j) {
                    const int oc = wn * WTN + j * 32 + (lane & 31);
                    *reinterpret_cast<float*>(sb + lr * ST_RBP + oc * 4) = acc[i][j][r];
                  }
                }
              }
            }
            lds_barrier();
#pragma unroll
            for (int c0 = 0; c0 < GP * 32 * CPR; c0 += 64 * NW) {
              const int c = c0 + tid;
              const int lr = c / CPR, ch = c % CPR;
              const int row = (h0 + (lr >> 5)) * WTM + i * 32 + (lr & 31);
              const int col = tile.n0 + ch * (16 / ST_ESZ);
              if (c < GP * 32 * CPR && row < tile.rows && col < p.N) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sb + lr * ST_RBP + ch * 16);
                char* dst = cbase + ((static_cast<int64_t>(tile.row0) + row) * p.ldc + col) * ST_ESZ;
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
              }
            }
            lds_barrier();
          }
        }
      }
      return;
    }
  }
  if (kn > 1) {  // fp32 partials, columns in B-row order of the tile
    const int64_t nv = static_cast<int64_t>(ntn) * BN;
    const int64_t cb = static_cast<int64_t>(tile.n0 / BN_OUT) * BN + wn * WTN + (lane & 31);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row >= tile.rows) continue;
        float* dst = p.partial + (static_cast<int64_t>(ks) * p.M + tile.row0 + row) * nv + cb;
#pragma unroll
        for (int j = 0; j < FN; ++j) dst[j * 32] = acc[i][j][r];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (row >= tile.rows) continue;
      const int64_t orow = tile.row0 + row;
      if (EPI == EPI_SITU) {
#pragma unroll
        for (int j = 0; j < FN; j += 2) {
          const int grp = wn * FN + j;  // even: gate group, odd: its up group
          const int col = tile.n0 + (grp >> 1) * 32 + (lane & 31);
          if (col < p.N) {
            store_bf16(p, orow * p.ldc + col, situ_glu(acc[i][j][r], acc[i][j + 1][r]));
            if (p.save_g) {
              p.save_g[orow * p.ldc + col] = acc[i][j][r];
              p.save_u[orow * p.ldc + col] = acc[i][j + 1][r];
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = tile.n0 + wn * WTN + j * 32 + (lane & 31);
          if (col >= p.N) continue;
          if (EPI == EPI_SIGMOID) {
            float x = acc[i][j][r];
            if (p.col_add) x += p.col_add[col];
            static_cast<float*>(p.C)[orow * p.ldc + col] = 1.0f / (1.0f + expf(-x));
          } else if (EPI == EPI_F32) {
            static_cast<float*>(p.C)[cgrp + orow * p.ldc + col] = acc[i][j][r];
          } else {
            store_bf16(p, orow * p.ldc + col, acc[i][j][r]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined kernel with MXFP4 B operands (bf16 A).
//
// Same ring as gemm_pipe with 64 K-elements per stage; the B stage holds the
// raw codes (32 bytes per row), copied straight to LDS.  The E8M0 scales of
// the block's B rows for the whole K range (K/32 bytes per row) are copied to
// an LDS panel once, before the ring starts.  The K order inside a stage is
// permuted identically for A and B so that each lane's codes for a whole
// stage are one 16-byte LDS read under a single scale byte: MFMA step kk of
// lane half h uses the 8 elements of chunk 4h + kk.  Codes are decoded with
// v_cvt_scalef32_pk_bf16_fp4 (two E2M1 values times the block scale per
// instruction).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load_lds16_raw(const void* g, void* lds) { load_lds16_asm(g, lds); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 8 E2M1 codes (one word, element 0 in the low nibble) times the scale -> 8 bf16
__device__ __forceinline__ bf16x8_t decode8_hw(uint32_t q, float scale) {
  bf16x8_t out = {};
#if defined(__HIP_DEVICE_COMPILE__)
  const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  out[0] = v0[0]; out[1] = v0[1]; out[2] = v1[0]; out[3] = v1[1];
  out[4] = v2[0]; out[5] = v2[1]; out[6] = v3[0]; out[7] = v3[1];
#endif
  return out;
}

// E8M0 byte -> fp32 2^(e-127) (e = 0 gives the subnormal 2^-127, 255 NaN)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e == 255u ? 0x7FC00000u : e ? (e << 23) : 0x00400000u);
}

// NW: waves per block.  SR: the E8M0 scales travel through the ring (4 bytes
// per B row per stage: the scale bytes of this stage and its neighbour)
// instead of a per-block panel of the whole K range, which leaves room for
// 320-row tiles at any K.
// AF (with SR): the format of quantised A operands, 8 for MXFP8 (E4M3 codes,
// one byte per element) or 4 for MXFP4 (E2M1 codes, two per byte, element 2i
// in the low nibble); 0 for bf16 A.  With quantised A a stage spans 128 K
// elements: 128 bytes of E4M3 A per row (laid out like a bf16 stage of 64) or
// 64 bytes of E2M1 A (laid out like the B codes), 64 bytes of B codes per row
// (16-byte chunks XOR-swizzled by (row / 2) mod 4) and one 4-byte word of E8M0
// scales per row for each of A and B.  Two scaled MFMAs
// (v_mfma_scale_f32_32x32x64_f8f6f4) per fragment pair and stage.
template <int BM, int BN, int WM, int EPI, int NW, bool SR, int AF = 0, int NSF = 3>
__global__ __launch_bounds__(64 * NW, (NW == 4 && BM < 160) ? 2 : 1) void gemm_pipe_fp4(Params p) {
  static_assert(AF == 0 || AF == 8 || AF == 4, "A format: bf16, E4M3 or E2M1");
  constexpr bool A4 = AF == 4, AQ = AF != 0;
  static_assert(!AQ || SR, "quantised A needs the scale ring");
  static_assert(NSF >= 2 && NSF <= 6, "ring depth");
  constexpr int BKP = 64;              // bf16 elements of A per row and stage (128 bytes)
  constexpr int KST = AQ ? 128 : 64;   // K elements per stage
  constexpr int AROW = A4 ? 64 : 128;  // bytes of A per row and stage
  constexpr int QROW = KST / 2;        // E2M1 code bytes per B row and stage
  constexpr int NTH = 64 * NW;
  constexpr int WN = NW / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold 32x32 blocks");
  static_assert(EPI != EPI_SITU || FN % 2 == 0, "SiTU needs gate/up fragment pairs");
  constexpr int BN_OUT = (EPI == EPI_SITU) ? BN / 2 : BN;
  // A: 8 rows of 128 bytes (16 of 64) per instruction; B: 1 KB of codes per
  // instruction
  constexpr int A_RPI = 1024 / AROW, Q_RPI = 1024 / QROW;
  constexpr int NA = BM / A_RPI, NQ = BN / Q_RPI;
  static_assert(NA * A_RPI == BM && NQ * Q_RPI == BN, "tile rows per instruction");
  constexpr int MA = (NA + NW - 1) / NW, MQ = NQ / NW;
  static_assert(NA >= NW && NQ % NW == 0, "uniform load instructions per wave");
  // surplus A instructions repeat the wave's own instruction i-1
  auto a_ins = [](int w, int i) { const int x = w + NW * i; return x < NA ? x : x - NW; };
  // A scales: 64 rows per instruction, waves past them repeat a neighbour's
  constexpr int NSA = AQ ? (BM + 63) / 64 : 1;
  static_assert(!AQ || NSA <= NW, "one A scale instruction per wave");
  // scale ring: one 4-byte piece per B row and stage, 64 rows per instruction;
  // waves past the BN / 64 that are needed repeat a neighbour's instruction
  constexpr int NS = BN / 64;
  constexpr int MS = (SR ? 1 : 0) + (AQ ? 1 : 0);
  static_assert(!SR || (NS <= NW && NS * 64 == BN), "one scale instruction per wave");

  // NSF ring stages: A rows (bf16 or E4M3 codes), B codes, B scales, A scales
  __shared__ __attribute__((aligned(1024))) bf16_t sA[NSF][BM * AROW / 2];
  __shared__ __attribute__((aligned(1024))) uint8_t sQ[NSF][BN * QROW];
  __shared__ __attribute__((aligned(16))) uint8_t sS[NSF][SR ? BN * 4 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sT[NSF][AQ ? NSA * 256 : 16];
  // scale panel [BN][K/32], sized by the launch (not used with SR)
  extern __shared__ __attribute__((aligned(16))) uint8_t sP[];

  const int ntn = (p.N + BN_OUT - 1) / BN_OUT;
  Tile tile;
  if (!locate_tile<BM>(p, ntn, BN_OUT, tile)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const Seg& g = p.seg[0];  // one K segment (checked by the launcher)

  // tile row -> B row (gate/up groups of 32 for SiTU), clamped below N
  auto b_row_of = [&](int r, bool& up) {
    int row;
    if (EPI == EPI_SITU) {
      const int grp = r >> 5;
      up = grp & 1;
      row = tile.n0 + (grp >> 1) * 32 + (r & 31);
    } else {
      up = false;
      row = tile.n0 + r;
    }
    return static_cast<int64_t>(row < p.N ? row : p.N - 1);
  };

  // scale panel: 16-byte pieces of each B row's K/32 scale bytes
  const int sp = static_cast<int>(g.ldb >> 4);  // scale bytes per row (multiple of 16)
  if (!SR) {
    const uint8_t* S = g.Bs + static_cast<int64_t>(tile.expert) * p.bs_expert_stride;
    const uint8_t* S2 = g.Bs2 + static_cast<int64_t>(tile.expert) * p.bs_expert_stride;
    const int per_row = sp >> 4;
    const int total = BN * per_row;
    for (int f = tid; f < total; f += NTH) {
      const int r = f / per_row, c = f - (f / per_row) * per_row;
      bool up;
      const int64_t row = b_row_of(r, up);
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>((up ? S2 : S) + row * sp + c * 16);
      *reinterpret_cast<u32x4_t*>(sP + r * sp + c * 16) = v;
    }
  }

  int64_t a_off[MA];
  int a_chunk[MA];
#pragma unroll
  for (int i = 0; i < MA; ++i) {
    int r;
    if (A4) {  // 64-byte rows: four 16-byte chunks, swizzled by (row / 2) mod 4
      r = a_ins(wave, i) * 16 + (lane >> 2);
      a_chunk[i] = (lane & 3) ^ ((r >> 1) & 3);
    } else {
      r = a_ins(wave, i) * 8 + (lane >> 3);
      a_chunk[i] = (lane & 7) ^ (r & 7);
    }
    r = r < tile.rows ? r : 0;
    const int slot = tile.row0 + r;
    a_off[i] = p.a_rows ? p.a_rows[slot] : slot;
  }
  const uint8_t* pq[MQ];
  const bf16_t* pa[MA];
  const uint8_t* ps = nullptr;  // this lane's scale row (SR)
  const int s_ins = wave % NS;  // scale instruction of this wave (SR)
  const uint8_t* pt = nullptr;  // this lane's A scale row (quantised A)
  const int t_ins = wave % NSA;
  if (AQ) {
    int r = t_ins * 64 + lane;
    r = r < tile.rows ? r : 0;
    const int slot = tile.row0 + r;
    const int64_t row = p.a_rows ? p.a_rows[slot] : slot;
    pt = g.As + row * (g.K / 32);
  }
  {
    const bf16_t* A = static_cast<const bf16_t*>(g.A);
    const uint8_t* Q = static_cast<const uint8_t*>(g.B) + static_cast<int64_t>(tile.expert) * p.b_expert_stride;
    const uint8_t* Q2 = static_cast<const uint8_t*>(g.B2) + static_cast<int64_t>(tile.expert) * p.b_expert_stride;
#pragma unroll
    for (int i = 0; i < MA; ++i)
      pa[i] = AQ ? reinterpret_cast<const bf16_t*>(reinterpret_cast<const uint8_t*>(g.A) +
                                                   a_off[i] * g.lda + a_chunk[i] * 16)
                 : A + a_off[i] * g.lda + a_chunk[i] * 8;
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      bool up;
      if (AQ) {  // 64-byte rows: four 16-byte chunks, swizzled by (row / 2) mod 4
        const int r = (wave + NW * i) * 16 + (lane >> 2);
        const int chunk = (lane & 3) ^ ((r >> 1) & 3);
        const int64_t row = b_row_of(r, up);
        pq[i] = (up ? Q2 : Q) + row * g.ldb + chunk * 16;
      } else {
        const int r = (wave + NW * i) * 32 + (lane >> 1);
        const int half = (lane & 1) ^ ((r >> 2) & 1);
        const int64_t row = b_row_of(r, up);
        pq[i] = (up ? Q2 : Q) + row * g.ldb + half * 16;
      }
    }
    if (SR) {
      bool up;
      const int64_t row = b_row_of(s_ins * 64 + lane, up);
      ps = (up ? g.Bs2 : g.Bs) + static_cast<int64_t>(tile.expert) * p.bs_expert_stride + row * sp;
    }
  }
  const int ktot = g.K / KST;

  int issued = 0;  // stages issued so far
  // the scale word of a stage: bytes 2kt .. 2kt+1 inside the aligned word at
  // (2kt) & ~3 (64-element stages), or exactly bytes 4kt .. 4kt+3 (128)
  auto scale_word = [&]() { return AQ ? 4 * issued : (2 * issued) & ~3; };
  auto issue = [&](bf16_t* As, uint8_t* Qs, uint8_t* Ss, uint8_t* Ts) {
#pragma unroll
    for (int i = 0; i < MA; ++i) {
      // one instruction fills 1 KB: 8 rows of 128 bytes (bf16, E4M3) or 16
      // rows of 64 (E2M1)
      load_lds16_raw(pa[i], As + a_ins(wave, i) * 512);
      pa[i] += AROW / 2;
    }
    if (AQ) load_lds4_asm(pt + scale_word(), Ts + t_ins * 256);
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      load_lds16_raw(pq[i], Qs + (wave + NW * i) * 1024);
      pq[i] += QROW;
    }
    if (SR)  // scale bytes 2kt, 2kt+1 of stage kt sit in the aligned word at (2kt) & ~3
      load_lds4_asm(ps + scale_word(), Ss + s_ins * 256);
    ++issued;
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int kt, const bf16_t* As, const uint8_t* Qs, const uint8_t* Ss,
                     const uint8_t* Ts) {
    const int hi = lane >> 5, sw = lane & 7;
    if constexpr (AQ) {
      // lane (r, h): B codes of K [32h, 32h+32); E4M3 A codes of K
      // [16h, 16h+16) and [32+16h, 32+16h+16), or E2M1 A codes of K
      // [32h, 32h+32) like B; scale registers of block h on both sides
      typedef int v8i_t __attribute__((ext_vector_type(8)));
      typedef int v4i_t __attribute__((ext_vector_type(4)));
      const uint8_t* Ab = reinterpret_cast<const uint8_t*>(As);
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {  // the stage's two 64-element MFMA steps
        v8i_t bq[FN];
        int sb[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int rb = wn * WTN + j * 32 + (lane & 31);
          const v4i_t q = *reinterpret_cast<const v4i_t*>(
              Qs + rb * 64 + (((2 * q2 + hi) ^ ((rb >> 1) & 3)) * 16));
          // E2M1 B occupies the first four registers; the other four are not read
          bq[j] = __builtin_shufflevector(q, q, 0, 1, 2, 3, -1, -1, -1, -1);
          sb[j] = Ss[rb * 4 + 2 * q2 + hi];
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int ra = wm * WTM + i * 32 + (lane & 31);
          v8i_t aq;
          if constexpr (A4) {
            const v4i_t qa = *reinterpret_cast<const v4i_t*>(
                Ab + ra * 64 + (((2 * q2 + hi) ^ ((ra >> 1) & 3)) * 16));
            aq = __builtin_shufflevector(qa, qa, 0, 1, 2, 3, -1, -1, -1, -1);
          } else {
            const int s = ra & 7;
            const u32x4_t lo =
                *reinterpret_cast<const u32x4_t*>(Ab + ra * 128 + (((4 * q2 + hi) ^ s) * 16));
            const u32x4_t up =
                *reinterpret_cast<const u32x4_t*>(Ab + ra * 128 + (((4 * q2 + 2 + hi) ^ s) * 16));
            aq = v8i_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]),
                       static_cast<int>(lo[2]), static_cast<int>(lo[3]),
                       static_cast<int>(up[0]), static_cast<int>(up[1]),
                       static_cast<int>(up[2]), static_cast<int>(up[3])};
          }
          const int sa = Ts[ra * 4 + 2 * q2 + hi];
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                aq, bq[j], acc[i][j], A4 ? 4 : 0, 4, 0, sa, 0, sb[j]);
        }
      }
      return;
    }
    u32x4_t q[FN];
    float sc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int rb = wn * WTN + j * 32 + (lane & 31);
      q[j] = *reinterpret_cast<const u32x4_t*>(Qs + rb * 32 + ((hi ^ ((rb >> 2) & 1)) * 16));
      sc[j] = e8m0_to_f32(SR ? Ss[rb * 4 + (kt & 1) * 2 + hi] : sP[rb * sp + kt * 2 + hi]);
    }
#pragma unroll
    for (int kk = 0; kk < BKP / 16; ++kk) {
      const int ch = ((hi * 4 + kk) ^ sw) * 8;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * WTM + i * 32 + (lane & 31)) * BKP + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = decode8_hw(q[j][kk], sc[j]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // the panel's LDS writes complete before the first barrier of the ring
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  static_assert((NSF - 2) * (MA + MQ + MS) < 64, "loads in flight exceed the vmcnt range");
#pragma unroll
  for (int s = 0; s < NSF - 1; ++s)
    if (s < ktot) issue(sA[s], sQ[s], sS[s], sT[s]);
  // one ring step: wait for stage kt (the NSF - 2 issued after it may stay in
  // flight), refill the slot stage kt-1 used, multiply stage kt
  auto ring = [&](int kt, int c, int nx) {
    if (kt < ktot) {
      const int ahead = min(NSF - 2, ktot - 1 - kt);
      wait_stages<NSF - 2, MA + MQ + MS>(ahead);
      lds_barrier();
      if (kt + NSF - 1 < ktot) issue(sA[nx], sQ[nx], sS[nx], sT[nx]);
      compute(kt, sA[c], sQ[c], sS[c], sT[c]);
    }
  };
  for (int kt = 0; kt < ktot; kt += NSF) {
#pragma unroll
    for (int s = 0; s < NSF; ++s) ring(kt + s, s, (s + NSF - 1) % NSF);
  }

  // Staged output (grouped problems, Params::stage_out), as in gemm_pipe:
  // per pass one 32-row fragment of every row group of waves (of one group
  // when the A ring cannot hold them all), through the A ring, then whole
  // rows, 16 bytes per lane, non-temporal.  Bit-identical to the direct
  // stores below.
  constexpr int ST_ESZ = (EPI == EPI_SITU) ? 2 : 4;
  constexpr int ST_RB = BN_OUT * ST_ESZ, ST_RBP = ST_RB + 32;
  if constexpr ((EPI == EPI_F32 || EPI == EPI_SITU) && 32 * ST_RBP <= sizeof(sA) &&
                ST_RB % 16 == 0) {
    if (p.stage_out) {
      typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
      constexpr int GP = WM * 32 * ST_RBP <= sizeof(sA) ? WM : 1;  // row groups per pass
      constexpr int CPR = ST_RB / 16;  // 16-byte chunks per output row
      char* const sb = reinterpret_cast<char*>(&sA[0][0]);
      lds_barrier();  // every wave is done with the ring
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int h0 = 0; h0 < WM; h0 += GP) {
          if (h0 * WTM + i * 32 < tile.rows) {  // uniform: the pass holds valid rows
            if (wm >= h0 && wm < h0 + GP) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int lr = (wm - h0) * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if constexpr (EPI == EPI_SITU) {
#pragma unroll
                  for (int j = 0; j < FN; j += 2) {
                    const int oc = ((wn * FN + j) >> 1) * 32 + (lane & 31);
                    *reinterpret_cast<bf16_t*>(sb + lr * ST_RBP + oc * 2) =
                        f32_to_bf16(situ_glu(acc[i][j][r], acc[i][j + 1][r]));
                  }
                } else {
#pragma unroll
                  for (int j = 0; j < FN; ++j) {
                    const int oc = wn * WTN + j * 32 + (lane & 31);
                    *reinterpret_cast<float*>(sb + lr * ST_RBP + oc * 4) = acc[i][j][r];
                  }
                }
              }
            }
            lds_barrier();
#pragma unroll
            for (int c0 = 0; c0 < GP * 32 * CPR; c0 += NTH) {
              const int c = c0 + tid;
              const int lr = c / CPR, ch = c % CPR;
              const int row = (h0 + (lr >> 5)) * WTM + i * 32 + (lr & 31);
              const int col = tile.n0 + ch * (16 / ST_ESZ);
              if (c < GP * 32 * CPR && row < tile.rows && col < p.N) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sb + lr * ST_RBP + ch * 16);
                char* dst = static_cast<char*>(p.C) +
                            ((static_cast<int64_t>(tile.row0) + row) * p.ldc + col) * ST_ESZ;
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
              }
            }
            lds_barrier();
          }
        }
      }
      return;
    }
  }

#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (row >= tile.rows) continue;
      const int64_t orow = tile.row0 + row;
      if (EPI == EPI_SITU) {
#pragma unroll
        for (int j = 0; j < FN; j += 2) {
          const int grp = wn * FN + j;
          const int col = tile.n0 + (grp >> 1) * 32 + (lane & 31);
          if (col < p.N)
            store_bf16(p, orow * p.ldc + col, situ_glu(acc[i][j][r], acc[i][j + 1][r]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = tile.n0 + wn * WTN + j * 32 + (lane & 31);
          if (col >= p.N) continue;
          if (EPI == EPI_F32)
            static_cast<float*>(p.C)[orow * p.ldc + col] = acc[i][j][r];
          else
            static_cast<bf16_t*>(p.C)[orow * p.ldc + col] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (fp32 activations and weights): 64x64 tiles, 4x4 per thread,
// BK = 16, same tile scheduling, segments, gather and epilogues.
// ---------------------------------------------------------------------------
constexpr int FB = 64;
constexpr int FK = 16;

template <int EPI>
__global__ __launch_bounds__(NTHREADS) void gemm_f32(Params p) {
  constexpr int BN_OUT = (EPI == EPI_SITU) ? FB / 2 : FB;
  __shared__ float As[FK][FB + 4];
  __shared__ float Bs[FK][FB + 4];
  __shared__ float Ct[FB][FB + 4];
  const int ntn = (p.N + BN_OUT - 1) / BN_OUT;
  Tile tile;
  if (!locate_tile<FB>(p, ntn, BN_OUT, tile)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  // loader: each thread loads 4 elements of A and of B per K step
  const int lr = tid >> 2;          // 0..63 row within the tile
  const int lk = (tid & 3) * 4;     // 0,4,8,12
  const bool a_ok = lr < tile.rows;
  const int slot = tile.row0 + lr;
  const int arow = a_ok ? (p.a_rows ? p.a_rows[slot] : slot) : 0;
  int brow;
  bool bup;
  if (EPI == EPI_SITU) {
    bup = lr >= FB / 2;
    brow = tile.n0 + (lr % (FB / 2));
  } else {
    bup = false;
    brow = tile.n0 + lr;
  }
  const bool b_ok = brow < p.N;
  for (int s = 0; s < p.nseg; ++s) {
    const Seg& g = p.seg[s];
    const float* A = static_cast<const float*>(g.A);
    const float* B = static_cast<const float*>(bup ? g.B2 : g.B) +
                     static_cast<int64_t>(tile.expert) * p.b_expert_stride;
    for (int k0 = 0; k0 < g.K; k0 += FK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        As[lk + e][lr] = a_ok ? A[static_cast<int64_t>(arow) * g.lda + k0 + lk + e] : 0.f;
        Bs[lk + e][lr] = b_ok ? B[static_cast<int64_t>(brow) * g.ldb + k0 + lk + e] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < FK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Ct[ty * 4 + i][tx * 4 + j] = acc[i][j];
  __syncthreads();
  for (int idx = tid; idx < FB * BN_OUT; idx += NTHREADS) {
    const int r = idx / BN_OUT, c = idx % BN_OUT;
    const int col = tile.n0 + c;
    if (r >= tile.rows || col >= p.N) continue;
    float x = (EPI == EPI_SITU) ? situ_glu(Ct[r][c], Ct[r][c + FB / 2]) : Ct[r][c];
    if (EPI == EPI_SIGMOID) {
      if (p.col_add) x += p.col_add[col];
      x = 1.0f / (1.0f + expf(-x));
    }
    static_cast<float*>(p.C)[static_cast<int64_t>(tile.row0 + r) * p.ldc + col] = x;
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction: C = epilogue(sum over splits of the fp32 partials).  The
// partial columns follow the B-row order of a BN-wide tile; for SiTU-GLU the
// gate and up rows of an output column are 32 apart inside its 64-row group.
// ---------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ part, int kn, int M,
                                                      int N, int64_t nv, int bn, void* C, void* C2,
                                                      int64_t ldc, const float* col_add,
                                                      float* save_g, float* save_u) {
  const int64_t total = static_cast<int64_t>(M) * N;
  const int64_t plane = static_cast<int64_t>(M) * nv;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = i / N;
    const int c = static_cast<int>(i - row * N);
    const float* pr = part + row * nv;
    if (EPI == EPI_SITU) {
      const int half = bn / 2;
      const int64_t vg = static_cast<int64_t>(c / half) * bn + ((c % half) / 32) * 64 + (c % 32);
      float g = 0.f, u = 0.f;
      for (int q = 0; q < kn; ++q) {
        g += pr[q * plane + vg];
        u += pr[q * plane + vg + 32];
      }
      store_bf16(C, C2, row * ldc + c, situ_glu(g, u));
      if (save_g) {
        save_g[row * ldc + c] = g;
        save_u[row * ldc + c] = u;
      }
    } else {
      float x = 0.f;
      for (int q = 0; q < kn; ++q) x += pr[q * plane + c];
      if (EPI == EPI_SIGMOID) {
        if (col_add) x += col_add[c];
        static_cast<float*>(C)[row * ldc + c] = 1.0f / (1.0f + expf(-x));
      } else if (EPI == EPI_F32) {
        static_cast<float*>(C)[row * ldc + c] = x;
      } else {
        store_bf16(C, C2, row * ldc + c, x);
      }
    }
  }
}

// Tile shape and K split of a bf16 dense problem.  Row tiles follow M (32,
// 64, else 128 x 128); when the output tiles cannot fill the chip the K
// range is split so that about one wave of blocks runs, each split keeping
// at least 4 stages.
struct DensePlan {
  int cfg;  // 0: 32x256 BKP 64, 1: 64x256 BKP 64, 2: 128x128 BKP 32,
            // 3: 256x128 BKP 32, 4: 256x256 BKP 32
  int bm, bn, bkp;
  int ntn, mt;
  int ks;
  size_t bytes;
};

static int tiles_of(int M, int N, int bm, int bn, int epi) {
  const int bn_out = epi == EPI_SITU ? bn / 2 : bn;
  return ((M + bm - 1) / bm) * ((N + bn_out - 1) / bn_out);
}

static DensePlan plan_dense(int M, int N, int K, int epi) {
  DensePlan d{};
  int target;
  if (M <= 32) {
    d.cfg = 0; d.bm = 32; d.bn = 256; d.bkp = 64; target = 256;
  } else if (M <= 64) {
    d.cfg = 1; d.bm = 64; d.bn = 256; d.bkp = 64; target = 256;
  } else if (M >= 256 && epi != EPI_SIGMOID && tiles_of(M, N, 256, 256, epi) >= 256) {
    // large products: 128 x 64 per wave, 8 waves
    d.cfg = 4; d.bm = 256; d.bn = 256; d.bkp = 64; target = 256;
  } else if (M >= 1024 && epi == EPI_SIGMOID) {
    // the router (few columns, K = 3 d): 256 x 256 tiles, split along K
    // until they fill the chip
    d.cfg = 4; d.bm = 256; d.bn = 256; d.bkp = 64; target = 256;
  } else if (M >= 256 && tiles_of(M, N, 256, 128, epi) >= 256) {
    d.cfg = 3; d.bm = 256; d.bn = 128; d.bkp = 32; target = 512;
  } else {
    d.cfg = 2; d.bm = 128; d.bn = 128; d.bkp = 32; target = 512;
  }
  const int bn_out = epi == EPI_SITU ? d.bn / 2 : d.bn;
  d.ntn = (N + bn_out - 1) / bn_out;
  d.mt = (M + d.bm - 1) / d.bm;
  const int64_t tiles = static_cast<int64_t>(d.mt) * d.ntn;
  const int kall = K / d.bkp;
  d.ks = 1;
  if (tiles > 0 && tiles < target / 2 && kall >= 8) {
    int ks = static_cast<int>((target + tiles - 1) / tiles);
    ks = ks < kall / 4 ? ks : kall / 4;
    d.ks = ks > 1 ? ks : 1;
  }
  d.bytes = d.ks > 1 ? static_cast<size_t>(d.ks) * M * d.ntn * d.bn * sizeof(float) : 0;
  return d;
}

size_t splitk_bytes(int M, int N, int K, int epi) {
  if (M <= 0 || N <= 0) return 0;
  return plan_dense(M, N, K, epi).bytes;
}

template <int EPI>
static int run_reduce(const Params& p, const DensePlan& d, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(p.M) * p.N;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce<EPI>, dim3(static_cast<unsigned>(blocks < 8192 ? blocks : 8192)),
                     dim3(256), 0, stream, p.partial, d.ks, p.M, p.N,
                     static_cast<int64_t>(d.ntn) * d.bn, d.bn, p.C, p.C2, p.ldc, p.col_add,
                     p.save_g, p.save_u);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int EPI, int BFMT>
static int run_bf16(const Params& p, hipStream_t stream) {
  constexpr int BN_OUT = (EPI == EPI_SITU) ? BN / 2 : BN;
  const int ntn = (p.N + BN_OUT - 1) / BN_OUT;
  const int mt = p.tiles ? p.max_mtiles : (p.M + BM - 1) / BM;
  const int64_t G = static_cast<int64_t>(mt) * ntn;
  if (G <= 0) return MOE_OK;
  const int64_t G8 = (G + 7) / 8 * 8;
  const size_t ab = static_cast<size_t>(2) * (BM + BN) * LDK * sizeof(bf16_t);
  const size_t ct = static_cast<size_t>(BM) * (BN + 4) * sizeof(float);
  const size_t smem = ab > ct ? ab : ct;
  static bool configured = false;
  if (!configured) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16<BM, BN, WM, EPI, BFMT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(smem)) != hipSuccess)
      return MOE_EHIP;
    configured = true;
  }
  hipLaunchKernelGGL((gemm_bf16<BM, BN, WM, EPI, BFMT>), dim3(static_cast<unsigned>(G8)),
                     dim3(NTHREADS), smem, stream, p);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Whether a grouped launch may write its output rows 16 bytes per lane
// (Params::stage_out): fp32 or SiTU-GLU outputs without residue or
// pre-activation stores, whole 16-byte chunks per row, aligned rows.
static int row_stores_ok(const Params& q, int epi) {
  return (epi == EPI_F32 || epi == EPI_SITU) && !q.C2 && !q.save_g && q.N % 8 == 0 &&
         q.ldc % 8 == 0 && reinterpret_cast<uintptr_t>(q.C) % 16 == 0;
}

template <int BM, int BN, int WM, int EPI, int BKP, int NST, bool BNT, int NW = 4, bool BKN = false>
static int run_pipe(const Params& p, hipStream_t stream, size_t pad_lds = 0) {
  constexpr int BN_OUT = (EPI == EPI_SITU) ? BN / 2 : BN;
  for (int s = 0; s < p.nseg; ++s)
    if (p.seg[s].K % BKP != 0) return MOE_EUNSUPPORTED;
  const int ntn = (p.N + BN_OUT - 1) / BN_OUT;
  const int mt = p.tiles ? p.max_mtiles : (p.M + BM - 1) / BM;
  const int64_t G = static_cast<int64_t>(mt) * ntn * (p.ksplit > 1 ? p.ksplit : 1) *
                    (p.kgroups > 0 ? p.kgroups : 1);
  if (G <= 0) return MOE_OK;
  const int64_t G8 = (G + 7) / 8 * 8;
  if (pad_lds > 0) {  // unused dynamic LDS that caps the blocks per CU
    static std::atomic<bool> configured{false};
    if (!configured.load(std::memory_order_relaxed)) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_pipe<BM, BN, WM, EPI, BKP, NST, BNT, NW, BKN>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(pad_lds)) != hipSuccess)
        return MOE_EHIP;
      configured.store(true, std::memory_order_relaxed);
    }
  }
  hipLaunchKernelGGL((gemm_pipe<BM, BN, WM, EPI, BKP, NST, BNT, NW, BKN>), dim3(static_cast<unsigned>(G8)),
                     dim3(64 * NW), pad_lds, stream, p);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Ring depth: 3 stages (a fourth measured no faster on the weight-streaming
// 32-row tiles once the loads stay in flight across the LDS reads); the
// 8-wave tiles take two 64-element stages (half the barriers per K of three
// 32-element ones, 2 - 5% faster), their second wave per SIMD covering the
// shorter prefetch.
template <int BM, int BN, int BKP, int NW>
constexpr int pipe_stages() {
  return (NW == 8 && BKP == 64) ? 2 : 3;
}

// BNT: B rows are read by exactly one block (grouped problems with one row
// tile per expert), so they are streamed with the non-temporal policy.
// NW: waves per block; 8 (two per SIMD) for the 256- and 320-row MFMA-bound
// tiles, so one wave's MFMAs cover the other's LDS and barrier waits.
template <int BM, int BN, int WM, int BKP, bool BNT = false, int NW = 4>
static int dispatch_pipe(const Params& p, int epi, hipStream_t s) {
  constexpr int NST = pipe_stages<BM, BN, BKP, NW>();
  switch (epi) {
    case EPI_BF16: return run_pipe<BM, BN, WM, EPI_BF16, BKP, NST, BNT, NW>(p, s);
    case EPI_F32: return run_pipe<BM, BN, WM, EPI_F32, BKP, NST, BNT, NW>(p, s);
    case EPI_SIGMOID: return run_pipe<BM, BN, WM, EPI_SIGMOID, BKP, NST, BNT, NW>(p, s);
    case EPI_SITU: return run_pipe<BM, BN, WM, EPI_SITU, BKP, NST, BNT, NW>(p, s);
    default: return MOE_EUNSUPPORTED;
  }
}

// Static LDS of the MXFP4 kernel (an upper bound: 1 KB is left for the
// placement of the small arrays), and the LDS a block may use in all (two
// blocks per CU up to 128-row tiles, one block per CU for taller tiles).
template <int BM, int BN>
constexpr size_t fp4_static_lds() {
  return static_cast<size_t>(3) * (BM * 64 * 2 + BN * 32) + 1024;
}
template <int BM>
constexpr size_t fp4_lds_budget() {
  return BM >= 160 ? 160 * 1024 : 80 * 1024;
}

size_t fp4_tall_tile_fits(int K) {
  return K % 512 == 0 && fp4_static_lds<160, 256>() + static_cast<size_t>(256) * (K / 32) <=
                             fp4_lds_budget<160>();
}

bool fp4_tile320_fits(int K) { return K > 0 && K % 128 == 0; }

// Returns 1 when the shape does not fit the pipelined MXFP4 kernel (the caller
// then uses the register-staged kernel).  SR: scales through the ring (K a
// multiple of 128, so that every stage's scale word lies inside its row).
template <int BM, int BN, int WM, int EPI, int NW = 4, bool SR = false, int AF = 0>
static int run_pipe_fp4(const Params& p, hipStream_t stream) {
  // W4A8: two 128-element stages (117 KB); W4A4: three 128-element stages
  // (114 KB); bf16-A: three 64-element stages
  constexpr int NSF = AF == 8 ? 2 : 3;
  constexpr int BN_OUT = (EPI == EPI_SITU) ? BN / 2 : BN;
  if (p.nseg != 1 || p.seg[0].K % (SR ? 128 : 512) != 0) return 1;
  const Seg& g = p.seg[0];
  const uintptr_t align = reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B) |
                          reinterpret_cast<uintptr_t>(g.B2) | reinterpret_cast<uintptr_t>(g.Bs) |
                          reinterpret_cast<uintptr_t>(g.Bs2) | reinterpret_cast<uintptr_t>(g.As) |
                          static_cast<uintptr_t>(g.lda * (AF ? 1 : 2)) |
                          static_cast<uintptr_t>(p.b_expert_stride) |
                          static_cast<uintptr_t>(p.bs_expert_stride);
  if (align % 16 != 0) return 1;
  const size_t panel = SR ? 0 : static_cast<size_t>(BN) * (p.seg[0].K / 32);
  if (fp4_static_lds<BM, BN>() + panel > fp4_lds_budget<BM>()) return 1;
  const int ntn = (p.N + BN_OUT - 1) / BN_OUT;
  const int mt = p.tiles ? p.max_mtiles : (p.M + BM - 1) / BM;
  const int64_t G = static_cast<int64_t>(mt) * ntn;
  if (G <= 0) return MOE_OK;
  const int64_t G8 = (G + 7) / 8 * 8;
  static bool configured = false;
  if (!SR && !configured) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_pipe_fp4<BM, BN, WM, EPI, NW, SR, AF, NSF>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(fp4_lds_budget<BM>() - fp4_static_lds<BM, BN>())) !=
        hipSuccess)
      return MOE_EHIP;
    configured = true;
  }
  // staged row stores for grouped launches; the W4A8 down-projection keeps
  // the direct stores (staged, it measured 2.44 -> 2.50 ms at T = 16384,
  // while every other grouped MXFP4 launch gained 1 - 5%)
  Params q = p;
  q.stage_out = p.tiles && !(AF == 8 && EPI == EPI_F32) ? row_stores_ok(p, EPI) : 0;
  hipLaunchKernelGGL((gemm_pipe_fp4<BM, BN, WM, EPI, NW, SR, AF, NSF>), dim3(static_cast<unsigned>(G8)),
                     dim3(64 * NW), panel, stream, q);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <int EPI>
static int run_f32(const Params& p, hipStream_t stream) {
  constexpr int BN_OUT = (EPI == EPI_SITU) ? FB / 2 : FB;
  const int ntn = (p.N + BN_OUT - 1) / BN_OUT;
  const int mt = p.tiles ? p.max_mtiles : (p.M + FB - 1) / FB;
  const int64_t G = static_cast<int64_t>(mt) * ntn;
  if (G <= 0) return MOE_OK;
  const int64_t G8 = (G + 7) / 8 * 8;
  hipLaunchKernelGGL(gemm_f32<EPI>, dim3(static_cast<unsigned>(G8)), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <int BM, int BN, int WM, int BFMT>
static int dispatch_epi(const Params& p, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_BF16: return run_bf16<BM, BN, WM, EPI_BF16, BFMT>(p, s);
    case EPI_F32: return run_bf16<BM, BN, WM, EPI_F32, BFMT>(p, s);
    case EPI_SIGMOID: return run_bf16<BM, BN, WM, EPI_SIGMOID, BFMT>(p, s);
    case EPI_SITU: return run_bf16<BM, BN, WM, EPI_SITU, BFMT>(p, s);
    default: return MOE_EUNSUPPORTED;
  }
}

int launch(const Params& p, int epi, int bfmt, bool act_bf16, int bm_hint, hipStream_t stream) {
  // low parts are written by the dense bf16 kernels and their split-K reduction
  if (p.C2 && !(act_bf16 && bfmt == B_DENSE && !p.tiles && (epi == EPI_BF16 || epi == EPI_SITU)))
    return MOE_EUNSUPPORTED;
  // pre-activations are stored by the pipelined bf16 kernels and their split-K reduction
  if ((p.save_g != nullptr) != (p.save_u != nullptr) ||
      (p.save_g && !(act_bf16 && bfmt == B_DENSE && epi == EPI_SITU)))
    return MOE_EUNSUPPORTED;
  if (!act_bf16) {
    if (bfmt != B_DENSE) return MOE_EUNSUPPORTED;
    switch (epi) {
      case EPI_F32: return run_f32<EPI_F32>(p, stream);
      case EPI_SIGMOID: return run_f32<EPI_SIGMOID>(p, stream);
      case EPI_SITU: return run_f32<EPI_SITU>(p, stream);
      default: return MOE_EUNSUPPORTED;
    }
  }
  for (int s = 0; s < p.nseg; ++s)
    if (p.seg[s].K % BK != 0) return MOE_EUNSUPPORTED;
  if (p.kgroups > 0) {
    // K-grouped weight gradients: fp32 outputs, one segment, no gather or
    // split; 256 x 256 tiles on 8 waves
    if (bfmt != B_DENSE || (epi != EPI_F32 && epi != EPI_SGD) || p.nseg != 1 || p.tiles ||
        p.a_rows || !p.kofs || p.C2)
      return MOE_EUNSUPPORTED;
    // the in-place update writes 8 bf16 weights per 16-byte access
    if (epi == EPI_SGD && (p.N % 8 != 0 || p.ldc % 8 != 0 || p.c_group_stride % 8 != 0 ||
                           reinterpret_cast<uintptr_t>(p.C) % 16 != 0))
      return MOE_EUNSUPPORTED;
    Params q = p;
    q.ksplit = 1;
    q.stage_out = epi == EPI_F32 && q.c_group_stride % 8 == 0 ? row_stores_ok(q, epi) : 0;
    if (epi == EPI_SGD) return run_pipe<256, 256, 2, EPI_SGD, 64, 2, false, 8>(q, stream);
    return dispatch_pipe<256, 256, 2, 64, false, 8>(q, epi, stream);
  }
  if (bfmt == B_DENSE_KN) {
    // grouped problems whose B is stored [K][N] (the experts' weights read
    // transposed), fp32 outputs; the tiles of the B_DENSE grouped problems
    if (!p.tiles || epi != EPI_F32 || p.C2 || p.N % 8 != 0 || p.b_expert_stride % 8 != 0)
      return MOE_EUNSUPPORTED;
    for (int s = 0; s < p.nseg; ++s)
      if (p.seg[s].ldb % 8 != 0 || reinterpret_cast<uintptr_t>(p.seg[s].B) % 16 != 0 ||
          p.seg[s].B2)
        return MOE_EUNSUPPORTED;
    Params q = p;
    q.ksplit = 1;
    q.stage_out = row_stores_ok(q, epi);
    if (bm_hint <= 32) return run_pipe<32, 256, 1, EPI_F32, 64, 3, true, 4, true>(q, stream);
    if (bm_hint <= 96) return run_pipe<96, 256, 1, EPI_F32, 64, 3, true, 4, true>(q, stream);
    if (bm_hint == 160) return run_pipe<160, 256, 1, EPI_F32, 64, 3, false, 4, true>(q, stream);
    if (bm_hint == 320) return run_pipe<320, 256, 2, EPI_F32, 64, 2, true, 8, true>(q, stream);
    if (bm_hint == 256) return run_pipe<256, 256, 2, EPI_F32, 64, 2, false, 8, true>(q, stream);
    return run_pipe<128, 128, 2, EPI_F32, 32, 3, false, 4, true>(q, stream);
  }
  if (bfmt == B_DENSE && p.tiles) {
    // grouped problems stream expert weights: tiles as tall as the expected
    // rows per expert and 256 columns wide (fewer re-reads of the gathered
    // rows per weight byte)
    Params q = p;
    q.ksplit = 1;
    q.stage_out = row_stores_ok(q, epi);
    // about one row tile per expert: each weight byte is read once
    if (bm_hint <= 32) return dispatch_pipe<32, 256, 1, 64, true>(q, epi, stream);
    if (bm_hint <= 96)  // 128-byte row pieces per stage, one block per CU
      return dispatch_pipe<96, 256, 1, 64, true>(q, epi, stream);
    // tall experts (MFMA-bound): 160 x 64, 160 x 64 (8 waves) or 128 x 64
    // (8 waves) per wave; up to 320 rows an expert is one row tile, so its
    // weights stream with the non-temporal policy
    if (bm_hint == 160) return dispatch_pipe<160, 256, 1, 64>(q, epi, stream);
    if (bm_hint == 320) return dispatch_pipe<320, 256, 2, 64, true, 8>(q, epi, stream);
    if (bm_hint == 256) return dispatch_pipe<256, 256, 2, 64, false, 8>(q, epi, stream);
    return dispatch_pipe<128, 128, 2, 32>(q, epi, stream);
  }
  if (bfmt == B_DENSE) {
    int K = 0;
    for (int s = 0; s < p.nseg; ++s) K += p.seg[s].K;
    const DensePlan d = plan_dense(p.M, p.N, K, epi);
    Params q = p;
    q.ksplit = 1;
    if (d.ks > 1 && p.partial && p.partial_bytes >= d.bytes) q.ksplit = d.ks;
    int rc;
    if (d.cfg == 0)
      rc = dispatch_pipe<32, 256, 1, 64>(q, epi, stream);
    else if (d.cfg == 1)
      rc = dispatch_pipe<64, 256, 1, 64>(q, epi, stream);
    else if (d.cfg == 4)
      rc = dispatch_pipe<256, 256, 2, 64, false, 8>(q, epi, stream);
    else if (d.cfg == 3)
      rc = dispatch_pipe<256, 128, 2, 32>(q, epi, stream);
    else
      rc = dispatch_pipe<128, 128, 2, 32>(q, epi, stream);
    if (rc != MOE_OK || q.ksplit == 1) return rc;
    switch (epi) {
      case EPI_BF16: return run_reduce<EPI_BF16>(q, d, stream);
      case EPI_F32: return run_reduce<EPI_F32>(q, d, stream);
      case EPI_SIGMOID: return run_reduce<EPI_SIGMOID>(q, d, stream);
      case EPI_SITU: return run_reduce<EPI_SITU>(q, d, stream);
      default: return MOE_EUNSUPPORTED;
    }
  }
  if (bfmt == B_MXFP4_A8 || bfmt == B_MXFP4_A4) {
    // W4A8 / W4A4: 320-row tiles on 8 waves, E4M3 or E2M1 A and E2M1 B
    // multiplied by the scaled MFMA; no other tile height takes these operands
    if (bm_hint != 320) return MOE_EUNSUPPORTED;
    int rcq = 1;
    if (bfmt == B_MXFP4_A8) {
      if (epi == EPI_SITU)
        rcq = run_pipe_fp4<320, 256, 2, EPI_SITU, 8, true, 8>(p, stream);
      else if (epi == EPI_F32)
        rcq = run_pipe_fp4<320, 256, 2, EPI_F32, 8, true, 8>(p, stream);
    } else {
      if (epi == EPI_SITU)
        rcq = run_pipe_fp4<320, 256, 2, EPI_SITU, 8, true, 4>(p, stream);
      else if (epi == EPI_F32)
        rcq = run_pipe_fp4<320, 256, 2, EPI_F32, 8, true, 4>(p, stream);
    }
    return rcq == 1 ? MOE_EUNSUPPORTED : rcq;
  }
  // MXFP4 routed experts: codes straight to LDS, scales in a per-block panel,
  // decoded per fragment; shapes outside that kernel's limits use the
  // register-staged kernel that decodes while writing LDS
  int rc = 1;
  if (bm_hint == 320) {
    // 320-row tiles, 8 waves, scales through the ring
    if (epi == EPI_SITU)
      rc = run_pipe_fp4<320, 256, 2, EPI_SITU, 8, true>(p, stream);
    else if (epi == EPI_BF16)
      rc = run_pipe_fp4<320, 256, 2, EPI_BF16, 8, true>(p, stream);
    else if (epi == EPI_F32)
      rc = run_pipe_fp4<320, 256, 2, EPI_F32, 8, true>(p, stream);
    return rc == 1 ? MOE_EUNSUPPORTED : rc;
  }
  if (bm_hint == 160) {
    // tiles were cut 160 rows tall: only the pipelined kernel takes them
    if (epi == EPI_SITU)
      rc = run_pipe_fp4<160, 256, 1, EPI_SITU>(p, stream);
    else if (epi == EPI_BF16)
      rc = run_pipe_fp4<160, 256, 1, EPI_BF16>(p, stream);
    else if (epi == EPI_F32)
      rc = run_pipe_fp4<160, 256, 1, EPI_F32>(p, stream);
    return rc == 1 ? MOE_EUNSUPPORTED : rc;
  }
  if (epi == EPI_SITU)
    rc = bm_hint <= 32 ? run_pipe_fp4<32, 256, 1, EPI_SITU>(p, stream)
                       : run_pipe_fp4<128, 128, 2, EPI_SITU>(p, stream);
  else if (epi == EPI_BF16)
    rc = bm_hint <= 32 ? run_pipe_fp4<32, 256, 1, EPI_BF16>(p, stream)
                       : run_pipe_fp4<128, 128, 2, EPI_BF16>(p, stream);
  else if (epi == EPI_F32)
    rc = bm_hint <= 32 ? run_pipe_fp4<32, 256, 1, EPI_F32>(p, stream)
                       : run_pipe_fp4<128, 128, 2, EPI_F32>(p, stream);
  if (rc != 1) return rc;
  if (bm_hint <= 32) return dispatch_epi<32, 256, 1, B_MXFP4>(p, epi, stream);
  return dispatch_epi<128, 128, 2, B_MXFP4>(p, epi, stream);
}

}  // namespace gemm
}  // namespace moe

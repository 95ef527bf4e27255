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
// bf16 kernel: 256 threads as a WM x WN grid of waves, v_mfma_f32_32x32x16_bf16
// on 32x32 blocks, BK = 64, double-buffered LDS with rows padded by 16 bytes
// (conflict-free 16-byte fragment reads), global loads for tile k+1 issued
// before the MFMAs of tile k.  MXFP4 B tiles are decoded to bf16 (exact:
// E2M1 value with the E8M0 exponent added) when they are written to LDS.
// The epilogue goes through LDS so that stores are row-contiguous.
#include "gemm.hpp"

namespace moe {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)
constexpr int NTHREADS = 256;

struct Tile {
  int expert, row0, rows, n0;
};

// Block -> tile, with consecutive tiles kept on one XCD (blocks are dealt to
// the 8 XCDs round robin), M-tile-major so one XCD's L2 reuses the A rows.
template <int BM>
__device__ __forceinline__ bool locate_tile(const Params& p, int ntn, int bn_out, Tile& t) {
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int tau = (b & 7) * (G >> 3) + (b >> 3);
  const int mt = tau / ntn, nt = tau - (tau / ntn) * ntn;
  if (p.tiles) {
    if (mt >= *p.ntiles) return false;
    const int32_t* q = p.tiles + 4 * mt;
    t.expert = q[0];
    t.row0 = q[1];
    t.rows = q[2];
  } else {
    t.expert = 0;
    t.row0 = mt * BM;
    if (t.row0 >= p.M) return false;
    t.rows = min(BM, p.M - t.row0);
  }
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

// 8 MXFP4 codes (one 32-bit word, element 0 in the low nibble) -> 8 bf16.
__device__ __forceinline__ u32x4_t decode8(uint32_t q, int32_t exp_add) {
  u32x4_t out;
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
        const int32_t ea = (rsc[i] - 127) << 7;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<u32x4_t*>(b_s + r * LDK + half * 32 + w * 8) = decode8(rb[i][w], ea);
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
    case EPI_SIGMOID: return run_bf16<BM, BN, WM, EPI_SIGMOID, BFMT>(p, s);
    case EPI_SITU: return run_bf16<BM, BN, WM, EPI_SITU, BFMT>(p, s);
    default: return MOE_EUNSUPPORTED;
  }
}

int launch(const Params& p, int epi, int bfmt, bool act_bf16, int bm_hint, hipStream_t stream) {
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
  if (bm_hint <= 32) {
    return bfmt == B_DENSE ? dispatch_epi<32, 256, 1, B_DENSE>(p, epi, stream)
                           : dispatch_epi<32, 256, 1, B_MXFP4>(p, epi, stream);
  }
  return bfmt == B_DENSE ? dispatch_epi<128, 128, 2, B_DENSE>(p, epi, stream)
                         : dispatch_epi<128, 128, 2, B_MXFP4>(p, epi, stream);
}

}  // namespace gemm
}  // namespace moe

// Forward pass of the Stable LatentMoE layer: router -> QB routing ->
// token permutation -> latent down-projection and shared gate/up ->
// routed gate/up with SiTU-GLU -> routed down -> weighted combine + RMSNorm
// -> up-projection fused with the shared down-projection.
//
// Sources: "Kimi K3 — LatentMoE" (dimsnsums.com), section "Why does the
// router need three moves?" (latent space of half the width, RMSNorm on the
// combined routed signal, SiTU-GLU); xhh.club "Kimi K3 模型结构（5）：宽度维度，
// Stable LatentMoE", Q&A on routing, SiTU-GLU, RMSNorm placement (after the
// latent aggregation, before the up-projection) and the shared expert (two
// experts merged into one MLP of width 6144 at full width, added to the
// routed output).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "gemm.hpp"
#include "layer_kernels.hpp"
#include "prof.hpp"
#include "route.hpp"

namespace moe {


namespace layer {

// Exact split of an fp32 matrix into three bf16 matrices, w = hi + mid + lo
// (each step rounds to nearest even and carries the exact fp32 remainder).
__global__ void split3(const float* __restrict__ w, bf16_t* hi, bf16_t* mid, bf16_t* lo,
                       int64_t count) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float v = w[i];
    const bf16_t h = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h);
    const bf16_t m = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(m);
    hi[i] = h;
    mid[i] = m;
    lo[i] = f32_to_bf16(r2);
  }
}

__global__ void copy_f32(const float* __restrict__ in, float* __restrict__ out, int64_t count) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    out[i] = in[i];
}

__global__ void fill_u32(uint32_t* p, uint32_t v, int64_t count) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// offs = exclusive scan of loads; grouped tile list for tile height bm.
__global__ __launch_bounds__(1024) void scan_and_tiles(const int32_t* loads, int n, int bm,
                                                       int32_t* offs, int32_t* tiles,
                                                       int32_t* ntiles) {
  __shared__ int32_t s_l[1024], s_t[1024];
  const int e = threadIdx.x;
  const int32_t L = e < n ? loads[e] : 0;
  const int32_t nt = (L + bm - 1) / bm;
  s_l[e] = L;
  s_t[e] = nt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t a = e >= off ? s_l[e - off] : 0;
    const int32_t b = e >= off ? s_t[e - off] : 0;
    __syncthreads();
    s_l[e] += a;
    s_t[e] += b;
    __syncthreads();
  }
  const int32_t lo = s_l[e] - L, to = s_t[e] - nt;
  if (e < n) {
    offs[e] = lo;
    for (int i = 0; i < nt; ++i) {
      int32_t* q = tiles + 4 * (to + i);
      q[0] = e;
      q[1] = lo + i * bm;
      q[2] = min(bm, L - i * bm);
      q[3] = 0;
    }
  }
  if (e == n - 1) {
    offs[n] = s_l[e];
    *ntiles = s_t[e];
  }
}

// sel[e][t] = j + 1 when token t chose expert e as its j-th expert.
__global__ void scatter_sel(const int32_t* idx, int T, int k, uint8_t* sel) {
  const int64_t total = static_cast<int64_t>(T) * k;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = i / k;
    const int j = static_cast<int>(i - t * k);
    sel[static_cast<int64_t>(idx[i]) * T + t] = static_cast<uint8_t>(j + 1);
  }
}

// One block per expert: the tokens that chose e, in increasing token order,
// take the slots offs[e], offs[e]+1, ...: perm[slot] = token, inv[t][j] = slot.
__global__ __launch_bounds__(256) void expert_slots(const uint8_t* sel, int T, int k,
                                                    const int32_t* offs, int32_t* perm,
                                                    int32_t* inv) {
  __shared__ int32_t s_wave[4];
  __shared__ int32_t s_base;
  const int e = blockIdx.x;
  const uint8_t* row = sel + static_cast<int64_t>(e) * T;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_base = offs[e];
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += 256) {
    const int t = t0 + threadIdx.x;
    const int j = t < T ? row[t] : 0;
    const uint64_t bal = __ballot(j != 0);
    const int before = __popcll(bal & ((uint64_t(1) << lane) - 1));
    if (lane == 0) s_wave[wv] = __popcll(bal);
    __syncthreads();
    int wbase = s_base;
    for (int w = 0; w < wv; ++w) wbase += s_wave[w];
    if (j != 0) {
      const int slot = wbase + before;
      perm[slot] = t;
      inv[static_cast<int64_t>(t) * k + (j - 1)] = slot;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_base += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
  }
}

// One element v / 2^X -> E4M3 code: nearest value, ties to the even mantissa,
// saturating at 448; the sign bit is q's.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const float a = fabsf(q);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a >= 0.015625f) {  // normal E4M3: 3 mantissa bits, round half to even
    const uint32_t bits = __float_as_uint(a);
    uint32_t keep = (bits >> 20) & 7u, field = ((bits >> 23) & 255u) - 127u + 7u;
    const uint32_t rem = bits & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) {
      keep = 0u;
      ++field;
    }
    code = (field << 3) | keep;
  } else {  // subnormal: multiples of 2^-9 (8 * 2^-9 is the smallest normal, code 8)
    code = static_cast<uint32_t>(rintf(a * 512.f));
  }
  return code | ((__float_as_uint(q) >> 31) << 7);
}

// bf16 rows -> MXFP8 (OCP Microscaling: E4M3 elements, one E8M0 scale per 32
// consecutive elements of a row).  Per block: shared exponent
// X = floor(log2 amax) - 8 (8 = E4M3's largest exponent), stored as X + 127
// clamped to [0, 254] (0 for an all-zero block); elements v / 2^X rounded to
// the nearest E4M3 value, ties to the even mantissa, saturating at 448.
// Each lane takes 8 consecutive elements (one 16-byte load, one 8-byte store),
// four lanes a block; blocks are consecutive in the row-major input.
__global__ __launch_bounds__(256) void mx8_quantize(const bf16_t* __restrict__ in, int64_t nblk,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales) {
  const int64_t tot = nblk * 4;  // 8-element pieces
  const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
  // the stride is a multiple of 4, so the four lanes of a block stay together
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < tot; g += step) {
    const uint4 raw = reinterpret_cast<const uint4*>(in)[g];
    float v[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
    int sb = 0;
    if (amax > 0.f) {
      const uint32_t ab = __float_as_uint(amax);
      const int e = static_cast<int>((ab >> 23) & 255u);
      const int fl = e ? e - 127 : (31 - __clz(ab & 0x7fffffu)) - 149;  // floor(log2 amax)
      sb = min(max(fl - 8 + 127, 0), 254);
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_code(ldexpf(v[i], 127 - sb)) << (8 * i);      // exact power-of-two scaling
      hi |= e4m3_code(ldexpf(v[4 + i], 127 - sb)) << (8 * i);
    }
    reinterpret_cast<uint2*>(codes)[g] = make_uint2(lo, hi);
    if ((g & 3) == 0) scales[g >> 2] = static_cast<uint8_t>(sb);
  }
}

// One element q = v / 2^X -> E2M1 code: the nearest of 0, .5, 1, 1.5, 2, 3,
// 4, 6, ties to the even code (the one with a zero mantissa bit), magnitudes
// above 6 saturating to 6; bit 3 carries q's sign.  The comparisons are exact:
// q is a bf16 value scaled by a power of two.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const float a = fabsf(q);
  uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
             : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return c | ((__float_as_uint(q) >> 31) << 3);
}

// bf16 rows -> MXFP4 (OCP Microscaling: E2M1 elements, two per byte with
// element 2i in the low nibble, one E8M0 scale per 32 consecutive elements of
// a row).  Per block: X = floor(log2 amax) - 2 (2 = E2M1's largest exponent),
// stored as X + 127 clamped to [0, 254] (0 for an all-zero block).  Each lane
// takes 8 consecutive elements (one 16-byte load, one 4-byte store), four
// lanes a block.
__global__ __launch_bounds__(256) void mx4_quantize(const bf16_t* __restrict__ in, int64_t nblk,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales) {
  const int64_t tot = nblk * 4;  // 8-element pieces
  const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
  // the stride is a multiple of 4, so the four lanes of a block stay together
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < tot; g += step) {
    const uint4 raw = reinterpret_cast<const uint4*>(in)[g];
    float v[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
    int sb = 0;
    if (amax > 0.f) {
      const uint32_t ab = __float_as_uint(amax);
      const int e = static_cast<int>((ab >> 23) & 255u);
      const int fl = e ? e - 127 : (31 - __clz(ab & 0x7fffffu)) - 149;  // floor(log2 amax)
      sb = min(max(fl - 2 + 127, 0), 254);
    }
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= e2m1_code(ldexpf(v[i], 127 - sb)) << (4 * i);
    reinterpret_cast<uint32_t*>(codes)[g] = word;
    if ((g & 3) == 0) scales[g >> 2] = static_cast<uint8_t>(sb);
  }
}

// y_t = sum_j w[t][j] * yp[inv[t][j]] in fp32 (j ascending), then
// RMSNorm: y * rsqrt(mean(y^2) + eps) * gamma.  One block per token; each
// lane owns groups of 4 consecutive columns (16-byte loads of the slot rows,
// which are read once: non-temporal).  With bf16 output, out_lo (when given)
// receives bf16(v - bf16(v)), so that the up-projection can take the
// normalised row to about 16 bits.  L is a multiple of 4 and at most 4096.
template <typename ACT>
__global__ __launch_bounds__(256) void combine_rmsnorm(const float* __restrict__ yp,
                                                       const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w,
                                                       const float* __restrict__ gamma, int k,
                                                       int L, float eps, ACT* __restrict__ out,
                                                       bf16_t* __restrict__ out_lo) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int MAXG = 4;  // column groups of 4 per lane: L <= 256 * 4 * MAXG
  __shared__ float s_red[256];
  const int t = blockIdx.x;
  const int L4 = L >> 2;
  f32x4_t acc[MAXG];
#pragma unroll
  for (int i = 0; i < MAXG; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // four slot rows per round trip: their loads are all in flight together
  constexpr int RB = 4;
  for (int j0 = 0; j0 < k; j0 += RB) {
    f32x4_t v[RB][MAXG];
    float wj[RB];
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int j = j0 + q;
      wj[q] = j < k ? w[static_cast<int64_t>(t) * k + j] : 0.f;
      const f32x4_t* src =
          j < k ? reinterpret_cast<const f32x4_t*>(
                      yp + static_cast<int64_t>(inv[static_cast<int64_t>(t) * k + j]) * L)
                : nullptr;
#pragma unroll
      for (int i = 0; i < MAXG; ++i) {
        const int c4 = threadIdx.x + 256 * i;
        v[q][i] = (src && c4 < L4) ? __builtin_nontemporal_load(src + c4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < RB; ++q)
#pragma unroll
      for (int i = 0; i < MAXG; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wj[q], v[q][i][e], acc[i][e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXG; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(acc[i][e], acc[i][e], ss);
  s_red[threadIdx.x] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) s_red[threadIdx.x] += s_red[threadIdx.x + s];
    __syncthreads();
  }
  const float scale = rsqrtf(s_red[0] / static_cast<float>(L) + eps);
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    const int c4 = threadIdx.x + 256 * i;
    if (c4 < L4) {
      const int64_t o0 = static_cast<int64_t>(t) * L + 4 * c4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[i][e] * scale * gamma[4 * c4 + e];
        const ACT o = from_f32<ACT>(v);
        out[o0 + e] = o;
        if (out_lo) out_lo[o0 + e] = f32_to_bf16(v - static_cast<float>(to_f32(o)));
      }
    }
  }
}

struct ForwardWorkspace {
  RouteWorkspace route;
  float* scores;
  int32_t* idx;
  float* w;
  int32_t* loads;
  int32_t* info;
  bf16_t* wsplit;     // [3][n][d] (bf16 activations)
  void* z;            // [T][latent]
  void* hs;           // [T][shared]
  bf16_t* hs_lo;      // [T][shared] bf16 residue of hs (bf16 activations)
  int32_t* offs;      // [n+1]
  int32_t* tiles;     // [max_mtiles][4]
  int32_t* ntiles;
  uint8_t* sel;       // [n][T]
  int32_t* perm;      // [T*k]
  int32_t* inv;       // [T*k]
  void* h;            // [T*k][inter]
  void* yp;           // [T*k][latent]
  void* yhat;         // [T][latent]
  bf16_t* yhat_lo;    // [T][latent] bf16 residue of yhat (bf16 activations)
  uint8_t* zq;        // W4A8 / W4A4: z as E4M3 codes [T][latent] (E2M1: [T][latent/2])
  uint8_t* zq_scale;  //   and E8M0 scales [T][latent/32]
  uint8_t* hq;        // W4A8 / W4A4: h as E4M3 codes [T*k][inter] (E2M1: [T*k][inter/2])
  uint8_t* hq_scale;  //   and scales [T*k][inter/32]
  int bm;
  int max_mtiles;
  float* partial;     // split-K partial sums of the dense GEMMs (used one at a time)
  size_t partial_bytes;
  // training forward: pre-activations of the routed and shared SiTU-GLU
  // (fp32), stored beside h and hs; null otherwise
  float *save_g, *save_u, *save_gs, *save_us;
};

size_t saved_layout(const moe_shape_t& s, SavedActivations* out, void* base) {
  Carver cv(base);
  SavedActivations a{};
  const int64_t T = s.T, S = static_cast<int64_t>(s.T) * s.top_k;
  a.z = cv.take<bf16_t>(T * s.latent);
  a.g = cv.take<float>(S * s.inter);
  a.u = cv.take<float>(S * s.inter);
  a.h = cv.take<bf16_t>(S * s.inter);
  a.yp = cv.take<float>(S * s.latent);
  a.gs = cv.take<float>(T * s.shared_inter);
  a.us = cv.take<float>(T * s.shared_inter);
  a.hs = cv.take<bf16_t>(T * s.shared_inter);
  if (out) *out = a;
  return cv.bytes();
}

// Tile height of the grouped expert GEMMs, from the mean rows per expert
// (exact under QB): 32 for decode-like batches, then 96, 160 or 320 rows
// (one tile per expert up to 320 rows), else 256; MXFP4 takes 160 when its
// pipelined kernel applies, else 128.
int grouped_bm(const moe_shape_t& s) {
  const int64_t avg = (static_cast<int64_t>(s.T) * s.top_k + s.n_experts - 1) / s.n_experts;
  if (s.act_dtype != MOE_BF16) return 64;
  if (s.routed_dtype == MOE_MXFP4_A8 || s.routed_dtype == MOE_MXFP4_A4)
    return 320;  // the only tile of quantised activations
  if (avg <= 32) return 32;
  if (s.routed_dtype == MOE_MXFP4) {
    // MFMA-bound: 320-row tiles on 8 waves for 161 - 320 rows per expert,
    // else 160-row tiles (5 x 2 fragments per wave), when the pipelined
    // MXFP4 kernels take both K widths
    if (avg > 160 && avg <= 320 && gemm::fp4_tile320_fits(s.latent) &&
        gemm::fp4_tile320_fits(s.inter))
      return 320;
    if (gemm::fp4_tall_tile_fits(s.latent) && gemm::fp4_tall_tile_fits(s.inter)) return 160;
    return 128;
  }
  if (avg <= 96) return 96;
  if (avg <= 160) return 160;
  if (avg <= 320) return 320;
  return 256;
}

static size_t forward_layout(const moe_shape_t& s, ForwardWorkspace* fw, void* base) {
  Carver cv(base);
  ForwardWorkspace f{};
  const size_t es = s.act_dtype == MOE_BF16 ? 2 : 4;
  const int64_t T = s.T, n = s.n_experts, k = s.top_k;
  // the routing workspace is carved first, at offset 0
  const size_t rb = route_workspace_layout(s.T, s.n_experts, &f.route, base);
  cv.off = rb;
  f.scores = cv.take<float>(T * n);
  f.idx = cv.take<int32_t>(T * k);
  f.w = cv.take<float>(T * k);
  f.loads = cv.take<int32_t>(n);
  f.info = cv.take<int32_t>(4);
  f.wsplit = cv.take<bf16_t>(s.act_dtype == MOE_BF16 ? 3 * n * s.d : 0);
  f.z = cv.take<char>(T * s.latent * es);
  f.hs = cv.take<char>(T * s.shared_inter * es);
  f.hs_lo = cv.take<bf16_t>(es == 2 ? T * s.shared_inter : 0);
  f.bm = grouped_bm(s);
  f.max_mtiles = static_cast<int>((T * k + f.bm - 1) / f.bm + n);
  f.offs = cv.take<int32_t>(n + 1);
  f.tiles = cv.take<int32_t>(4 * static_cast<size_t>(f.max_mtiles));
  f.ntiles = cv.take<int32_t>(1);
  f.sel = cv.take<uint8_t>(align_up(static_cast<size_t>(n * T), 4));
  f.perm = cv.take<int32_t>(T * k);
  f.inv = cv.take<int32_t>(T * k);
  f.h = cv.take<char>(T * k * s.inter * es);
  f.yp = cv.take<float>(T * k * s.latent);  // fp32: the combine sums unrounded products
  f.yhat = cv.take<char>(T * s.latent * es);
  f.yhat_lo = cv.take<bf16_t>(es == 2 ? T * s.latent : 0);
  const bool a8 = s.routed_dtype == MOE_MXFP4_A8, a4 = s.routed_dtype == MOE_MXFP4_A4;
  const int64_t qdiv = a4 ? 2 : 1;  // elements per code byte
  f.zq = cv.take<uint8_t>(a8 || a4 ? T * s.latent / qdiv : 0);
  f.zq_scale = cv.take<uint8_t>(a8 || a4 ? T * s.latent / 32 : 0);
  f.hq = cv.take<uint8_t>(a8 || a4 ? T * k * s.inter / qdiv : 0);
  f.hq_scale = cv.take<uint8_t>(a8 || a4 ? T * k * s.inter / 32 : 0);
  // The dense GEMMs that may split K never overlap in time: the router runs
  // before the shared branch forks, the two shared-branch products run in
  // order on one stream, and the up-projection runs after the join.
  size_t pb = 0;
  if (s.act_dtype == MOE_BF16) {
    const int epi_store = gemm::EPI_BF16;
    const size_t c[4] = {gemm::splitk_bytes(s.T, s.n_experts, 3 * s.d, gemm::EPI_SIGMOID),
                         gemm::splitk_bytes(s.T, s.latent, s.d, epi_store),
                         gemm::splitk_bytes(s.T, s.shared_inter, s.d, gemm::EPI_SITU),
                         gemm::splitk_bytes(s.T, s.d, s.latent + s.shared_inter, epi_store)};
    for (size_t v : c) pb = v > pb ? v : pb;
  }
  f.partial = cv.take<float>(pb / sizeof(float));
  f.partial_bytes = pb;
  if (fw) *fw = f;
  return cv.bytes();
}

static int validate(const moe_shape_t* sp, const moe_weights_t* w) {
  if (!sp) return MOE_EINVAL;
  const moe_shape_t& s = *sp;
  int st = route_validate(s.T, s.n_experts, s.top_k);
  if (st != MOE_OK) return st;
  if (s.d <= 0 || s.latent <= 0 || s.inter <= 0 || s.shared_inter <= 0) return MOE_EINVAL;
  if (s.d % 64 || s.latent % 64 || s.inter % 64 || s.shared_inter % 64) return MOE_EUNSUPPORTED;
  if (s.latent > 256 * 16) return MOE_EUNSUPPORTED;
  if (s.act_dtype != MOE_F32 && s.act_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  const bool mx = s.routed_dtype == MOE_MXFP4 || s.routed_dtype == MOE_MXFP4_A8 ||
                  s.routed_dtype == MOE_MXFP4_A4;
  if (!(s.routed_dtype == s.act_dtype || (mx && s.act_dtype == MOE_BF16))) return MOE_EUNSUPPORTED;
  // W4A8 scale words stay inside their rows when K is a multiple of 128
  if ((s.routed_dtype == MOE_MXFP4_A8 || s.routed_dtype == MOE_MXFP4_A4) &&
      (s.latent % 128 || s.inter % 128))
    return MOE_EUNSUPPORTED;
  if (s.qb_mode != MOE_QB_BATCH && s.qb_mode != MOE_QB_FROZEN) return MOE_EINVAL;
  if (!(s.rms_eps >= 0.f)) return MOE_EINVAL;
  if (w) {
    if (!w->w_router || !w->w_down || !w->w_up || !w->w_gate || !w->w_uproj || !w->w_dn ||
        !w->rms_gamma || !w->ws_gate || !w->ws_up || !w->ws_down)
      return MOE_EINVAL;
    if (mx && (!w->s_gate || !w->s_uproj || !w->s_dn)) return MOE_EINVAL;
  }
  return MOE_OK;
}

// Per-device side stream (default priority, non-blocking) on which the
// routing-independent shared branch runs while the caller's stream does the
// latency-bound routing; two events fork it from and join it back into the
// caller's stream.  A per-device mutex is held for the whole forward call so
// that concurrent calls on one device cannot interleave on the shared events.
struct SideStream {
  std::mutex mu;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ok = false;
};

// Joins a forked side stream back into the caller's stream when a forward
// returns early (an error after the fork), so that no side-stream work can
// outlive the call and touch a workspace the caller then frees.
struct SideJoin {
  SideStream* side = nullptr;
  hipStream_t st = nullptr;
  bool joined = false;
  ~SideJoin() {
    if (side && !joined && hipEventRecord(side->join, side->s) == hipSuccess)
      (void)hipStreamWaitEvent(st, side->join, 0);
  }
};

static SideStream* side_stream() {
  static SideStream tab[64];
  static std::mutex init_mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(init_mu);
  SideStream& ss = tab[dev];
  if (!ss.ok) {
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) return nullptr;
    ss.ok = true;
  }
  return &ss;
}


static int forward(const moe_shape_t& s, const moe_weights_t& wt, const void* x, void* out,
                   double* bias, const float* scores_in, float* scores_out, int32_t* idx_out,
                   float* w_out, int32_t* loads_out, int32_t* info_out,
                   const ForwardWorkspace& f, hipStream_t st) {
  const bool bf = s.act_dtype == MOE_BF16;
  const int T = s.T, n = s.n_experts, k = s.top_k, d = s.d, L = s.latent, m = s.inter,
            ms = s.shared_inter;
  const int store_epi = bf ? gemm::EPI_BF16 : gemm::EPI_F32;
  const int64_t es = bf ? 2 : 4;
  int rc;
  float* scores = scores_out ? scores_out : f.scores;
  int32_t* idx = idx_out ? idx_out : f.idx;
  float* w = w_out ? w_out : f.w;
  int32_t* info = info_out ? info_out : f.info;

  // 1. router: s = sigmoid(x W_r^T + p)
  {
  prof::Scope sc(prof::ST_ROUTER, st);
  if (scores_in) {
    if (scores_out && T > 0)
      hipLaunchKernelGGL(copy_f32, dim3(1024), dim3(256), 0, st, scores_in, scores_out,
                         static_cast<int64_t>(T) * n);
  } else if (T > 0) {
    gemm::Params p{};
    p.M = T;
    p.N = n;
    p.C = scores;
    p.ldc = n;
    p.col_add = wt.router_logit_offset;
    p.partial = f.partial;
    p.partial_bytes = f.partial_bytes;
    if (bf) {
      const int64_t cnt = static_cast<int64_t>(n) * d;
      bf16_t* hi = f.wsplit;
      hipLaunchKernelGGL(split3, dim3(2048), dim3(256), 0, st, wt.w_router, hi, hi + cnt,
                         hi + 2 * cnt, cnt);
      p.nseg = 3;
      for (int q = 0; q < 3; ++q) p.seg[q] = seg(x, d, hi + q * cnt, d, d);
    } else {
      p.nseg = 1;
      p.seg[0] = seg(x, d, wt.w_router, d, d);
    }
    if ((rc = gemm::launch(p, gemm::EPI_SIGMOID, gemm::B_DENSE, bf, 128, st)) != MOE_OK) return rc;
  }
  }
  const float* route_scores = scores_in ? scores_in : scores;

  // 2. shared branch (independent of routing) on the side stream:
  //    z = x W_down^T, hs = SiTU(x Wgs^T, x Wus^T)
  SideStream* side = T > 0 ? side_stream() : nullptr;
  std::unique_lock<std::mutex> side_lock;
  SideJoin side_join;  // destroyed before side_lock is released
  hipStream_t sst = st;
  if (side) {
    side_lock = std::unique_lock<std::mutex>(side->mu);
    MOE_HIP_CHECK(hipEventRecord(side->fork, st));
    side_join.side = side;
    side_join.st = st;
    MOE_HIP_CHECK(hipStreamWaitEvent(side->s, side->fork, 0));
    sst = side->s;
  }
  // 3. routing (QB or frozen bias), enqueued before the shared-branch GEMMs:
  // the balancing loop is one persistent launch that takes whole CUs; with
  // the side stream running beside it, it takes 1/cu_share of them and the
  // shared-branch GEMMs run on the rest.
  {
    prof::Scope sc(prof::ST_ROUTING, st);
    // Above 8192 tokens the side-stream GEMMs are long enough that the
    // batch loop is given half of the compute units and the GEMMs the rest;
    // below that the loop is short and takes every unit.
    const int cu_share = side && s.qb_mode == MOE_QB_BATCH && T > 8192 ? 2 : 1;
    if ((rc = route_run(route_scores, T, n, k, s.qb_mode, s.qb_max_rounds, bias, idx, w, f.loads,
                        info, f.route, st, cu_share)) != MOE_OK)
      return rc;
  }
  const int side_hint = 128;
  if (T > 0) {
    gemm::Params p{};
    p.M = T;
    p.N = L;
    p.nseg = 1;
    p.seg[0] = seg(x, d, wt.w_down, d, d);
    p.C = f.z;
    p.ldc = L;
    p.partial = f.partial;
    p.partial_bytes = f.partial_bytes;
    {
      prof::Scope sc(prof::ST_LATENT_DOWN, sst);
      if ((rc = gemm::launch(p, store_epi, gemm::B_DENSE, bf, side_hint, sst)) != MOE_OK) return rc;
      if (s.routed_dtype == MOE_MXFP4_A8 || s.routed_dtype == MOE_MXFP4_A4) {
        // z -> MXFP8 / MXFP4 for the routed experts
        const int64_t nblk = static_cast<int64_t>(T) * (L / 32);
        const dim3 grid(static_cast<unsigned>(std::min<int64_t>((nblk + 63) / 64, 8192)));
        if (s.routed_dtype == MOE_MXFP4_A8)
          hipLaunchKernelGGL(mx8_quantize, grid, dim3(256), 0, sst,
                             static_cast<const bf16_t*>(f.z), nblk, f.zq, f.zq_scale);
        else
          hipLaunchKernelGGL(mx4_quantize, grid, dim3(256), 0, sst,
                             static_cast<const bf16_t*>(f.z), nblk, f.zq, f.zq_scale);
        MOE_LAUNCH_CHECK();
      }
    }
    gemm::Params q{};
    q.M = T;
    q.N = ms;
    q.nseg = 1;
    q.seg[0] = seg(x, d, wt.ws_gate, d, d);
    q.seg[0].B2 = wt.ws_up;
    q.C = f.hs;
    q.C2 = bf ? f.hs_lo : nullptr;
    q.ldc = ms;
    q.save_g = f.save_gs;
    q.save_u = f.save_us;
    q.partial = f.partial;
    q.partial_bytes = f.partial_bytes;
    {
      prof::Scope sc(prof::ST_SHARED_GATE_UP, sst);
      if ((rc = gemm::launch(q, gemm::EPI_SITU, gemm::B_DENSE, bf, side_hint, sst)) != MOE_OK)
        return rc;
    }
  }
  if (side) MOE_HIP_CHECK(hipEventRecord(side->join, side->s));
  if (loads_out)
    MOE_HIP_CHECK(hipMemcpyAsync(loads_out, f.loads, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st));
  if (T == 0) return MOE_OK;

  // 4. permutation: slots grouped by expert, tokens ascending inside a group
  {
  prof::Scope sc(prof::ST_PERMUTE, st);
  hipLaunchKernelGGL(scan_and_tiles, dim3(1), dim3(1024), 0, st, f.loads, n, f.bm, f.offs,
                     f.tiles, f.ntiles);
  const int64_t selw = static_cast<int64_t>(align_up(static_cast<size_t>(n) * T, 4) / 4);
  hipLaunchKernelGGL(fill_u32, dim3(1024), dim3(256), 0, st, reinterpret_cast<uint32_t*>(f.sel),
                     0u, selw);
  hipLaunchKernelGGL(scatter_sel, dim3(1024), dim3(256), 0, st, idx, T, k, f.sel);
  hipLaunchKernelGGL(expert_slots, dim3(n), dim3(256), 0, st, f.sel, T, k, f.offs, f.perm, f.inv);
  MOE_LAUNCH_CHECK();
  }

  if (side) {
    MOE_HIP_CHECK(hipStreamWaitEvent(st, side->join, 0));
    side_join.joined = true;
  }
  const bool a8 = s.routed_dtype == MOE_MXFP4_A8, a4 = s.routed_dtype == MOE_MXFP4_A4;
  const bool mx = s.routed_dtype == MOE_MXFP4 || a8 || a4;
  const int bfmt = a8 ? gemm::B_MXFP4_A8
                 : a4 ? gemm::B_MXFP4_A4
                 : mx ? gemm::B_MXFP4 : gemm::B_DENSE;
  // 5. routed gate/up with SiTU-GLU: h[slot] = SiTU(z[perm[slot]] Wg_e^T, z[perm[slot]] Wu_e^T)
  {
    gemm::Params p{};
    p.N = m;
    p.nseg = 1;
    if (a8)  // W4A8: the E4M3 codes of z, one byte per element
      p.seg[0] = seg(f.zq, L, wt.w_gate, L / 2, L);
    else if (a4)  // W4A4: the E2M1 codes of z, two per byte
      p.seg[0] = seg(f.zq, L / 2, wt.w_gate, L / 2, L);
    else
      p.seg[0] = seg(f.z, L, wt.w_gate, mx ? L / 2 : L, L);
    p.seg[0].As = f.zq_scale;
    p.seg[0].B2 = wt.w_uproj;
    p.seg[0].Bs = wt.s_gate;
    p.seg[0].Bs2 = wt.s_uproj;
    p.b_expert_stride = mx ? static_cast<int64_t>(m) * L / 2 : static_cast<int64_t>(m) * L;
    p.bs_expert_stride = static_cast<int64_t>(m) * L / 32;
    p.tiles = f.tiles;
    p.ntiles = f.ntiles;
    p.max_mtiles = f.max_mtiles;
    p.a_rows = f.perm;
    p.C = f.h;
    p.ldc = m;
    p.save_g = f.save_g;
    p.save_u = f.save_u;
    prof::Scope sc(prof::ST_ROUTED_GATE_UP, st);
    if ((rc = gemm::launch(p, gemm::EPI_SITU, bfmt, bf, f.bm, st)) != MOE_OK) return rc;
  }
  if (a8 || a4) {  // h -> MXFP8 / MXFP4 for the down-projection
    const int64_t nblk = static_cast<int64_t>(T) * k * (m / 32);
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>((nblk + 63) / 64, 8192)));
    if (a8)
      hipLaunchKernelGGL(mx8_quantize, grid, dim3(256), 0, st, static_cast<const bf16_t*>(f.h), nblk,
                         f.hq, f.hq_scale);
    else
      hipLaunchKernelGGL(mx4_quantize, grid, dim3(256), 0, st, static_cast<const bf16_t*>(f.h), nblk,
                         f.hq, f.hq_scale);
    MOE_LAUNCH_CHECK();
  }
  // 6. routed down: yp[slot] = h[slot] Wd_e^T
  {
    gemm::Params p{};
    p.N = L;
    p.nseg = 1;
    if (a8)
      p.seg[0] = seg(f.hq, m, wt.w_dn, m / 2, m);
    else if (a4)
      p.seg[0] = seg(f.hq, m / 2, wt.w_dn, m / 2, m);
    else
      p.seg[0] = seg(f.h, m, wt.w_dn, mx ? m / 2 : m, m);
    p.seg[0].As = f.hq_scale;
    p.seg[0].Bs = wt.s_dn;
    p.b_expert_stride = mx ? static_cast<int64_t>(L) * m / 2 : static_cast<int64_t>(L) * m;
    p.bs_expert_stride = static_cast<int64_t>(L) * m / 32;
    p.tiles = f.tiles;
    p.ntiles = f.ntiles;
    p.max_mtiles = f.max_mtiles;
    p.C = f.yp;
    p.ldc = L;
    prof::Scope sc(prof::ST_ROUTED_DOWN, st);
    if ((rc = gemm::launch(p, gemm::EPI_F32, bfmt, bf, f.bm, st)) != MOE_OK) return rc;
  }
  // 7. weighted combine in the latent space + RMSNorm
  {
  prof::Scope sc(prof::ST_COMBINE_RMSNORM, st);
  if (bf)
    hipLaunchKernelGGL(combine_rmsnorm<bf16_t>, dim3(T), dim3(256), 0, st,
                       static_cast<const float*>(f.yp), f.inv, w, wt.rms_gamma, k, L, s.rms_eps,
                       static_cast<bf16_t*>(f.yhat), f.yhat_lo);
  else
    hipLaunchKernelGGL(combine_rmsnorm<float>, dim3(T), dim3(256), 0, st,
                       static_cast<const float*>(f.yp), f.inv, w, wt.rms_gamma, k, L, s.rms_eps,
                       static_cast<float*>(f.yhat), nullptr);
  MOE_LAUNCH_CHECK();
  }
  // 8. out = yhat W_up^T + hs Ws_down^T (one GEMM, K concatenated); with bf16
  // activations each of yhat and hs enters as its bf16 value plus the bf16
  // residue, two K segments against the same weights
  {
    gemm::Params p{};
    p.M = T;
    p.N = d;
    if (bf) {
      p.nseg = 4;
      p.seg[0] = seg(f.yhat, L, wt.w_up, L, L);
      p.seg[1] = seg(f.yhat_lo, L, wt.w_up, L, L);
      p.seg[2] = seg(f.hs, ms, wt.ws_down, ms, ms);
      p.seg[3] = seg(f.hs_lo, ms, wt.ws_down, ms, ms);
    } else {
      p.nseg = 2;
      p.seg[0] = seg(f.yhat, L, wt.w_up, L, L);
      p.seg[1] = seg(f.hs, ms, wt.ws_down, ms, ms);
    }
    p.C = out;
    p.ldc = d;
    p.partial = f.partial;
    p.partial_bytes = f.partial_bytes;
    prof::Scope sc(prof::ST_UP_SHARED_DOWN, st);
    if ((rc = gemm::launch(p, store_epi, gemm::B_DENSE, bf, 128, st)) != MOE_OK) return rc;
  }
  (void)es;
  return MOE_OK;
}

}  // namespace layer
}  // namespace moe

extern "C" size_t moe_forward_workspace_bytes(const moe_shape_t* shape) {
  if (moe::layer::validate(shape, nullptr) != MOE_OK) return 0;
  return moe::layer::forward_layout(*shape, nullptr, nullptr);
}

extern "C" int moe_latent_forward(const moe_shape_t* shape, const moe_weights_t* weights,
                                  const void* x, void* out, double* bias, const float* scores_in,
                                  float* scores_out, int32_t* topk_idx, float* topk_w,
                                  int32_t* loads, int32_t* qb_info, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int st = moe::layer::validate(shape, weights);
  if (st != MOE_OK) return st;
  if (!weights || !bias || !workspace) return MOE_EINVAL;
  if (shape->T > 0 && (!x || !out)) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MOE_EINVAL;
  moe::layer::ForwardWorkspace fw;
  const size_t need = moe::layer::forward_layout(*shape, &fw, workspace);
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  return moe::layer::forward(*shape, *weights, x, out, bias, scores_in, scores_out, topk_idx,
                             topk_w, loads, qb_info, fw, static_cast<hipStream_t>(stream));
}

extern "C" size_t moe_saved_activations_bytes(const moe_shape_t* shape) {
  if (moe::layer::validate(shape, nullptr) != MOE_OK || shape->act_dtype != MOE_BF16 ||
      shape->routed_dtype != MOE_BF16)
    return 0;
  // never 0 for a shape the calls take (0 means "not taken"): at least 256 bytes
  return std::max<size_t>(moe::layer::saved_layout(*shape, nullptr, nullptr), 256);
}

extern "C" int moe_latent_forward_train(const moe_shape_t* shape, const moe_weights_t* weights,
                                        const void* x, void* out, double* bias,
                                        const float* scores_in, float* scores_out,
                                        int32_t* topk_idx, float* topk_w, int32_t* loads,
                                        int32_t* qb_info, void* saved, size_t saved_bytes,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = moe::layer::validate(shape, weights);
  if (st != MOE_OK) return st;
  if (shape->act_dtype != MOE_BF16 || shape->routed_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (!weights || !bias || !workspace || !saved) return MOE_EINVAL;
  if (shape->T > 0 && (!x || !out)) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      reinterpret_cast<uintptr_t>(saved) % 256 != 0)
    return MOE_EINVAL;
  moe::layer::ForwardWorkspace fw;
  const size_t need = moe::layer::forward_layout(*shape, &fw, workspace);
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  moe::layer::SavedActivations sv;
  if (saved_bytes < moe::layer::saved_layout(*shape, &sv, saved)) return MOE_EWORKSPACE;
  // z, h, the experts' outputs and hs live in the saved buffer; the SiTU-GLU
  // GEMMs also store their pre-activations there
  fw.z = sv.z;
  fw.h = sv.h;
  fw.yp = sv.yp;
  fw.hs = sv.hs;
  fw.save_g = sv.g;
  fw.save_u = sv.u;
  fw.save_gs = sv.gs;
  fw.save_us = sv.us;
  return moe::layer::forward(*shape, *weights, x, out, bias, scores_in, scores_out, topk_idx,
                             topk_w, loads, qb_info, fw, static_cast<hipStream_t>(stream));
}

extern "C" int moe_mxfp8_quantize(const void* x, int64_t rows, int64_t K, uint8_t* codes,
                                  uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_EINVAL;
  if (rows > 0 && (!x || !codes || !scales)) return MOE_EINVAL;
  if (rows > 0 && (reinterpret_cast<uintptr_t>(x) % 16 != 0 ||
                   reinterpret_cast<uintptr_t>(codes) % 8 != 0))
    return MOE_EINVAL;
  if (rows > (int64_t(1) << 56) / K) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  const int64_t nblk = rows * (K / 32);
  hipLaunchKernelGGL(moe::layer::mx8_quantize,
                     dim3(static_cast<unsigned>(std::min<int64_t>((nblk + 63) / 64, 8192))), dim3(256),
                     0, static_cast<hipStream_t>(stream), static_cast<const moe::bf16_t*>(x), nblk,
                     codes, scales);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

extern "C" int moe_mxfp4_quantize(const void* x, int64_t rows, int64_t K, uint8_t* codes,
                                  uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_EINVAL;
  if (rows > 0 && (!x || !codes || !scales)) return MOE_EINVAL;
  if (rows > 0 && (reinterpret_cast<uintptr_t>(x) % 16 != 0 ||
                   reinterpret_cast<uintptr_t>(codes) % 4 != 0))
    return MOE_EINVAL;
  if (rows > (int64_t(1) << 56) / K) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  const int64_t nblk = rows * (K / 32);
  hipLaunchKernelGGL(moe::layer::mx4_quantize,
                     dim3(static_cast<unsigned>(std::min<int64_t>((nblk + 63) / 64, 8192))), dim3(256),
                     0, static_cast<hipStream_t>(stream), static_cast<const moe::bf16_t*>(x), nblk,
                     codes, scales);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

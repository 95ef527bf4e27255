// Backward pass of the Stable LatentMoE layer with the expert selection held
// fixed (the QB bias acts on selection only, "Kimi K3 模型结构（5）：宽度维度，
// Stable LatentMoE", Q&A on routing): gradients reach the router through the
// renormalised raw scores w = s_sel / sum(s_sel), and every step after
// routing is differentiated as written (SiTU-GLU, Q&A on SiTU-GLU; RMSNorm
// after the aggregation, Q&A on RMSNorm; the merged shared MLP, Q&A on the
// shared expert).
//
// The call recomputes the forward activations from x and the forward's
// routing (scores, idx, w), or reads those a training forward kept, then
// runs the backward products on the same pipelined MFMA GEMM (C = A B^T).  The experts' weights enter the products
// through them as [K][N] B operands read in place (transposing LDS reads);
// other operands that are not K-contiguous take transposed copies; the
// weight gradients of the routed experts are K-grouped products over each
// expert's slots (zero-padded to 64), optionally applied to the weights in
// their epilogue (the SGD step of a training step).  MFMA operands are bf16,
// accumulations and gradients fp32.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "gemm.hpp"
#include "layer_kernels.hpp"

namespace moe {
namespace bwd {

constexpr int TB = 64;  // transpose tile

// loads[e] = number of slots of expert e (loads zeroed before).
__global__ void count_loads(const int32_t* idx, int64_t total, int32_t* loads) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    atomicAdd(&loads[idx[i]], 1);
}

// poffs = exclusive scan of loads rounded up to 64 (one block of 1024).
__global__ __launch_bounds__(1024) void pad_offsets(const int32_t* loads, int n, int32_t* poffs) {
  __shared__ int32_t s[1024];
  const int e = threadIdx.x;
  const int32_t v = e < n ? (loads[e] + 63) / 64 * 64 : 0;
  s[e] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t a = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += a;
    __syncthreads();
  }
  if (e < n) poffs[e] = s[e] - v;
  if (e == n - 1) poffs[n] = s[e];
}

// pcol[slot] = the slot's column in the padded per-expert layout.
__global__ void slot_cols(const int32_t* offs, const int32_t* poffs, int32_t* pcol) {
  const int e = blockIdx.x;
  for (int s = offs[e] + threadIdx.x; s < offs[e + 1]; s += blockDim.x)
    pcol[s] = poffs[e] + (s - offs[e]);
}

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p, int64_t i) {
  return to_f32(p[i]);
}

// out[b][c][r] = in[b][r][c] (r < R, c < C), converted to bf16.  64 x 64
// tiles through LDS; blockIdx.z is the batch.
template <typename TI>
__global__ __launch_bounds__(256) void transpose_k(const TI* __restrict__ in, int64_t R, int64_t C,
                                                   int64_t ldi, int64_t bsi,
                                                   bf16_t* __restrict__ out, int64_t ldo,
                                                   int64_t bso) {
  __shared__ float tile[TB][TB + 1];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * TB, c0 = static_cast<int64_t>(blockIdx.x) * TB;
  const TI* src = in + static_cast<int64_t>(blockIdx.z) * bsi;
  bf16_t* dst = out + static_cast<int64_t>(blockIdx.z) * bso;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < TB; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? ld_f32(src, r * ldi + c) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < TB; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < R) dst[c * ldo + r] = f32_to_bf16(tile[tx][i]);
  }
}

// bf16 -> bf16 transpose with 16-byte accesses: 64 x 64 tiles, each lane
// loads 8 consecutive elements of a row and stores 8 consecutive elements of
// an output row (R, C multiples of 8 and 16-byte aligned rows; the launcher
// checks and otherwise uses transpose_k).
__global__ __launch_bounds__(256) void transpose16_k(const bf16_t* __restrict__ in, int64_t R,
                                                     int64_t C, int64_t ldi, int64_t bsi,
                                                     bf16_t* __restrict__ out, int64_t ldo,
                                                     int64_t bso) {
  __shared__ uint16_t tile[TB][TB + 2];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * TB, c0 = static_cast<int64_t>(blockIdx.x) * TB;
  const bf16_t* src = in + static_cast<int64_t>(blockIdx.z) * bsi;
  bf16_t* dst = out + static_cast<int64_t>(blockIdx.z) * bso;
  // load: lane -> (row r0 + tid / 8 + 32 i, columns c0 + 8 (tid % 8) .. +8)
  const int lr = threadIdx.x >> 3, lc = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = r0 + lr + 32 * i, c = c0 + lc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < R && c < C) v = *reinterpret_cast<const uint4*>(src + r * ldi + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[lr + 32 * i][lc + 2 * j] = static_cast<uint16_t>(w[j] & 0xFFFFu);
      tile[lr + 32 * i][lc + 2 * j + 1] = static_cast<uint16_t>(w[j] >> 16);
    }
  }
  __syncthreads();
  // store: lane -> (output row c0 + tid / 8 + 32 i, output columns r0 + 8 (tid % 8) .. +8)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t c = c0 + lr + 32 * i, r = r0 + lc;
    if (c < C && r < R) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = static_cast<uint32_t>(tile[lc + 2 * j][lr + 32 * i]) |
               (static_cast<uint32_t>(tile[lc + 2 * j + 1][lr + 32 * i]) << 16);
      *reinterpret_cast<uint4*>(dst + c * ldo + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// out[c][pcol[s]] = in[src(s)][c] for slots s < S, c < C (src(s) = rowmap[s]
// or s), converted to bf16: rows grouped by expert become K ranges.
template <typename TI>
__global__ __launch_bounds__(256) void slot_transpose_k(const TI* __restrict__ in, int64_t ldi,
                                                        const int32_t* __restrict__ rowmap,
                                                        const int32_t* __restrict__ pcol,
                                                        int64_t S, int64_t C,
                                                        bf16_t* __restrict__ out, int64_t ldo) {
  __shared__ float tile[TB][TB + 1];
  const int64_t s0 = static_cast<int64_t>(blockIdx.y) * TB, c0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < TB; i += 4) {
    const int64_t s = s0 + i, c = c0 + tx;
    float v = 0.f;
    if (s < S && c < C) {
      const int64_t row = rowmap ? rowmap[s] : s;
      v = ld_f32(in, row * ldi + c);
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < TB; i += 4) {
    const int64_t c = c0 + i, s = s0 + tx;
    if (c < C && s < S) out[c * ldo + pcol[s]] = f32_to_bf16(tile[tx][i]);
  }
}

// SiTU-GLU parts: gc = 4 tanh(g/4), uc = 25 tanh(u/25), h = SiLU(gc) uc.
__device__ __forceinline__ void situ_parts(float g, float u, float& gc, float& sg, float& uc) {
  gc = 4.0f * tanh_fast(g * 0.25f);
  uc = 25.0f * tanh_fast(u * 0.04f);
  sg = 1.0f / (1.0f + __expf(-gc));
}

// h = SiTU-GLU(g, u) in bf16 (the forward's recomputation).
__global__ void situ_fwd_k(const float* __restrict__ g, const float* __restrict__ u, int64_t count,
                           bf16_t* __restrict__ h) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float gc, sg, uc;
    situ_parts(g[i], u[i], gc, sg, uc);
    h[i] = f32_to_bf16(gc * sg * uc);
  }
}

// 1 - tanh(x)^2 = 4 e / (1 + e)^2 with e = exp(-2|x|): no cancellation where
// tanh(x) is close to +-1.
__device__ __forceinline__ float sech2(float x) {
  const float e = __expf(-2.0f * fabsf(x));
  const float q = 1.0f + e;
  return __fdividef(4.0f * e, q * q);
}

// dg = dh * uc * SiLU'(gc) * sech^2(g/4), du = dh * SiLU(gc) * sech^2(u/25)
// with SiLU'(x) = s (1 + x (1 - s)), s = sigmoid(x); outputs in bf16.
__global__ void situ_bwd_k(const float* __restrict__ g, const float* __restrict__ u,
                           const float* __restrict__ dh, int64_t count, bf16_t* __restrict__ dg,
                           bf16_t* __restrict__ du) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float gc, sg, uc;
    const float gv = g[i], uv = u[i];
    situ_parts(gv, uv, gc, sg, uc);
    const float d = dh[i];
    dg[i] = f32_to_bf16(d * uc * sg * (1.0f + gc * (1.0f - sg)) * sech2(gv * 0.25f));
    du[i] = f32_to_bf16(d * gc * sg * sech2(uv * 0.04f));
  }
}

constexpr int MAXV = 16;  // latent <= 256 * MAXV

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// One block (256 threads) per token: y = sum_j w_j yp[inv[t][j]] (j
// ascending, as the forward), r = rsqrt(mean(y^2) + eps), yhat = y r gamma;
// from dyhat: gd = gamma dyhat, dy = r gd - y r^3 (gd . y) / L; then
// dy_slot = w_j dy (bf16), dw_j = dy . yp_slot, q = dyhat y r (for dgamma).
__global__ __launch_bounds__(256) void norm_bwd_k(const float* __restrict__ yp,
                                                  const int32_t* __restrict__ inv,
                                                  const float* __restrict__ w,
                                                  const float* __restrict__ gamma,
                                                  const float* __restrict__ dyhat, int k, int L,
                                                  float eps, bf16_t* __restrict__ yhat,
                                                  bf16_t* __restrict__ dy_slot,
                                                  float* __restrict__ dw, float* __restrict__ q) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  float y[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) y[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const float* src = yp + static_cast<int64_t>(inv[t * k + j]) * L;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < L) y[i] = fmaf(wj, src[c], y[i]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) ss = fmaf(y[i], y[i], ss);
  const float r = rsqrtf(block_sum(ss, red) / static_cast<float>(L) + eps);
  float gdy = 0.f;
  float gd[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + 256 * i;
    gd[i] = 0.f;
    if (c < L) {
      const float dv = dyhat[t * L + c];
      gd[i] = gamma[c] * dv;
      gdy = fmaf(gd[i], y[i], gdy);
      yhat[t * L + c] = f32_to_bf16(y[i] * r * gamma[c]);
      q[t * L + c] = dv * y[i] * r;
    }
  }
  const float cc = block_sum(gdy, red) * r * r * r / static_cast<float>(L);
#pragma unroll
  for (int i = 0; i < MAXV; ++i) gd[i] = r * gd[i] - y[i] * cc;  // dy
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const int64_t slot = inv[t * k + j];
    const float* src = yp + slot * L;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < L) {
        part = fmaf(gd[i], src[c], part);
        dy_slot[slot * L + c] = f32_to_bf16(wj * gd[i]);
      }
    }
    const float s = block_sum(part, red);
    if (threadIdx.x == 0) dw[t * k + j] = s;
  }
}

// Router: w_i = s_i / S (S = sum of the chosen scores), so
// ds_i = (dw_i - sum_j w_j dw_j) / S and dlogit_i = ds_i s_i (1 - s_i); one
// thread per token, written per (t, j) and per slot.
__global__ void router_bwd_k(const float* __restrict__ scores, const int32_t* __restrict__ idx,
                             const float* __restrict__ w, const float* __restrict__ dw,
                             const int32_t* __restrict__ inv, int T, int n, int k,
                             float* __restrict__ dlogit, float* __restrict__ dlogit_slot) {
  const int64_t t = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (t >= T) return;
  float S = 0.f, wd = 0.f;
  for (int j = 0; j < k; ++j) {
    S += scores[t * n + idx[t * k + j]];
    wd = fmaf(w[t * k + j], dw[t * k + j], wd);
  }
  for (int j = 0; j < k; ++j) {
    const float s = scores[t * n + idx[t * k + j]];
    const float v = (dw[t * k + j] - wd) / S * s * (1.0f - s);
    dlogit[t * k + j] = v;
    dlogit_slot[inv[t * k + j]] = v;
  }
}

// dz_t = sum_j dz_slot[inv[t][j]] (j ascending) in bf16; one block per token.
__global__ __launch_bounds__(256) void dz_gather_k(const float* __restrict__ dz_slot,
                                                   const int32_t* __restrict__ inv, int k, int L,
                                                   bf16_t* __restrict__ dz) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < L; c += 256) {
    float a = 0.f;
    for (int j = 0; j < k; ++j) a += dz_slot[static_cast<int64_t>(inv[t * k + j]) * L + c];
    dz[t * L + c] = f32_to_bf16(a);
  }
}

// dx_t = dx_acc_t + sum_j dlogit_tj W_r[idx_tj] (j ascending), in the
// activation dtype; one block per token.
template <typename ACT>
__global__ __launch_bounds__(256) void dx_final_k(const float* __restrict__ dx_acc,
                                                  const float* __restrict__ dlogit,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ w_router, int k, int d,
                                                  ACT* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += 256) {
    float a = dx_acc[t * d + c];
    for (int j = 0; j < k; ++j)
      a = fmaf(dlogit[t * k + j], w_router[static_cast<int64_t>(idx[t * k + j]) * d + c], a);
    dx[t * d + c] = from_f32<ACT>(a);
  }
}

// Router weight gradients: dW_r[e] = sum over e's slots (in slot order) of
// dlogit_slot x_token, d_offset[e] = sum of dlogit_slot; one block per
// (expert, 256 columns).
template <typename ACT>
__global__ __launch_bounds__(256) void router_wgrad_k(const ACT* __restrict__ x,
                                                      const int32_t* __restrict__ offs,
                                                      const int32_t* __restrict__ perm,
                                                      const float* __restrict__ dlogit_slot, int d,
                                                      float* __restrict__ dwr,
                                                      float* __restrict__ doff) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  float a = 0.f, o = 0.f;
  for (int s = offs[e]; s < offs[e + 1]; ++s) {
    const float g = dlogit_slot[s];
    o += g;
    if (c < d) a = fmaf(g, to_f32(x[static_cast<int64_t>(perm[s]) * d + c]), a);
  }
  if (c < d) dwr[static_cast<int64_t>(e) * d + c] = a;
  if (doff && blockIdx.x == 0 && threadIdx.x == 0) doff[e] = o;
}

// dgamma[c] = sum_t q[t][c] in two fixed-order passes: partial sums over
// chunks of 64 tokens (one thread per (chunk, column)), then over the chunks.
__global__ void gamma_part_k(const float* __restrict__ q, int64_t T, int L, float* __restrict__ part) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * 64;
  if (c >= L) return;
  float a = 0.f;
  for (int64_t t = t0; t < t0 + 64 && t < T; ++t) a += q[t * L + c];
  part[blockIdx.y * static_cast<int64_t>(L) + c] = a;
}

__global__ void gamma_grad_k(const float* __restrict__ part, int64_t chunks, int L,
                             float* __restrict__ dg) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= L) return;
  float a = 0.f;
  for (int64_t i = 0; i < chunks; ++i) a += part[i * L + c];
  dg[c] = a;
}

__global__ void fill_f32(float* p, int64_t count) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

// ---------------------------------------------------------------------------
struct BackwardWorkspace {
  int32_t *loads, *offs, *poffs, *tiles, *ntiles, *perm, *inv, *pcol;
  uint8_t* sel;
  bf16_t *w_upT, *w_dsT, *w_gsT, *w_usT, *w_downT;
  bf16_t *z, *h, *hs, *yhat, *dy_slot, *dg, *du, *dgs, *dus, *dz;
  float *g, *u, *yp, *gs, *us, *dyhat, *dh, *dz_slot, *dhs, *dx_acc, *q, *gpart, *dw, *dlogit,
      *dlogit_slot;
  bf16_t *xT, *doutT, *yhatT, *hsT, *dgsT, *dusT, *dzT;     // [.][Tp]
  bf16_t *z_slotT, *hT, *dy_slotT, *dgT, *duT;              // [.][Sp]
  int bm, max_mtiles;
  int64_t Tp, Sp;
};

static size_t backward_layout(const moe_shape_t& s, BackwardWorkspace* out, void* base) {
  Carver cv(base);
  BackwardWorkspace f{};
  const int64_t T = s.T, n = s.n_experts, k = s.top_k, d = s.d, L = s.latent, m = s.inter,
                ms = s.shared_inter;
  const int64_t S = T * k;
  f.Tp = (T + 63) / 64 * 64;
  f.Sp = S + 64 * n;
  f.bm = layer::grouped_bm(s);
  f.max_mtiles = static_cast<int>((S + f.bm - 1) / f.bm + n);
  f.loads = cv.take<int32_t>(n);
  f.offs = cv.take<int32_t>(n + 1);
  f.poffs = cv.take<int32_t>(n + 1);
  f.tiles = cv.take<int32_t>(4 * static_cast<size_t>(f.max_mtiles));
  f.ntiles = cv.take<int32_t>(1);
  f.perm = cv.take<int32_t>(S);
  f.inv = cv.take<int32_t>(S);
  f.pcol = cv.take<int32_t>(S);
  f.sel = cv.take<uint8_t>(align_up(static_cast<size_t>(n * T), 4));
  f.w_upT = cv.take<bf16_t>(L * d);
  f.w_dsT = cv.take<bf16_t>(ms * d);
  f.w_gsT = cv.take<bf16_t>(d * ms);
  f.w_usT = cv.take<bf16_t>(d * ms);
  f.w_downT = cv.take<bf16_t>(d * L);
  f.z = cv.take<bf16_t>(T * L);
  f.h = cv.take<bf16_t>(S * m);
  f.hs = cv.take<bf16_t>(T * ms);
  f.yhat = cv.take<bf16_t>(T * L);
  f.dy_slot = cv.take<bf16_t>(S * L);
  f.dg = cv.take<bf16_t>(S * m);
  f.du = cv.take<bf16_t>(S * m);
  f.dgs = cv.take<bf16_t>(T * ms);
  f.dus = cv.take<bf16_t>(T * ms);
  f.dz = cv.take<bf16_t>(T * L);
  f.g = cv.take<float>(S * m);
  f.u = cv.take<float>(S * m);
  f.yp = cv.take<float>(S * L);
  f.gs = cv.take<float>(T * ms);
  f.us = cv.take<float>(T * ms);
  f.dyhat = cv.take<float>(T * L);
  f.dh = cv.take<float>(S * m);
  f.dz_slot = cv.take<float>(S * L);
  f.dhs = cv.take<float>(T * ms);
  f.dx_acc = cv.take<float>(T * d);
  f.q = cv.take<float>(T * L);
  f.gpart = cv.take<float>((T + 63) / 64 * L);
  f.dw = cv.take<float>(S);
  f.dlogit = cv.take<float>(S);
  f.dlogit_slot = cv.take<float>(S);
  f.xT = cv.take<bf16_t>(d * f.Tp);
  f.doutT = cv.take<bf16_t>(d * f.Tp);
  f.yhatT = cv.take<bf16_t>(L * f.Tp);
  f.hsT = cv.take<bf16_t>(ms * f.Tp);
  f.dgsT = cv.take<bf16_t>(ms * f.Tp);
  f.dusT = cv.take<bf16_t>(ms * f.Tp);
  f.dzT = cv.take<bf16_t>(L * f.Tp);
  f.z_slotT = cv.take<bf16_t>(L * f.Sp);
  f.hT = cv.take<bf16_t>(m * f.Sp);
  f.dy_slotT = cv.take<bf16_t>(L * f.Sp);
  f.dgT = cv.take<bf16_t>(m * f.Sp);
  f.duT = cv.take<bf16_t>(m * f.Sp);
  if (out) *out = f;
  return cv.bytes();
}

static int validate(const moe_shape_t* sp) {
  if (!sp) return MOE_EINVAL;
  const moe_shape_t& s = *sp;
  if (s.T < 0 || s.n_experts < 1 || s.top_k < 1 || s.top_k > s.n_experts) return MOE_EINVAL;
  if (s.d <= 0 || s.latent <= 0 || s.inter <= 0 || s.shared_inter <= 0) return MOE_EINVAL;
  if (s.d % 64 || s.latent % 64 || s.inter % 64 || s.shared_inter % 64) return MOE_EINVAL;
  if (s.n_experts > 1024 || s.top_k > 64 || s.latent > 256 * MAXV || s.T > MOE_MAX_TOKENS)
    return MOE_EUNSUPPORTED;
  if (s.act_dtype != MOE_BF16 || s.routed_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (!(s.rms_eps >= 0.f)) return MOE_EINVAL;
  return MOE_OK;
}

static unsigned grid_of(int64_t count) {
  return static_cast<unsigned>(std::min<int64_t>((count + 255) / 256, 8192));
}

// out[b][c][r] = in[b][r][c] in bf16
template <typename TI>
static void transpose(const TI* in, int64_t R, int64_t C, int64_t ldi, bf16_t* out, int64_t ldo,
                      int batch, int64_t bsi, int64_t bso, hipStream_t st) {
  dim3 grid(static_cast<unsigned>((C + TB - 1) / TB), static_cast<unsigned>((R + TB - 1) / TB),
            static_cast<unsigned>(batch));
  const bool vec = std::is_same<TI, bf16_t>::value && R % 8 == 0 && C % 8 == 0 && ldi % 8 == 0 &&
                   ldo % 8 == 0 && bsi % 8 == 0 && bso % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(out) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(transpose16_k, grid, dim3(256), 0, st,
                       reinterpret_cast<const bf16_t*>(in), R, C, ldi, bsi, out, ldo, bso);
  else
    hipLaunchKernelGGL(transpose_k<TI>, grid, dim3(256), 0, st, in, R, C, ldi, bsi, out, ldo, bso);
}

template <typename TI>
static void slot_transpose(const TI* in, int64_t ldi, const int32_t* rowmap, const int32_t* pcol,
                           int64_t S, int64_t C, bf16_t* out, int64_t ldo, hipStream_t st) {
  dim3 grid(static_cast<unsigned>((C + TB - 1) / TB), static_cast<unsigned>((S + TB - 1) / TB));
  hipLaunchKernelGGL(slot_transpose_k<TI>, grid, dim3(256), 0, st, in, ldi, rowmap, pcol, S, C, out,
                     ldo);
}

static void zero(void* p, int64_t bytes, hipStream_t st) {
  hipLaunchKernelGGL(layer::fill_u32, dim3(grid_of(bytes / 4)), dim3(256), 0, st,
                     static_cast<uint32_t*>(p), 0u, bytes / 4);
}

// sgd_lr: when not null, the routed experts' weight gradients are not
// stored: each is applied to its weight in the GEMM epilogue (w <- w - lr * g,
// the step of moe_sgd_step), after every read of those weights.
// saved: the activations a training forward kept (else they are recomputed).
static int backward(const moe_shape_t& s, const moe_weights_t& wt, const void* xv,
                    const float* scores, const int32_t* idx, const float* w, const void* doutv,
                    const moe_grads_t& gr, const BackwardWorkspace& fws, hipStream_t st,
                    const float* sgd_lr = nullptr,
                    const layer::SavedActivations* saved = nullptr) {
  BackwardWorkspace f = fws;
  if (saved) {  // read-only from here on
    f.z = saved->z;
    f.g = saved->g;
    f.u = saved->u;
    f.h = saved->h;
    f.yp = saved->yp;
    f.gs = saved->gs;
    f.us = saved->us;
    f.hs = saved->hs;
  }
  using layer::seg;
  const int T = s.T, n = s.n_experts, k = s.top_k, d = s.d, L = s.latent, m = s.inter,
            ms = s.shared_inter;
  const int64_t S = static_cast<int64_t>(T) * k;
  const bf16_t* x = static_cast<const bf16_t*>(xv);
  const bf16_t* dout = static_cast<const bf16_t*>(doutv);
  int rc;
  auto dense = [&](const void* A, int64_t lda, const void* B, int64_t ldb, int K, int M, int N,
                   void* C, int64_t ldc, int epi) {
    gemm::Params p{};
    p.M = M;
    p.N = N;
    p.nseg = 1;
    p.seg[0] = seg(A, lda, B, ldb, K);
    p.C = C;
    p.ldc = ldc;
    return gemm::launch(p, epi, gemm::B_DENSE, true, 128, st);
  };
  // bfmt B_DENSE: B [N][K] per expert; B_DENSE_KN: B [K][N] per expert (the
  // experts' weights read transposed in place)
  auto grouped = [&](const void* A, int64_t lda, const int32_t* rows, const void* B, int64_t ldb,
                     int64_t bstride, int K, int N, float* C, int64_t ldc, int bfmt = gemm::B_DENSE,
                     const void* A2 = nullptr, const void* B2 = nullptr) {
    gemm::Params p{};
    p.N = N;
    p.nseg = A2 ? 2 : 1;
    p.seg[0] = seg(A, lda, B, ldb, K);
    if (A2) p.seg[1] = seg(A2, lda, B2, ldb, K);
    p.b_expert_stride = bstride;
    p.tiles = f.tiles;
    p.ntiles = f.ntiles;
    p.max_mtiles = f.max_mtiles;
    p.a_rows = rows;
    p.C = C;
    p.ldc = ldc;
    return gemm::launch(p, gemm::EPI_F32, bfmt, true, f.bm, st);
  };
  auto kgrouped = [&](const bf16_t* A, const bf16_t* B, int M, int N, void* C) {
    gemm::Params p{};
    p.M = M;
    p.N = N;
    p.nseg = 1;
    p.seg[0] = seg(A, f.Sp, B, f.Sp, 0);
    p.kofs = f.poffs;
    p.kgroups = n;
    p.c_group_stride = static_cast<int64_t>(M) * N;
    p.C = C;
    p.ldc = N;
    if (sgd_lr) p.sgd_lr = *sgd_lr;
    return gemm::launch(p, sgd_lr ? gemm::EPI_SGD : gemm::EPI_F32, gemm::B_DENSE, true, 0, st);
  };

  // 0. the forward's token permutation, and each expert's padded K range
  zero(f.loads, 4 * n, st);
  hipLaunchKernelGGL(count_loads, dim3(grid_of(S)), dim3(256), 0, st, idx, S, f.loads);
  hipLaunchKernelGGL(layer::scan_and_tiles, dim3(1), dim3(1024), 0, st, f.loads, n, f.bm, f.offs,
                     f.tiles, f.ntiles);
  zero(f.sel, static_cast<int64_t>(align_up(static_cast<size_t>(n) * T, 4)), st);
  hipLaunchKernelGGL(layer::scatter_sel, dim3(grid_of(S)), dim3(256), 0, st, idx, T, k, f.sel);
  hipLaunchKernelGGL(layer::expert_slots, dim3(n), dim3(256), 0, st, f.sel, T, k, f.offs, f.perm,
                     f.inv);
  hipLaunchKernelGGL(pad_offsets, dim3(1), dim3(1024), 0, st, f.loads, n, f.poffs);
  hipLaunchKernelGGL(slot_cols, dim3(n), dim3(256), 0, st, f.offs, f.poffs, f.pcol);
  MOE_LAUNCH_CHECK();

  // 1. transposed dense weights (B operands of the products through them;
  // the experts' weights are read in place as [K][N] operands)
  const bf16_t* W_down = static_cast<const bf16_t*>(wt.w_down);
  const bf16_t* W_up = static_cast<const bf16_t*>(wt.w_up);
  const bf16_t* W_g = static_cast<const bf16_t*>(wt.w_gate);
  const bf16_t* W_u = static_cast<const bf16_t*>(wt.w_uproj);
  const bf16_t* W_dn = static_cast<const bf16_t*>(wt.w_dn);
  const bf16_t* W_gs = static_cast<const bf16_t*>(wt.ws_gate);
  const bf16_t* W_us = static_cast<const bf16_t*>(wt.ws_up);
  const bf16_t* W_ds = static_cast<const bf16_t*>(wt.ws_down);
  transpose(W_up, d, L, L, f.w_upT, d, 1, 0, 0, st);          // [L][d]
  transpose(W_ds, d, ms, ms, f.w_dsT, d, 1, 0, 0, st);        // [ms][d]
  transpose(W_gs, ms, d, d, f.w_gsT, ms, 1, 0, 0, st);        // [d][ms]
  transpose(W_us, ms, d, d, f.w_usT, ms, 1, 0, 0, st);        // [d][ms]
  transpose(W_down, L, d, d, f.w_downT, L, 1, 0, 0, st);      // [d][L]
  const int64_t es = static_cast<int64_t>(m) * L;
  MOE_LAUNCH_CHECK();

  // 2. forward activations (unless the forward kept them)
  if (!saved) {
  if ((rc = dense(x, d, W_down, d, d, T, L, f.z, L, gemm::EPI_BF16)) != MOE_OK) return rc;
  if ((rc = grouped(f.z, L, f.perm, W_g, L, es, L, m, f.g, m)) != MOE_OK) return rc;
  if ((rc = grouped(f.z, L, f.perm, W_u, L, es, L, m, f.u, m)) != MOE_OK) return rc;
  hipLaunchKernelGGL(situ_fwd_k, dim3(grid_of(S * m)), dim3(256), 0, st, f.g, f.u, S * m, f.h);
  MOE_LAUNCH_CHECK();
  if ((rc = grouped(f.h, m, nullptr, W_dn, m, es, m, L, f.yp, L)) != MOE_OK) return rc;
  if ((rc = dense(x, d, W_gs, d, d, T, ms, f.gs, ms, gemm::EPI_F32)) != MOE_OK) return rc;
  if ((rc = dense(x, d, W_us, d, d, T, ms, f.us, ms, gemm::EPI_F32)) != MOE_OK) return rc;
  hipLaunchKernelGGL(situ_fwd_k, dim3(grid_of(static_cast<int64_t>(T) * ms)), dim3(256), 0, st,
                     f.gs, f.us, static_cast<int64_t>(T) * ms, f.hs);
  MOE_LAUNCH_CHECK();
  }

  // 3. up-projection and RMSNorm / combine, router
  if ((rc = dense(dout, d, f.w_upT, d, d, T, L, f.dyhat, L, gemm::EPI_F32)) != MOE_OK) return rc;
  hipLaunchKernelGGL(norm_bwd_k, dim3(T), dim3(256), 0, st, f.yp, f.inv, w, wt.rms_gamma, f.dyhat,
                     k, L, s.rms_eps, f.yhat, f.dy_slot, f.dw, f.q);
  hipLaunchKernelGGL(router_bwd_k, dim3((T + 255) / 256), dim3(256), 0, st, scores, idx, w, f.dw,
                     f.inv, T, n, k, f.dlogit, f.dlogit_slot);
  MOE_LAUNCH_CHECK();

  // 4. routed experts: dh = dy_slot W_dn, SiTU-GLU, dz_slot = dg W_g + du W_u
  if ((rc = grouped(f.dy_slot, L, nullptr, W_dn, m, es, L, m, f.dh, m, gemm::B_DENSE_KN)) != MOE_OK)
    return rc;
  hipLaunchKernelGGL(situ_bwd_k, dim3(grid_of(S * m)), dim3(256), 0, st, f.g, f.u, f.dh, S * m,
                     f.dg, f.du);
  MOE_LAUNCH_CHECK();
  if ((rc = grouped(f.dg, m, nullptr, W_g, L, es, m, L, f.dz_slot, L, gemm::B_DENSE_KN, f.du,
                    W_u)) != MOE_OK)
    return rc;
  hipLaunchKernelGGL(dz_gather_k, dim3(T), dim3(256), 0, st, f.dz_slot, f.inv, k, L, f.dz);

  // 5. shared branch and dx
  if ((rc = dense(dout, d, f.w_dsT, d, d, T, ms, f.dhs, ms, gemm::EPI_F32)) != MOE_OK) return rc;
  hipLaunchKernelGGL(situ_bwd_k, dim3(grid_of(static_cast<int64_t>(T) * ms)), dim3(256), 0, st,
                     f.gs, f.us, f.dhs, static_cast<int64_t>(T) * ms, f.dgs, f.dus);
  MOE_LAUNCH_CHECK();
  {
    gemm::Params p{};
    p.M = T;
    p.N = d;
    p.nseg = 3;
    p.seg[0] = seg(f.dgs, ms, f.w_gsT, ms, ms);
    p.seg[1] = seg(f.dus, ms, f.w_usT, ms, ms);
    p.seg[2] = seg(f.dz, L, f.w_downT, L, L);
    p.C = f.dx_acc;
    p.ldc = d;
    if ((rc = gemm::launch(p, gemm::EPI_F32, gemm::B_DENSE, true, 128, st)) != MOE_OK) return rc;
  }
  hipLaunchKernelGGL(dx_final_k<bf16_t>, dim3(T), dim3(256), 0, st, f.dx_acc, f.dlogit, idx,
                     wt.w_router, k, d, static_cast<bf16_t*>(gr.dx));
  hipLaunchKernelGGL(router_wgrad_k<bf16_t>, dim3((d + 255) / 256, n), dim3(256), 0, st, x, f.offs,
                     f.perm, f.dlogit_slot, d, gr.d_w_router, gr.d_router_logit_offset);
  const int64_t chunks = (static_cast<int64_t>(T) + 63) / 64;
  hipLaunchKernelGGL(gamma_part_k, dim3((L + 255) / 256, static_cast<unsigned>(chunks)), dim3(256),
                     0, st, f.q, static_cast<int64_t>(T), L, f.gpart);
  hipLaunchKernelGGL(gamma_grad_k, dim3((L + 255) / 256), dim3(256), 0, st, f.gpart, chunks, L,
                     gr.d_rms_gamma);
  MOE_LAUNCH_CHECK();

  // 6. dense weight gradients: [out][in] = sum over tokens (K = T, padded)
  const int64_t Tp = f.Tp;
  zero(f.xT, 2 * static_cast<int64_t>(d) * Tp, st);
  zero(f.doutT, 2 * static_cast<int64_t>(d) * Tp, st);
  zero(f.yhatT, 2 * static_cast<int64_t>(L) * Tp, st);
  zero(f.hsT, 2 * static_cast<int64_t>(ms) * Tp, st);
  zero(f.dgsT, 2 * static_cast<int64_t>(ms) * Tp, st);
  zero(f.dusT, 2 * static_cast<int64_t>(ms) * Tp, st);
  zero(f.dzT, 2 * static_cast<int64_t>(L) * Tp, st);
  transpose(x, T, d, d, f.xT, Tp, 1, 0, 0, st);
  transpose(dout, T, d, d, f.doutT, Tp, 1, 0, 0, st);
  transpose(f.yhat, T, L, L, f.yhatT, Tp, 1, 0, 0, st);
  transpose(f.hs, T, ms, ms, f.hsT, Tp, 1, 0, 0, st);
  transpose(f.dgs, T, ms, ms, f.dgsT, Tp, 1, 0, 0, st);
  transpose(f.dus, T, ms, ms, f.dusT, Tp, 1, 0, 0, st);
  transpose(f.dz, T, L, L, f.dzT, Tp, 1, 0, 0, st);
  MOE_LAUNCH_CHECK();
  const int Ki = static_cast<int>(Tp);
  if ((rc = dense(f.doutT, Tp, f.yhatT, Tp, Ki, d, L, gr.d_w_up, L, gemm::EPI_F32)) != MOE_OK)
    return rc;
  if ((rc = dense(f.doutT, Tp, f.hsT, Tp, Ki, d, ms, gr.d_ws_down, ms, gemm::EPI_F32)) != MOE_OK)
    return rc;
  if ((rc = dense(f.dgsT, Tp, f.xT, Tp, Ki, ms, d, gr.d_ws_gate, d, gemm::EPI_F32)) != MOE_OK)
    return rc;
  if ((rc = dense(f.dusT, Tp, f.xT, Tp, Ki, ms, d, gr.d_ws_up, d, gemm::EPI_F32)) != MOE_OK)
    return rc;
  if ((rc = dense(f.dzT, Tp, f.xT, Tp, Ki, L, d, gr.d_w_down, d, gemm::EPI_F32)) != MOE_OK)
    return rc;

  // 7. routed-expert weight gradients: per expert, K = its slots (padded)
  const int64_t Sp = f.Sp;
  zero(f.z_slotT, 2 * static_cast<int64_t>(L) * Sp, st);
  zero(f.hT, 2 * static_cast<int64_t>(m) * Sp, st);
  zero(f.dy_slotT, 2 * static_cast<int64_t>(L) * Sp, st);
  zero(f.dgT, 2 * static_cast<int64_t>(m) * Sp, st);
  zero(f.duT, 2 * static_cast<int64_t>(m) * Sp, st);
  slot_transpose(f.z, L, f.perm, f.pcol, S, L, f.z_slotT, Sp, st);
  slot_transpose(f.h, m, nullptr, f.pcol, S, m, f.hT, Sp, st);
  slot_transpose(f.dy_slot, L, nullptr, f.pcol, S, L, f.dy_slotT, Sp, st);
  slot_transpose(f.dg, m, nullptr, f.pcol, S, m, f.dgT, Sp, st);
  slot_transpose(f.du, m, nullptr, f.pcol, S, m, f.duT, Sp, st);
  MOE_LAUNCH_CHECK();
  void* g_dn = sgd_lr ? const_cast<void*>(wt.w_dn) : static_cast<void*>(gr.d_w_dn);
  void* g_gate = sgd_lr ? const_cast<void*>(wt.w_gate) : static_cast<void*>(gr.d_w_gate);
  void* g_up = sgd_lr ? const_cast<void*>(wt.w_uproj) : static_cast<void*>(gr.d_w_uproj);
  if ((rc = kgrouped(f.dy_slotT, f.hT, L, m, g_dn)) != MOE_OK) return rc;
  if ((rc = kgrouped(f.dgT, f.z_slotT, m, L, g_gate)) != MOE_OK) return rc;
  if ((rc = kgrouped(f.duT, f.z_slotT, m, L, g_up)) != MOE_OK) return rc;
  return MOE_OK;
}

}  // namespace bwd
}  // namespace moe

namespace moe {
namespace bwd {

// w <- round(w - round(lr * g)) elementwise (sgd_value: fp32 operations
// rounded to nearest even, no fused multiply-add), stored in the weight's
// type; eight elements per thread and iteration when the count allows.
template <typename W>
__global__ __launch_bounds__(256) void sgd_k(W* __restrict__ w, const float* __restrict__ g,
                                             int64_t count, float lr) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += stride) {
    w[i] = from_f32<W>(sgd_value(to_f32<W>(w[i]), g[i], lr));
  }
}

__global__ __launch_bounds__(256) void sgd_bf16x8_k(bf16_t* __restrict__ w,
                                                    const float* __restrict__ g, int64_t groups,
                                                    float lr) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < groups;
       i += stride) {
    uint4 wv = reinterpret_cast<const uint4*>(w)[i];
    const float4 g0 = reinterpret_cast<const float4*>(g)[2 * i];
    const float4 g1 = reinterpret_cast<const float4*>(g)[2 * i + 1];
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = sgd_value(bf16_to_f32(static_cast<bf16_t>(words[q] & 0xFFFFu)), gv[2 * q], lr);
      const float hi = sgd_value(bf16_to_f32(static_cast<bf16_t>(words[q] >> 16)), gv[2 * q + 1], lr);
      words[q] = static_cast<uint32_t>(f32_to_bf16(lo)) |
                 (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    reinterpret_cast<uint4*>(w)[i] = make_uint4(words[0], words[1], words[2], words[3]);
  }
}

template <typename W>
static void sgd(W* w, const float* g, int64_t count, float lr, hipStream_t st) {
  if (count <= 0) return;
  if constexpr (std::is_same<W, bf16_t>::value) {
    if (count % 8 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(g) % 32 == 0) {
      hipLaunchKernelGGL(sgd_bf16x8_k, dim3(grid_of(count / 8)), dim3(256), 0, st, w, g, count / 8,
                         lr);
      return;
    }
  }
  hipLaunchKernelGGL(sgd_k<W>, dim3(grid_of(count)), dim3(256), 0, st, w, g, count, lr);
}

}  // namespace bwd
}  // namespace moe

namespace moe {
namespace bwd {

// Weights and gradients present as the step needs them (experts: whether the
// routed experts' gradients are read).
static bool sgd_args_ok(const moe_weights_t& w, const moe_grads_t& g, bool experts) {
  if (!w.w_router || !w.w_down || !w.w_up || !w.w_gate || !w.w_uproj || !w.w_dn || !w.rms_gamma ||
      !w.ws_gate || !w.ws_up || !w.ws_down)
    return false;
  if (!g.d_w_router || !g.d_w_down || !g.d_w_up || !g.d_rms_gamma || !g.d_ws_gate || !g.d_ws_up ||
      !g.d_ws_down)
    return false;
  if (experts && (!g.d_w_gate || !g.d_w_uproj || !g.d_w_dn)) return false;
  return (w.router_logit_offset == nullptr) == (g.d_router_logit_offset == nullptr);
}

// Every gradient of a batch without tokens: zero.
static int zero_grads(const moe_shape_t& s, const moe_grads_t& g, hipStream_t st) {
  const int64_t n = s.n_experts, d = s.d, L = s.latent, m = s.inter, ms = s.shared_inter;
  float* outs[] = {g.d_w_router, g.d_router_logit_offset, g.d_w_down, g.d_w_up, g.d_w_gate,
                   g.d_w_uproj, g.d_w_dn, g.d_rms_gamma, g.d_ws_gate, g.d_ws_up, g.d_ws_down};
  const int64_t cnt[] = {n * d, n, L * d, d * L, n * m * L, n * m * L, n * L * m, L, ms * d, ms * d,
                         d * ms};
  for (int i = 0; i < 11; ++i)
    if (outs[i])
      hipLaunchKernelGGL(fill_f32, dim3(grid_of(cnt[i])), dim3(256), 0, st, outs[i], cnt[i]);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// The step on every weight (experts: the routed experts' weights too).
static int apply_sgd(const moe_shape_t& s, const moe_weights_t& w, const moe_grads_t& g, float lr,
                     bool experts, hipStream_t hs) {
  const int64_t n = s.n_experts, d = s.d, L = s.latent, m = s.inter, ms = s.shared_inter;
  auto f32 = [](const float* p) { return const_cast<float*>(p); };
  auto b16 = [](const void* p) { return static_cast<bf16_t*>(const_cast<void*>(p)); };
  sgd(f32(w.w_router), g.d_w_router, n * d, lr, hs);
  if (w.router_logit_offset) sgd(f32(w.router_logit_offset), g.d_router_logit_offset, n, lr, hs);
  sgd(b16(w.w_down), g.d_w_down, L * d, lr, hs);
  sgd(b16(w.w_up), g.d_w_up, d * L, lr, hs);
  if (experts) {
    sgd(b16(w.w_gate), g.d_w_gate, n * m * L, lr, hs);
    sgd(b16(w.w_uproj), g.d_w_uproj, n * m * L, lr, hs);
    sgd(b16(w.w_dn), g.d_w_dn, n * L * m, lr, hs);
  }
  sgd(f32(w.rms_gamma), g.d_rms_gamma, L, lr, hs);
  sgd(b16(w.ws_gate), g.d_ws_gate, ms * d, lr, hs);
  sgd(b16(w.ws_up), g.d_ws_up, ms * d, lr, hs);
  sgd(b16(w.ws_down), g.d_ws_down, d * ms, lr, hs);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace bwd
}  // namespace moe

extern "C" int moe_sgd_step(const moe_shape_t* shape, const moe_weights_t* weights,
                            const moe_grads_t* grads, float lr, void* stream) {
  int st = moe::bwd::validate(shape);
  if (st != MOE_OK) return st;
  if (!weights || !grads || !std::isfinite(lr)) return MOE_EINVAL;
  if (!moe::bwd::sgd_args_ok(*weights, *grads, true)) return MOE_EINVAL;
  return moe::bwd::apply_sgd(*shape, *weights, *grads, lr, true, static_cast<hipStream_t>(stream));
}

extern "C" size_t moe_backward_workspace_bytes(const moe_shape_t* shape) {
  if (moe::bwd::validate(shape) != MOE_OK) return 0;
  return moe::bwd::backward_layout(*shape, nullptr, nullptr);
}

extern "C" int moe_latent_backward(const moe_shape_t* shape, const moe_weights_t* weights,
                                   const void* x, const float* scores, const int32_t* topk_idx,
                                   const float* topk_w, const void* dout, const moe_grads_t* grads,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = moe::bwd::validate(shape);
  if (st != MOE_OK) return st;
  if (!weights || !grads || !workspace) return MOE_EINVAL;
  const moe_weights_t& w = *weights;
  const moe_grads_t& g = *grads;
  if (!w.w_router || !w.w_down || !w.w_up || !w.w_gate || !w.w_uproj || !w.w_dn || !w.rms_gamma ||
      !w.ws_gate || !w.ws_up || !w.ws_down)
    return MOE_EINVAL;
  if (!g.d_w_router || !g.d_w_down || !g.d_w_up || !g.d_w_gate || !g.d_w_uproj || !g.d_w_dn ||
      !g.d_rms_gamma || !g.d_ws_gate || !g.d_ws_up || !g.d_ws_down)
    return MOE_EINVAL;
  if ((w.router_logit_offset == nullptr) != (g.d_router_logit_offset == nullptr)) return MOE_EINVAL;
  if (shape->T > 0 && (!x || !scores || !topk_idx || !topk_w || !dout || !g.dx)) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MOE_EINVAL;
  moe::bwd::BackwardWorkspace f;
  const size_t need = moe::bwd::backward_layout(*shape, &f, workspace);
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape->T == 0) return moe::bwd::zero_grads(*shape, g, s);  // no tokens: zero gradients
  return moe::bwd::backward(*shape, w, x, scores, topk_idx, topk_w, dout, g, f, s);
}

extern "C" int moe_latent_backward_train(const moe_shape_t* shape, const moe_weights_t* weights,
                                         const void* x, const float* scores,
                                         const int32_t* topk_idx, const float* topk_w,
                                         const void* dout, const void* saved, size_t saved_bytes,
                                         const moe_grads_t* grads, int apply_sgd, float lr,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  int st = moe::bwd::validate(shape);
  if (st != MOE_OK) return st;
  if (!weights || !grads || !workspace || !saved) return MOE_EINVAL;
  if (apply_sgd != 0 && apply_sgd != 1) return MOE_EINVAL;
  if (apply_sgd && !std::isfinite(lr)) return MOE_EINVAL;
  const moe_weights_t& w = *weights;
  const moe_grads_t& g = *grads;
  if (!moe::bwd::sgd_args_ok(w, g, !apply_sgd)) return MOE_EINVAL;
  if (shape->T > 0 && (!x || !scores || !topk_idx || !topk_w || !dout || !g.dx)) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      reinterpret_cast<uintptr_t>(saved) % 256 != 0)
    return MOE_EINVAL;
  moe::bwd::BackwardWorkspace f;
  const size_t need = moe::bwd::backward_layout(*shape, &f, workspace);
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  moe::layer::SavedActivations sv;
  if (saved_bytes < moe::layer::saved_layout(*shape, &sv, const_cast<void*>(saved)))
    return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape->T == 0) return apply_sgd ? MOE_OK : moe::bwd::zero_grads(*shape, g, s);
  if (!apply_sgd) return moe::bwd::backward(*shape, w, x, scores, topk_idx, topk_w, dout, g, f, s,
                                            nullptr, &sv);
  moe_grads_t gx = g;  // the experts' gradients are applied where they are formed
  gx.d_w_gate = gx.d_w_uproj = gx.d_w_dn = nullptr;
  st = moe::bwd::backward(*shape, w, x, scores, topk_idx, topk_w, dout, gx, f, s, &lr, &sv);
  if (st != MOE_OK) return st;
  return moe::bwd::apply_sgd(*shape, w, gx, lr, false, s);
}

extern "C" int moe_latent_backward_sgd(const moe_shape_t* shape, const moe_weights_t* weights,
                                       const void* x, const float* scores,
                                       const int32_t* topk_idx, const float* topk_w,
                                       const void* dout, const moe_grads_t* grads, float lr,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = moe::bwd::validate(shape);
  if (st != MOE_OK) return st;
  if (!weights || !grads || !workspace || !std::isfinite(lr)) return MOE_EINVAL;
  const moe_weights_t& w = *weights;
  const moe_grads_t& g = *grads;
  if (!moe::bwd::sgd_args_ok(w, g, false)) return MOE_EINVAL;
  if (shape->T > 0 && (!x || !scores || !topk_idx || !topk_w || !dout || !g.dx)) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MOE_EINVAL;
  moe::bwd::BackwardWorkspace f;
  const size_t need = moe::bwd::backward_layout(*shape, &f, workspace);
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape->T == 0) return MOE_OK;  // no tokens: zero gradients, nothing moves
  // the experts' gradient pointers are not used: their updates happen in place
  moe_grads_t gx = g;
  gx.d_w_gate = gx.d_w_uproj = gx.d_w_dn = nullptr;
  st = moe::bwd::backward(*shape, w, x, scores, topk_idx, topk_w, dout, gx, f, s, &lr);
  if (st != MOE_OK) return st;
  return moe::bwd::apply_sgd(*shape, w, gx, lr, false, s);
}

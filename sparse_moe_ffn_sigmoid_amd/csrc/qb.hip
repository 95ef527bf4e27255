// Quantile Balancing routing on gfx950.
//
// Routing rule (xhh.club "Kimi K3 模型结构（5）：宽度维度，Stable LatentMoE",
// Q&A on routing): top-k of the biased sigmoid scores, mixture weights = the
// chosen raw scores renormalised.  Balancing rule (same page, Q&A on
// Quantile Balancing and 延伸解读 "Quantile Balancing与DeepSeek-V3路由的异同"):
// each unbalanced expert's bias jumps to minus the (1 - C_e/T) quantile of
// its margin -- the exact coordinate minimiser of the dual of the balanced
// assignment problem -- and a common offset is removed at the end.
//
// Arithmetic is exact: scores and biases live on a 2^-40 fixed-point grid in
// int64 and every comparison uses the packed key
//     ((sfx + bias + 2^51) << 10) | (1023 - e),
// so "higher biased score first, ties to the lower expert index".
//
// Coordinate rounds alone stall with a few experts off by one (the dual is
// piecewise linear), so once the count of unbalanced experts stops reaching
// new minima the balance is completed by shortest augmenting paths on the
// same dual: Bellman-Ford over experts on a sparse edge list holding every
// (token, chosen A, unchosen B) whose reduced cost is at most Delta; the
// distances up to D* are exact whenever D* <= Delta, otherwise Delta grows.
//
// Control flow lives on the device: a step is [top-k pass, status, quantile
// round] and every kernel reads the phase word first, so the host only
// launches batches of steps and polls the phase.  A quantile round becomes
// live in the next step: the top-k pass reads its biases from the idle
// buffer, the status pass commits it; an augmenting-path move is made by the
// status pass itself.
#include "prof.hpp"
#include "route.hpp"

namespace moe {
namespace qb {

constexpr int FRAC_BITS = 40;
constexpr int IDX_BITS = 10;
constexpr int64_t KEY_OFFSET = int64_t(1) << 51;
constexpr int64_t BIAS_LIMIT = int64_t(1) << 50;
constexpr int64_t DIST_INF = int64_t(1) << 52;
constexpr uint64_t PACKED_INF = uint64_t(DIST_INF) << IDX_BITS;
constexpr int MAX_NJ = 16;            // keys per lane: n <= 1024
constexpr int TOPK_BLOCK = 256;       // 4 waves, one token per wave at a time
constexpr int MAX_K = 64;
constexpr int STALL_ROUNDS = 3;
constexpr int MAX_SAP_MOVES = 4096;
constexpr int EDGE_LIST_MAX = 64;     // per token: low chosen / high unchosen candidates
constexpr int64_t DELTA_START = int64_t(1) << 30;
constexpr int64_t DELTA_MAX = int64_t(1) << 44;
constexpr int64_t DELTA_MIN = int64_t(1) << 16;
// The top-k pass adds its per-block loads into one of ACC_COPIES copies of
// the load counters (chosen by block index), so that the device-wide atomics
// on one counter do not serialise across every block; the status pass sums
// the copies.
constexpr int ACC_COPIES = 32;
constexpr int TOPK_MAX_GRID = 768;    // top-k blocks: three resident per CU; waves loop over tokens

enum Phase : int64_t { PH_ROUNDS = 0, PH_SAP = 1, PH_DONE = 2, PH_FAILED = 3, PH_FROZEN = 4 };
enum Ctrl {
  C_PHASE = 0, C_ROUNDS, C_BEST, C_SINCE, C_MOVES, C_IMB, C_RESID, C_STATUS, C_DELTA,
  C_EDGES_VALID, C_CUR, C_ROUND, C_MAX_ROUNDS, C_LAST_D, C_LAST_HOPS, C_BF_PASSES,
  C_PIVOT,  // th[].k1 holds every token's (k+1)-th key of the last top-k pass
  C_DROP,   // largest bias decrease (grid units) since that pass
  C_COUNT = 32
};
// The edge list is split into EDGE_SEGS segments with one counter each
// (chosen by block index), for the same reason as the load counters.
constexpr int EDGE_SEGS = 256;
enum Cnt { N_OVERFLOW = 1, N_BIASRANGE = 2, N_SEG0 = 8, N_COUNT = N_SEG0 + EDGE_SEGS };

__host__ __device__ __forceinline__ int64_t target(int64_t T, int64_t n, int64_t k, int64_t e) {
  return (T * k) / n + (e < (T * k) % n ? 1 : 0);
}

// rint(s * 2^40) for a score s in [0, 1] with integer operations only:
// s = m * 2^(E-150) with m the 24-bit significand, so s * 2^40 = m * 2^(E-110);
// a right shift rounds half to even.  Zero and subnormals give 0.
__device__ __forceinline__ int64_t score_fixed(float s) {
  const uint32_t u = __float_as_uint(s);
  const int E = static_cast<int>((u >> 23) & 255u);
  const uint32_t m = (u & 0x7FFFFFu) | 0x800000u;
  const int sh = E - 110;
  if (sh >= 0) return static_cast<int64_t>(static_cast<uint64_t>(m) << sh);  // s >= 2^-17: exact
  if (E == 0) return 0;
  const int r = -sh;
  if (r > 24) return 0;  // m < 2^24 <= 2^(r-1): below one half
  const uint32_t q = m >> r;                       // r <= 24: 32-bit arithmetic suffices
  const uint32_t rem = m & ((1u << r) - 1u);
  const uint32_t half = 1u << (r - 1);
  return static_cast<int64_t>(q + ((rem > half) || (rem == half && (q & 1u))));
}

__device__ __forceinline__ uint64_t pack_key(int64_t sfx, int64_t b, int e) {
  return (static_cast<uint64_t>(sfx + b + KEY_OFFSET) << IDX_BITS) |
         static_cast<uint64_t>(1023 - e);
}

// floor((a + b) / 2^11) without overflowing int64.
__device__ __forceinline__ int64_t floor_mid(int64_t a, int64_t b) {
  return (a >> 11) + (b >> 11) + (((a & 2047) + (b & 2047)) >> 11);
}

// Wave-wide maximum with DPP row operations fused into v_max_u32 (quad
// swaps, row shifts, row broadcasts; lanes without a source read 0, neutral
// for an unsigned max); lane 63 ends with the maximum, broadcast through a
// scalar register.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t w =
      static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
  return v > w ? v : w;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x114>(v);  // row_shr:4
  v = dpp_max_step<0x118>(v);  // row_shr:8
  v = dpp_max_step<0x142>(v);  // row_bcast:15
  v = dpp_max_step<0x143>(v);  // row_bcast:31
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// 64-bit maximum: the high words first, then the low words of the lanes that
// hold the highest high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32), lo = static_cast<uint32_t>(v);
  const uint32_t H = wave_max_u32(hi);
  const uint32_t L = wave_max_u32(hi == H ? lo : 0u);
  return (static_cast<uint64_t>(H) << 32) | L;
}

struct Args {
  const float* scores;   // [T][n]
  const float* scoresT;  // [n][T]
  int T, n, k;
  int64_t* bfx;          // [2][n] biases, ctrl[C_CUR] selects the live half
  KeyPair* th;           // [T]
  int32_t* loads;        // [n]
  int32_t* acc;          // [ACC_COPIES][n] loads accumulated by the top-k pass
  int64_t* ctrl;         // [C_COUNT]
  int32_t* cnt;          // [N_COUNT]
  uint64_t* edges;       // [EDGE_SEGS][edge_cap / EDGE_SEGS]
  int32_t edge_cap;
  int32_t* idx;          // [T][k] or null
  float* w;              // [T][k] or null
};

// ---------------------------------------------------------------------------
// Top-k pass: one wave per token.  Finds the k-th and (k+1)-th keys by k+1
// rounds of wave-wide max extraction, counts loads per block, and (by flag)
// writes the ordered outputs or the sparse edges of the augmenting-path phase.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(TOPK_BLOCK) void topk_pass(Args a, int emit_out) {
  const int64_t phase = a.ctrl[C_PHASE];
  if (phase == PH_DONE || phase == PH_FAILED) {
    if (!emit_out) return;
  }
  const bool emit_edges = (phase == PH_SAP) && !emit_out;
  extern __shared__ unsigned char smem_raw[];
  int32_t* sload = reinterpret_cast<int32_t*>(smem_raw);                 // [1024]
  int64_t* lowKp = reinterpret_cast<int64_t*>(sload + 1024);             // [4][64]
  int64_t* highKp = lowKp + 4 * EDGE_LIST_MAX;                           // [4][64]
  int32_t* lowE = reinterpret_cast<int32_t*>(highKp + 4 * EDGE_LIST_MAX);  // [4][64]
  int32_t* highE = lowE + 4 * EDGE_LIST_MAX;                             // [4][64]
  int32_t* nList = highE + 4 * EDGE_LIST_MAX;                            // [4][2]
  int64_t* oSfx = reinterpret_cast<int64_t*>(nList + 8);                 // [4][64]
  float* oS = reinterpret_cast<float*>(oSfx + 4 * MAX_K);                // [4][64]
  int32_t* oE = reinterpret_cast<int32_t*>(oS + 4 * MAX_K);              // [4][64]
  float* oSorted = reinterpret_cast<float*>(oE + 4 * MAX_K);             // [4][64]

  uint64_t* cand = reinterpret_cast<uint64_t*>(oSorted + 4 * MAX_K);      // [4][64]
  uint64_t* thv = cand + 4 * 64;                                         // [4][2]
  int64_t* sbias = reinterpret_cast<int64_t*>(thv + 4 * 2);              // [1024]

  const int n = a.n, k = a.k, T = a.T;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nj = (n + 63) >> 6;
  // this wave's tokens: t_first, t_first + 4 * gridDim.x, ...; each token's
  // scores are requested while the previous token is ranked
  const int t_first = blockIdx.x * 4 + wv;
  float sv[MAX_NJ];
  auto load_scores = [&](int t) {
    const float* row = a.scores + static_cast<size_t>(t) * n;
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j) {
      const int e = lane + 64 * j;
      sv[j] = (j < nj && e < n) ? row[e] : 0.f;
    }
  };
  if (t_first < T) load_scores(t_first);  // in flight during the bias staging
  // A quantile round of the previous step is committed by the status pass
  // that follows this one; until then its biases (in the idle buffer) are
  // the live ones, and the largest bias decrease is taken here.
  const bool pending = a.ctrl[C_PHASE] == PH_ROUNDS && a.ctrl[C_ROUND] != 0;
  const int cur = static_cast<int>(a.ctrl[C_CUR] & 1) ^ (pending ? 1 : 0);
  const int64_t* gbias = a.bfx + cur * n;
  const int64_t* obias = a.bfx + (cur ^ 1) * n;
  uint64_t dmax = 0;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    sload[e] = 0;
    const int64_t b = gbias[e];
    sbias[e] = b;
    if (pending) {
      const int64_t dec = obias[e] - b;
      dmax = dec > static_cast<int64_t>(dmax) ? static_cast<uint64_t>(dec) : dmax;
    }
  }
  __shared__ uint64_t s_dmax[TOPK_BLOCK / 64];
  if (pending) {
    const uint64_t m = wave_max_u64(dmax);
    if (lane == 0) s_dmax[wv] = m;
  }
  __syncthreads();
  // Pivot: every key of the last pass's top k+1 has dropped by at most
  // `drop`, so at least k+1 keys are >= th.k1 - drop; when at most 64 are,
  // the k-th and (k+1)-th keys are found by ranking those candidates.
  const bool use_pivot = a.ctrl[C_PIVOT] != 0 && k < n;
  uint64_t drop = static_cast<uint64_t>(a.ctrl[C_DROP]);
  if (pending) {
    drop = 0;
    for (int i = 0; i < TOPK_BLOCK / 64; ++i) drop = s_dmax[i] > drop ? s_dmax[i] : drop;
  }
  const uint64_t drop_key = drop << IDX_BITS;

  const int64_t* bias = sbias;
  const int64_t delta = a.ctrl[C_DELTA];
  const int seg = blockIdx.x & (EDGE_SEGS - 1);
  const int seg_cap = a.edge_cap / EDGE_SEGS;
  const int rounds = (k < n) ? k + 1 : k;

  const int stride = gridDim.x * 4;
  for (int t = t_first; t < T; t += stride) {
    const float* row = a.scores + static_cast<size_t>(t) * n;
    // the pivot is requested before the next token's scores, so waiting for
    // it leaves that prefetch in flight
    const uint64_t prev = use_pivot ? static_cast<uint64_t>(a.th[t].k1) : 0;
    uint64_t key[MAX_NJ];
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j) {
      const int e = lane + 64 * j;
      key[j] = 0;
      if (j < nj && e < n) key[j] = pack_key(score_fixed(sv[j]), bias[e], e);
    }
    if (t + stride < T) load_scores(t + stride);
    uint64_t thk = 0, thk1 = 0;
    bool found = false;
    // Exact k-th and (k+1)-th keys from a pivot P with k+1 <= #{keys >= P}
    // <= 64: the keys >= P are compacted into LDS and ranked.
    auto try_pivot = [&](uint64_t P) -> bool {
      int c = 0;
#pragma unroll
      for (int j = 0; j < MAX_NJ; ++j) c += __popcll(__ballot(key[j] >= P));
      if (c < k + 1 || c > 64) return false;
      int base = 0;
#pragma unroll
      for (int j = 0; j < MAX_NJ; ++j) {
        const bool in = key[j] >= P;
        const uint64_t bal = __ballot(in);
        if (in) cand[wv * 64 + base + __popcll(bal & ((uint64_t(1) << lane) - 1))] = key[j];
        base += __popcll(bal);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (lane < c) {
        const uint64_t v = cand[wv * 64 + lane];
        const uint64_t* cw = cand + wv * 64;
        int rank = 0, i = 0;
        for (; i + 8 <= c; i += 8) {
#pragma unroll
          for (int q = 0; q < 8; ++q) rank += cw[i + q] > v;
        }
        for (; i < c; ++i) rank += cw[i] > v;
        if (rank == k - 1) thv[wv * 2] = v;
        if (rank == k) thv[wv * 2 + 1] = v;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      thk = thv[wv * 2];
      thk1 = thv[wv * 2 + 1];
      __builtin_amdgcn_wave_barrier();
      return true;
    };
    if (use_pivot) found = try_pivot(prev > drop_key ? prev - drop_key : 1);
    if (!found && k < n && k + 1 <= 64) {
      // Second pivot: the (k+1)-th largest of the 64 lane maxima.  At least
      // k+1 keys (those maxima) are >= it; usually few more are.
      uint64_t lm = key[0];
#pragma unroll
      for (int j = 1; j < MAX_NJ; ++j) lm = key[j] > lm ? key[j] : lm;
      if (lane == 0) thv[wv * 2] = 1;  // lanes without keys tie at 0: P = 1 then
      cand[wv * 64 + lane] = lm;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      int r = 0;
      const uint64_t* cw = cand + wv * 64;
#pragma unroll 8
      for (int q = 0; q < 64; ++q) r += cw[q] > lm;
      __builtin_amdgcn_wave_barrier();
      if (r == k && lm != 0) thv[wv * 2] = lm;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      const uint64_t P = thv[wv * 2];
      __builtin_amdgcn_wave_barrier();
      found = try_pivot(P);
    }
    if (!found) {
      // k+1 rounds of wave-wide maximum: each lane offers its largest
      // remaining key, the winner (keys are distinct) removes it; removed
      // keys are rebuilt afterwards.
      uint32_t removed = 0;
      for (int r = 0; r < rounds; ++r) {
        uint64_t lm = key[0];
#pragma unroll
        for (int j = 1; j < MAX_NJ; ++j) lm = key[j] > lm ? key[j] : lm;
        const uint64_t wm = wave_max_u64(lm);
        if (lm == wm) {
#pragma unroll
          for (int j = 0; j < MAX_NJ; ++j)
            if (key[j] == wm) {
              key[j] = 0;
              removed |= 1u << j;
            }
        }
        if (r == k - 1) thk = wm;
        if (r == k) thk1 = wm;
      }
#pragma unroll
      for (int j = 0; j < MAX_NJ; ++j)
        if ((removed >> j) & 1u) {
          const int e = lane + 64 * j;
          key[j] = pack_key(score_fixed(row[e]), bias[e], e);
        }
    }
    if (lane == 0) a.th[t] = KeyPair{static_cast<int64_t>(thk), static_cast<int64_t>(thk1)};
    uint32_t selmask = 0;
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j)
      if (key[j] != 0 && key[j] >= thk) {
        selmask |= 1u << j;
        atomicAdd(&sload[lane + 64 * j], 1);
      }

    if (emit_out) {
      // gather the k chosen (sfx, s, e) into this wave's LDS slots
      int base = 0;
#pragma unroll
      for (int j = 0; j < MAX_NJ; ++j) {
        const bool sel = (selmask >> j) & 1u;
        const uint64_t bal = __ballot(sel);
        if (sel) {
          const int pos = base + __popcll(bal & ((uint64_t(1) << lane) - 1));
          const int e = lane + 64 * j;
          const float sval = row[e];
          oSfx[wv * MAX_K + pos] = score_fixed(sval);
          oS[wv * MAX_K + pos] = sval;
          oE[wv * MAX_K + pos] = e;
        }
        base += __popcll(bal);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      int rank = 0;
      int64_t my_sfx = 0;
      int my_e = 0;
      float my_s = 0.f;
      if (lane < k) {
        my_sfx = oSfx[wv * MAX_K + lane];
        my_e = oE[wv * MAX_K + lane];
        my_s = oS[wv * MAX_K + lane];
        for (int i = 0; i < k; ++i) {
          const int64_t si = oSfx[wv * MAX_K + i];
          const int ei = oE[wv * MAX_K + i];
          rank += (si > my_sfx) || (si == my_sfx && ei < my_e);
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (lane < k) oSorted[wv * MAX_K + rank] = my_s;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (lane < k) {
        float sum = 0.f;
        for (int i = 0; i < k; ++i) sum += oSorted[wv * MAX_K + i];
        a.idx[static_cast<size_t>(t) * k + rank] = my_e;
        a.w[static_cast<size_t>(t) * k + rank] = my_s / sum;
      }
      __builtin_amdgcn_wave_barrier();
    }

    if (emit_edges) {
      // reduced cost rho_t(A,B) = Kp_A - Kp_B - [A > B] with Kp = sfx + bias
      const int64_t kpk = static_cast<int64_t>(thk >> IDX_BITS) - KEY_OFFSET;
      const int64_t kpk1 = (k < n) ? static_cast<int64_t>(thk1 >> IDX_BITS) - KEY_OFFSET : 0;
      if (k < n && kpk - kpk1 <= delta + 1) {
        int nlow = 0, nhigh = 0;
#pragma unroll
        for (int j = 0; j < MAX_NJ; ++j) {
          const int e = lane + 64 * j;
          const bool valid = key[j] != 0;
          const int64_t kp = static_cast<int64_t>(key[j] >> IDX_BITS) - KEY_OFFSET;  // sfx + bias
          const bool sel = (selmask >> j) & 1u;
          const bool isLow = valid && sel && (kp - kpk <= delta + 1);
          const bool isHigh = valid && !sel && (kpk1 - kp <= delta + 1);
          const uint64_t bl = __ballot(isLow);
          const uint64_t bh = __ballot(isHigh);
          if (isLow) {
            const int pos = nlow + __popcll(bl & ((uint64_t(1) << lane) - 1));
            if (pos < EDGE_LIST_MAX) {
              lowKp[wv * EDGE_LIST_MAX + pos] = kp;
              lowE[wv * EDGE_LIST_MAX + pos] = e;
            }
          }
          if (isHigh) {
            const int pos = nhigh + __popcll(bh & ((uint64_t(1) << lane) - 1));
            if (pos < EDGE_LIST_MAX) {
              highKp[wv * EDGE_LIST_MAX + pos] = kp;
              highE[wv * EDGE_LIST_MAX + pos] = e;
            }
          }
          nlow += __popcll(bl);
          nhigh += __popcll(bh);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        if (nlow > EDGE_LIST_MAX || nhigh > EDGE_LIST_MAX) {
          if (lane == 0) atomicOr(&a.cnt[N_OVERFLOW], 1);
        } else {
          // the token's edges: lane ia pairs low candidate ia with every
          // high one (broadcast LDS reads); counted first, then one atomic
          // reserves them all
          const bool has = lane < nlow;
          const int A = has ? lowE[wv * EDGE_LIST_MAX + lane] : 0;
          const int64_t kA = has ? lowKp[wv * EDGE_LIST_MAX + lane] : 0;
          int mine = 0;
          for (int ib = 0; ib < nhigh; ++ib) {
            const int B = highE[wv * EDGE_LIST_MAX + ib];
            mine += has && kA - highKp[wv * EDGE_LIST_MAX + ib] - (A > B ? 1 : 0) <= delta;
          }
          int incl = mine;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(incl, off);
            if (lane >= off) incl += u;
          }
          const int total = __shfl(incl, 63);
          if (total > 0) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&a.cnt[N_SEG0 + seg], total);
            base = __shfl(base, 0);
            int pos = base + incl - mine;
            bool over = false;
            for (int ib = 0; ib < nhigh; ++ib) {
              const int B = highE[wv * EDGE_LIST_MAX + ib];
              const int64_t rho = kA - highKp[wv * EDGE_LIST_MAX + ib] - (A > B ? 1 : 0);
              if (has && rho <= delta) {
                if (pos < seg_cap)
                  a.edges[static_cast<size_t>(seg) * seg_cap + pos] =
                      (static_cast<uint64_t>(rho) << 20) | (static_cast<uint64_t>(A) << 10) |
                      static_cast<uint64_t>(B);
                else
                  over = true;
                ++pos;
              }
            }
            if (__ballot(over) != 0 && lane == 0) atomicOr(&a.cnt[N_OVERFLOW], 1);
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  // per-block counts, one global atomic per expert the block selected
  __syncthreads();
  int32_t* acc = a.acc + (blockIdx.x & (ACC_COPIES - 1)) * n;
  for (int e = threadIdx.x; e < n; e += blockDim.x)
    if (sload[e]) atomicAdd(&acc[e], sload[e]);
  if (emit_edges && blockIdx.x == 0 && threadIdx.x == 0) a.ctrl[C_EDGES_VALID] = 1;
}

// ---------------------------------------------------------------------------
// One augmenting-path move (all 1024 threads of the status block): shortest
// distances from the overloaded experts over this step's sparse edge list,
// then every expert drops by D - min(d, D) and the path to the nearest
// underloaded expert is shifted by one grid unit per hop.
// ---------------------------------------------------------------------------
__device__ void sap_move(const Args& a, int edge_cache) {
  int64_t* c = a.ctrl;
  const int n = a.n;
  const int tid = threadIdx.x;
  __shared__ uint64_t d[1024];
  __shared__ int64_t s_red[1024];
  __shared__ int s_flag[3];  // rotating 'lowered a distance <= D' flags, one per pass
  __shared__ int16_t s_path[1032];
  __shared__ int s_len;
  // edge cache: the status kernel's dynamic LDS (edge_cache entries, 0 = none)
  extern __shared__ uint64_t s_edges[];
  __shared__ int s_seg_off[EDGE_SEGS + 1];


  const int cur = static_cast<int>(c[C_CUR] & 1);
  int64_t* bias = a.bfx + cur * n;
  const int64_t delta = c[C_DELTA];
  const int seg_cap = a.edge_cap / EDGE_SEGS;
  {  // segment offsets: exclusive scan of the (capped) segment counts
    static_assert(EDGE_SEGS == 256, "scan below: four waves of 64");
    __shared__ int s_wsum[4];
    const int lane = tid & 63, wid = tid >> 6;
    int m = 0;
    if (tid < EDGE_SEGS) {
      m = a.cnt[N_SEG0 + tid];
      m = m < seg_cap ? m : seg_cap;
    }
    int incl = m;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off);
      if (lane >= off) incl += u;
    }
    if (tid < EDGE_SEGS && lane == 63) s_wsum[wid] = incl;
    __syncthreads();
    if (tid < EDGE_SEGS) {
      int before = 0;
      for (int w = 0; w < wid; ++w) before += s_wsum[w];
      s_seg_off[tid] = before + incl - m;
      if (tid == EDGE_SEGS - 1) s_seg_off[EDGE_SEGS] = before + incl;
    }
  }
  const bool overflow = a.cnt[N_OVERFLOW] != 0;
  __syncthreads();
  // segment of edge i (0 <= i < nedges): the last sg with s_seg_off[sg] <= i
  auto seg_of = [&](int i) {
    int lo = 0, hi = EDGE_SEGS - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_seg_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  const int nedges = s_seg_off[EDGE_SEGS];
  // every segment counter is cleared by the end of the move
  auto clear_edges = [&]() {
    if (tid < EDGE_SEGS) a.cnt[N_SEG0 + tid] = 0;
    if (tid == 0) c[C_EDGES_VALID] = 0;
  };
  if (overflow) {
    if (tid == 0) {
      if (delta / 4 < DELTA_MIN) {
        c[C_PHASE] = PH_FAILED;
        c[C_STATUS] = MOE_QB_STATUS_NOT_BALANCED;
      } else {
        c[C_DELTA] = delta / 4;
      }
      a.cnt[N_OVERFLOW] = 0;
    }
    clear_edges();
    return;
  }
  // sources: overloaded experts at distance 0
  __shared__ uint8_t s_over[1024], s_under[1024];
  __shared__ int16_t s_pos[1024];
  __shared__ int s_bad;
  bool under_e = false;
  if (tid < n) {
    const int64_t C = target(a.T, n, a.k, tid);
    const int32_t L = a.loads[tid];
    s_over[tid] = L > C;
    under_e = L < C;
    s_under[tid] = under_e;
    s_pos[tid] = 0;
    d[tid] = L > C ? static_cast<uint64_t>(tid) : PACKED_INF;
  }
  const bool cached = nedges <= edge_cache;
  if (cached)
    for (int i = tid; i < nedges; i += blockDim.x) {
      const int sg = seg_of(i);
      s_edges[i] = a.edges[static_cast<size_t>(sg) * seg_cap + (i - s_seg_off[sg])];
    }
  // Relaxation passes.  s_D is the running minimum distance of an
  // underloaded expert (it only decreases); a pass that lowers some distance
  // to at most s_D asks for another pass.  Flagging against the running value
  // flags a superset of "changed at or below the final D*", so the passes
  // stop only when every distance <= D* and its predecessor is final.
  __shared__ unsigned long long s_D;
  if (tid == 0) {
    s_D = static_cast<unsigned long long>(DIST_INF);
    s_bad = 0;
  }
  __syncthreads();
  if (tid < n && under_e && static_cast<int64_t>(d[tid] >> IDX_BITS) < DIST_INF)
    atomicMin(&s_D, static_cast<unsigned long long>(d[tid] >> IDX_BITS));
  // One barrier per pass: pass p raises s_flag[p % 3]; thread 0 clears the
  // flag of pass p + 1 during pass p (its last readers finished before the
  // barrier that ended pass p - 1).
  if (tid < 3) s_flag[tid] = 0;
  __syncthreads();
  int passes = 0;
  while (true) {
    const int fi = passes % 3;
    if (tid == 0) s_flag[(passes + 1) % 3] = 0;
    for (int i = tid; i < nedges; i += blockDim.x) {
      uint64_t ed;
      if (cached) {
        ed = s_edges[i];
      } else {
        const int sg = seg_of(i);
        ed = a.edges[static_cast<size_t>(sg) * seg_cap + (i - s_seg_off[sg])];
      }
      const int B = static_cast<int>(ed & 1023);
      const int A = static_cast<int>((ed >> 10) & 1023);
      const int64_t rho = static_cast<int64_t>(ed >> 20);
      const int64_t dA = static_cast<int64_t>(d[A] >> IDX_BITS);
      if (dA >= DIST_INF) continue;
      const int64_t cand = dA + rho;
      if (cand >= DIST_INF) continue;
      const uint64_t pk = (static_cast<uint64_t>(cand) << IDX_BITS) | static_cast<uint64_t>(A);
      if (pk < d[B]) {
        const uint64_t old = atomicMin(reinterpret_cast<unsigned long long*>(&d[B]), pk);
        if (pk < old) {
          if (s_under[B]) atomicMin(&s_D, static_cast<unsigned long long>(cand));
          if (static_cast<uint64_t>(cand) <= s_D) s_flag[fi] = 1;
        }
      }
    }
    __syncthreads();
    ++passes;
    if (!s_flag[fi] || passes > 4 * 1024) break;
  }
  const int64_t D = static_cast<int64_t>(s_D);
  if (D >= DIST_INF || D > delta) {
    if (tid == 0) {
      if (delta >= DELTA_MAX) {
        c[C_PHASE] = PH_FAILED;
        c[C_STATUS] = MOE_QB_STATUS_NOT_BALANCED;
      } else {
        c[C_DELTA] = delta * 16;
      }
    }
    clear_edges();
    return;
  }
  // u* = lowest underloaded expert at distance D
  {
    int u = (tid < n && under_e && static_cast<int64_t>(d[tid] >> IDX_BITS) == D) ? tid : 1 << 30;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) u = min(u, __shfl_xor(u, off));
    if ((tid & 63) == 0) s_red[tid >> 6] = u;
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) u = min(u, static_cast<int>(s_red[w]));
      s_red[0] = u;
    }
    __syncthreads();
  }
  // the path from u* back to its source (an overloaded expert), in LDS
  if (tid == 0) {
    int v = static_cast<int>(s_red[0]);
    int len = 0;
    bool ok = true;
    while (true) {
      s_path[len++] = static_cast<int16_t>(v);
      if (s_over[v]) break;
      v = static_cast<int>(d[v] & 1023);
      if (len > n) {
        ok = false;
        break;
      }
    }
    s_len = ok ? len : -1;
  }
  __syncthreads();
  const int len = s_len;
  if (len < 0) {
    if (tid == 0) {
      c[C_PHASE] = PH_FAILED;
      c[C_STATUS] = MOE_QB_STATUS_NOT_BALANCED;
    }
    clear_edges();
    return;
  }
  // the i-th expert from the source gains i grid units (s_path[len-1] is the
  // source, s_path[0] = u*); a vertex appears once on a predecessor path
  if (tid < len) s_pos[s_path[len - 1 - tid]] = static_cast<int16_t>(tid);
  __syncthreads();
  // every expert drops by D - min(d, D), then the path shift is added
  if (tid < n) {
    const int64_t dv = static_cast<int64_t>(d[tid] >> IDX_BITS);
    const int64_t nbv = bias[tid] + ((dv < D ? dv : D) - D) + s_pos[tid];
    bias[tid] = nbv;
    if (nbv >= BIAS_LIMIT || nbv <= -BIAS_LIMIT) s_bad = 1;
  }
  __syncthreads();
  if (tid == 0) {
    c[C_MOVES] += 1;
    c[C_DROP] = D;  // no bias fell by more than D
    c[C_LAST_D] = D;
    c[C_LAST_HOPS] = len - 1;
    c[C_BF_PASSES] += passes;
    if (s_bad) {
      c[C_PHASE] = PH_FAILED;
      c[C_STATUS] = MOE_QB_STATUS_BIAS_RANGE;
    }
  }
  clear_edges();
}

// ---------------------------------------------------------------------------
// Status (one block of 1024 threads): commit the quantile round of the
// previous step, take the accumulated loads (clearing the accumulators),
// decide the next phase exactly as the schedule prescribes (rounds until the
// unbalanced count stalls, then augmenting paths, then done) and, in the
// augmenting-path phase, make this step's move.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void status_pass(Args a, int edge_cache) {
  __shared__ int32_t s_imb[16], s_res[16];
  __shared__ int s_move;
  const int n = a.n;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int imb = 0, res = 0;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    int32_t L = 0;
    for (int r0 = 0; r0 < ACC_COPIES; r0 += 8) {
      int32_t part[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) part[r] = a.acc[(r0 + r) * n + e];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        L += part[r];
        a.acc[(r0 + r) * n + e] = 0;
      }
    }
    a.loads[e] = L;
    const int64_t d = static_cast<int64_t>(L) - target(a.T, n, a.k, e);
    imb += d != 0;
    const int ad = static_cast<int>(d < 0 ? -d : d);
    res = res > ad ? res : ad;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    imb += __shfl_xor(imb, off);
    res = max(res, __shfl_xor(res, off));
  }
  if (lane == 0) {
    s_imb[wid] = imb;
    s_res[wid] = res;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    imb = 0;
    res = 0;
    for (int w = 0; w < 16; ++w) {
      imb += s_imb[w];
      res = max(res, s_res[w]);
    }
    int64_t* c = a.ctrl;
    if (c[C_ROUND] != 0) {  // the previous step's quantile round becomes live
      c[C_ROUND] = 0;
      c[C_CUR] ^= 1;
      c[C_ROUNDS] += 1;
      if (a.cnt[N_BIASRANGE]) {
        c[C_PHASE] = PH_FAILED;
        c[C_STATUS] = MOE_QB_STATUS_BIAS_RANGE;
      }
    }
    c[C_IMB] = imb;
    c[C_RESID] = res;
    c[C_PIVOT] = 1;  // th[].k1 now holds this pass's keys; biases unchanged so far
    c[C_DROP] = 0;
    const int64_t ph = c[C_PHASE];
    if (ph == PH_ROUNDS) {
      bool round = false;
      if (imb == 0) {
        c[C_PHASE] = PH_DONE;
      } else if (c[C_ROUNDS] >= c[C_MAX_ROUNDS]) {
        c[C_PHASE] = PH_SAP;
      } else if (c[C_BEST] < 0 || imb < c[C_BEST]) {
        c[C_BEST] = imb;
        c[C_SINCE] = 0;
        round = true;
      } else if (++c[C_SINCE] >= STALL_ROUNDS) {
        c[C_PHASE] = PH_SAP;
      } else {
        round = true;
      }
      c[C_ROUND] = round ? 1 : 0;  // the quantile kernel runs; the next status commits it
    } else if (ph == PH_SAP) {
      if (imb == 0) {
        c[C_PHASE] = PH_DONE;
      } else if (c[C_MOVES] >= MAX_SAP_MOVES) {
        c[C_PHASE] = PH_FAILED;
        c[C_STATUS] = MOE_QB_STATUS_NOT_BALANCED;
      }
    }
    s_move = c[C_PHASE] == PH_SAP && c[C_EDGES_VALID] != 0;
  }
  __syncthreads();
  if (s_move) sap_move(a, edge_cache);
}

// ---------------------------------------------------------------------------
// Fixed-step sign update (DeepSeek-V3's bias rule, the baseline QB is
// compared with; xhh.club "Kimi K3 模型结构（5）", 延伸解读 "Quantile
// Balancing与DeepSeek-V3路由的异同": sign descent on the same dual with a
// hand-tuned step).  One block of 1024 threads after each top-k pass: loads,
// then b_e += step * sign(C_e - L_e) unless balanced or out of rounds.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void sign_status(Args a, int64_t step) {
  __shared__ int32_t s_imb[16], s_res[16];
  __shared__ int s_upd, s_bad;
  const int n = a.n;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int imb = 0, res = 0;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    int32_t L = 0;
    for (int r = 0; r < ACC_COPIES; ++r) {
      L += a.acc[r * n + e];
      a.acc[r * n + e] = 0;
    }
    a.loads[e] = L;
    const int64_t d = static_cast<int64_t>(L) - target(a.T, n, a.k, e);
    imb += d != 0;
    const int ad = static_cast<int>(d < 0 ? -d : d);
    res = res > ad ? res : ad;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    imb += __shfl_xor(imb, off);
    res = max(res, __shfl_xor(res, off));
  }
  if (lane == 0) {
    s_imb[wid] = imb;
    s_res[wid] = res;
  }
  __syncthreads();
  int64_t* c = a.ctrl;
  if (threadIdx.x == 0) {
    imb = 0;
    res = 0;
    for (int w = 0; w < 16; ++w) {
      imb += s_imb[w];
      res = max(res, s_res[w]);
    }
    c[C_IMB] = imb;
    c[C_RESID] = res;
    c[C_PIVOT] = 1;  // th[].k1 holds this pass's keys
    c[C_DROP] = 0;
    int upd = 0;
    if (c[C_PHASE] == PH_ROUNDS) {
      if (imb == 0) {
        c[C_PHASE] = PH_DONE;
      } else if (c[C_ROUNDS] >= c[C_MAX_ROUNDS]) {
        c[C_PHASE] = PH_FAILED;
        c[C_STATUS] = MOE_QB_STATUS_NOT_BALANCED;
      } else {
        upd = 1;
        c[C_ROUNDS] += 1;
        c[C_DROP] = step;  // no bias falls by more than the step
      }
    }
    s_upd = upd;
    s_bad = 0;
  }
  __syncthreads();
  if (!s_upd) return;
  int64_t* bias = a.bfx + (c[C_CUR] & 1) * n;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int64_t L = a.loads[e], C = target(a.T, n, a.k, e);
    const int64_t b = bias[e] + (L < C ? step : (L > C ? -step : 0));
    bias[e] = b;
    if (b >= BIAS_LIMIT || b <= -BIAS_LIMIT) s_bad = 1;
  }
  __syncthreads();
  if (threadIdx.x == 0 && s_bad) {
    c[C_PHASE] = PH_FAILED;
    c[C_STATUS] = MOE_QB_STATUS_BIAS_RANGE;
  }
}

// Bias and counters of a sign-update run (no common offset is removed).
__global__ void sign_export(Args a, double* bias_out, int32_t* info) {
  const int n = a.n;
  int64_t* c = a.ctrl;
  const int64_t* bias = a.bfx + (c[C_CUR] & 1) * n;
  for (int e = threadIdx.x; e < n; e += blockDim.x)
    bias_out[e] = static_cast<double>(bias[e]) * (1.0 / 1099511627776.0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t ph = c[C_PHASE];
    if (ph != PH_DONE && c[C_STATUS] == MOE_QB_STATUS_OK)
      c[C_STATUS] = MOE_QB_STATUS_NOT_BALANCED;  // the host's step cap ended the loop
    c[C_DROP] = 0;  // biases unchanged since the last pass
    if (info) {
      info[0] = static_cast<int32_t>(c[C_ROUNDS]);
      info[1] = static_cast<int32_t>(c[C_STATUS]);
      info[3] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// One quantile round (one block per expert, reading the transposed scores so
// the column is contiguous): an unbalanced expert finds the C-th and
// (C+1)-th largest margins over all tokens exactly and jumps to minus their
// midpoint.  New biases go to the idle bias buffer, which the next step
// reads as live.
//
// Selection: one pass bins d = margin - cut (the cut is -1024*bias; d > 0 iff
// the token currently picks the expert) into 2048 order-preserving buckets
// that are exact near zero and ~6% wide far from it, a block scan finds the
// buckets holding the two ranks, a second pass gathers those one or two
// buckets into LDS and the ranks are resolved by exact counting.  A bucket
// too large for LDS falls back to an MSB-first radix select.
// ---------------------------------------------------------------------------
constexpr int SEL_BLOCK = 1024;
constexpr int SEL_WAVES = SEL_BLOCK / 64;
constexpr int QREG = 16;  // margins held in registers per thread: one memory pass for T <= 16384
constexpr int NBUCKET = 2048;
constexpr int GATHER_CAP = 4096;
constexpr int DIG = 10;
constexpr int NBIN = 1 << DIG;

// Margin of token t for expert e: its key without the bias minus the key the
// expert has to beat (the k-th key when e is not chosen, the (k+1)-th when it is).
__device__ __forceinline__ int64_t margin_from(float s, KeyPair th, int64_t be, int e) {
  const int64_t sfx = score_fixed(s);
  const uint64_t key = pack_key(sfx, be, e);
  const bool sel = static_cast<int64_t>(key) >= th.k;
  return static_cast<int64_t>(pack_key(sfx, 0, e)) - (sel ? th.k1 : th.k);
}

__device__ __forceinline__ int64_t margin_of(const Args& a, const int64_t* bias, int e, int t) {
  return margin_from(a.scoresT[static_cast<size_t>(e) * a.T + t], a.th[t], bias[e], e);
}

__device__ __forceinline__ int log_code(uint64_t x) {
  if (x < 16) return static_cast<int>(x);
  const int msb = 63 - __clzll(static_cast<long long>(x));
  return 16 + (msb - 4) * 16 + static_cast<int>((x >> (msb - 4)) & 15);
}

// order-preserving bucket of d: [0, 1024) for d <= 0, [1024, 2048) for d > 0
__device__ __forceinline__ int bucket_of(int64_t d) {
  return d > 0 ? 1024 + log_code(static_cast<uint64_t>(d - 1))
               : 1023 - log_code(static_cast<uint64_t>(-d));
}

// Exact value of descending ranks r1 <= r2 among all margins (radix select on
// the order-preserving uint64 image); used when a bucket overflows LDS.
__device__ void radix_select2(const Args& a, const int64_t* bias, int e, int64_t r1, int64_t r2,
                              int32_t* h1, int32_t* h2, int64_t* out) {
  __shared__ uint64_t s_pre[2];
  __shared__ int64_t s_rem[2];
  if (threadIdx.x == 0) {
    s_pre[0] = s_pre[1] = 0;
    s_rem[0] = r1;
    s_rem[1] = r2;
  }
  __syncthreads();
  uint64_t mask = 0;
  for (int shift = 64; shift > 0;) {
    const int nbits = shift >= DIG ? DIG : shift;
    shift -= nbits;
    for (int i = threadIdx.x; i < NBIN; i += SEL_BLOCK) h1[i] = h2[i] = 0;
    __syncthreads();
    const uint64_t p1 = s_pre[0], p2 = s_pre[1];
    const uint64_t dmask = (uint64_t(1) << nbits) - 1;
    for (int t = threadIdx.x; t < a.T; t += SEL_BLOCK) {
      const uint64_t u = static_cast<uint64_t>(margin_of(a, bias, e, t)) ^ (uint64_t(1) << 63);
      const int dg = static_cast<int>((u >> shift) & dmask);
      if ((u & mask) == p1) atomicAdd(&h1[dg], 1);
      if ((u & mask) == p2) atomicAdd(&h2[dg], 1);
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      int32_t* h = threadIdx.x == 0 ? h1 : h2;
      int64_t rem = s_rem[threadIdx.x];
      int dsel = 0;
      for (int dgt = static_cast<int>(dmask); dgt >= 0; --dgt) {
        if (rem <= h[dgt]) {
          dsel = dgt;
          break;
        }
        rem -= h[dgt];
      }
      s_rem[threadIdx.x] = rem;
      s_pre[threadIdx.x] |= static_cast<uint64_t>(dsel) << shift;
    }
    mask |= dmask << shift;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = static_cast<int64_t>(s_pre[0] ^ (uint64_t(1) << 63));
    out[1] = static_cast<int64_t>(s_pre[1] ^ (uint64_t(1) << 63));
  }
  __syncthreads();
}

__global__ __launch_bounds__(SEL_BLOCK) void quantile_round(Args a) {
  if (a.ctrl[C_PHASE] != PH_ROUNDS || a.ctrl[C_ROUND] == 0) return;
  const int e = blockIdx.x;
  const int n = a.n, T = a.T;
  const int cur = static_cast<int>(a.ctrl[C_CUR] & 1);
  const int64_t* bias = a.bfx + cur * n;
  int64_t* nb = a.bfx + (cur ^ 1) * n;
  const int64_t C = target(T, n, a.k, e);
  if (a.loads[e] == C) {  // the lazy rule: balanced experts keep their bias
    if (threadIdx.x == 0) nb[e] = bias[e];
    return;
  }
  __shared__ int32_t hist[NBUCKET];
  __shared__ int64_t gat[GATHER_CAP];
  __shared__ int32_t wsum[SEL_WAVES];
  __shared__ int s_bucket[2];
  __shared__ int64_t s_above[2];
  __shared__ int s_cnt;
  __shared__ int64_t s_val[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int64_t be = bias[e];
  const int64_t cut = -be * 1024;

  for (int i = tid; i < NBUCKET; i += SEL_BLOCK) hist[i] = 0;
  if (tid == 0) s_cnt = 0;
  // every operand of this thread's first QREG tokens is requested before
  // any is used, so the loads overlap instead of forming a chain
  const float* col = a.scoresT + static_cast<size_t>(e) * T;
  float sv[QREG];
  KeyPair thv[QREG];
#pragma unroll
  for (int i = 0; i < QREG; ++i) {
    const int t = tid + i * SEL_BLOCK;
    if (t < T) {
      sv[i] = col[t];
      thv[i] = a.th[t];
    }
  }
  int64_t mreg[QREG];
#pragma unroll
  for (int i = 0; i < QREG; ++i)
    mreg[i] = tid + i * SEL_BLOCK < T ? margin_from(sv[i], thv[i], be, e) : 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < QREG; ++i)
    if (tid + i * SEL_BLOCK < T) atomicAdd(&hist[bucket_of(mreg[i] - cut)], 1);
  for (int t = tid + QREG * SEL_BLOCK; t < T; t += SEL_BLOCK)
    atomicAdd(&hist[bucket_of(margin_of(a, bias, e, t) - cut)], 1);
  __syncthreads();

  // descending ranks: r1 = C, r2 = C+1, or a single rank at the edges
  int64_t r1 = C, r2 = C + 1;
  if (C == 0) r1 = r2 = 1;
  if (C == T) r1 = r2 = T;
  // thread i owns the PER buckets below 2048 - PER*i: counts in descending
  // order; inclusive block scan = shuffle scan in the wave + wave offsets
  constexpr int PER = NBUCKET / SEL_BLOCK;
  int32_t own = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) own += hist[NBUCKET - 1 - (tid * PER + j)];
  int32_t incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (tid < 64) {
    int32_t w = tid < SEL_WAVES ? wsum[tid] : 0;
#pragma unroll
    for (int off = 1; off < SEL_WAVES; off <<= 1) {
      const int32_t u = __shfl_up(w, off);
      if (lane >= off) w += u;
    }
    if (tid < SEL_WAVES) wsum[tid] = w;
  }
  __syncthreads();
  if (wid > 0) incl += wsum[wid - 1];
  const int64_t before = incl - own;  // values in buckets above this thread's chunk
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t r = q == 0 ? r1 : r2;
    if (before < r && r <= incl) {
      int64_t acc = before;
      for (int j = 0; j < PER; ++j) {
        const int b = NBUCKET - 1 - (tid * PER + j);
        if (acc + hist[b] >= r) {
          s_bucket[q] = b;
          s_above[q] = acc;
          break;
        }
        acc += hist[b];
      }
    }
  }
  __syncthreads();
  const int b1 = s_bucket[0], b2 = s_bucket[1];  // b2 <= b1
  auto gather = [&](int64_t M) {
    const int b = bucket_of(M - cut);
    if (b <= b1 && b >= b2) {
      const int pos = atomicAdd(&s_cnt, 1);
      if (pos < GATHER_CAP) gat[pos] = M;
    }
  };
#pragma unroll
  for (int i = 0; i < QREG; ++i)
    if (tid + i * SEL_BLOCK < T) gather(mreg[i]);
  for (int t = tid + QREG * SEL_BLOCK; t < T; t += SEL_BLOCK) gather(margin_of(a, bias, e, t));
  __syncthreads();
  const int cnt = s_cnt;
  if (cnt <= GATHER_CAP) {
    // ranks inside the gathered set (everything in buckets above b1 is larger)
    const int64_t q1 = r1 - s_above[0], q2 = r2 - s_above[0];
    for (int i = tid; i < cnt; i += SEL_BLOCK) {
      const int64_t v = gat[i];
      int64_t g = 0, ge = 0;
      for (int j = 0; j < cnt; ++j) {
        const int64_t w = gat[j];
        g += w > v;
        ge += w >= v;
      }
      if (g < q1 && q1 <= ge) s_val[0] = v;
      if (g < q2 && q2 <= ge) s_val[1] = v;
    }
    __syncthreads();
  } else {
    radix_select2(a, bias, e, r1, r2, hist, hist + NBIN, s_val);
  }
  if (tid == 0) {
    const int64_t m1 = s_val[0], m2 = s_val[1];
    int64_t b;
    if (C == 0)
      b = -(m1 >> IDX_BITS) - 1;
    else if (C == T)
      b = -(m1 >> IDX_BITS) + 1;
    else
      b = -floor_mid(m1, m2);
    nb[e] = b;
    if (b >= BIAS_LIMIT || b <= -BIAS_LIMIT) atomicOr(&a.cnt[N_BIASRANGE], 1);
  }
}

// ---------------------------------------------------------------------------
// Small helpers: init, transposition, centring, bias conversion.
// ---------------------------------------------------------------------------
__global__ void init_ctrl(Args a, const double* bias_in, int mode, int max_rounds) {
  const int n = a.n;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const double b = bias_in ? bias_in[e] : 0.0;
    const double bf = rint(b * 1099511627776.0);
    int64_t v = 0;
    if (!(fabs(bf) < static_cast<double>(BIAS_LIMIT))) {
      atomicOr(&a.cnt[N_BIASRANGE], 1);
    } else {
      v = static_cast<int64_t>(bf);
    }
    a.bfx[e] = v;
    a.bfx[n + e] = v;
  }
  for (int i = threadIdx.x; i < ACC_COPIES * n; i += blockDim.x) a.acc[i] = 0;
  if (threadIdx.x == 0) {
    int64_t* c = a.ctrl;
    for (int i = 0; i < C_COUNT; ++i) c[i] = 0;
    // an empty batch is balanced: every target is zero
    c[C_PHASE] = mode == MOE_QB_BATCH ? (a.T > 0 ? PH_ROUNDS : PH_DONE) : PH_FROZEN;
    c[C_BEST] = -1;
    c[C_DELTA] = DELTA_START;
    c[C_MAX_ROUNDS] = max_rounds;
  }
}

__global__ void zero_cnt(Args a) {
  for (int i = threadIdx.x; i < N_COUNT; i += blockDim.x) a.cnt[i] = 0;
}

__global__ void check_range(Args a) {
  // bias given out of range: report instead of routing with a clamped bias
  if (threadIdx.x == 0 && a.cnt[N_BIASRANGE]) {
    a.ctrl[C_PHASE] = PH_FAILED;
    a.ctrl[C_STATUS] = MOE_QB_STATUS_BIAS_RANGE;
  }
}

__global__ void transpose_scores(const float* __restrict__ in, float* __restrict__ out, int T,
                                 int n) {
  __shared__ float tile[64][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 256 threads: 64 x 4
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + r, e = e0 + tx;
    tile[r][tx] = (t < T && e < n) ? in[static_cast<size_t>(t) * n + e] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int e = e0 + r, t = t0 + tx;
    if (e < n && t < T) out[static_cast<size_t>(e) * T + t] = tile[tx][r];
  }
}

__global__ void center_and_export(Args a, double* bias_out, int32_t* info) {
  __shared__ long long s[1024];
  const int n = a.n;
  int64_t* c = a.ctrl;
  // a quantile round left uncommitted when the host's step cap ended the loop
  const bool pending = c[C_PHASE] == PH_ROUNDS && c[C_ROUND] != 0;
  const int cur = static_cast<int>(c[C_CUR] & 1) ^ (pending ? 1 : 0);
  int64_t* bias = a.bfx + cur * n;
  const bool balanced = c[C_PHASE] == PH_DONE;
  __syncthreads();
  if (pending && threadIdx.x == 0) {
    c[C_ROUND] = 0;
    c[C_CUR] = cur;
    c[C_ROUNDS] += 1;
    if (a.cnt[N_BIASRANGE]) c[C_STATUS] = MOE_QB_STATUS_BIAS_RANGE;
  }
  long long acc = 0;
  for (int e = threadIdx.x; e < n; e += blockDim.x) acc += bias[e];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) s[threadIdx.x] += s[threadIdx.x + st];
    __syncthreads();
  }
  long long sum = s[0];
  long long off = sum / n;
  if ((sum % n != 0) && (sum < 0)) off -= 1;  // floor division
  if (!balanced) off = 0;
  __syncthreads();
  if (threadIdx.x == 0) c[C_DROP] = off > 0 ? off : 0;  // every bias moves by -off
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    bias[e] -= off;
    if (bias_out) bias_out[e] = static_cast<double>(bias[e]) * (1.0 / 1099511627776.0);
  }
  if (threadIdx.x == 0 && c[C_PHASE] != PH_DONE && c[C_PHASE] != PH_FROZEN &&
      c[C_STATUS] == MOE_QB_STATUS_OK)
    c[C_STATUS] = MOE_QB_STATUS_NOT_BALANCED;  // the host's step cap ended the loop
  if (threadIdx.x == 0 && info) {
    info[0] = static_cast<int32_t>(c[C_ROUNDS]);
    info[1] = static_cast<int32_t>(c[C_STATUS]);
    info[3] = static_cast<int32_t>(c[C_MOVES]);
  }
}

__global__ void export_resid(Args a, int32_t* info) {
  if (threadIdx.x == 0 && info) info[2] = static_cast<int32_t>(a.ctrl[C_RESID]);
}

size_t topk_smem_bytes() {
  return 1024 * 4 + 4 * EDGE_LIST_MAX * (8 + 8 + 4 + 4) + 8 * 4 + 4 * MAX_K * (8 + 4 + 4 + 4) +
         4 * 64 * 8 + 4 * 2 * 8 + 1024 * 8;
}

}  // namespace qb

// ---------------------------------------------------------------------------
// Host driver shared by moe_route_qb and moe_latent_forward.
// ---------------------------------------------------------------------------

// Edge list: 16 per token on average plus, in every segment, room for the
// largest list one token can emit (64 x 64).
static int32_t edge_capacity(int32_t T) { return 16 * T + qb::EDGE_SEGS * 4096; }

size_t route_workspace_layout(int32_t T, int32_t n, RouteWorkspace* ws, void* base) {
  Carver cv(base);
  RouteWorkspace w;
  w.scoresT = cv.take<float>(static_cast<size_t>(T) * n);
  w.bfx = cv.take<int64_t>(2 * static_cast<size_t>(n));
  w.th = cv.take<KeyPair>(T);
  w.loads = cv.take<int32_t>(n);
  w.acc = cv.take<int32_t>(static_cast<size_t>(qb::ACC_COPIES) * n);
  w.ctrl = cv.take<int64_t>(qb::C_COUNT);
  w.cnt = cv.take<int32_t>(qb::N_COUNT);
  w.edge_cap = edge_capacity(T);
  w.edges = cv.take<uint64_t>(w.edge_cap);
  if (ws) *ws = w;
  return cv.bytes();
}

// Pinned host words and events of the balancing loop (per host thread and
// device, created on first use and kept for the life of the process): batch
// i copies the phase word into slot i % 2 and records event i % 2.
struct PollState {
  int64_t* word = nullptr;  // [2][8] (one 64-byte line per slot)
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool ok = false;
};

// Edges the status kernel caches in dynamic LDS once the host has seen the
// augmenting-path phase (128 KB); before that it runs with a small LDS
// footprint, so that its block can be resident beside other kernels' blocks.
constexpr int SAP_EDGE_CACHE = 16384;

static PollState* poll_state() {
  constexpr int MAX_DEVICES = 64;
  thread_local PollState st[MAX_DEVICES];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  PollState& p = st[dev];
  if (!p.ok) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(qb::status_pass),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            SAP_EDGE_CACHE * static_cast<int>(sizeof(uint64_t))) != hipSuccess)
      return nullptr;
    if (!p.word) {
      void* w = nullptr;
      if (hipHostMalloc(&w, 128, hipHostMallocDefault) != hipSuccess) return nullptr;
      p.word = static_cast<int64_t*>(w);
    }
    for (int i = 0; i < 2; ++i)
      if (!p.ev[i] && hipEventCreateWithFlags(&p.ev[i], hipEventDisableTiming) != hipSuccess)
        return nullptr;
    p.ok = true;
  }
  return &p;
}

int route_validate(int32_t T, int32_t n, int32_t k) {
  if (T < 0 || n < 1 || k < 1 || k > n) return MOE_EINVAL;
  if (n > 1024 || k > qb::MAX_K) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Routes T tokens from fp32 scores.  Outputs may be null except the internal
// loads buffer; `loads_out` receives a copy when given.
int route_run(const float* scores, int32_t T, int32_t n, int32_t k, int32_t mode,
              int32_t max_rounds, double* bias, int32_t* idx, float* w, int32_t* loads_out,
              int32_t* info, const RouteWorkspace& ws, hipStream_t stream) {
  using namespace qb;
  Args a{};
  a.scores = scores;
  a.scoresT = ws.scoresT;
  a.T = T;
  a.n = n;
  a.k = k;
  a.bfx = ws.bfx;
  a.th = ws.th;
  a.loads = ws.loads;
  a.acc = ws.acc;
  a.ctrl = ws.ctrl;
  a.cnt = ws.cnt;
  a.edges = ws.edges;
  a.edge_cap = ws.edge_cap;
  a.idx = idx;
  a.w = w;
  const int grid = T > 0 ? std::min((T + 3) / 4, TOPK_MAX_GRID) : 1;  // 4 waves per block
  if (max_rounds <= 0) max_rounds = 64;
  const size_t smem = topk_smem_bytes();

  hipLaunchKernelGGL(zero_cnt, dim3(1), dim3(64), 0, stream, a);
  hipLaunchKernelGGL(init_ctrl, dim3(1), dim3(1024), 0, stream, a,
                     mode == MOE_QB_BATCH ? bias : static_cast<const double*>(bias), mode,
                     max_rounds);
  hipLaunchKernelGGL(check_range, dim3(1), dim3(64), 0, stream, a);
  MOE_LAUNCH_CHECK();

  if (mode == MOE_QB_BATCH && T > 0) {
    dim3 tg((T + 63) / 64, (n + 63) / 64);
    hipLaunchKernelGGL(transpose_scores, tg, dim3(256), 0, stream, scores, ws.scoresT, T, n);
    MOE_LAUNCH_CHECK();
  }
  if (mode == MOE_QB_BATCH && T > 0) {
    // Batches of steps; while batch i runs the host waits for the phase word
    // of batch i-1, so the queue never drains for a poll.  Steps launched
    // after the loop has ended return at once.
    const int batch = 4;
    const int max_steps = max_rounds + 8 * MAX_SAP_MOVES + 64;
    PollState* ps = poll_state();
    if (!ps) return MOE_EHIP;
    int steps = 0, launched = 0;
    bool sap_seen = false;  // edge cache from the first batch after the phase was seen
    while (true) {
      const int slot = launched & 1;
      const int cache = sap_seen ? SAP_EDGE_CACHE : 0;
      for (int i = 0; i < batch; ++i) {
        hipLaunchKernelGGL(topk_pass, dim3(grid), dim3(TOPK_BLOCK), smem, stream, a, 0);
        hipLaunchKernelGGL(status_pass, dim3(1), dim3(1024), cache * sizeof(uint64_t), stream, a,
                           cache);
        // the augmenting-path phase never returns to quantile rounds
        if (!sap_seen) hipLaunchKernelGGL(quantile_round, dim3(n), dim3(SEL_BLOCK), 0, stream, a);
      }
      MOE_LAUNCH_CHECK();
      MOE_HIP_CHECK(hipMemcpyAsync(ps->word + 8 * slot, ws.ctrl + C_PHASE, sizeof(int64_t),
                                   hipMemcpyDeviceToHost, stream));
      MOE_HIP_CHECK(hipEventRecord(ps->ev[slot], stream));
      ++launched;
      steps += batch;
      if (launched >= 2) {
        const int prev = slot ^ 1;
        MOE_HIP_CHECK(hipEventSynchronize(ps->ev[prev]));
        const int64_t phase = ps->word[8 * prev];
        if (phase == PH_DONE || phase == PH_FAILED) break;
        if (phase == PH_SAP) sap_seen = true;
      }
      if (steps >= max_steps) break;
    }
  }
  // final pass: centred bias, ordered outputs, loads
  hipLaunchKernelGGL(center_and_export, dim3(1), dim3(1024), 0, stream, a,
                     mode == MOE_QB_BATCH ? bias : nullptr, info);
  hipLaunchKernelGGL(topk_pass, dim3(grid), dim3(TOPK_BLOCK), smem, stream, a, 1);
  hipLaunchKernelGGL(status_pass, dim3(1), dim3(1024), 0, stream, a, 0);
  hipLaunchKernelGGL(export_resid, dim3(1), dim3(64), 0, stream, a, info);
  if (loads_out)
    MOE_HIP_CHECK(hipMemcpyAsync(loads_out, ws.loads, sizeof(int32_t) * n,
                                 hipMemcpyDeviceToDevice, stream));
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// The sign-update baseline on the same workspace: top-k pass and sign status
// per step, in polled batches like the balancing loop; then the outputs.
int route_sign_run(const float* scores, int32_t T, int32_t n, int32_t k, int64_t step,
                   int32_t max_rounds, double* bias, int32_t* idx, float* w, int32_t* loads_out,
                   int32_t* info, const RouteWorkspace& ws, hipStream_t stream) {
  using namespace qb;
  Args a{};
  a.scores = scores;
  a.scoresT = ws.scoresT;
  a.T = T;
  a.n = n;
  a.k = k;
  a.bfx = ws.bfx;
  a.th = ws.th;
  a.loads = ws.loads;
  a.acc = ws.acc;
  a.ctrl = ws.ctrl;
  a.cnt = ws.cnt;
  a.edges = ws.edges;
  a.edge_cap = ws.edge_cap;
  a.idx = idx;
  a.w = w;
  const int grid = T > 0 ? std::min((T + 3) / 4, TOPK_MAX_GRID) : 1;
  const size_t smem = topk_smem_bytes();
  hipLaunchKernelGGL(zero_cnt, dim3(1), dim3(64), 0, stream, a);
  hipLaunchKernelGGL(init_ctrl, dim3(1), dim3(1024), 0, stream, a, static_cast<const double*>(bias),
                     static_cast<int>(MOE_QB_BATCH), max_rounds);
  hipLaunchKernelGGL(check_range, dim3(1), dim3(64), 0, stream, a);
  MOE_LAUNCH_CHECK();
  if (T > 0) {
    const int batch = 4;
    const int max_steps = max_rounds + 2 * batch + 1;
    PollState* ps = poll_state();
    if (!ps) return MOE_EHIP;
    int steps = 0, launched = 0;
    while (true) {
      const int slot = launched & 1;
      for (int i = 0; i < batch; ++i) {
        hipLaunchKernelGGL(topk_pass, dim3(grid), dim3(TOPK_BLOCK), smem, stream, a, 0);
        hipLaunchKernelGGL(sign_status, dim3(1), dim3(1024), 0, stream, a, step);
      }
      MOE_LAUNCH_CHECK();
      MOE_HIP_CHECK(hipMemcpyAsync(ps->word + 8 * slot, ws.ctrl + C_PHASE, sizeof(int64_t),
                                   hipMemcpyDeviceToHost, stream));
      MOE_HIP_CHECK(hipEventRecord(ps->ev[slot], stream));
      ++launched;
      steps += batch;
      if (launched >= 2) {
        const int prev = slot ^ 1;
        MOE_HIP_CHECK(hipEventSynchronize(ps->ev[prev]));
        const int64_t phase = ps->word[8 * prev];
        if (phase == PH_DONE || phase == PH_FAILED) break;
      }
      if (steps >= max_steps) break;
    }
  }
  hipLaunchKernelGGL(sign_export, dim3(1), dim3(1024), 0, stream, a, bias, info);
  hipLaunchKernelGGL(topk_pass, dim3(grid), dim3(TOPK_BLOCK), smem, stream, a, 1);
  hipLaunchKernelGGL(status_pass, dim3(1), dim3(1024), 0, stream, a, 0);
  hipLaunchKernelGGL(export_resid, dim3(1), dim3(64), 0, stream, a, info);
  if (loads_out)
    MOE_HIP_CHECK(hipMemcpyAsync(loads_out, ws.loads, sizeof(int32_t) * n,
                                 hipMemcpyDeviceToDevice, stream));
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe

extern "C" size_t moe_route_workspace_bytes(int32_t T, int32_t n, int32_t k) {
  if (moe::route_validate(T, n, k) != MOE_OK) return 0;
  return moe::route_workspace_layout(T, n, nullptr, nullptr);
}

extern "C" int moe_route_qb(const float* scores, int32_t T, int32_t n, int32_t k, int32_t mode,
                            int32_t max_rounds, double* bias, int32_t* topk_idx, float* topk_w,
                            int32_t* loads, int32_t* qb_info, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = moe::route_validate(T, n, k);
  if (st != MOE_OK) return st;
  if (mode != MOE_QB_BATCH && mode != MOE_QB_FROZEN) return MOE_EINVAL;
  if ((T > 0 && (!scores || !topk_idx || !topk_w)) || !bias || !workspace) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MOE_EINVAL;
  moe::RouteWorkspace ws;
  const size_t need = moe::route_workspace_layout(T, n, &ws, workspace);
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  moe::prof::Scope sc(moe::prof::ST_ROUTING, static_cast<hipStream_t>(stream));
  return moe::route_run(scores, T, n, k, mode, max_rounds, bias, topk_idx, topk_w, loads, qb_info,
                        ws, static_cast<hipStream_t>(stream));
}

extern "C" int moe_route_sign(const float* scores, int32_t T, int32_t n, int32_t k, double step,
                              int32_t max_rounds, double* bias, int32_t* topk_idx, float* topk_w,
                              int32_t* loads, int32_t* qb_info, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int st = moe::route_validate(T, n, k);
  if (st != MOE_OK) return st;
  if (max_rounds < 0 || !(step > 0.0)) return MOE_EINVAL;
  const double sf = rint(step * 1099511627776.0);
  if (!(sf >= 1.0 && sf < static_cast<double>(moe::qb::BIAS_LIMIT))) return MOE_EINVAL;
  if ((T > 0 && (!scores || !topk_idx || !topk_w)) || !bias || !workspace) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MOE_EINVAL;
  moe::RouteWorkspace ws;
  const size_t need = moe::route_workspace_layout(T, n, &ws, workspace);
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  moe::prof::Scope sc(moe::prof::ST_ROUTING, static_cast<hipStream_t>(stream));
  return moe::route_sign_run(scores, T, n, k, static_cast<int64_t>(sf), max_rounds, bias, topk_idx,
                             topk_w, loads, qb_info, ws, static_cast<hipStream_t>(stream));
}

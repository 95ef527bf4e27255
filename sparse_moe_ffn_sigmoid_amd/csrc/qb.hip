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
// The whole loop is one persistent launch (one block per CU), so a call
// never returns control to the host and never synchronises the stream.  A
// step is two phases separated by grid barriers:
//   A. every wave ranks its tokens under the live biases (the k-th and
//      (k+1)-th keys, per-expert loads; in the augmenting-path phase also the
//      sparse edges);
//   B. every block reads all loads and takes the same decision; in a quantile
//      round the unbalanced experts are shared out over the blocks, each
//      writing its new bias to the idle buffer; an augmenting-path move (or a
//      sign-rule update) is made by block 0 alone.
// Words that one block writes and another reads go through device-scope
// (sc1) loads and stores or device atomics: the L2 of an XCD is not coherent
// with the other XCDs' inside one launch.
#include <algorithm>
#include <type_traits>
#include <mutex>

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
constexpr int MAX_K = 64;
constexpr int NT = 512;               // threads per block
constexpr int NW = NT / 64;           // waves per block
constexpr int STALL_ROUNDS = 3;
constexpr int MAX_SAP_MOVES = 4096;
constexpr int EDGE_LIST_MAX = 64;     // per token: low chosen / high unchosen candidates
constexpr int64_t DELTA_START = int64_t(1) << 28;
constexpr int64_t DELTA_MAX = int64_t(1) << 44;
constexpr int64_t DELTA_MIN = int64_t(1) << 16;
// Per-expert load counters: each block adds its per-block counts into one of
// ACC_COPIES copies (chosen by block index), so that the device atomics on
// one counter do not serialise over every block.
constexpr int ACC_COPIES = 8;
// The edge list is split into EDGE_SEGS segments with one counter each.
constexpr int EDGE_SEGS = 256;
// Grid barrier: blocks arrive on one of several group counters; the last
// arrival of a group bumps the top counter on which every block waits.
constexpr int BAR_GROUP = 16;
constexpr int BAR_LINE = 64;          // uint32 words per counter (one 256-byte line)
constexpr int MAX_GRID = 1024;
// top counter, abort word, per-group arrival counters, per-group release words
constexpr int BAR_WORDS = BAR_LINE * (2 + 2 * (MAX_GRID / BAR_GROUP));
// Every block reads the whole bias vector each step; the writers keep
// BIAS_COPIES copies of it so that the blocks' device-scope reads spread
// over several memory locations instead of all hitting one.
constexpr int BIAS_COPIES = 16;

enum Mode : int { MODE_FROZEN = 0, MODE_QB = 1, MODE_SIGN = 2 };
enum Phase : int { PH_ROUNDS = 0, PH_SAP = 1, PH_DONE = 2, PH_FAILED = 3, PH_FROZEN = 4 };
// ctrl words (int64)
// C_SMALL: some score of the batch lies below 2^-17 (or is zero or subnormal),
// where the fixed-point conversion has to round
enum Ctrl { C_STATUS0 = 0, C_OUTCOME, C_DELTA, C_SMALL, C_COUNT = 16 };
enum Outcome : int64_t { O_MOVED = 0, O_RETRY = 1, O_FAILED = 2, O_RANGE = 3 };
// cnt words (int32)
// N_DEG0 + A: edges leaving expert A in the current list (grouping by source)
enum Cnt { N_OVERFLOW = 1, N_BIASRANGE = 2, N_SEG0 = 8, N_DEG0 = N_SEG0 + EDGE_SEGS,
           N_COUNT = N_DEG0 + 1024 };

// Status reported when a grid barrier wait ran out of time (the grid could
// not become resident, e.g. beside other persistent launches): the routing
// outputs are then not valid.
constexpr int STATUS_ABORTED = 3;

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
  if (__builtin_expect(sh >= 0, 1))
    return static_cast<int64_t>(static_cast<uint64_t>(m) << sh);  // s >= 2^-17: exact
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

// score_fixed(s) << 10 without branches: for s >= 2^-17 (exponent field
// E >= 110) the significand shifted into place; below, the significand
// shifted right by 110 - E (at most 25 places) with round-half-even; zero
// and subnormals give 0.
__device__ __forceinline__ uint64_t score_fixed10(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t E = (u >> 23) & 255u;
  const uint32_t m = (u & 0x7FFFFFu) | 0x800000u;
  const uint64_t big = static_cast<uint64_t>(m) << ((E - 100u) & 63u);
  const uint32_t r = min(110u - E, 25u);           // meaningful when E < 110
  const uint32_t q = m >> r;
  const uint32_t rem = m & ((1u << r) - 1u);
  const uint32_t half = 1u << (r - 1u);
  const uint32_t small = q + ((rem > half) | ((rem == half) & q & 1u));
  const uint64_t sm = static_cast<uint64_t>(E == 0u ? 0u : small) << 10;
  return E >= 110u ? big : sm;
}

// score_fixed(s) << 10 for s >= 2^-17: the significand shifted into place.
__device__ __forceinline__ uint64_t score_fixed10_normal(float s) {
  const uint32_t u = __float_as_uint(s);
  return static_cast<uint64_t>((u & 0x7FFFFFu) | 0x800000u) << (((u >> 23) & 255u) - 100u);
}

// The bias part of a key: key = (sfx << 10) + key_bias(b, e).
__device__ __forceinline__ uint64_t key_bias(int64_t b, int e) {
  return (static_cast<uint64_t>(b + KEY_OFFSET) << IDX_BITS) | static_cast<uint64_t>(1023 - e);
}

// floor((a + b) / 2^11) without overflowing int64.
__device__ __forceinline__ int64_t floor_mid(int64_t a, int64_t b) {
  return (a >> 11) + (b >> 11) + (((a & 2047) + (b & 2047)) >> 11);
}

// ---------------------------------------------------------------------------
// Device-scope accesses for words exchanged between blocks of one launch.
// ---------------------------------------------------------------------------
template <typename V>
__device__ __forceinline__ V ldc(const V* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void stc(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void addc(V* p, V v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The thread index through an opaque copy: values derived from it are
// recomputed where a phase uses them instead of being hoisted out of the
// persistent loop and kept live across every phase.
__device__ __forceinline__ int opaque_tid() {
  int v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(static_cast<int>(threadIdx.x)));
  return v;
}

// This thread's earlier stores and atomics have completed (and the compiler
// keeps memory operations on their side of this point).
__device__ __forceinline__ void writes_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
  const float* scoresT;  // [n][T] (quantile rounds only)
  int T, n, k;
  int mode;              // Mode
  int max_rounds;
  int64_t step;          // sign rule: bias step in grid units
  int64_t* bfx;          // [BIAS_COPIES][2][n]
  KeyPair* th;           // [T]
  int32_t* acc;          // [2][ACC_COPIES][n]
  uint32_t* bar;         // [BAR_WORDS]
  int64_t* ctrl;         // [C_COUNT]
  int32_t* cnt;          // [N_COUNT]
  uint64_t* edges;       // [EDGE_SEGS][edge_cap / EDGE_SEGS]
  int32_t edge_cap;
  int32_t edge_cache;    // edges block 0 keeps in LDS during a move
  int32_t bucket_cap;    // tokens whose margin bucket a quantile block keeps in LDS
  uint64_t timeout;      // grid-barrier wait limit in wall-clock ticks
  int32_t* idx;          // [T][k]
  float* w;              // [T][k]
  int32_t* loads;        // [n]
  int32_t* info;         // [4] or null
  double* bias_out;      // [n] or null
};

// Bias buffer `buf` (0/1) of copy `c`.
__device__ __forceinline__ int64_t* bias_buf(const Args& a, int c, int buf) {
  return a.bfx + (static_cast<size_t>(c) * 2 + buf) * a.n;
}
// Writes bias v of expert e into buffer `buf` of every copy (BIAS_COPIES
// consecutive threads may share the work: lane q of them writes copy q).
__device__ __forceinline__ void put_bias(const Args& a, int buf, int e, int64_t v) {
#pragma unroll
  for (int c = 0; c < BIAS_COPIES; ++c) stc(&bias_buf(a, c, buf)[e], v);
}

// ---------------------------------------------------------------------------
// LDS of the persistent block: a fixed part and per-phase scratch (union).
// ---------------------------------------------------------------------------
constexpr int NBUCKET = 2048;
constexpr int GATHER_CAP = 4096;
constexpr int DIG = 10;
constexpr int NBIN = 1 << DIG;

constexpr int THB = 32;  // tokens per wave whose key pair is held in LDS before the write-out

struct TopkScratch {
  uint64_t cand[NW][64];
  uint64_t thv[NW][2];
  KeyPair thb[NW][THB];  // this wave's (k-th, (k+1)-th) keys, written out in bursts
  union {
    struct {
      int64_t sfx[NW][MAX_K];
      float s[NW][MAX_K];
      int32_t e[NW][MAX_K];
      float sorted[NW][MAX_K];
    } emit;
    struct {
      int64_t lowKp[NW][EDGE_LIST_MAX];
      int64_t highKp[NW][EDGE_LIST_MAX];
      int32_t lowE[NW][EDGE_LIST_MAX];
      int32_t highE[NW][EDGE_LIST_MAX];
    } edge;
  };
};

struct QuantScratch {
  int32_t hist[NBUCKET];
  int64_t gat[GATHER_CAP];
  int32_t wsum[NW];
  int bucket[2];
  int64_t above[2];
  int cnt;
  int64_t val[2];
  uint64_t pre[2];
  int64_t rem[2];
};

// (The distances of a move live in Fixed::kb and the per-source cursors in
// Fixed::sload: neither is in use outside the top-k pass.)
struct SapScratch {
  int32_t off[1025];    // edges grouped by source: [off[A], off[A+1])
  int16_t front[2][1024];  // experts to relax in this pass / the next
  int nfront[2];
  uint32_t inq[256];    // byte flags: expert already in the next pass's list
  int32_t seg_off[EDGE_SEGS + 1];
  int32_t wsum4[4];
  int16_t path[1032];
  int16_t pos[1024];
  uint8_t over[1024];
  uint8_t under[1024];
  int flag[3];
  int len;
  int bad;
  int red[NW];
  unsigned long long D;
};

struct Fixed {
  uint64_t kb[1024];    // key_bias of the staged biases
  float bf[1024];       // the staged biases in score units, rounded to fp32 (-inf past n)
  uint64_t piv[NW][32]; // (k+1)-th key of each wave's first 32 tokens in the last pass
  int64_t pb[1024];     // biases staged by the previous pass (largest decrease since)
  int32_t sload[1024];  // this block's selections per expert in the current pass
  int32_t sL[1024];     // loads of the step (every block)
  int16_t ulist[1024];  // unbalanced experts, ascending
  int32_t red_i[NW];
  int64_t red_l[NW];
  uint64_t red_u[NW];
  int nu;
  int ok;
};

constexpr size_t align16(size_t v) { return (v + 15) & ~size_t(15); }
constexpr size_t SCRATCH_MIN =
    sizeof(TopkScratch) > sizeof(QuantScratch) ? sizeof(TopkScratch) : sizeof(QuantScratch);

__host__ __device__ constexpr size_t lds_bytes(int edge_cache) {
  return align16(sizeof(Fixed)) +
         (SCRATCH_MIN > align16(sizeof(SapScratch)) + size_t(edge_cache) * 8
              ? SCRATCH_MIN
              : align16(sizeof(SapScratch)) + size_t(edge_cache) * 8);
}

// ---------------------------------------------------------------------------
// Grid barrier.  Barrier number `idx` is complete once the top counter has
// reached (idx + 1) * groups.  Every wait is bounded: a block that times out
// (or sees another block's timeout) raises the abort word and the whole grid
// leaves the loop.
// ---------------------------------------------------------------------------
__device__ __attribute__((always_inline)) inline bool grid_sync(const Args& a, Fixed& F, uint32_t& idx) {
  writes_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t G = gridDim.x;
    const uint32_t g = blockIdx.x / BAR_GROUP;
    const uint32_t gsize = min(static_cast<uint32_t>(BAR_GROUP), G - g * BAR_GROUP);
    const uint32_t ng = (G + BAR_GROUP - 1) / BAR_GROUP;
    uint32_t* top = a.bar;
    uint32_t* abort_w = a.bar + BAR_LINE;
    uint32_t* grp = a.bar + BAR_LINE * (2 + g);
    uint32_t* rel = a.bar + BAR_LINE * (2 + MAX_GRID / BAR_GROUP + g);
    // the last arrival of a group bumps the top counter; the last group to
    // arrive releases every group (one release word per group, so that each
    // word is polled by one group's blocks only)
    const uint32_t old =
        __hip_atomic_fetch_add(grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (idx + 1) * gsize) {
      const uint32_t o2 = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 + 1 == (idx + 1) * ng)
        for (uint32_t q = 0; q < ng; ++q)
          stc(a.bar + BAR_LINE * (2 + MAX_GRID / BAR_GROUP + q), idx + 1);
    }
    const uint32_t want = idx + 1;
    int ok = 1;
    if (ldc(rel) < want) {
      const uint64_t t0 = wall_clock64();
      int it = 0;
      while (ldc(rel) < want) {
        __builtin_amdgcn_s_sleep(1);
        if ((++it & 63) == 0 && (ldc(abort_w) != 0u || wall_clock64() - t0 > a.timeout)) {
          addc(abort_w, 1u);
          ok = 0;
          break;
        }
      }
    }
    F.ok = ok;
  }
  __syncthreads();
  ++idx;
  return F.ok != 0;
}

// ---------------------------------------------------------------------------
// Phase A for one token (one wave): the k-th and (k+1)-th keys, the chosen
// set, per-block load counts, and by flag the sparse edges or the ordered
// outputs.
// ---------------------------------------------------------------------------
struct TokenCtx {
  int n, k, lane, wv, seg, seg_cap, slot;
  int64_t delta;
  uint64_t drop_key;
  double err;  // bound on |fp32(s + bf) - (sfx + b) 2^-40| over the staged biases
};

// emit: 0 ranks only, 1 also the sparse edges, 2 also the ordered outputs.
// kbr[j] is key_bias of expert lane + 64 j (0 past n); a key is 0 past n.
template <int NJ>
__device__ __attribute__((always_inline)) inline uint64_t topk_token(
    const Args& a, Fixed& F, TopkScratch& X, const TokenCtx& c, const float (&sv)[NJ],
    const float (&bfr)[NJ], int t, uint64_t prev, bool use_pivot, int emit, bool small) {
  const int n = c.n, k = c.k, lane = c.lane, wv = c.wv;
  constexpr int MAX_NJ = NJ;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  if (emit == 0 && use_pivot && k < n) {
    // Coarse prefilter: every key >= P has score + bias >= P's value in score
    // units, so fp32(s + bf) >= that value - err.  The candidates (at most 64)
    // get their exact keys; the top k+1 keys are >= P, hence candidates, and
    // their ranks among the candidates are their ranks among all keys.
    const uint64_t P = prev > c.drop_key ? prev - c.drop_key : 1;
    const double Vp =
        static_cast<double>(static_cast<int64_t>(P >> IDX_BITS) - KEY_OFFSET) * 0x1p-40;
    const float Pf = static_cast<float>(Vp - c.err - (fabs(Vp) + 1.0) * 0x1p-23);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j) cnt += __popcll(__ballot(sv[j] + bfr[j] >= Pf));
    if (cnt >= k + 1 && cnt <= 64) {
      int base = 0;
#pragma unroll
      for (int j = 0; j < MAX_NJ; ++j) {
        const bool in = sv[j] + bfr[j] >= Pf;
        const uint64_t mj = __ballot(in);
        if (in)
          X.cand[wv][base + __popcll(mj & lt_mask)] =
              (static_cast<uint64_t>(__float_as_uint(sv[j])) << 32) | static_cast<uint64_t>(lane + 64 * j);
        base += __popcll(mj);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      uint64_t kx = 0;
      int ex = 0;
      if (lane < cnt) {
        const uint64_t v = X.cand[wv][lane];
        ex = static_cast<int>(v & 0xFFFFu);
        kx = score_fixed10(__uint_as_float(static_cast<uint32_t>(v >> 32))) + F.kb[ex];
      }
      // the pivot bound holds whenever the previous pass's keys were exact
      if (__popcll(__ballot(lane < cnt && kx >= P)) >= k + 1) {
        // ranks by broadcasting every candidate key (no LDS round trips)
        int rank = 0;
        const uint32_t klo = static_cast<uint32_t>(kx), khi = static_cast<uint32_t>(kx >> 32);
        for (int i = 0; i < cnt; ++i) {
          const uint64_t ki =
              (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(khi), i))) << 32) |
              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(klo), i));
          rank += ki > kx;
        }
        const uint64_t at_k = __ballot(lane < cnt && rank == k - 1);
        const uint64_t at_k1 = __ballot(lane < cnt && rank == k);
        const int lk = __ffsll(static_cast<long long>(at_k)) - 1, lk1 = __ffsll(static_cast<long long>(at_k1)) - 1;
        const uint64_t thk =
            (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(khi), lk))) << 32) |
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(klo), lk));
        const uint64_t thk1 =
            (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(khi), lk1))) << 32) |
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(klo), lk1));
        if (lane < cnt && kx >= thk) atomicAdd(&F.sload[ex], 1);
        if (lane == 0) X.thb[wv][c.slot] = KeyPair{static_cast<int64_t>(thk), static_cast<int64_t>(thk1)};
        return thk1;
      }
    }
  }
  // Exact path.  Keys: (sfx << 10) + key_bias, 0 for lanes past the last
  // expert (their key_bias in LDS is 0).  The opaque lane keeps the compiler
  // from computing these keys ahead of the prefilter above.
  const int xl = opaque_tid() & 63;
  uint64_t key[MAX_NJ];
#pragma unroll
  for (int j = 0; j < MAX_NJ; ++j) {
    const uint64_t kb = F.kb[xl + 64 * j];
    key[j] = (score_fixed10_normal(sv[j]) + kb) & (0ull - static_cast<uint64_t>(kb != 0));
  }
  if (__builtin_expect(small, 0)) {
    // the batch holds scores below 2^-17: round those on the grid
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j) {
      const uint64_t kb = F.kb[lane + 64 * j];
      if (((__float_as_uint(sv[j]) >> 23) & 255u) < 110u)
        key[j] = (score_fixed10(sv[j]) + kb) & (0ull - static_cast<uint64_t>(kb != 0));
    }
  }
  uint64_t thk = 0, thk1 = 0;
  bool found = false;
  // Exact k-th and (k+1)-th keys from a pivot P with k+1 <= #{keys >= P}
  // <= 64: the keys >= P are compacted into LDS and ranked.
  auto try_pivot = [&](uint64_t P) __attribute__((always_inline)) -> bool {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j) cnt += __popcll(__ballot(key[j] >= P));
    if (cnt < k + 1 || cnt > 64) return false;
    int base = 0;
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j) {
      const bool in = key[j] >= P;
      const uint64_t bal = __ballot(in);
      if (in) X.cand[wv][base + __popcll(bal & ((uint64_t(1) << lane) - 1))] = key[j];
      base += __popcll(bal);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (lane < cnt) {
      const uint64_t v = X.cand[wv][lane];
      int rank = 0, i = 0;
      for (; i + 8 <= cnt; i += 8) {
#pragma unroll
        for (int q = 0; q < 8; ++q) rank += X.cand[wv][i + q] > v;
      }
      for (; i < cnt; ++i) rank += X.cand[wv][i] > v;
      if (rank == k - 1) X.thv[wv][0] = v;
      if (rank == k) X.thv[wv][1] = v;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    thk = X.thv[wv][0];
    thk1 = X.thv[wv][1];
    __builtin_amdgcn_wave_barrier();
    return true;
  };
  if (use_pivot && k < n) found = try_pivot(prev > c.drop_key ? prev - c.drop_key : 1);
  if (!found && k < n && k + 1 <= 64) {
    // Second pivot: the (k+1)-th largest of the 64 lane maxima.  At least
    // k+1 keys (those maxima) are >= it; usually few more are.
    uint64_t lm = key[0];
#pragma unroll
    for (int j = 1; j < MAX_NJ; ++j) lm = key[j] > lm ? key[j] : lm;
    if (lane == 0) X.thv[wv][0] = 1;  // lanes without keys tie at 0: P = 1 then
    X.cand[wv][lane] = lm;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    int r = 0;
#pragma unroll 8
    for (int q = 0; q < 64; ++q) r += X.cand[wv][q] > lm;
    __builtin_amdgcn_wave_barrier();
    if (r == k && lm != 0) X.thv[wv][0] = lm;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const uint64_t P = X.thv[wv][0];
    __builtin_amdgcn_wave_barrier();
    found = try_pivot(P);
  }
  if (!found) {
    // k+1 rounds of wave-wide maximum: each lane offers its largest
    // remaining key, the winner (keys are distinct) removes it; removed
    // keys are rebuilt afterwards.
    const int rounds = (k < n) ? k + 1 : k;
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
        const uint64_t kb = F.kb[lane + 64 * j];
        key[j] = (score_fixed10(sv[j]) + kb) & (0ull - static_cast<uint64_t>(kb != 0));
      }
  }
  // the key pair goes to the wave's LDS buffer; the caller writes the buffer
  // out in bursts (global stores inside the token loop would make every
  // token wait for the previous one's store acknowledgements)
  if (lane == 0) X.thb[wv][c.slot] = KeyPair{static_cast<int64_t>(thk), static_cast<int64_t>(thk1)};
  uint32_t selmask = 0;
#pragma unroll
  for (int j = 0; j < MAX_NJ; ++j)
    if (key[j] != 0 && key[j] >= thk) {
      selmask |= 1u << j;
      atomicAdd(&F.sload[lane + 64 * j], 1);
    }

  if (emit == 2) {
    // the k chosen (sfx, s, e) into this wave's LDS slots, then ranked by
    // descending raw score (ties to the lower index)
    int base = 0;
#pragma unroll
    for (int j = 0; j < MAX_NJ; ++j) {
      const bool sel = (selmask >> j) & 1u;
      const uint64_t bal = __ballot(sel);
      if (sel) {
        const int pos = base + __popcll(bal & ((uint64_t(1) << lane) - 1));
        X.emit.sfx[wv][pos] = score_fixed(sv[j]);
        X.emit.s[wv][pos] = sv[j];
        X.emit.e[wv][pos] = lane + 64 * j;
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
      my_sfx = X.emit.sfx[wv][lane];
      my_e = X.emit.e[wv][lane];
      my_s = X.emit.s[wv][lane];
      for (int i = 0; i < k; ++i) {
        const int64_t si = X.emit.sfx[wv][i];
        const int ei = X.emit.e[wv][i];
        rank += (si > my_sfx) || (si == my_sfx && ei < my_e);
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < k) X.emit.sorted[wv][rank] = my_s;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (lane < k) {
      float sum = 0.f;
      for (int i = 0; i < k; ++i) sum += X.emit.sorted[wv][i];
      a.idx[static_cast<size_t>(t) * k + rank] = my_e;
      a.w[static_cast<size_t>(t) * k + rank] = my_s / sum;
    }
    __builtin_amdgcn_wave_barrier();
  }

  if (emit == 1 && k < n) {
    // reduced cost rho_t(A,B) = Kp_A - Kp_B - [A > B] with Kp = sfx + bias
    const int64_t delta = c.delta;
    const int64_t kpk = static_cast<int64_t>(thk >> IDX_BITS) - KEY_OFFSET;
    const int64_t kpk1 = static_cast<int64_t>(thk1 >> IDX_BITS) - KEY_OFFSET;
    if (kpk - kpk1 <= delta + 1) {
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
            X.edge.lowKp[wv][pos] = kp;
            X.edge.lowE[wv][pos] = e;
          }
        }
        if (isHigh) {
          const int pos = nhigh + __popcll(bh & ((uint64_t(1) << lane) - 1));
          if (pos < EDGE_LIST_MAX) {
            X.edge.highKp[wv][pos] = kp;
            X.edge.highE[wv][pos] = e;
          }
        }
        nlow += __popcll(bl);
        nhigh += __popcll(bh);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (nlow > EDGE_LIST_MAX || nhigh > EDGE_LIST_MAX) {
        if (lane == 0) __hip_atomic_fetch_or(&a.cnt[N_OVERFLOW], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      } else {
        // the token's edges: lane ia pairs low candidate ia with every high
        // one (broadcast LDS reads); counted first, then one atomic reserves
        // them all
        const bool has = lane < nlow;
        const int A = has ? X.edge.lowE[wv][lane] : 0;
        const int64_t kA = has ? X.edge.lowKp[wv][lane] : 0;
        int mine = 0;
        for (int ib = 0; ib < nhigh; ++ib) {
          const int B = X.edge.highE[wv][ib];
          mine += has && kA - X.edge.highKp[wv][ib] - (A > B ? 1 : 0) <= delta;
        }
        int incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int u = __shfl_up(incl, off);
          if (lane >= off) incl += u;
        }
        const int total = __shfl(incl, 63);
        if (has && mine > 0) addc(&a.cnt[N_DEG0 + A], mine);
        if (total > 0) {
          int base = 0;
          if (lane == 0)
            base = __hip_atomic_fetch_add(&a.cnt[N_SEG0 + c.seg], total, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
          base = __shfl(base, 0);
          int pos = base + incl - mine;
          bool over = false;
          for (int ib = 0; ib < nhigh; ++ib) {
            const int B = X.edge.highE[wv][ib];
            const int64_t rho = kA - X.edge.highKp[wv][ib] - (A > B ? 1 : 0);
            if (has && rho <= delta) {
              if (pos < c.seg_cap)
                stc(&a.edges[static_cast<size_t>(c.seg) * c.seg_cap + pos],
                    (static_cast<uint64_t>(rho) << 20) | (static_cast<uint64_t>(A) << 10) |
                        static_cast<uint64_t>(B));
              else
                over = true;
              ++pos;
            }
          }
          if (__ballot(over) != 0 && lane == 0)
            __hip_atomic_fetch_or(&a.cnt[N_OVERFLOW], 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  return thk1;
}

// ---------------------------------------------------------------------------
// Quantile round for one unbalanced expert (whole block): the C-th and
// (C+1)-th largest margins over all tokens, exactly, and the new bias = minus
// their midpoint.
//
// Selection: one pass bins d = margin - cut (the cut is -1024*bias; d > 0 iff
// the token currently picks the expert) into 2048 order-preserving buckets
// that are exact near zero and ~6% wide far from it, a block scan finds the
// buckets holding the two ranks, a second pass gathers those one or two
// buckets into LDS and the ranks are resolved by exact counting.  A bucket
// too large for LDS falls back to an MSB-first radix select.
// ---------------------------------------------------------------------------
constexpr int QCH = 8;  // tokens per thread whose operands are requested together

// Margin of token t for expert e: its key without the bias minus the key the
// expert has to beat (the k-th key when e is not chosen, the (k+1)-th when it is).
__device__ __forceinline__ int64_t margin_from(float s, int64_t thk, int64_t thk1, int64_t be,
                                               int e, bool small) {
  const uint64_t base = (small ? score_fixed10(s) : score_fixed10_normal(s)) + key_bias(0, e);
  const bool sel = static_cast<int64_t>(base + (static_cast<uint64_t>(be) << IDX_BITS)) >= thk;
  return static_cast<int64_t>(base) - (sel ? thk1 : thk);
}

// th[] was written by other blocks in this launch: device-scope loads (an
// L2 invalidation instead would also evict the score rows every pass reads).
__device__ __forceinline__ int64_t margin_of(const Args& a, int64_t be, int e, int t, bool small) {
  return margin_from(a.scoresT[static_cast<size_t>(e) * a.T + t], ldc(&a.th[t].k),
                     ldc(&a.th[t].k1), be, e, small);
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
__device__ __attribute__((always_inline)) inline void radix_select2(const Args& a, QuantScratch& Q, bool small, int64_t be, int e, int64_t r1,
                              int64_t r2) {
  int32_t* h1 = Q.hist;
  int32_t* h2 = Q.hist + NBIN;
  if (threadIdx.x == 0) {
    Q.pre[0] = Q.pre[1] = 0;
    Q.rem[0] = r1;
    Q.rem[1] = r2;
  }
  __syncthreads();
  uint64_t mask = 0;
  for (int shift = 64; shift > 0;) {
    const int nbits = shift >= DIG ? DIG : shift;
    shift -= nbits;
    for (int i = threadIdx.x; i < NBIN; i += NT) h1[i] = h2[i] = 0;
    __syncthreads();
    const uint64_t p1 = Q.pre[0], p2 = Q.pre[1];
    const uint64_t dmask = (uint64_t(1) << nbits) - 1;
    for (int t = threadIdx.x; t < a.T; t += NT) {
      const uint64_t u = static_cast<uint64_t>(margin_of(a, be, e, t, small)) ^ (uint64_t(1) << 63);
      const int dg = static_cast<int>((u >> shift) & dmask);
      if ((u & mask) == p1) atomicAdd(&h1[dg], 1);
      if ((u & mask) == p2) atomicAdd(&h2[dg], 1);
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      int32_t* h = threadIdx.x == 0 ? h1 : h2;
      int64_t rem = Q.rem[threadIdx.x];
      int dsel = 0;
      for (int dgt = static_cast<int>(dmask); dgt >= 0; --dgt) {
        if (rem <= h[dgt]) {
          dsel = dgt;
          break;
        }
        rem -= h[dgt];
      }
      Q.rem[threadIdx.x] = rem;
      Q.pre[threadIdx.x] |= static_cast<uint64_t>(dsel) << shift;
    }
    mask |= dmask << shift;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    Q.val[0] = static_cast<int64_t>(Q.pre[0] ^ (uint64_t(1) << 63));
    Q.val[1] = static_cast<int64_t>(Q.pre[1] ^ (uint64_t(1) << 63));
  }
  __syncthreads();
}

// New bias of unbalanced expert e (returned to every thread).  One pass over
// the tokens bins the margins (and, when bcache has room for T entries,
// keeps each token's bucket in LDS); the gather pass then recomputes only
// the margins that fall in the buckets holding the wanted ranks.
__device__ __attribute__((always_inline)) inline int64_t quantile_bias(const Args& a,
                                                                      QuantScratch& Q,
                                                                      int16_t* bcache, int e,
                                                                      int64_t be, bool small) {
  const int T = a.T;
  const int64_t C = target(T, a.n, a.k, e);
  const int tid = opaque_tid();
  const int lane = tid & 63, wid = tid >> 6;
  const int64_t cut = -be * 1024;
  // LDS after the scratch: every margin (8 bytes a token) when it fits, else
  // every token's bucket (2 bytes), else every token's coarse bucket (1 byte:
  // the bucket / 8; the gather recomputes the margins of the tokens whose
  // coarse bucket can hold the wanted ranks), else nothing (the gather
  // recomputes every margin)
  const bool mcached = T <= a.bucket_cap / 4;
  const bool cached = !mcached && T <= a.bucket_cap;
  const bool ccached = !mcached && !cached && T <= 2 * a.bucket_cap;
  int64_t* mcache = reinterpret_cast<int64_t*>(bcache);
  uint8_t* ccache = reinterpret_cast<uint8_t*>(bcache);

  for (int i = tid; i < NBUCKET; i += NT) Q.hist[i] = 0;
  if (tid == 0) Q.cnt = 0;
  __syncthreads();
  const float* col = a.scoresT + static_cast<size_t>(e) * T;
  for (int t0 = 0; t0 < T; t0 += NT * QCH) {
    // every operand of the chunk is requested before any is used
    float sv[QCH];
    KeyPair thv[QCH];
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int t = t0 + tid + i * NT;
      if (t < T) {
        sv[i] = col[t];
        thv[i].k = ldc(&a.th[t].k);
        thv[i].k1 = ldc(&a.th[t].k1);
      }
    }
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int t = t0 + tid + i * NT;
      if (t < T) {
        const int64_t M = margin_from(sv[i], thv[i].k, thv[i].k1, be, e, small);
        const int b = bucket_of(M - cut);
        atomicAdd(&Q.hist[b], 1);
        if (mcached) mcache[t] = M;
        if (cached) bcache[t] = static_cast<int16_t>(b);
        if (ccached) ccache[t] = static_cast<uint8_t>(b >> 3);
      }
    }
  }
  __syncthreads();

  // descending ranks: r1 = C, r2 = C+1, or a single rank at the edges
  int64_t r1 = C, r2 = C + 1;
  if (C == 0) r1 = r2 = 1;
  if (C == T) r1 = r2 = T;
  // thread i owns the PER buckets below 2048 - PER*i: counts in descending
  // order; inclusive block scan = shuffle scan in the wave + wave offsets
  constexpr int PER = NBUCKET / NT;
  int32_t own = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) own += Q.hist[NBUCKET - 1 - (tid * PER + j)];
  int32_t incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) Q.wsum[wid] = incl;
  __syncthreads();
  if (tid < 64) {
    int32_t wsv = tid < NW ? Q.wsum[tid] : 0;
#pragma unroll
    for (int off = 1; off < NW; off <<= 1) {
      const int32_t u = __shfl_up(wsv, off);
      if (lane >= off) wsv += u;
    }
    if (tid < NW) Q.wsum[tid] = wsv;
  }
  __syncthreads();
  if (wid > 0) incl += Q.wsum[wid - 1];
  const int64_t before = incl - own;  // values in buckets above this thread's chunk
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t r = q == 0 ? r1 : r2;
    if (before < r && r <= incl) {
      int64_t acc = before;
      for (int j = 0; j < PER; ++j) {
        const int b = NBUCKET - 1 - (tid * PER + j);
        if (acc + Q.hist[b] >= r) {
          Q.bucket[q] = b;
          Q.above[q] = acc;
          break;
        }
        acc += Q.hist[b];
      }
    }
  }
  __syncthreads();
  const int b1 = Q.bucket[0], b2 = Q.bucket[1];  // b2 <= b1
  auto gather = [&](int64_t M) __attribute__((always_inline)) {
    const int pos = atomicAdd(&Q.cnt, 1);
    if (pos < GATHER_CAP) Q.gat[pos] = M;
  };
  if (mcached) {
    for (int t = tid; t < T; t += NT) {
      const int64_t M = mcache[t];
      const int b = bucket_of(M - cut);
      if (b <= b1 && b >= b2) gather(M);
    }
  } else if (cached) {
    for (int t = tid; t < T; t += NT) {
      const int b = bcache[t];
      if (b <= b1 && b >= b2) gather(margin_of(a, be, e, t, small));
    }
  } else if (ccached) {
    const int c1 = b1 >> 3, c2 = b2 >> 3;
    for (int t = tid; t < T; t += NT) {
      const int cb = ccache[t];
      if (cb <= c1 && cb >= c2) {
        const int64_t M = margin_of(a, be, e, t, small);
        const int b = bucket_of(M - cut);
        if (b <= b1 && b >= b2) gather(M);
      }
    }
  } else {
    for (int t = tid; t < T; t += NT) {
      const int64_t M = margin_of(a, be, e, t, small);
      const int b = bucket_of(M - cut);
      if (b <= b1 && b >= b2) gather(M);
    }
  }
  __syncthreads();
  const int cnt = Q.cnt;
  if (cnt <= GATHER_CAP) {
    // ranks inside the gathered set (everything in buckets above b1 is larger)
    const int64_t q1 = r1 - Q.above[0], q2 = r2 - Q.above[0];
    for (int i = tid; i < cnt; i += NT) {
      const int64_t v = Q.gat[i];
      int64_t g = 0, ge = 0;
      for (int j = 0; j < cnt; ++j) {
        const int64_t wv = Q.gat[j];
        g += wv > v;
        ge += wv >= v;
      }
      if (g < q1 && q1 <= ge) Q.val[0] = v;
      if (g < q2 && q2 <= ge) Q.val[1] = v;
    }
    __syncthreads();
  } else {
    radix_select2(a, Q, small, be, e, r1, r2);
  }
  const int64_t m1 = Q.val[0], m2 = Q.val[1];
  int64_t b;
  if (C == 0)
    b = -(m1 >> IDX_BITS) - 1;
  else if (C == T)
    b = -(m1 >> IDX_BITS) + 1;
  else
    b = -floor_mid(m1, m2);
  __syncthreads();  // the scratch is reused by the next expert
  return b;
}

// ---------------------------------------------------------------------------
// One augmenting-path move (block 0): shortest distances from the overloaded
// experts over this step's sparse edge list, then every expert drops by
// D - min(d, D) and the path to the nearest underloaded expert is shifted by
// one grid unit per hop.  The outcome goes to the ctrl words.
//
// The edges are grouped by source expert in LDS (counts come from the top-k
// pass) and relaxed level by level by the whole block: each pass relaxes the
// out-edges of the experts whose distance fell in the previous pass (16
// lanes per expert), until no distance falls.  Candidates above the best
// underloaded distance so far cannot lie on a path of length <= D*, so they
// are dropped; every distance <= D* and its predecessor (ties to the lower
// index, through the packed minimum) come out as the full relaxation gives
// them.  When the list outgrows the LDS cache the relaxation runs over the
// list in device memory instead.
// ---------------------------------------------------------------------------
__device__ __attribute__((always_inline)) inline void sap_move(const Args& a, Fixed& F,
                                                               SapScratch& P, uint64_t* csr,
                                                               int cur, int64_t delta) {
  const int n = a.n;
  const int tid = opaque_tid();
  const int lane = tid & 63, wid = tid >> 6;
  uint64_t* d = F.kb;          // packed (distance << 10 | predecessor)
  int32_t* cursor = F.sload;   // scatter cursors per source
  const int seg_cap = a.edge_cap / EDGE_SEGS;
  {  // segment offsets: exclusive scan of the (capped) segment counts
    static_assert(EDGE_SEGS == 256, "scan below: four waves of 64");
    int m = 0;
    if (tid < EDGE_SEGS) {
      m = ldc(&a.cnt[N_SEG0 + tid]);
      m = m < seg_cap ? m : seg_cap;
    }
    int incl = m;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off);
      if (lane >= off) incl += u;
    }
    if (tid < EDGE_SEGS && lane == 63) P.wsum4[wid] = incl;
    __syncthreads();
    if (tid < EDGE_SEGS) {
      int before = 0;
      for (int w = 0; w < wid; ++w) before += P.wsum4[w];
      P.seg_off[tid] = before + incl - m;
      if (tid == EDGE_SEGS - 1) P.seg_off[EDGE_SEGS] = before + incl;
    }
  }
  const bool overflow = ldc(&a.cnt[N_OVERFLOW]) != 0;
  __syncthreads();
  auto seg_of = [&](int i) __attribute__((always_inline)) {
    int lo = 0, hi = EDGE_SEGS - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (P.seg_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto edge_at = [&](int i) __attribute__((always_inline)) {
    const int sg = seg_of(i);
    return ldc(&a.edges[static_cast<size_t>(sg) * seg_cap + (i - P.seg_off[sg])]);
  };
  const int nedges = P.seg_off[EDGE_SEGS];
  // every segment counter, source count and the overflow flag are cleared by
  // the end of the move
  auto clear_edges = [&]() __attribute__((always_inline)) {
    if (tid < EDGE_SEGS) stc(&a.cnt[N_SEG0 + tid], 0);
    for (int e = tid; e < n; e += NT) stc(&a.cnt[N_DEG0 + e], 0);
    if (tid == 0) stc(&a.cnt[N_OVERFLOW], 0);
  };
  if (overflow) {
    if (tid == 0) {
      if (delta / 4 < DELTA_MIN) {
        stc(&a.ctrl[C_OUTCOME], static_cast<int64_t>(O_FAILED));
      } else {
        stc(&a.ctrl[C_OUTCOME], static_cast<int64_t>(O_RETRY));
        stc(&a.ctrl[C_DELTA], delta / 4);
      }
    }
    clear_edges();
    return;
  }
  // sources: overloaded experts at distance 0
  for (int e = tid; e < n; e += NT) {
    const int64_t C = target(a.T, n, a.k, e);
    const int32_t L = F.sL[e];
    P.over[e] = L > C;
    P.under[e] = L < C;
    P.pos[e] = 0;
    d[e] = L > C ? static_cast<uint64_t>(e) : PACKED_INF;
  }
  if (tid == 0) {
    P.D = static_cast<unsigned long long>(DIST_INF);
    P.bad = 0;
  }
  // (the source counts add up to the list length whenever nothing overflowed)
  const bool grouped = nedges <= a.edge_cache;
  if (grouped) {
    // sources' edge counts -> offsets (exclusive scan over the experts)
    {
      int c0 = 0, c1 = 0;
      static_assert(2 * NT >= 1024, "two experts per thread cover n <= 1024");
      const int e0 = 2 * tid, e1 = 2 * tid + 1;  // two experts per thread: n <= 1024
      if (e0 < n) c0 = ldc(&a.cnt[N_DEG0 + e0]);
      if (e1 < n) c1 = ldc(&a.cnt[N_DEG0 + e1]);
      const int own = c0 + c1;
      int incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
      }
      if (lane == 63) P.red[wid] = incl;
      __syncthreads();
      int before = 0;
      for (int w = 0; w < wid; ++w) before += P.red[w];
      const int ex = before + incl - own;
      if (e0 < n) { P.off[e0] = ex; cursor[e0] = ex; }
      if (e1 < n) { P.off[e1] = ex + c0; cursor[e1] = ex + c0; }
      if (tid == NT - 1) P.off[n] = before + incl;
      __syncthreads();
    }
    // one thread per segment, eight loads in flight at a time
    if (tid < EDGE_SEGS) {
      const int m = P.seg_off[tid + 1] - P.seg_off[tid];
      const uint64_t* src = a.edges + static_cast<size_t>(tid) * seg_cap;
      for (int i0 = 0; i0 < m; i0 += 8) {
        uint64_t ed[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) ed[q] = i0 + q < m ? ldc(&src[i0 + q]) : 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (i0 + q < m) {
            const int A = static_cast<int>((ed[q] >> 10) & 1023);
            const int at = atomicAdd(&cursor[A], 1);
            if (at < a.edge_cache) csr[at] = ((ed[q] >> 20) << 10) | (ed[q] & 1023);  // rho << 10 | B
          }
        }
      }
    }
    // Level-synchronous relaxation over the grouped edges: pass p relaxes the
    // out-edges of the experts whose distance fell (to at most P.D) in pass
    // p - 1; groups of 16 lanes take one expert each, the lanes its edges.
    for (int i = tid; i < 256; i += NT) P.inq[i] = 0;
    if (tid == 0) P.nfront[0] = P.nfront[1] = 0;
    __syncthreads();
    for (int e = tid; e < n; e += NT)  // the sources, in any order
      if (P.over[e]) P.front[0][atomicAdd(&P.nfront[0], 1)] = static_cast<int16_t>(e);
    __syncthreads();
    const int grp = tid >> 4, gl = tid & 15;
    constexpr int NGRP = NT / 16;
    int buf = 0, passes = 0;
    while (true) {
      const int ncur = P.nfront[buf];
      if (ncur == 0) break;
      if (++passes > 4096) {
        if (tid == 0) P.bad = 2;
        break;
      }
      for (int i = tid; i < ncur; i += NT) {
        const int v = P.front[buf][i];
        atomicAnd(&P.inq[v >> 2], ~(0xFFu << (8 * (v & 3))));
      }
      if (tid == 0) P.nfront[buf ^ 1] = 0;
      __syncthreads();
      for (int i = grp; i < ncur; i += NGRP) {
        const int v = P.front[buf][i];
        const int64_t dv = static_cast<int64_t>(d[v] >> IDX_BITS);
        if (dv > static_cast<int64_t>(P.D)) continue;
        const int jend = P.off[v + 1];
        for (int j = P.off[v] + gl; j < jend; j += 16) {
          const uint64_t ce = csr[j];
          const int B = static_cast<int>(ce & 1023);
          const int64_t cand = dv + static_cast<int64_t>(ce >> 10);
          if (cand > static_cast<int64_t>(P.D)) continue;
          const uint64_t pk = (static_cast<uint64_t>(cand) << IDX_BITS) | static_cast<uint64_t>(v);
          if (pk >= d[B]) continue;
          const uint64_t old = atomicMin(reinterpret_cast<unsigned long long*>(&d[B]), pk);
          if (pk >= old) continue;
          if (P.under[B]) atomicMin(&P.D, static_cast<unsigned long long>(cand));
          const uint32_t bit = 1u << (8 * (B & 3));
          if ((atomicOr(&P.inq[B >> 2], bit) & bit) == 0) {
            const int at = atomicAdd(&P.nfront[buf ^ 1], 1);
            P.front[buf ^ 1][at] = static_cast<int16_t>(B);
          }
        }
      }
      __syncthreads();
      buf ^= 1;
    }
    __syncthreads();
  } else {
    // Too many edges for LDS: Bellman-Ford passes over the list in memory.
    // A pass that lowers some distance to at most P.D asks for another pass;
    // flagging against the running value flags a superset of "changed at or
    // below the final D*", so the passes stop only when every distance <= D*
    // and its predecessor is final.
    if (tid < 3) P.flag[tid] = 0;
    __syncthreads();
    int passes = 0;
    while (true) {
      const int fi = passes % 3;
      if (tid == 0) P.flag[(passes + 1) % 3] = 0;
      for (int i = tid; i < nedges; i += NT) {
        const uint64_t ed = edge_at(i);
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
            if (P.under[B]) atomicMin(&P.D, static_cast<unsigned long long>(cand));
            if (static_cast<uint64_t>(cand) <= P.D) P.flag[fi] = 1;
          }
        }
      }
      __syncthreads();
      ++passes;
      if (!P.flag[fi] || passes > 4 * 1024) break;
    }
  }
  const int64_t D = static_cast<int64_t>(P.D);
  if (P.bad == 2) {  // the relaxation did not settle (cannot happen with costs >= 0)
    if (tid == 0) stc(&a.ctrl[C_OUTCOME], static_cast<int64_t>(O_FAILED));
    clear_edges();
    return;
  }
  if (D >= DIST_INF || D > delta) {
    if (tid == 0) {
      if (delta >= DELTA_MAX) {
        stc(&a.ctrl[C_OUTCOME], static_cast<int64_t>(O_FAILED));
      } else {
        stc(&a.ctrl[C_OUTCOME], static_cast<int64_t>(O_RETRY));
        stc(&a.ctrl[C_DELTA], delta * 16);
      }
    }
    clear_edges();
    return;
  }
  // u* = lowest underloaded expert at distance D
  {
    int u = 1 << 30;
    for (int e = tid; e < n; e += NT)
      if (P.under[e] && static_cast<int64_t>(d[e] >> IDX_BITS) == D) u = min(u, e);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) u = min(u, __shfl_xor(u, off));
    if (lane == 0) P.red[wid] = u;
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NW; ++w) u = min(u, P.red[w]);
      P.red[0] = u;
    }
    __syncthreads();
  }
  // the path from u* back to its source (an overloaded expert), in LDS
  if (tid == 0) {
    int v = P.red[0];
    int len = 0;
    bool ok = true;
    while (true) {
      P.path[len++] = static_cast<int16_t>(v);
      if (P.over[v]) break;
      v = static_cast<int>(d[v] & 1023);
      if (len > n) {
        ok = false;
        break;
      }
    }
    P.len = ok ? len : -1;
  }
  __syncthreads();
  const int len = P.len;
  if (len < 0) {
    if (tid == 0) stc(&a.ctrl[C_OUTCOME], static_cast<int64_t>(O_FAILED));
    clear_edges();
    return;
  }
  // the i-th expert from the source gains i grid units (P.path[len-1] is the
  // source, P.path[0] = u*); a vertex appears once on a predecessor path
  for (int i = tid; i < len; i += NT) P.pos[P.path[len - 1 - i]] = static_cast<int16_t>(i);
  __syncthreads();
  // every expert drops by D - min(d, D), then the path shift is added
  for (int e = tid; e < n; e += NT) {
    const int64_t dv = static_cast<int64_t>(d[e] >> IDX_BITS);
    const int64_t nbv = F.pb[e] + ((dv < D ? dv : D) - D) + P.pos[e];
    put_bias(a, cur, e, nbv);
    if (nbv >= BIAS_LIMIT || nbv <= -BIAS_LIMIT) P.bad = 1;
  }
  __syncthreads();
  if (tid == 0) stc(&a.ctrl[C_OUTCOME], static_cast<int64_t>(P.bad ? O_RANGE : O_MOVED));
  clear_edges();
}

// ---------------------------------------------------------------------------
// Block reductions (every thread gets the result).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_sum_i(Fixed& F, int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) F.red_i[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += F.red_i[w];
  return s;
}

__device__ __forceinline__ int block_max_i(Fixed& F, int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) F.red_i[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = F.red_i[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s = max(s, F.red_i[w]);
  return s;
}

__device__ __forceinline__ long long block_sum_l(Fixed& F, long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) F.red_l[threadIdx.x >> 6] = v;
  __syncthreads();
  long long s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += F.red_l[w];
  return s;
}

__device__ __forceinline__ uint64_t block_max_u(Fixed& F, uint64_t v) {
  v = wave_max_u64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) F.red_u[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s = F.red_u[w] > s ? F.red_u[w] : s;
  return s;
}

// ---------------------------------------------------------------------------
// The persistent routing loop (NJ = keys per lane, n <= 64 NJ).  Each wave
// ranks the tokens gw, gw + GW, ... and requests the next token's scores
// while the current one is ranked.
// ---------------------------------------------------------------------------
template <int NJ>
__global__ __launch_bounds__(NT) void route_loop(Args a) {
  extern __shared__ __align__(16) unsigned char lds[];
  Fixed& F = *reinterpret_cast<Fixed*>(lds);
  unsigned char* scratch = lds + align16(sizeof(Fixed));
  TopkScratch& X = *reinterpret_cast<TopkScratch*>(scratch);
  QuantScratch& Q = *reinterpret_cast<QuantScratch*>(scratch);
  SapScratch& P = *reinterpret_cast<SapScratch*>(scratch);
  uint64_t* ecache = reinterpret_cast<uint64_t*>(scratch + align16(sizeof(SapScratch)));
  int16_t* bcache = reinterpret_cast<int16_t*>(scratch + align16(sizeof(QuantScratch)));

  const int n = a.n, k = a.k, T = a.T;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int G = gridDim.x;
  const int gw = blockIdx.x * NW + wv, GW = G * NW;
  uint32_t bar_idx = 0;
  const bool small = ldc(&a.ctrl[C_SMALL]) != 0;

  // Lanes past the last expert read the last expert's score (in bounds, no
  // branch); their keys are zeroed (key_bias 0 in LDS).
  auto load_row = [&](float (&dst)[NJ], int t, int ln) __attribute__((always_inline)) {
    const float* row = a.scores + static_cast<size_t>(t) * n;
#pragma unroll
    for (int j = 0; j < NJ; ++j) dst[j] = row[min(ln + 64 * j, n - 1)];
  };

  // block-uniform state: every block takes the same decisions
  int phase;
  int status = static_cast<int>(ldc(&a.ctrl[C_STATUS0]));
  if (a.mode == MODE_FROZEN)
    phase = PH_FROZEN;
  else if (status != MOE_QB_STATUS_OK)
    phase = PH_FAILED;
  else
    phase = T > 0 ? PH_ROUNDS : PH_DONE;
  int cur = 0, par = 0, rounds = 0, moves = 0, best = -1, since = 0, steps = 0;
  int64_t delta = DELTA_START;
  bool pivots = false;  // piv / th[].k1 hold the last pass's (k+1)-th keys
  const int max_steps = a.mode == MODE_SIGN ? a.max_rounds + 2
                                            : a.max_rounds + 8 * MAX_SAP_MOVES + 64;

  TokenCtx c;
  c.n = n;
  c.k = k;
  c.lane = lane;
  c.wv = wv;
  c.seg = blockIdx.x & (EDGE_SEGS - 1);
  c.seg_cap = a.edge_cap / EDGE_SEGS;

  // Stages the live biases into LDS and returns the largest decrease since
  // the previous staging.
  auto stage = [&](int buf) __attribute__((always_inline)) -> uint64_t {
    const int64_t* b = bias_buf(a, blockIdx.x % BIAS_COPIES, buf);
    constexpr int SH = (1024 + NT - 1) / NT;  // experts per thread: n <= 1024
    int64_t v[SH];
#pragma unroll
    for (int h = 0; h < SH; ++h) {
      const int e = tid + h * NT;
      v[h] = e < n ? ldc(&b[e]) : 0;
    }
    uint64_t dmax = 0, bmax = 0;
#pragma unroll
    for (int h = 0; h < SH; ++h) {
      const int e = tid + h * NT;
      if (e >= n && e < 64 * NJ) {
        F.kb[e] = 0;
        F.bf[e] = -__builtin_huge_valf();
      }
      if (e < n) {
        const int64_t dec = F.pb[e] - v[h];
        if (dec > static_cast<int64_t>(dmax)) dmax = static_cast<uint64_t>(dec);
        const uint64_t ab = static_cast<uint64_t>(v[h] < 0 ? -v[h] : v[h]);
        bmax = ab > bmax ? ab : bmax;
        F.pb[e] = v[h];
        F.kb[e] = key_bias(v[h], e);
        F.bf[e] = static_cast<float>(static_cast<double>(v[h]) * 0x1p-40);
        F.sload[e] = 0;
      }
    }
    // |fp32(s + bf) - exact| <= (1 + 2 max|b|) 2^-24 + 2^-41; twice that
    c.err = (1.0 + 2.0 * static_cast<double>(block_max_u(F, bmax)) * 0x1p-40) * 0x1p-23 + 0x1p-40;
    return block_max_u(F, dmax);
  };

  // Phase A over this wave's tokens (the first token's operands are
  // requested before the live biases are staged).
  auto pass = [&](int emit) __attribute__((always_inline)) {
    const int otid = opaque_tid();
    const int ln = otid & 63, owv = otid >> 6;
    c.lane = ln;
    c.wv = owv;
    // the next token's scores are in flight while one is ranked
    float row[NJ], nxt[NJ];
    int t = gw;
    if (t < T) load_row(row, t, ln);
    const uint64_t drop = stage(cur);
    c.drop_key = drop << IDX_BITS;
    c.delta = delta;
    float bfr[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[j] = F.bf[ln + 64 * j];
    // key pairs of the buffered tokens gw + (first + i) GW, i < count
    auto flush_th = [&](int first, int count) __attribute__((always_inline)) {
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      if (ln < count) {
        const KeyPair v = X.thb[owv][ln];
        const int tt = gw + (first + ln) * GW;
        stc(&a.th[tt].k, v.k);
        stc(&a.th[tt].k1, v.k1);
      }
      __builtin_amdgcn_wave_barrier();
    };
    int i_tok = 0;
    c.slot = 0;
    for (; t < T; t += GW) {
      if (t + GW < T) load_row(nxt, t + GW, ln);
      // a wave's first 32 pivots live in LDS, later ones are read back
      uint64_t prev = 0;
      if (pivots)
        prev = i_tok < 32 ? F.piv[owv][i_tok] : static_cast<uint64_t>(ldc(&a.th[t].k1));
      const uint64_t k1 = topk_token<NJ>(a, F, X, c, row, bfr, t, prev, pivots, emit, small);
      if (i_tok < 32 && ln == 0) F.piv[owv][i_tok] = k1;
#pragma unroll
      for (int j = 0; j < NJ; ++j) row[j] = nxt[j];
      ++i_tok;
      if (++c.slot == THB) {
        flush_th(i_tok - THB, THB);
        c.slot = 0;
      }
    }
    if (c.slot) flush_th(i_tok - c.slot, c.slot);
    // per-block counts, one device atomic per expert the block selected
    __syncthreads();
    int32_t* acc = a.acc + (static_cast<size_t>(par) * ACC_COPIES + (blockIdx.x % ACC_COPIES)) * n;
    for (int e = tid; e < n; e += NT)
      if (F.sload[e]) addc(&acc[e], F.sload[e]);
  };

  // Loads of the pass into F.sL (every block), clearing the other parity's
  // counters for the next pass; returns (unbalanced count, max |L - C|).
  auto read_loads = [&](int& imb, int& res) __attribute__((always_inline)) {
    const int32_t* acc = a.acc + static_cast<size_t>(par) * ACC_COPIES * n;
    int my_imb = 0, my_res = 0;
    int32_t part[2][ACC_COPIES];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + h * NT;
#pragma unroll
      for (int r = 0; r < ACC_COPIES; ++r)
        part[h][r] = e < n ? ldc(&acc[static_cast<size_t>(r) * n + e]) : 0;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + h * NT;
      if (e >= n) continue;
      int32_t L = 0;
#pragma unroll
      for (int r = 0; r < ACC_COPIES; ++r) L += part[h][r];
      F.sL[e] = L;
      const int64_t d = static_cast<int64_t>(L) - target(T, n, k, e);
      my_imb += d != 0;
      const int ad = static_cast<int>(d < 0 ? -d : d);
      my_res = my_res > ad ? my_res : ad;
    }
    // this block's share of the other parity's counters
    int32_t* other = a.acc + static_cast<size_t>(par ^ 1) * ACC_COPIES * n;
    const int tot = ACC_COPIES * n;
    for (int i = blockIdx.x * NT + tid; i < tot; i += G * NT) stc(&other[i], 0);
    imb = block_sum_i(F, my_imb);
    res = block_max_i(F, my_res);
  };

  while (true) {
    // the last pass (loop over) writes the ordered outputs and the final
    // loads; the common offset (QB, balanced) moves every key of a token
    // alike, so the outputs are taken before it is removed
    const bool last = !(phase == PH_ROUNDS || phase == PH_SAP);
    if (T > 0) pass(last ? 2 : (phase == PH_SAP ? 1 : 0));
    if (!grid_sync(a, F, bar_idx)) return;
    if (last) break;
    pivots = true;
    int imb, res;
    read_loads(imb, res);
    ++steps;
    // decisions: the oracle's schedule, step by step
    bool do_round = false, do_move = false, do_sign = false;
    if (a.mode == MODE_SIGN) {
      if (imb == 0) {
        phase = PH_DONE;
      } else if (rounds >= a.max_rounds) {
        phase = PH_FAILED;
        status = MOE_QB_STATUS_NOT_BALANCED;
      } else {
        do_sign = true;
      }
    } else if (phase == PH_ROUNDS) {
      if (imb == 0) {
        phase = PH_DONE;
      } else if (rounds >= a.max_rounds) {
        phase = PH_SAP;
      } else if (best < 0 || imb < best) {
        best = imb;
        since = 0;
        do_round = true;
      } else if (++since >= STALL_ROUNDS) {
        phase = PH_SAP;
      } else {
        do_round = true;
      }
      // the pass that found the switch carried no edges: the next one does
    } else {  // PH_SAP
      if (imb == 0) {
        phase = PH_DONE;
      } else if (moves >= MAX_SAP_MOVES) {
        phase = PH_FAILED;
        status = MOE_QB_STATUS_NOT_BALANCED;
      } else {
        do_move = true;
      }
    }
    if (do_round) {
      // unbalanced experts in ascending order, shared out over the blocks
      if (tid == 0) F.nu = 0;
      __syncthreads();
      for (int e0 = 0; e0 < n; e0 += 64 * NW) {
        const int e = e0 + tid;
        const bool u = e < n && F.sL[e] != static_cast<int32_t>(target(T, n, k, e));
        const uint64_t bal = __ballot(u);
        if (lane == 0) F.red_i[wv] = __popcll(bal);
        __syncthreads();
        int before = F.nu;
        for (int w = 0; w < wv; ++w) before += F.red_i[w];
        if (u) F.ulist[before + __popcll(bal & ((uint64_t(1) << lane) - 1))] = static_cast<int16_t>(e);
        __syncthreads();
        if (tid == 0) {
          int s = 0;
          for (int w = 0; w < NW; ++w) s += F.red_i[w];
          F.nu += s;
        }
        __syncthreads();
      }
      const int nu = F.nu;
      // the lazy rule: balanced experts keep their bias
      for (int e = blockIdx.x * NT + tid; e < n; e += G * NT)
        if (F.sL[e] == static_cast<int32_t>(target(T, n, k, e))) put_bias(a, cur ^ 1, e, F.pb[e]);
      for (int i = blockIdx.x; i < nu; i += G) {
        const int e = F.ulist[i];
        const int64_t b = quantile_bias(a, Q, bcache, e, F.pb[e], small);
        if (tid < BIAS_COPIES) stc(&bias_buf(a, tid, cur ^ 1)[e], b);
        if (tid == 0 && (b >= BIAS_LIMIT || b <= -BIAS_LIMIT))
          __hip_atomic_fetch_or(&a.cnt[N_BIASRANGE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (do_move && blockIdx.x == 0) sap_move(a, F, P, ecache, cur, delta);
    if (do_sign && blockIdx.x == 0) {
      int bad = 0;
      for (int e = tid; e < n; e += NT) {
        const int64_t L = F.sL[e], C = target(T, n, k, e);
        const int64_t v = F.pb[e] + (L < C ? a.step : (L > C ? -a.step : 0));
        put_bias(a, cur, e, v);
        bad |= (v >= BIAS_LIMIT || v <= -BIAS_LIMIT);
      }
      if (bad)
        __hip_atomic_fetch_or(&a.cnt[N_BIASRANGE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!grid_sync(a, F, bar_idx)) return;
    par ^= 1;
    if (do_round) {
      cur ^= 1;
      rounds += 1;
      if (ldc(&a.cnt[N_BIASRANGE]) != 0) {
        phase = PH_FAILED;
        status = MOE_QB_STATUS_BIAS_RANGE;
      }
    }
    if (do_sign) {
      rounds += 1;
      if (ldc(&a.cnt[N_BIASRANGE]) != 0) {
        phase = PH_FAILED;
        status = MOE_QB_STATUS_BIAS_RANGE;
      }
    }
    if (do_move) {
      const int64_t o = ldc(&a.ctrl[C_OUTCOME]);
      if (o == O_MOVED || o == O_RANGE) {
        moves += 1;
        if (o == O_RANGE) {
          phase = PH_FAILED;
          status = MOE_QB_STATUS_BIAS_RANGE;
        }
      } else if (o == O_RETRY) {
        delta = ldc(&a.ctrl[C_DELTA]);
      } else {
        phase = PH_FAILED;
        status = MOE_QB_STATUS_NOT_BALANCED;
      }
    }
    if ((phase == PH_ROUNDS || phase == PH_SAP) && steps >= max_steps) {
      phase = PH_FAILED;
      status = MOE_QB_STATUS_NOT_BALANCED;
    }
  }

  if (blockIdx.x != 0) return;
  int imb, res;
  {
    const int32_t* acc = a.acc + static_cast<size_t>(par) * ACC_COPIES * n;
    int my_res = 0;
    for (int e = tid; e < n; e += NT) {
      int32_t L = 0;
#pragma unroll
      for (int r = 0; r < ACC_COPIES; ++r) L += ldc(&acc[static_cast<size_t>(r) * n + e]);
      a.loads[e] = L;
      const int64_t d = static_cast<int64_t>(L) - target(T, n, k, e);
      const int ad = static_cast<int>(d < 0 ? -d : d);
      my_res = my_res > ad ? my_res : ad;
    }
    res = block_max_i(F, my_res);
    (void)imb;
  }
  const int64_t* b = bias_buf(a, 0, cur);
  long long off = 0;
  if (a.mode == MODE_QB && phase == PH_DONE) {
    long long my = 0;
    for (int e = tid; e < n; e += NT) my += ldc(&b[e]);
    const long long sum = block_sum_l(F, my);
    off = sum / n;
    if ((sum % n != 0) && (sum < 0)) off -= 1;  // floor division
  }
  if (a.bias_out)
    for (int e = tid; e < n; e += NT)
      a.bias_out[e] = static_cast<double>(ldc(&b[e]) - off) * (1.0 / 1099511627776.0);
  if (tid == 0 && a.info) {
    a.info[0] = rounds;
    a.info[1] = status;
    a.info[2] = res;
    a.info[3] = a.mode == MODE_QB ? moves : 0;
  }
}

// ---------------------------------------------------------------------------
// Set-up and wrap-up kernels.
// ---------------------------------------------------------------------------
// One block of 1024: biases from the caller (fp64 -> grid units, with a range
// check), every counter, flag and barrier word cleared.
__global__ void route_init(Args a, const double* bias_in) {
  const int n = a.n;
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const double b = bias_in ? bias_in[e] : 0.0;
    const double bf = rint(b * 1099511627776.0);
    int64_t v = 0;
    if (!(fabs(bf) < static_cast<double>(BIAS_LIMIT)))
      s_bad = 1;
    else
      v = static_cast<int64_t>(bf);
    for (int c = 0; c < 2 * BIAS_COPIES; ++c) a.bfx[static_cast<size_t>(c) * n + e] = v;
  }
  for (int i = threadIdx.x; i < 2 * ACC_COPIES * n; i += blockDim.x) a.acc[i] = 0;
  for (int i = threadIdx.x; i < BAR_WORDS; i += blockDim.x) a.bar[i] = 0;
  for (int i = threadIdx.x; i < N_COUNT; i += blockDim.x) a.cnt[i] = 0;
  __syncthreads();
  if (threadIdx.x < C_COUNT) a.ctrl[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    a.ctrl[C_STATUS0] = s_bad ? MOE_QB_STATUS_BIAS_RANGE : MOE_QB_STATUS_OK;
    if (a.info) a.info[0] = a.info[1] = a.info[2] = a.info[3] = 0;
  }
}

// After the loop: a barrier wait that timed out voids the outputs.
__global__ void route_finish(Args a) {
  if (threadIdx.x == 0 && a.info && a.bar[BAR_LINE] != 0u) a.info[1] = STATUS_ABORTED;
}

// Scores before the loop: the transposed copy [n][T] (quantile rounds only)
// and the flag of scores below 2^-17 (zero and subnormals included).
__global__ void prep_scores(const float* __restrict__ in, float* __restrict__ out, int T, int n,
                            int64_t* ctrl) {
  __shared__ float tile[64][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 256 threads: 64 x 4
  int small = 0;
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + r, e = e0 + tx;
    const float v = (t < T && e < n) ? in[static_cast<size_t>(t) * n + e] : 1.f;
    small |= ((__float_as_uint(v) >> 23) & 255u) < 110u;
    tile[r][tx] = v;
  }
  small = __syncthreads_or(small);
  if (small && threadIdx.x == 0)
    atomicOr(reinterpret_cast<unsigned long long*>(&ctrl[C_SMALL]), 1ull);
  if (!out) return;
  for (int r = ty; r < 64; r += 4) {
    const int e = e0 + r, t = t0 + tx;
    if (e < n && t < T) out[static_cast<size_t>(e) * T + t] = tile[tx][r];
  }
}

}  // namespace qb

// ---------------------------------------------------------------------------
// Host driver.
// ---------------------------------------------------------------------------

// Edge list: 16 per token on average plus, in every segment, room for the
// largest list one token can emit (64 x 64); T <= MOE_MAX_TOKENS keeps it in
// 32 bits.
static int32_t edge_capacity(int32_t T) { return 16 * T + qb::EDGE_SEGS * 4096; }
static_assert(16ll * MOE_MAX_TOKENS + qb::EDGE_SEGS * 4096ll < (1ll << 31), "edge count in 32 bits");

size_t route_workspace_layout(int32_t T, int32_t n, RouteWorkspace* ws, void* base) {
  Carver cv(base);
  RouteWorkspace w;
  w.scoresT = cv.take<float>(static_cast<size_t>(T) * n);
  w.bfx = cv.take<int64_t>(2 * static_cast<size_t>(qb::BIAS_COPIES) * n);
  w.th = cv.take<KeyPair>(T);
  w.loads = cv.take<int32_t>(n);
  w.acc = cv.take<int32_t>(2 * static_cast<size_t>(qb::ACC_COPIES) * n);
  w.bar = cv.take<uint32_t>(qb::BAR_WORDS);
  w.ctrl = cv.take<int64_t>(qb::C_COUNT);
  w.cnt = cv.take<int32_t>(qb::N_COUNT);
  w.edge_cap = edge_capacity(T);
  w.edges = cv.take<uint64_t>(w.edge_cap);
  if (ws) *ws = w;
  return cv.bytes();
}

int route_validate(int32_t T, int32_t n, int32_t k) {
  if (T < 0 || n < 1 || k < 1 || k > n) return MOE_EINVAL;
  if (n > 1024 || k > qb::MAX_K || T > MOE_MAX_TOKENS) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

namespace {

// Per-device launch facts (filled once per device, under a mutex).
struct LoopDevice {
  bool ok = false;
  int cus = 0;
  uint64_t ticks_per_s = 0;
};

constexpr int LDS_CACHE_MAX = 13824;  // edges (108 KB)
static_assert(qb::lds_bytes(LDS_CACHE_MAX) <= 160 * 1024, "LDS of one block");

// Instantiated key counts per lane; a batch takes the smallest >= ceil(n / 64).
constexpr int NJ_VARIANTS[6] = {1, 2, 4, 8, 14, 16};

const void* loop_fn(int vi) {
  switch (vi) {
    case 0: return reinterpret_cast<const void*>(qb::route_loop<1>);
    case 1: return reinterpret_cast<const void*>(qb::route_loop<2>);
    case 2: return reinterpret_cast<const void*>(qb::route_loop<4>);
    case 3: return reinterpret_cast<const void*>(qb::route_loop<8>);
    case 4: return reinterpret_cast<const void*>(qb::route_loop<14>);
    default: return reinterpret_cast<const void*>(qb::route_loop<16>);
  }
}

LoopDevice* loop_device() {
  static LoopDevice tab[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  LoopDevice& d = tab[dev];
  if (!d.ok) {
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return nullptr;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      khz = 100000;  // 100 MHz
    d.ticks_per_s = static_cast<uint64_t>(khz) * 1000ull;
    const int lds = static_cast<int>(qb::lds_bytes(LDS_CACHE_MAX));
    for (int vi = 0; vi < 6; ++vi) {
      if (hipFuncSetAttribute(loop_fn(vi), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
          hipSuccess)
        return nullptr;
    }
    d.ok = true;
  }
  return &d;
}

}  // namespace

// Routes T tokens from fp32 scores: mode MOE_QB_FROZEN / MOE_QB_BATCH, or the
// sign rule (sign_step > 0).  Every launch goes onto `stream`; nothing waits
// on the host.
static int route_launch(const float* scores, int32_t T, int32_t n, int32_t k, int mode,
                        int32_t max_rounds, int64_t sign_step, double* bias_in,
                        double* bias_out, int32_t* idx, float* w, int32_t* loads_out,
                        int32_t* info, const RouteWorkspace& ws, hipStream_t stream,
                        int cu_share) {
  using namespace qb;
  LoopDevice* dv = loop_device();
  if (!dv) return MOE_EHIP;
  Args a{};
  a.scores = scores;
  a.scoresT = ws.scoresT;
  a.T = T;
  a.n = n;
  a.k = k;
  a.mode = mode;
  a.max_rounds = max_rounds;
  a.step = sign_step;
  a.bfx = ws.bfx;
  a.th = ws.th;
  a.acc = ws.acc;
  a.bar = ws.bar;
  a.ctrl = ws.ctrl;
  a.cnt = ws.cnt;
  a.edges = ws.edges;
  a.edge_cap = ws.edge_cap;
  a.timeout = 2ull * dv->ticks_per_s;  // 2 s per barrier wait
  a.idx = idx;
  a.w = w;
  a.loads = loads_out ? loads_out : ws.loads;
  a.info = info;
  a.bias_out = bias_out;

  // grid: one block per CU (fewer for tiny batches is not worth a second
  // code path: idle blocks only join the barriers)
  // cu_share: fraction of the CUs (1/cu_share) the loop may take, leaving the
  // rest to work on other streams
  const int G = std::max(1, std::min(dv->cus / std::max(cu_share, 1), MAX_GRID));
  const int nj = (n + 63) / 64;
  int vi = 0;
  while (NJ_VARIANTS[vi] < nj) ++vi;
  int cache = static_cast<int>(std::min<int64_t>(LDS_CACHE_MAX, std::max<int64_t>(2048, 2 * int64_t(T))));
  const size_t lds = lds_bytes(cache);
  a.edge_cache = cache;
  a.bucket_cap = static_cast<int32_t>(
      (lds - align16(sizeof(Fixed)) - align16(sizeof(QuantScratch))) / sizeof(int16_t));
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, loop_fn(vi), NT, lds) != hipSuccess ||
      occ < 1)
    return MOE_EHIP;

  hipLaunchKernelGGL(route_init, dim3(1), dim3(1024), 0, stream, a, bias_in);
  MOE_LAUNCH_CHECK();
  if (T > 0) {
    dim3 tg((T + 63) / 64, (n + 63) / 64);
    hipLaunchKernelGGL(prep_scores, tg, dim3(256), 0, stream, scores,
                       mode == MODE_QB ? ws.scoresT : nullptr, T, n, ws.ctrl);
    MOE_LAUNCH_CHECK();
  }
  switch (vi) {
    case 0: hipLaunchKernelGGL(route_loop<1>, dim3(G), dim3(NT), lds, stream, a); break;
    case 1: hipLaunchKernelGGL(route_loop<2>, dim3(G), dim3(NT), lds, stream, a); break;
    case 2: hipLaunchKernelGGL(route_loop<4>, dim3(G), dim3(NT), lds, stream, a); break;
    case 3: hipLaunchKernelGGL(route_loop<8>, dim3(G), dim3(NT), lds, stream, a); break;
    case 4: hipLaunchKernelGGL(route_loop<14>, dim3(G), dim3(NT), lds, stream, a); break;
    default: hipLaunchKernelGGL(route_loop<16>, dim3(G), dim3(NT), lds, stream, a); break;
  }
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(route_finish, dim3(1), dim3(64), 0, stream, a);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int route_run(const float* scores, int32_t T, int32_t n, int32_t k, int32_t mode,
              int32_t max_rounds, double* bias, int32_t* idx, float* w, int32_t* loads_out,
              int32_t* info, const RouteWorkspace& ws, hipStream_t stream, int cu_share) {
  if (max_rounds <= 0) max_rounds = 64;
  const bool batch = mode == MOE_QB_BATCH;
  return route_launch(scores, T, n, k, batch ? qb::MODE_QB : qb::MODE_FROZEN, max_rounds, 0, bias,
                      batch ? bias : nullptr, idx, w, loads_out, info, ws, stream, cu_share);
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
                        ws, static_cast<hipStream_t>(stream), 1);
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
  return moe::route_launch(scores, T, n, k, moe::qb::MODE_SIGN, max_rounds,
                           static_cast<int64_t>(sf), bias, bias, topk_idx, topk_w, loads, qb_info,
                           ws, static_cast<hipStream_t>(stream), 1);
}

// ---------------------------------------------------------------------------
// Routing without a caller workspace: the scratch lives in a file-scope
// device array of MOE_ROUTE_SCRATCH_BYTES, one per GPU, whose device address
// is looked up once per device.  Every call on a GPU reuses that GPU's array
// (the routing kernels clear what must start at zero), so calls that overlap
// on one GPU race.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[MOE_ROUTE_SCRATCH_BYTES];

// Device address of this device's scratch array (null when the lookup fails).
void* route_scratch() {
  static void* addr[64] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" int moe_route_qb_noalloc(const float* scores, int32_t T, int32_t n, int32_t k,
                                    int32_t mode, int32_t max_rounds, double* bias,
                                    int32_t* topk_idx, float* topk_w, int32_t* loads,
                                    int32_t* qb_info, void* stream) {
  int st = moe::route_validate(T, n, k);
  if (st != MOE_OK) return st;
  if (mode != MOE_QB_BATCH && mode != MOE_QB_FROZEN) return MOE_EINVAL;
  if ((T > 0 && (!scores || !topk_idx || !topk_w)) || !bias) return MOE_EINVAL;
  if (moe::route_workspace_layout(T, n, nullptr, nullptr) > MOE_ROUTE_SCRATCH_BYTES)
    return MOE_EWORKSPACE;
  void* base = route_scratch();
  if (!base) return MOE_EHIP;
  moe::RouteWorkspace ws;
  moe::route_workspace_layout(T, n, &ws, base);
  moe::prof::Scope sc(moe::prof::ST_ROUTING, static_cast<hipStream_t>(stream));
  return moe::route_run(scores, T, n, k, mode, max_rounds, bias, topk_idx, topk_w, loads, qb_info,
                        ws, static_cast<hipStream_t>(stream), 1);
}

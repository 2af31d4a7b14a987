// Budget eviction, compaction and append of the new token.
//
// CONF-KV summary, "Methodik: CONF-KV": tokens are ranked by the composite
// score, the newest P are never evicted (Token-Ranking und Eviktion), and
// the survivors are packed contiguously so attention reads a dense layout
// without indirection tables (Implementierung). Review "方法步骤详情"
// (Algorithm 1): if |C_l| > N evict the lowest-ranked unprotected tokens and
// compact the survivors; step 13 appends the new K/V in FP16.
//
// Plan kernel, one workgroup per (layer, sequence); thread t owns a contiguous
// run of logical indices:
//  1. k = n - N tokens leave, chosen among all but the newest P (the last P
//     logical entries): exactly the k smallest 64-bit keys (order-preserving
//     image of the fp32 score, position), so equal scores evict the older
//     token first. The k-th key is found from a 1024-bucket histogram of the
//     monotone bucket floor(score * 1024) (clamped), then by ranking the few
//     keys of the boundary bucket; radix selects on the score bits and then
//     on the tied positions cover crowded buckets and long caches.
//     Block eviction (B > 0) takes kb = min(full blocks, ceil(k / B)) whole
//     blocks of B consecutive candidates instead, the blocks with the
//     smallest (largest key in the block, block index), so k = kb * B.
//  2. Ballot bit-plane scans give each survivor its new logical index and
//     each region (INT8 ring, FP16 ring) its eviction count and first / last
//     hole.
//  3. Token eviction in the fill order (kFill) does everything in this
//     kernel: the surviving INT8 tokens at or beyond the new INT8 length fill
//     the holes below it (slot order; sources and destinations are disjoint,
//     so the rows move in one pass), the FP16 part is packed toward the end
//     that moves fewer rows (keep the base and shift the survivors after the
//     first hole down, or advance the base and shift the survivors before the
//     last hole up), and the new token's rows are appended. EMA / position
//     metadata are rewritten in place after a barrier that follows every
//     read. The fused form (FUSE) starts with the EMA update and rank scores
//     and may end with the window step of the quantisation.
//  4. Token eviction in the stable order (kStable, the default) and block
//     eviction (kBlock) pack both regions that way. A (layer, sequence)
//     with nothing to move is finished here (append, window step), and so
//     is every pair of a launch over at most kPlanMovePairs pairs (its rows
//     move in this workgroup, in rounds, as the move kernel moves them); the
//     others are flagged for:
// Move kernel (a fixed grid over the flagged (layer, sequence, kv head)
// items): the planned rows of a head's rings move in rounds (read all rows
// of a round, wait, write them) in an order that never overwrites an unread
// source; then the new token's rows are written to the FP16 rings, and in
// the fused form the head's window step follows.
#include <type_traits>

#include "confidence_dev.h"
#include "quantize_seq.h"

namespace confk {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRegKeys = 8;    // indices per thread held in registers
// plan kernel modes: token eviction with INT8 hole filling, token eviction
// with stable packing, block eviction (stable packing)
constexpr int kFill = 0, kStable = 1, kBlock = 2;
constexpr int kBuckets = 1024;
constexpr int kRankMax = 64;   // boundary-bucket keys ranked by one wave
constexpr int kHdr = 16;       // plan header words per (layer, sequence)
static_assert(2 * kMaxEvictBlocks <= kBuckets, "block keys and flags share the histogram");
// 16-byte pieces per thread per round of the move kernel (half K, half V):
// 192 INT8 or 96 FP16 rows of a head per round at d = 128
#ifndef CONFK_MOVE_ROUND
#define CONFK_MOVE_ROUND 12
#endif
constexpr int kMoveRound = CONFK_MOVE_ROUND;
constexpr int kMaxHeadDim = kMaxMoveHeadDim;  // move kernel's window step (scales in shared memory)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// plan header words (the move kernel's instructions for one (layer, sequence)):
// per region movers, packing side, evictions, first moved new index; the old
// ring bases; the new token's FP16 slot (-1: nothing left to do); the window
// step's token count and whether it calibrates; the new ring bases and INT8
// length after the packing
enum { H_MOV8 = 0, H_LEFT8, H_E8, H_JLO8, H_MOV16, H_LEFT16, H_E16, H_JLO16, H_BASE8, H_BASE16,
       H_APPEND, H_Q, H_CAL, H_B8N, H_B16N, H_M8 };
constexpr int kMoveThreads = 256;  // move kernel workgroup: one (layer, sequence, kv head) item at a time
constexpr int kMoveGrid = 1024;    // move kernel workgroups at most (4 per compute unit)
constexpr int kPlanMovePairs = 16; // launches over at most this many (layer, sequence) pairs move rows in the plan kernel

// Order-preserving uint32 image of an fp32 score; NaN sorts above +inf
// (0xFFFFFFFF stays free as the "not a candidate" key).
__device__ __forceinline__ uint32_t ord_bits(float f) {
  if (f != f) return 0xFFFFFFFEu;
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Monotone (non-decreasing) bucket of a score; NaN goes to the top.
__device__ __forceinline__ int bucket_of(float s) {
  if (!(s >= 0.f)) return s < 0.f ? 0 : kBuckets - 1;
  const float x = s * (float)kBuckets;
  return x >= (float)(kBuckets - 1) ? kBuckets - 1 : (int)x;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Wave exclusive prefix and total of small non-negative counts (< 16).
__device__ __forceinline__ int wave_prefix16(int x, int& total) {
  const uint64_t lt = lanemask_lt();
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint64_t m = __ballot((x >> b) & 1);
    pre += __popcll(m & lt) << b;
    tot += __popcll(m) << b;
  }
  total = tot;
  return pre;
}

// A pointer every lane holds the same value of, in scalar registers.
__device__ __forceinline__ unsigned char* uniform_ptr(const void* p) {
  const uint64_t rp = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)rp);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(rp >> 32));
  return (unsigned char*)(((uint64_t)hi << 32) | lo);
}

struct Shared {
  uint32_t hist[kBuckets];
  float rmax[kWaves];  // fused EMA: per-wave max EMA and position range
  int rpmin[kWaves], rpmax[kWaves];
  int wsum[4][kWaves];  // per-wave keeps, e8, e16, window-step tokens
  int wfill[2][kWaves];  // per-wave INT8 holes and tails
  int wfirst[2][kWaves], wlast[2][kWaves];
  uint64_t rank_keys[kRankMax];
  int rank_n;
  int sel_bucket, sel_below, sel_crowded;
  uint64_t kth;
  uint32_t sel_digit, sel_before;
};

// Tails' metadata and the fill lists of register-held runs (fewer than
// n8 / 2 <= kFillMax holes when n < kRegKeys * kThreads).
constexpr int kFillMax = kRegKeys * kThreads / 2;
struct FillShared {
  float e[kFillMax];
  int32_t p[kFillMax], i[kFillMax], h[kFillMax];
};
// The fused EMA phase hands its results (EMA, position per logical index)
// from lane-strided to run-contiguous ownership through the same LDS, before
// the fill lists are written.
union RegShared {
  FillShared fill;
  struct {
    float e[kRegKeys * kThreads];
    int32_t p[kRegKeys * kThreads];
  } x;
};

// Workspace words per (layer, sequence) for long caches: staged metadata of
// the survivors (EMA, position, old index) and the fill lists.
__host__ __device__ constexpr size_t stage_words(int cap) { return 5 * (size_t)cap + 8; }

struct Region {
  int rs, m, e, first_ev, last_ev;
  int left, movers, jlo;
};

__device__ __forceinline__ void plan_region(Region& r) {
  r.left = 1;
  r.movers = 0;
  r.jlo = 0;
  if (r.e == 0) return;
  const int mk = r.m - r.e;                           // survivors
  const int cost_l = mk - (r.first_ev - r.rs);        // survivors after the first hole
  const int cost_r = (r.last_ev - r.rs) - (r.e - 1);  // survivors before the last hole
  r.left = cost_l <= cost_r;
  r.movers = r.left ? cost_l : cost_r;
  r.jlo = r.left ? (r.first_ev - r.rs) : 0;
}

// Radix select of the kk-th smallest value val(j) among this workgroup's
// entries with part(j) (j < cnt of each thread's run); leaves in kk how many
// entries equal to the result are selected.
template <bool REG, typename Part, typename Val>
__device__ uint32_t radix_select(int& kk, int cnt, Part part, Val val, Shared& sh) {
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0;
    __syncthreads();
    auto count = [&](int j) {
      if (part(j)) {
        const uint32_t x = val(j);
        if ((x & mask) == prefix) atomicAdd(&sh.hist[(x >> shift) & 255u], 1u);
      }
    };
    if constexpr (REG) {
#pragma unroll
      for (int j = 0; j < kRegKeys; ++j)
        if (j < cnt) count(j);
    } else {
      for (int j = 0; j < cnt; ++j) count(j);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const uint32_t h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1], h2 = sh.hist[4 * lane + 2],
                     h3 = sh.hist[4 * lane + 3];
      const int s = (int)(h0 + h1 + h2 + h3);
      int incl = s;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const int excl = incl - s;
      if (excl < kk && kk <= incl) {
        const int c0 = excl + (int)h0, c1 = c0 + (int)h1, c2 = c1 + (int)h2;
        const int q = c0 >= kk ? 0 : (c1 >= kk ? 1 : (c2 >= kk ? 2 : 3));
        sh.sel_digit = (uint32_t)(4 * lane + q);
        sh.sel_before = (uint32_t)(q == 0 ? excl : (q == 1 ? c0 : (q == 2 ? c1 : c2)));
      }
    }
    __syncthreads();
    prefix |= sh.sel_digit << shift;
    mask |= 0xFFu << shift;
    kk -= (int)sh.sel_before;
  }
  return prefix;
}

// Stable packing of one ring kind (INT8, or FP16 with F16) of every kv head
// of a (layer, sequence), in the plan workgroup (small launches, where a
// second kernel's launch would cost more than the rounds here). lst holds
// the movers' region-local old indices in move order; mover r goes to
// region-local new index j = jlo + r (left) or jlo + mv - 1 - r, slot
// base + j (+ e on the right side). A round reads kPlanMoveRound (mover,
// head) rows of K and of V per thread, waits, and writes them; round r+1
// reads only slots beyond round r's destinations in the packing direction
// (per head), so a round needs one barrier. Thread t takes piece column
// t % P of (mover, head) pairs t / P, t / P + cpp, ... in mover-major order;
// loads and stores are unconditional (pairs past the last take the last
// pair's piece and write it again: same bytes, same place).
constexpr int kPlanMoveRound = 4;
template <bool F16>
__device__ __forceinline__ void move_ring(const CacheView& c, int lbc, int mv, int left, int e, int jlo, int base,
                                          const int32_t* lst) {
  typedef __attribute__((address_space(1))) u32x4 gvec;
  constexpr int U = kPlanMoveRound;
  if (mv == 0) return;  // uniform
  const int H = c.hkv, d = c.d;
  const int P = F16 ? d >> 3 : d >> 4;  // 16-byte pieces per row of one head
  const uint32_t rowb = F16 ? 2u * (uint32_t)d : (uint32_t)d;
  const int C = F16 ? c.cap16 : c.cap;
  const uint32_t ring = (uint32_t)C * rowb;  // bytes per ring of one head
  const size_t lbo = (size_t)lbc * H * ring;
  gvec* kg = (gvec*)uniform_ptr((F16 ? reinterpret_cast<const unsigned char*>(c.k16)
                                     : reinterpret_cast<const unsigned char*>(c.k8)) + lbo);
  gvec* vg = (gvec*)uniform_ptr((F16 ? reinterpret_cast<const unsigned char*>(c.v16)
                                     : reinterpret_cast<const unsigned char*>(c.v8)) + lbo);
  const int cpp = kThreads / P;  // (mover, head) pairs per pass
  const int q = threadIdx.x / P, pc = threadIdx.x - q * P;
  const int npair = mv * H;
  for (int c0 = 0; c0 < npair; c0 += U * cpp) {
    u32x4 v[2 * U];
    uint32_t dof[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cu = min(c0 + q + u * cpp, npair - 1);
      const int r = cu / H, h = cu - r * H;
      int ss = base + lst[r];
      ss = ss >= C ? ss - C : ss;
      const uint32_t hb = (uint32_t)h * ring + (uint32_t)pc * 16u;
      v[u] = kg[(hb + (uint32_t)ss * rowb) >> 4];
      v[U + u] = vg[(hb + (uint32_t)ss * rowb) >> 4];
      const int j = jlo + (left ? r : mv - 1 - r);
      int ds = base + (left ? j : j + e);
      ds = ds >= C ? ds - C : ds;
      dof[u] = (hb + (uint32_t)ds * rowb) >> 4;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every source of the round has been read
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kg[dof[u]] = v[u];
      vg[dof[u]] = v[U + u];
    }
  }
}

// FUSE: the EMA update and rank scores of ema_rank_kernel run first, in this
// kernel, with the same arithmetic and summation order (bit-identical).
// REG: the form for a cache of at most kRegKeys * kThreads tokens with the
// new one (keys and fill lists in registers and LDS); the long form stages
// through the workspace.
template <bool REG, int MODE, bool FUSE>
__device__ __forceinline__ void plan_body(const CompactArgs& a) {
  // MODE: kStable (token eviction, both regions packed stably), kBlock (block
  // eviction, packed stably) or kFill (token eviction, INT8 holes filled from
  // the INT8 tail). Stable packing leaves its row moves (and then the append
  // and the window step) to the move kernel, except in launches over few
  // (layer, sequence) pairs (a.plan_moves), which move them here as the fill
  // order moves its few rows.
  constexpr bool BLOCK = MODE == kBlock;   // block selection
  constexpr bool MOVEK = MODE != kFill;    // rows moved by the move kernel
  const CacheView& c = a.c;
  const int lb = blockIdx.x;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  const int cap = c.cap;
  int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  int32_t* hdr = a.plan + (size_t)lb * (kHdr + 2 * (size_t)cap);
  int32_t* src8 = hdr + kHdr;
  int32_t* src16 = src8 + cap;
  const int n = meta[CONFK_META_N];
  const int n8 = meta[CONFK_META_N8];
  const int base8 = meta[CONFK_META_BASE8];
  const int base16 = meta[CONFK_META_BASE16];
  const int P = a.protect;
  // Whole-step call (a.conf_merge, uniform): the budget comes from this
  // sequence's confidence. Wave 0 issues the loads of the per-chunk states
  // now and finishes the merge inside the EMA phase (token eviction), or
  // here (block eviction, which needs the budget first).
  const bool merge_late = FUSE && !BLOCK && a.conf_merge;
  const bool greedy = a.conf.choice == confm::kGreedy;
  const int brow = a.conf.nbl > 1 ? l : 0;  // budget row of this layer
  __shared__ float conf_c;
  confm::RowState crs{};
  if (a.conf_merge && threadIdx.x < 64)
    crs = greedy ? confm::conf_lane_state<confm::kGreedy>(a.conf, b, threadIdx.x)
                 : confm::conf_lane_state<confm::kNoChoice>(a.conf, b, threadIdx.x);
  auto conf_finish = [&]() {  // wave 0: c to shared memory; the first layer writes the outputs
    int tok;
    const float cc = greedy ? confm::conf_row_finish<confm::kGreedy>(a.conf, b, threadIdx.x, crs, tok)
                            : confm::conf_row_finish<confm::kNoChoice>(a.conf, b, threadIdx.x, crs, tok);
    if (threadIdx.x == 0) {
      conf_c = cc;
      if (l == 0) {
        a.conf.c_out[b] = cc;
        if (greedy) a.conf.token_out[b] = tok;
        if (cc != cc && a.conf.status) atomicOr(a.conf.status, (uint32_t)CONFK_STATUS_NONFINITE_LOGITS);
      }
      if (brow == l) a.conf.budget_out[(int64_t)brow * a.conf.batch + b] = confm::conf_budget(a.conf, brow, cc);
    }
  };
  int N = P;  // merge_late: set after the merge
  if (!a.conf_merge) {
    N = max(a.budget[l * a.budget_stride + b], P);
  } else if (!merge_late) {
    if (threadIdx.x < 64) conf_finish();
    __syncthreads();
    N = max(confm::conf_budget(a.conf, brow, conf_c), P);
  }
  float* ema = c.ema + (size_t)lbc * cap;
  int32_t* pos = c.pos + (size_t)lbc * cap;
  const float* score = a.score + (size_t)lb * cap;
  __shared__ Shared sh;
  __shared__ std::conditional_t<REG && (!MOVEK || FUSE), RegShared, char> rsh;
  // the new token's K and V rows into the FP16 rings at `slot`
  auto append_rows = [&](int slot) {
    const int H = c.hkv, d = c.d, p16 = d >> 3, rp16 = 2 * H * p16;
    const size_t ring16 = (size_t)c.cap16 * 2 * d;
    unsigned char* k16b = reinterpret_cast<unsigned char*>(c.k16) + (size_t)lbc * H * ring16;
    unsigned char* v16b = reinterpret_cast<unsigned char*>(c.v16) + (size_t)lbc * H * ring16;
    for (int q = threadIdx.x; q < rp16; q += kThreads) {
      const int ring = q / p16, pc = q - ring * p16, h = ring >> 1;
      const uint16_t* src = ((ring & 1) ? a.v_new : a.k_new) + ((size_t)lb * H + h) * d + pc * 8;
      unsigned char* dst = ((ring & 1) ? v16b : k16b) + (size_t)h * ring16 + (size_t)slot * 2 * d + pc * 16;
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
  };

  // Fused form with the window step: once the cache holds the step's
  // survivors and the new token, the FP16 tokens at positions <= t - W move
  // to INT8 in this workgroup, as the quantisation kernel would do next.
  auto quantize_tail = [&](int n_after, int n8_after, int base8_after, int base16_after) {
    if (!a.quantize) return;  // uniform (a kernel argument)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // the rows, positions and metadata written above are visible
    quantize_window<kThreads>(c, lbc, a.t, a.window, n_after, n8_after, base8_after, base16_after,
                              meta[CONFK_META_CALIB]);
  };

  const int nn = n + 1;  // tokens incl. the new one
  const int f = n - n8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (!meta_ok(n, n8, base8, base16, cap, c.cap16)) {  // no room: flag, leave the cache as it is
    if (merge_late && threadIdx.x < 64) conf_finish();  // the confidence outputs are still due
    if (threadIdx.x == 0) {
      atomicOr(c.status, (uint32_t)CONFK_STATUS_CAPACITY);
      meta[CONFK_META_EVICTED] = 0;
      meta[CONFK_META_MOVED] = 0;
      meta[CONFK_META_MOVED16] = 0;
      hdr[H_MOV8] = hdr[H_MOV16] = 0;
      hdr[H_APPEND] = -1;
      if constexpr (MOVEK) a.jobs[lb] = 0;
      if (a.evicted_out) a.evicted_out[lb] = 0;
    }
    return;
  }
  int k = n > N ? n - N : 0;
  const int ncand = n - P;  // candidates: logical [0, ncand)
  const int B = BLOCK ? a.block : 0;  // block eviction: whole blocks of B candidates
  int nb = 0, kb = 0;       // full candidate blocks; blocks that leave
  if (BLOCK && k > 0) {
    nb = ncand / B;
    kb = min(nb, (k + B - 1) / B);
    k = kb * B;
  }

  const int chunk = (nn + kThreads - 1) / kThreads;
  const int lo = min(nn, (int)threadIdx.x * chunk);
  const int cnt = min(nn, lo + chunk) - lo;
  // this thread's run: score keys, EMA and positions (read before any write)
  uint32_t kreg[REG ? kRegKeys : 1];
  float ereg[REG ? kRegKeys : 1];
  int preg[REG ? kRegKeys : 1];
  int bk[REG ? kRegKeys : 1];
  float sreg[REG && FUSE ? kRegKeys : 1];

  // ------------------------------------------------- 0. EMA + rank (fused)
  if constexpr (FUSE) {
    const int H = mass_rows(meta, c.hkv);  // rows of partial mass sums
    const float* mass = a.mass + (size_t)lb * c.hkv * cap;
    const float inv_hq = 1.f / (float)c.hq, lam = a.lambda, oml = 1.f - lam;
    float amax = 0.f;
    int pmin = INT32_MAX, pmax = INT32_MIN;
    // a_i = lam a_i + (1 - lam) Abar_i for cached tokens, (1 - lam) Abar_n for
    // the new one (zero prior); mass rows summed in order. Lane-strided
    // ownership (index threadIdx.x + r * kThreads) keeps the loads coalesced.
    if constexpr (REG) {
      float ms[kRegKeys], av[kRegKeys];
      int pv[kRegKeys];
#pragma unroll
      for (int r = 0; r < kRegKeys; ++r) {
        const int i = threadIdx.x + r * kThreads;
        ms[r] = 0.f;
        av[r] = i < n ? ema[i] : 0.f;
        pv[r] = i < n ? pos[i] : a.t;
      }
      for (int j0 = 0; j0 < H; j0 += 8) {
        float t8[8][kRegKeys];
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int r = 0; r < kRegKeys; ++r) {
            const int i = threadIdx.x + r * kThreads;
            t8[q][r] = (j0 + q < H && i < nn) ? mass[(size_t)(j0 + q) * cap + i] : 0.f;
          }
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int r = 0; r < kRegKeys; ++r)
            if (j0 + q < H) ms[r] += t8[q][r];
      }
#pragma unroll
      for (int r = 0; r < kRegKeys; ++r) {
        const int i = threadIdx.x + r * kThreads;
        if (i < n) {
          av[r] = fmaf(lam, av[r], oml * (ms[r] * inv_hq));
          amax = fmaxf(amax, av[r]);
          pmin = min(pmin, pv[r]);
          pmax = max(pmax, pv[r]);
        } else {
          av[r] = oml * (ms[r] * inv_hq);
        }
        if (i < nn) {
          rsh.x.e[i] = av[r];
          rsh.x.p[i] = pv[r];
        }
      }
    } else {
      // the same arithmetic over blocks of kRegKeys * kThreads tokens, a
      // thread's loads of a block issued together
      for (int base = 0; base < nn; base += kRegKeys * kThreads) {
        float ms[kRegKeys], bv[kRegKeys];
        int qv[kRegKeys];
#pragma unroll
        for (int r = 0; r < kRegKeys; ++r) {
          const int i = base + threadIdx.x + r * kThreads;
          ms[r] = 0.f;
          bv[r] = i < n ? ema[i] : 0.f;
          qv[r] = i < n ? pos[i] : 0;
        }
        for (int j0 = 0; j0 < H; j0 += 4) {  // four rows per round trip (register budget)
          float t4[4][kRegKeys];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < kRegKeys; ++r) {
              const int i = base + threadIdx.x + r * kThreads;
              t4[q][r] = (j0 + q < H && i < nn) ? mass[(size_t)(j0 + q) * cap + i] : 0.f;
            }
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < kRegKeys; ++r)
              if (j0 + q < H) ms[r] += t4[q][r];
        }
#pragma unroll
        for (int r = 0; r < kRegKeys; ++r) {
          const int i = base + threadIdx.x + r * kThreads;
          if (i < n) {
            const float v = fmaf(lam, bv[r], oml * (ms[r] * inv_hq));
            ema[i] = v;
            amax = fmaxf(amax, v);
            pmin = min(pmin, qv[r]);
            pmax = max(pmax, qv[r]);
          } else if (i == n) {
            ema[n] = oml * (ms[r] * inv_hq);
            pos[n] = a.t;
          }
        }
      }
    }
    amax = wave_max(amax);
    for (int o = 32; o > 0; o >>= 1) {
      pmin = min(pmin, __shfl_xor(pmin, o, 64));
      pmax = max(pmax, __shfl_xor(pmax, o, 64));
    }
    if (lane == 0) {
      sh.rmax[w] = amax;
      sh.rpmin[w] = pmin;
      sh.rpmax[w] = pmax;
    }
    if (merge_late && w == 0) conf_finish();
    __syncthreads();  // the exchange, the long-cache form's EMA writes and conf_c are visible
    if (merge_late) {
      N = max(confm::conf_budget(a.conf, brow, conf_c), P);
      k = n > N ? n - N : 0;
    }
    amax = sh.rmax[0];
    int p0 = sh.rpmin[0], p1 = sh.rpmax[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) {
      amax = fmaxf(amax, sh.rmax[q]);
      p0 = min(p0, sh.rpmin[q]);
      p1 = max(p1, sh.rpmax[q]);
    }
    const float inv_a = amax > 0.f ? 1.f / amax : 0.f;
    const float inv_r = p1 > p0 ? 1.f / (float)(p1 - p0) : 0.f;
    const float alpha = a.alpha;
    float* score_w = a.score_out + (size_t)lb * cap;  // this (layer, sequence)'s scores
    if constexpr (REG) {
#pragma unroll
      for (int r = 0; r < kRegKeys; ++r) {  // this thread's run, from the exchange
        const int i = lo + r;
        ereg[r] = r < cnt ? rsh.x.e[i] : 0.f;
        preg[r] = r < cnt ? rsh.x.p[i] : 0;
        sreg[r] = 0.f;
        if (r < cnt && i < n) {
          const float rh = p1 > p0 ? (float)(preg[r] - p0) * inv_r : 1.f;
          sreg[r] = fmaf(alpha, ereg[r] * inv_a, (1.f - alpha) * rh);
          score_w[i] = sreg[r];
        }
      }
    } else {  // lane-strided blocks, each thread's loads of a block together
      for (int base = 0; base < n; base += kRegKeys * kThreads) {
        float ev[kRegKeys];
        int qv[kRegKeys];
#pragma unroll
        for (int r = 0; r < kRegKeys; ++r) {
          const int i = base + threadIdx.x + r * kThreads;
          ev[r] = i < n ? ema[i] : 0.f;
          qv[r] = i < n ? pos[i] : 0;
        }
#pragma unroll
        for (int r = 0; r < kRegKeys; ++r) {
          const int i = base + threadIdx.x + r * kThreads;
          if (i < n) {
            const float rh = p1 > p0 ? (float)(qv[r] - p0) * inv_r : 1.f;
            score_w[i] = fmaf(alpha, ev[r] * inv_a, (1.f - alpha) * rh);
          }
        }
      }
      __syncthreads();  // scores are read back from memory below
    }
  }

  if (k == 0) {  // nothing leaves: the new token (metadata slot n) is appended
    if constexpr (FUSE && REG) {  // every entry stays: its updated EMA in place
#pragma unroll
      for (int r = 0; r < kRegKeys; ++r)
        if (r < cnt) {
          ema[lo + r] = ereg[r];
          if (lo + r == n) pos[n] = a.t;
        }
    }
    int slot = base16 + f;
    slot = slot >= c.cap16 ? slot - c.cap16 : slot;
    append_rows(slot);
    if (threadIdx.x == 0) {
      if constexpr (MOVEK) a.jobs[lb] = 0;  // the move kernel has nothing to do here
      meta[CONFK_META_N] = nn;
      meta[CONFK_META_EVICTED] = 0;
      meta[CONFK_META_MOVED] = 0;
      meta[CONFK_META_MOVED16] = 0;
      if (a.evicted_out) a.evicted_out[lb] = 0;
    }
    if constexpr (FUSE) quantize_tail(nn, n8, base8, base16);
    return;
  }

  if constexpr (REG) {
#pragma unroll
    for (int j = 0; j < kRegKeys; ++j) {
      const int i = lo + j;
      const bool in = j < cnt;
      const bool cand = in && i < ncand;
      const float s = cand ? (FUSE ? sreg[j] : score[i]) : 0.f;
      kreg[j] = cand ? ord_bits(s) : 0xFFFFFFFFu;
      bk[j] = cand ? bucket_of(s) : kBuckets;
      if constexpr (!FUSE) {
        ereg[j] = in ? ema[i] : 0.f;
        preg[j] = in ? pos[i] : 0;
      }
    }
  }
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (REG) {
      return kreg[j];
    } else {
      const int i = lo + j;
      return i < ncand ? ord_bits(score[i]) : 0xFFFFFFFFu;
    }
  };
  // position of logical index lo + j (the non-register form reads memory,
  // valid until the metadata is rewritten in place)
  auto pos_at = [&](int j) -> uint32_t {
    if constexpr (REG) {
      return (uint32_t)preg[j];
    } else {
      return (uint32_t)pos[lo + j];
    }
  };

  // ---------------------------------------------------------- 1. select
  // T64: the k-th smallest (key, position); every candidate at or below leaves.
  // Block eviction instead marks the kb blocks with the smallest (largest
  // key in the block, block index) in bsel.
  uint64_t T64 = 0;
  uint32_t* const bmax = sh.hist;                    // [nb] block keys
  uint32_t* const bsel = sh.hist + kMaxEvictBlocks;  // [nb] 1: the block leaves
  bool use_radix = !REG && !BLOCK;
  if constexpr (BLOCK) {
    for (int q = threadIdx.x; q < nb; q += kThreads) bmax[q] = 0u;  // below every key
    __syncthreads();
    const int span = nb * B;
    int cur = -1;
    uint32_t run = 0;
    auto fold = [&](int j) {
      const int i = lo + j;
      if (i < span) {
        const int q = i / B;
        if (q != cur) {
          if (cur >= 0) atomicMax(&bmax[cur], run);
          cur = q;
          run = 0u;
        }
        run = max(run, key_at(j));
      }
    };
    if constexpr (REG) {
#pragma unroll
      for (int j = 0; j < kRegKeys; ++j)
        if (j < cnt) fold(j);
    } else {
      for (int j = 0; j < cnt; ++j) fold(j);
    }
    if (cur >= 0) atomicMax(&bmax[cur], run);
    __syncthreads();
    for (int q = threadIdx.x; q < nb; q += kThreads) {
      const uint64_t mine = ((uint64_t)bmax[q] << 32) | (uint32_t)q;
      int rank = 0;
      for (int z = 0; z < nb; ++z) rank += (((uint64_t)bmax[z] << 32) | (uint32_t)z) < mine ? 1 : 0;
      bsel[q] = rank < kb ? 1u : 0u;
    }
    __syncthreads();
  } else if constexpr (REG) {
    for (int i = threadIdx.x; i < kBuckets; i += kThreads) sh.hist[i] = 0;
    if (threadIdx.x == 0) sh.rank_n = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegKeys; ++j)
      if (bk[j] < kBuckets) atomicAdd(&sh.hist[bk[j]], 1u);
    __syncthreads();
    if (threadIdx.x < 64) {
      constexpr int per = kBuckets / 64;
      int hsum = 0;
      uint32_t hv[per];
#pragma unroll
      for (int q = 0; q < per; ++q) {
        hv[q] = sh.hist[per * lane + q];
        hsum += (int)hv[q];
      }
      int incl = hsum;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const int excl = incl - hsum;
      if (excl < k && k <= incl) {
        int run = excl, bsel = per * lane, below = excl;
        bool found = false;
#pragma unroll
        for (int q = 0; q < per; ++q) {
          if (!found && run + (int)hv[q] >= k) {
            found = true;
            bsel = per * lane + q;
            below = run;
          }
          run += (int)hv[q];
        }
        sh.sel_bucket = bsel;
        sh.sel_below = below;
        sh.sel_crowded = (int)sh.hist[bsel] > kRankMax;
      }
    }
    __syncthreads();
    const int bsel = sh.sel_bucket;
    if (!sh.sel_crowded) {
#pragma unroll
      for (int j = 0; j < kRegKeys; ++j)
        if (bk[j] == bsel) sh.rank_keys[atomicAdd(&sh.rank_n, 1)] = ((uint64_t)kreg[j] << 32) | (uint32_t)preg[j];
      __syncthreads();
      if (threadIdx.x < 64) {
        // rank the boundary bucket's keys; the (k - below)-th smallest is T64
        const int m = sh.rank_n;
        const int want = k - sh.sel_below - 1;
        if (lane < m) {
          const uint64_t mine = sh.rank_keys[lane];
          int rank = 0;
          for (int q = 0; q < m; ++q) rank += sh.rank_keys[q] < mine ? 1 : 0;
          if (rank == want) sh.kth = mine;
        }
      }
      __syncthreads();
      T64 = sh.kth;
    } else {
      use_radix = true;
    }
  }
  if (use_radix) {
    // the k-th smallest key T, then the kk-th smallest position among the
    // candidates whose key is T (positions are unique)
    int kk = k;
    auto cand = [&](int j) { return lo + j < ncand; };
    const uint32_t T = radix_select<REG>(kk, cnt, cand, key_at, sh);
    auto tied = [&](int j) { return lo + j < ncand && key_at(j) == T; };
    const uint32_t Tp = radix_select<REG>(kk, cnt, tied, pos_at, sh);
    T64 = ((uint64_t)T << 32) | Tp;
  }

  // ------------------------------------------- 2. flags, scans, regions
  auto leaves = [&](int j) -> bool {
    const int i = lo + j;
    if constexpr (BLOCK) return i < nb * B && bsel[i / B] != 0u;
    return i < ncand && ((((uint64_t)key_at(j)) << 32) | pos_at(j)) <= T64;
  };
  uint32_t evm = 0;  // bit j: index lo + j leaves (register path)
  int keeps = 0, e8 = 0, e16 = 0;
  // fused window step after stable packing: the FP16 survivors that leave the
  // window (position at most t - window; the oldest ones, as the FP16 part is
  // in position order)
  const bool qcount = MOVEK && FUSE && a.quantize;
  int q16 = 0;
  int f8 = INT32_MAX, l8 = -1, f16 = INT32_MAX, l16 = -1;
  auto tally = [&](int j) {
    const int i = lo + j;
    if (leaves(j)) {
      if (j < 32) evm |= 1u << j;
      if (i < n8) {
        ++e8;
        f8 = min(f8, i);
        l8 = max(l8, i);
      } else {
        ++e16;
        f16 = min(f16, i);
        l16 = max(l16, i);
      }
    } else {
      ++keeps;
      if (qcount && i >= n8 && i < n && (int)pos_at(j) <= a.t - a.window) ++q16;
    }
  };
  if constexpr (REG) {
#pragma unroll
    for (int j = 0; j < kRegKeys; ++j)
      if (j < cnt) tally(j);
  } else {
    for (int j = 0; j < cnt; ++j) tally(j);
  }
  int tk, t8, t16, pre_keep;
  if constexpr (REG) {  // counts of at most kRegKeys: bit-plane ballots
    pre_keep = wave_prefix16(keeps, tk);
    wave_prefix16(e8, t8);
    wave_prefix16(e16, t16);
  } else {
    int incl = keeps;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    pre_keep = incl - keeps;
    tk = __shfl(incl, 63, 64);
    t8 = e8;
    t16 = e16;
    for (int o = 32; o > 0; o >>= 1) {
      t8 += __shfl_xor(t8, o, 64);
      t16 += __shfl_xor(t16, o, 64);
    }
  }
  // first / last holes: runs are contiguous, so the lowest (highest) lane
  // with a hole holds the wave's first (last)
  const uint64_t h8 = __ballot(e8 > 0), h16 = __ballot(e16 > 0);
  const int wf8 = h8 ? __shfl(f8, __ffsll((unsigned long long)h8) - 1, 64) : INT32_MAX;
  const int wl8 = h8 ? __shfl(l8, 63 - __clzll((long long)h8), 64) : -1;
  const int wf16 = h16 ? __shfl(f16, __ffsll((unsigned long long)h16) - 1, 64) : INT32_MAX;
  const int wl16 = h16 ? __shfl(l16, 63 - __clzll((long long)h16), 64) : -1;
  __syncthreads();  // the select's shared values other than bsel are no longer read
  const int tq = qcount ? wave_sum_i(q16) : 0;
  if (lane == 0) {
    sh.wsum[0][w] = tk;
    sh.wsum[1][w] = t8;
    sh.wsum[2][w] = t16;
    sh.wsum[3][w] = tq;
    sh.wfirst[0][w] = wf8;
    sh.wlast[0][w] = wl8;
    sh.wfirst[1][w] = wf16;
    sh.wlast[1][w] = wl16;
  }
  __syncthreads();
  int keep_base = pre_keep, nkeep = 0, nq = 0;
  Region r8{0, n8, 0, INT32_MAX, -1, 1, 0, 0}, r16{n8, f, 0, INT32_MAX, -1, 1, 0, 0};
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    keep_base += q < w ? sh.wsum[0][q] : 0;
    nkeep += sh.wsum[0][q];
    nq += sh.wsum[3][q];
    r8.e += sh.wsum[1][q];
    r16.e += sh.wsum[2][q];
    r8.first_ev = min(r8.first_ev, sh.wfirst[0][q]);
    r8.last_ev = max(r8.last_ev, sh.wlast[0][q]);
    r16.first_ev = min(r16.first_ev, sh.wfirst[1][q]);
    r16.last_ev = max(r16.last_ev, sh.wlast[1][q]);
  }
  plan_region(r8);
  plan_region(r16);
  const int js16 = n8 - r8.e;  // new logical index of the first FP16 survivor

  if constexpr (MODE != kFill) {
    // ------------- stable packing of both regions (token eviction in the
    // stable order, or block eviction)

    // ------------------------------------- 3. metadata and 4. move lists
    // List entries (the mover's region-local old index) are stored in move
    // order: ascending new index when packing toward the base, descending
    // otherwise.
    auto emit = [&](int i, int jn, float ev_, int pv_) {
      ema[jn] = ev_;
      pos[jn] = pv_;
      if (i < n8) {
        const int m = jn - r8.jlo;
        if (m >= 0 && m < r8.movers) src8[r8.left ? m : r8.movers - 1 - m] = i;
      } else if (i < n) {
        const int m = jn - js16 - r16.jlo;  // region-local new index minus the first mover's
        if (m >= 0 && m < r16.movers) src16[r16.left ? m : r16.movers - 1 - m] = i - n8;
      }
    };
    if constexpr (REG) {
      int jn = keep_base;
  #pragma unroll
      for (int j = 0; j < kRegKeys; ++j)
        if (j < cnt && !((evm >> j) & 1u)) emit(lo + j, jn++, ereg[j], preg[j]);
    } else {
      // long caches: each survivor's metadata and old index go through a
      // staging area, so that the in-place writes after the barrier need no
      // second look at the (by then rewritten) positions
      int32_t* st = a.stage + (size_t)lb * stage_words(cap);
      float* se = reinterpret_cast<float*>(st);
      int32_t* sp = st + cap;
      int32_t* si = st + 2 * cap;
      int jn = keep_base;
      for (int j = 0; j < cnt; ++j) {
        if (!leaves(j)) {
          se[jn] = ema[lo + j];
          sp[jn] = pos[lo + j];
          si[jn] = lo + j;
          ++jn;
        }
      }
      __syncthreads();
      for (jn = keep_base; jn < keep_base + keeps; ++jn) emit(si[jn], jn, se[jn], sp[jn]);
    }
    int b8 = base8, b16 = base16;  // ring bases after the packing
    if (!r8.left) {
      b8 += r8.e;
      if (b8 >= cap) b8 -= cap;
    }
    if (!r16.left) {
      b16 += r16.e;
      if (b16 >= c.cap16) b16 -= c.cap16;
    }
    int slot = b16 + (f - r16.e);  // the new token's FP16 slot
    slot = slot >= c.cap16 ? slot - c.cap16 : slot;
    const int m8 = n8 - r8.e;
    if (a.plan_moves || r8.movers + r16.movers == 0) {  // uniform
      // nothing moves (the evicted tokens sat at the packing ends), or a
      // small launch moves its rows here: append and window step here, the
      // move kernel skips this (layer, sequence). The append slot is no
      // FP16 source when no FP16 row moves, and every FP16 source has been
      // read (the last round's barrier) when one does.
      if (r8.movers + r16.movers > 0) {  // uniform
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // the move lists in the workspace are complete
        move_ring<false>(c, lbc, r8.movers, r8.left, r8.e, r8.jlo, base8, src8);
        move_ring<true>(c, lbc, r16.movers, r16.left, r16.e, r16.jlo, base16, src16);
      }
      append_rows(slot);
      if (threadIdx.x == 0) {
        a.jobs[lb] = 0;
        meta[CONFK_META_N] = nkeep;
        meta[CONFK_META_N8] = m8;
        meta[CONFK_META_BASE8] = b8;
        meta[CONFK_META_BASE16] = b16;
        meta[CONFK_META_EVICTED] = k;
        meta[CONFK_META_MOVED] = r8.movers;
        meta[CONFK_META_MOVED16] = r16.movers;
        if (a.evicted_out) a.evicted_out[lb] = k;
      }
      if constexpr (FUSE) quantize_tail(nkeep, m8, b8, b16);
    } else if (threadIdx.x == 0) {
      // the move kernel moves the rows, appends the new token and (fused
      // form) moves the nq oldest FP16 survivors to INT8; the header below
      // is the state after all of that
      const int calib = meta[CONFK_META_CALIB];
      int b16q = b16 + nq;
      b16q = b16q >= c.cap16 ? b16q - c.cap16 : b16q;
      hdr[H_MOV8] = r8.movers;
      hdr[H_LEFT8] = r8.left;
      hdr[H_E8] = r8.e;
      hdr[H_JLO8] = r8.jlo;
      hdr[H_MOV16] = r16.movers;
      hdr[H_LEFT16] = r16.left;
      hdr[H_E16] = r16.e;
      hdr[H_JLO16] = r16.jlo;
      hdr[H_BASE8] = base8;
      hdr[H_BASE16] = base16;
      hdr[H_APPEND] = slot;
      hdr[H_Q] = nq;
      hdr[H_CAL] = nq > 0 && !calib;
      hdr[H_B8N] = b8;
      hdr[H_B16N] = b16;
      hdr[H_M8] = m8;
      a.jobs[lb] = 1;
      meta[CONFK_META_N] = nkeep;
      meta[CONFK_META_N8] = m8 + nq;
      meta[CONFK_META_BASE8] = b8;
      meta[CONFK_META_BASE16] = b16q;
      meta[CONFK_META_CALIB] = calib | (nq > 0);
      meta[CONFK_META_EVICTED] = k;
      meta[CONFK_META_MOVED] = r8.movers;
      meta[CONFK_META_MOVED16] = r16.movers;
      if (a.evicted_out) a.evicted_out[lb] = k;
    }
  } else {
    // ------------- token eviction: INT8 hole filling, FP16 packing, append
    // Holes are the evicted INT8 entries below the new INT8 length m8, tails
    // the surviving INT8 entries at or beyond it; the r-th tail (slot order)
    // moves to the r-th hole. Tails and holes are disjoint slots, so those
    // moves need no ordering. The FP16 part is packed stably as planned above.
    const int m8 = js16;
    int nh = 0, nt = 0;
    auto hole_tail = [&](int j, bool lv) {
      const int i = lo + j;
      if (i < n8) {
        nh += (lv && i < m8) ? 1 : 0;
        nt += (!lv && i >= m8) ? 1 : 0;
      }
    };
    if constexpr (REG) {
#pragma unroll
      for (int j = 0; j < kRegKeys; ++j)
        if (j < cnt) hole_tail(j, (evm >> j) & 1u);
    } else {
      for (int j = 0; j < cnt; ++j) hole_tail(j, leaves(j));
    }
    int hbase, tbase, nholes = 0;  // this thread's first hole and tail rank; holes in all
    {
      int th, tt;
      if constexpr (REG) {
        hbase = wave_prefix16(nh, th);
        tbase = wave_prefix16(nt, tt);
      } else {
        int ih = nh, it = nt;
        for (int o = 1; o < 64; o <<= 1) {
          const int yh = __shfl_up(ih, o, 64), yt = __shfl_up(it, o, 64);
          if (lane >= o) {
            ih += yh;
            it += yt;
          }
        }
        hbase = ih - nh;
        tbase = it - nt;
        th = __shfl(ih, 63, 64);
        tt = __shfl(it, 63, 64);
      }
      if (lane == 0) {
        sh.wfill[0][w] = th;
        sh.wfill[1][w] = tt;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        hbase += q < w ? sh.wfill[0][q] : 0;
        tbase += q < w ? sh.wfill[1][q] : 0;
        nholes += sh.wfill[0][q];
      }
    }
    // fill lists and the tails' metadata: LDS for register-held runs, the
    // workspace otherwise (where the FP16 survivors' metadata is staged too:
    // every read of the metadata precedes the barrier, every write follows)
    int32_t* st = a.stage + (size_t)lb * stage_words(cap);
    const int half = (cap + 1) / 2;
    float* tse;
    int32_t *tsp, *tsi, *hd;
    if constexpr (REG) {
      tse = rsh.fill.e;
      tsp = rsh.fill.p;
      tsi = rsh.fill.i;
      hd = rsh.fill.h;
    } else {
      tse = reinterpret_cast<float*>(st + 3 * cap);
      tsp = st + 3 * cap + half;
      tsi = st + 3 * cap + 2 * half;
      hd = st + 3 * cap + 3 * half;
    }
    auto emit16 = [&](int i, int jn, float ev_, int pv_) {  // FP16 survivor or the new token
      ema[jn] = ev_;
      pos[jn] = pv_;
      if (i < n) {
        const int m = jn - m8 - r16.jlo;
        if (m >= 0 && m < r16.movers) src16[r16.left ? m : r16.movers - 1 - m] = i - n8;
      }
    };
    if constexpr (REG) {
      int h = hbase, t = tbase, jn = keep_base;
#pragma unroll
      for (int j = 0; j < kRegKeys; ++j) {
        if (j < cnt) {
          const int i = lo + j;
          if (!((evm >> j) & 1u)) {
            if (i >= n8) {
              emit16(i, jn, ereg[j], preg[j]);
            } else if (i < m8) {
              if constexpr (FUSE) ema[i] = ereg[j];  // stays in its slot
            } else {
              tse[t] = ereg[j];
              tsp[t] = preg[j];
              tsi[t] = i;
              ++t;
            }
            ++jn;
          } else if (i < m8) {
            hd[h++] = i;
          }
        }
      }
    } else {
      float* se = reinterpret_cast<float*>(st);
      int32_t* sp = st + cap;
      int32_t* si = st + 2 * cap;
      int h = hbase, t = tbase, jn = keep_base;
      for (int j = 0; j < cnt; ++j) {
        const int i = lo + j;
        if (!leaves(j)) {
          if (i >= n8) {
            se[jn] = ema[i];
            sp[jn] = pos[i];
            si[jn] = i;
          } else if (i >= m8) {
            tse[t] = ema[i];
            tsp[t] = pos[i];
            tsi[t] = i;
            ++t;
          }
          ++jn;
        } else if (i < m8) {
          hd[h++] = i;
        }
      }
    }
    __syncthreads();
    // each hole takes its tail's metadata
    for (int r = hbase; r < hbase + nh; ++r) {
      const int i = hd[r];
      ema[i] = tse[r];
      pos[i] = tsp[r];
    }
    if constexpr (!REG) {
      float* se = reinterpret_cast<float*>(st);
      int32_t* sp = st + cap;
      int32_t* si = st + 2 * cap;
      for (int jn = max(keep_base, m8); jn < keep_base + keeps; ++jn) emit16(si[jn], jn, se[jn], sp[jn]);
    }
    __syncthreads();  // fill lists and FP16 movers are complete

    // ---- the moves: all 512 threads, 16-byte pieces, consecutive threads
    // on consecutive pieces of a row
    const int H = c.hkv, d = c.d;
    const int p8 = d >> 4, rp8 = 2 * H * p8;   // pieces per INT8 row; per moved token
    const int p16 = d >> 3, rp16 = 2 * H * p16;  // same for FP16 rows
    const size_t ring8 = (size_t)cap * d, ring16 = (size_t)c.cap16 * 2 * d;  // bytes per ring
    unsigned char* k8b = reinterpret_cast<unsigned char*>(c.k8) + (size_t)lbc * H * ring8;
    unsigned char* v8b = reinterpret_cast<unsigned char*>(c.v8) + (size_t)lbc * H * ring8;
    unsigned char* k16b = reinterpret_cast<unsigned char*>(c.k16) + (size_t)lbc * H * ring16;
    unsigned char* v16b = reinterpret_cast<unsigned char*>(c.v16) + (size_t)lbc * H * ring16;
    const int tot8 = nholes * rp8;
    for (int q0 = threadIdx.x; q0 < tot8; q0 += 4 * kThreads) {
      u32x4 v[4];
      unsigned char* dp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * kThreads;
        dp[u] = nullptr;
        if (q < tot8) {
          const int r = q / rp8, rem = q - r * rp8;
          const int ring = rem / p8, pc = rem - ring * p8;
          unsigned char* rb = ((ring & 1) ? v8b : k8b) + (size_t)(ring >> 1) * ring8 + pc * 16;
          int ss = base8 + tsi[r], ds = base8 + hd[r];
          ss = ss >= cap ? ss - cap : ss;
          ds = ds >= cap ? ds - cap : ds;
          v[u] = *reinterpret_cast<const u32x4*>(rb + (size_t)ss * d);
          dp[u] = rb + (size_t)ds * d;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (dp[u]) *reinterpret_cast<u32x4*>(dp[u]) = v[u];
    }
    // FP16 packing in plan order: a round reads all of its rows, waits, and
    // writes them; round r+1 reads only slots beyond round r's destinations
    const int mv16 = r16.movers, C16 = c.cap16;
    const int rows16 = max(1, 4 * kThreads / rp16);
    for (int m0 = 0; m0 < mv16; m0 += rows16) {
      const int tot = min(rows16, mv16 - m0) * rp16;
      u32x4 v[4];
      unsigned char* dp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = threadIdx.x + u * kThreads;
        dp[u] = nullptr;
        if (q < tot) {
          const int rr = m0 + q / rp16, rem = q % rp16;
          const int ring = rem / p16, pc = rem - ring * p16;
          unsigned char* rb = ((ring & 1) ? v16b : k16b) + (size_t)(ring >> 1) * ring16 + pc * 16;
          const int j = r16.jlo + (r16.left ? rr : mv16 - 1 - rr);
          int ss = base16 + src16[rr], ds = base16 + (r16.left ? j : j + r16.e);
          ss = ss >= C16 ? ss - C16 : ss;
          ds = ds >= C16 ? ds - C16 : ds;
          v[u] = *reinterpret_cast<const u32x4*>(rb + (size_t)ss * 2 * d);
          dp[u] = rb + (size_t)ds * 2 * d;
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (dp[u]) *reinterpret_cast<u32x4*>(dp[u]) = v[u];
    }
    int b16 = base16;
    if (!r16.left) {
      b16 += r16.e;
      if (b16 >= C16) b16 -= C16;
    }
    int slot = b16 + (f - r16.e);
    slot = slot >= C16 ? slot - C16 : slot;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every FP16 source has been read before the append slot is written
    append_rows(slot);
    if (threadIdx.x == 0) {
      meta[CONFK_META_N] = nkeep;
      meta[CONFK_META_N8] = m8;
      meta[CONFK_META_BASE16] = b16;
      meta[CONFK_META_EVICTED] = k;
      meta[CONFK_META_MOVED] = nholes;
      meta[CONFK_META_MOVED16] = mv16;
      if (a.evicted_out) a.evicted_out[lb] = k;
    }
    if constexpr (FUSE) quantize_tail(nkeep, m8, base8, b16);
  }
}

// One workgroup per (layer, sequence). SHORTCAP: the capacity itself fits the
// register form. Otherwise each workgroup takes the register form when its
// own cache (with the new token) fits and the long form when it does not, so
// a long-capacity cache pays for the long form only while it is long.
template <bool SHORTCAP, int MODE, bool FUSE>
__global__ __launch_bounds__(kThreads) void compact_plan_kernel(CompactArgs a) {
  if constexpr (SHORTCAP) {
    plan_body<true, MODE, FUSE>(a);
  } else {
    const int lb = blockIdx.x, l = lb / a.c.B, b = lb - l * a.c.B;
    const int n = a.c.meta[((a.layer0 + l) * a.c.B + b) * CONFK_META_WORDS + CONFK_META_N];
    if (n + 1 <= kRegKeys * kThreads)  // uniform; a corrupt length is flagged by either form
      plan_body<true, MODE, FUSE>(a);
    else
      plan_body<false, MODE, FUSE>(a);
  }
}

// Move kernel: one workgroup of kMoveThreads per (layer, sequence, kv head).
// The planned rows of that head's four rings (K and V, INT8 and FP16) move in
// rounds, then the new token's K and V rows of the head are appended, then
// (fused form) the head's rows of the tokens that left the FP16 window are
// quantised. A (layer, sequence) whose plan needs no move (header slot -1) is
// finished by the plan kernel. Rounds follow plan order: round r+1 reads only
// slots beyond round r's destinations in the packing direction, and within a
// round every source is read before any destination is written. Thread t
// copies piece column t % P (P 16-byte pieces per row) of movers t / P,
// t / P + mpp, ... (mpp = kMoveThreads / P movers per pass), the K piece and
// the V piece at the same ring offset. Loads and stores are unconditional: a
// piece past the last mover takes the last mover's piece and writes it again
// (same bytes, same place), since branches around each piece would make every
// memory operation wait for all earlier ones; a thread past the last whole
// mover of a pass (P not dividing the workgroup) repeats the round's first.
__device__ __forceinline__ void move_rounds(unsigned char* kb, unsigned char* vb, uint32_t rowb, int C, int P,
                                            int mv, int left, int e, int jlo, int base, const int32_t* lst) {
  typedef __attribute__((address_space(1))) u32x4 gvec;
  constexpr int HALF = kMoveRound / 2;
  gvec* kg = (gvec*)kb;
  gvec* vg = (gvec*)vb;
  const int mpp = kMoveThreads / P;
  const int mq = threadIdx.x / P, pc = threadIdx.x - mq * P;
  const bool act = mq < mpp;  // threads past the last whole mover of a pass repeat the round's first
  for (int m0 = 0; m0 < mv; m0 += HALF * mpp) {
    u32x4 v[2 * HALF];
    uint32_t dof[HALF];
#pragma unroll
    for (int u = 0; u < HALF; ++u) {
      const int r = act ? min(m0 + mq + u * mpp, mv - 1) : m0;
      int ss = base + lst[r];
      ss = ss >= C ? ss - C : ss;
      const uint32_t off = ((uint32_t)ss * rowb + (uint32_t)pc * 16u) >> 4;
      v[u] = kg[off];
      v[HALF + u] = vg[off];
      const int j = jlo + (left ? r : mv - 1 - r);
      int ds = base + (left ? j : j + e);
      ds = ds >= C ? ds - C : ds;
      dof[u] = ((uint32_t)ds * rowb + (uint32_t)pc * 16u) >> 4;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every source of the round has been read
#pragma unroll
    for (int u = 0; u < HALF; ++u) {
      kg[dof[u]] = v[u];
      vg[dof[u]] = v[HALF + u];
    }
  }
}

// One (layer, sequence, kv head) item of the move kernel.
template <bool WINDOW>
__device__ __forceinline__ void move_item(const CompactArgs& a, const int lb, const int hh) {
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) u32x4 gvec;
  constexpr int HALF = kMoveRound / 2;
  const CacheView& c = a.c;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  const int H = c.hkv, d = c.d, cap = c.cap, cap16 = c.cap16;
  const int32_t* hdr = a.plan + (size_t)lb * (kHdr + 2 * (size_t)cap);
  const int32_t* src8 = hdr + kHdr;
  const int32_t* src16 = src8 + cap;
  const size_t hrow = (size_t)lbc * H + hh;
  const int P8 = d >> 4, p16 = d >> 3, g8 = d >> 3;
  const int mpp = kMoveThreads / P8;
  const int mq = threadIdx.x / P8, pc = threadIdx.x - mq * P8;

  // ---- round trip 1: everything whose address is known at launch: the
  // header, this thread's list entries of the first INT8 round and the first
  // mover's (speculatively, as the mover count is still unknown), the new
  // row, and the scales the window step needs
  const i32x4 hA = reinterpret_cast<const i32x4*>(hdr)[0];  // MOV8, LEFT8, E8, JLO8
  const i32x4 hB = reinterpret_cast<const i32x4*>(hdr)[1];  // MOV16, LEFT16, E16, JLO16
  const i32x4 hC = reinterpret_cast<const i32x4*>(hdr)[2];  // BASE8, BASE16, APPEND, Q
  const i32x4 hD = reinterpret_cast<const i32x4*>(hdr)[3];  // CAL, B8N, B16N, M8
  int lsp[HALF];
#pragma unroll
  for (int u = 0; u < HALF; ++u) lsp[u] = src8[min(mq + u * mpp, cap - 1)];
  const int l0 = src8[0];
  const bool nrow_lane = (int)threadIdx.x < 2 * p16;
  const int nkind = (int)threadIdx.x >= p16, npc = threadIdx.x - nkind * p16;
  u32x4 nv = {0u, 0u, 0u, 0u};
  if (nrow_lane) nv = *reinterpret_cast<const u32x4*>((nkind ? a.v_new : a.k_new) + ((size_t)lb * H + hh) * d + npc * 8);
  const bool q_lane = WINDOW && (int)threadIdx.x < 2 * g8;
  const int qkind = (int)threadIdx.x >= g8, qch = 8 * (threadIdx.x - qkind * g8);
  qf32x4 qs0 = {0.f, 0.f, 0.f, 0.f}, qs1 = qs0;
  if (q_lane) {
    const float* sp = (qkind ? c.vs : c.ks) + hrow * d + qch;
    qs0 = *reinterpret_cast<const qf32x4*>(sp);
    qs1 = *reinterpret_cast<const qf32x4*>(sp + 4);
  }
  asm volatile("" ::: "memory");  // the loads above are issued before the exit test

  const int append = hC[2];
  unsigned char* k8r = uniform_ptr(c.k8 + hrow * cap * d);
  unsigned char* v8r = uniform_ptr(c.v8 + hrow * cap * d);
  unsigned char* k16r = uniform_ptr(c.k16 + hrow * cap16 * d);
  unsigned char* v16r = uniform_ptr(c.v16 + hrow * cap16 * d);
  const int mv8 = hA[0], mv16 = hB[0], nq = WINDOW ? hC[3] : 0;
  const int cal = hD[0], b8n = hD[1], b16n = hD[2], m8 = hD[3];
  int* satp = c.meta + lbc * CONFK_META_WORDS + CONFK_META_SAT;

  if (mv8 <= HALF * mpp && mv16 == 0 && nq <= 1 && !(nq && cal)) {  // uniform
    // ---- the common case: one INT8 round, no FP16 row moves, at most one
    // token leaves the window and the scales exist. Round trip 2 reads the
    // movers' rows and the leaving token's FP16 row (no FP16 row moves, so
    // it is in place) and writes the appended row (its slot is no source).
    gvec* kg = (gvec*)k8r;
    gvec* vg = (gvec*)v8r;
    const int left = hA[1], e = hA[2], jlo = hA[3], base = hC[0];
    u32x4 v[2 * HALF];
    uint32_t dof[HALF];
    if (mv8 > 0) {
#pragma unroll
      for (int u = 0; u < HALF; ++u) {
        const int rr = mq + u * mpp;
        const bool in = rr < mv8;  // beyond the movers: repeat the first mover's piece
        const int r = in ? rr : 0;
        int ss = base + (in ? lsp[u] : l0);
        ss = ss >= cap ? ss - cap : ss;
        const uint32_t off = ((uint32_t)ss * (uint32_t)d + (uint32_t)pc * 16u) >> 4;
        v[u] = kg[off];
        v[HALF + u] = vg[off];
        const int j = jlo + (left ? r : mv8 - 1 - r);
        int ds = base + (left ? j : j + e);
        ds = ds >= cap ? ds - cap : ds;
        dof[u] = ((uint32_t)ds * (uint32_t)d + (uint32_t)pc * 16u) >> 4;
      }
    }
    if (nrow_lane) *reinterpret_cast<u32x4*>((nkind ? v16r : k16r) + (size_t)append * 2 * d + npc * 16) = nv;
    qu32x4 qh = {0u, 0u, 0u, 0u};
    if (nq && q_lane) qh = *reinterpret_cast<const qu32x4*>((qkind ? v16r : k16r) + ((size_t)b16n * d + qch) * 2);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every INT8 source has been read
    if (mv8 > 0) {
#pragma unroll
      for (int u = 0; u < HALF; ++u) {
        kg[dof[u]] = v[u];
        vg[dof[u]] = v[HALF + u];
      }
    }
    if (nq && q_lane) {
      int ds = b8n + m8;
      ds = ds >= cap ? ds - cap : ds;
      float s8[8];
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        s8[z] = qs0[z];
        s8[4 + z] = qs1[z];
      }
      int sat = 0;
      *reinterpret_cast<qu32x2*>((qkind ? v8r : k8r) + (size_t)ds * d + qch) = quant8(qh, s8, sat);
      if (sat) atomicAdd(satp, sat);
    }
    return;
  }

  // ---- the general form: rounds over the lists, then the append, then the
  // window step
  move_rounds(k8r, v8r, (uint32_t)d, cap, P8, mv8, hA[1], hA[2], hA[3], hC[0], src8);
  move_rounds(k16r, v16r, (uint32_t)(2 * d), cap16, p16, mv16, hB[1], hB[2], hB[3], hC[1], src16);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every FP16 source has been read before the append slot is written
  if (nrow_lane) *reinterpret_cast<u32x4*>((nkind ? v16r : k16r) + (size_t)append * 2 * d + npc * 16) = nv;
  if constexpr (WINDOW) {
    if (nq == 0) return;  // uniform
    // the window step of this head: the nq oldest FP16 survivors become INT8
    // (scales over every FP16 token of the head first, if the sequence has
    // none yet), as quantize_window does for all heads
    int fa = append - b16n;
    fa = (fa < 0 ? fa + cap16 : fa) + 1;  // FP16 tokens after the append
    __shared__ float sc[2 * kMaxHeadDim];
    __shared__ int red[kMoveThreads / 64];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // moved and appended rows are written
    for (int e = threadIdx.x; e < 2 * d; e += kMoveThreads) {
      const int kind = e >= d, ch = e - kind * d;
      float* sp = (kind ? c.vs : c.ks) + hrow * d + ch;
      if (cal) {
        const uint16_t* ring = reinterpret_cast<const uint16_t*>(kind ? v16r : k16r);
        float amax = 0.f;
        for (int j = 0; j < fa; ++j) {
          int slot = b16n + j;
          if (slot >= cap16) slot -= cap16;
          amax = fmaxf(amax, fabsf(half_bits_to_float(ring[(size_t)slot * d + ch])));
        }
        const float sv = __fdiv_rn(amax, 127.f);
        *sp = sv;
        sc[e] = sv;
      } else {
        sc[e] = *sp;
      }
    }
    __syncthreads();  // scales in shared memory
    int sat = 0;
    for (int i = 0; i < nq; ++i) {
      int ss = b16n + i;
      ss = ss >= cap16 ? ss - cap16 : ss;
      int ds = b8n + m8 + i;
      ds = ds >= cap ? ds - cap : ds;
      for (int g = threadIdx.x; g < 2 * g8; g += kMoveThreads) {
        const int kind = g >= g8, ch = 8 * (g - kind * g8);
        const qu32x4 h = *reinterpret_cast<const qu32x4*>((kind ? v16r : k16r) + ((size_t)ss * d + ch) * 2);
        *reinterpret_cast<qu32x2*>((kind ? v8r : k8r) + (size_t)ds * d + ch) = quant8(h, sc + kind * d + ch, sat);
      }
    }
    sat = wave_sum_i(sat);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sat;
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int q = 0; q < kMoveThreads / 64; ++q) tot += red[q];
      if (tot) atomicAdd(satp, tot);
    }
  }
}

// The move kernel: a grid of at most kMoveGrid workgroups. Each reads the job
// flags the plan kernel left (one per (layer, sequence): 1 when rows move),
// lists the flagged pairs in shared memory with wave ballots, and walks the
// items (flagged pair, kv head) from its own index in steps of the grid, so
// that the work, not the cache shape, sets how many workgroups run.
template <bool WINDOW>
__global__ __launch_bounds__(kMoveThreads) void compact_move_kernel(CompactArgs a) {
  extern __shared__ int jobl[];  // [nl * B]: the flagged (layer, sequence) pairs
  __shared__ int wtot[kMoveThreads / 64];
  const int npair = a.nl * a.c.B, H = a.c.hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int njobs = 0;
  for (int p0 = 0; p0 < npair; p0 += kMoveThreads) {
    const int p = p0 + (int)threadIdx.x;
    const bool f = p < npair && a.jobs[p] != 0;
    const uint64_t m = __ballot(f);
    const int pre = __popcll(m & lanemask_lt());
    if (lane == 0) wtot[w] = __popcll(m);
    __syncthreads();
    int base = njobs, tot = 0;
#pragma unroll
    for (int q = 0; q < kMoveThreads / 64; ++q) {
      base += q < w ? wtot[q] : 0;
      tot += wtot[q];
    }
    if (f) jobl[base + pre] = p;
    njobs += tot;
    __syncthreads();  // wtot is rewritten by the next chunk; jobl is complete after the last
  }
  for (int it = blockIdx.x; it < njobs * H; it += gridDim.x) {
    const int j = it / H;
    move_item<WINDOW>(a, jobl[j], it - j * H);
    __syncthreads();  // shared memory of the window step is reused by the next item
  }
}

}  // namespace

size_t compact_jobs_offset(int nlayers, int batch, int cap) {
  return (size_t)nlayers * batch * (kHdr + 2 * (size_t)cap) * 4;
}

size_t compact_plan_bytes(int nlayers, int batch, int cap) {
  // plan: header + two source lists per (layer, sequence), then one job flag
  // per (layer, sequence), padded to 256 bytes
  const size_t jobs = ((size_t)nlayers * batch * 4 + 255) / 256 * 256;
  return compact_jobs_offset(nlayers, batch, cap) + jobs;
}

size_t compact_ws_bytes(int nlayers, int batch, int cap) {
  // plan and job flags; staging of the long-cache path: EMA, positions and
  // old indices per (layer, sequence)
  const size_t stage = cap > kRegKeys * kThreads ? (size_t)nlayers * batch * stage_words(cap) * 4 : 0;
  return compact_plan_bytes(nlayers, batch, cap) + stage;
}

template <int MODE, bool FUSE>
hipError_t launch_plan(const CompactArgs& a, hipStream_t s) {
  const int blocks = a.nl * a.c.B;
  if (a.c.cap <= kRegKeys * kThreads)  // every cache fits the register form
    hipLaunchKernelGGL((compact_plan_kernel<true, MODE, FUSE>), dim3(blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((compact_plan_kernel<false, MODE, FUSE>), dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool FUSE>
hipError_t launch_compact_t(const CompactArgs& a, hipStream_t s) {
  // token eviction in the fill order: one kernel selects, fills, packs,
  // moves and appends
  if (a.block == 0 && !a.stable) return launch_plan<kFill, FUSE>(a, s);
  // stable packing (token eviction in the stable order, block eviction): the
  // plan kernel selects and plans, and finishes the (layer, sequence) pairs
  // with nothing to move; the move kernel does the rest, spread over kv heads
  // a launch over few (layer, sequence) pairs moves its rows in the plan
  // kernel: the move kernel's launch would cost more than the rounds there
  CompactArgs b = a;
  const int npair = a.nl * a.c.B;
  b.plan_moves = npair <= kPlanMovePairs;
  hipError_t e = b.block ? launch_plan<kBlock, FUSE>(b, s) : launch_plan<kStable, FUSE>(b, s);
  if (e != hipSuccess || b.plan_moves) return e;
  const dim3 mgrid(min(npair * a.c.hkv, kMoveGrid)), mblock(kMoveThreads);
  const size_t lds = (size_t)npair * sizeof(int);
  if (FUSE && a.quantize)
    hipLaunchKernelGGL(compact_move_kernel<true>, mgrid, mblock, lds, s, a);
  else
    hipLaunchKernelGGL(compact_move_kernel<false>, mgrid, mblock, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  return a.fuse ? launch_compact_t<true>(a, s) : launch_compact_t<false>(a, s);
}

}  // namespace confk

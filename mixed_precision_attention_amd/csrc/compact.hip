// Budget eviction, stable compaction and append of the new token.
//
// CONF-KV summary, "Methodik: CONF-KV": tokens are ranked by the composite
// score, the newest P are never evicted (Token-Ranking und Eviktion), and
// the survivors are packed contiguously so attention reads a dense layout
// without indirection tables (Implementierung). Review "方法步骤详情"
// (Algorithm 1): if |C_l| > N evict the lowest-ranked unprotected tokens and
// compact the survivors; step 13 appends the new K/V in FP16.
//
// One workgroup per (layer, sequence); thread t owns a contiguous run of
// logical indices. For caches of up to 4096 tokens the run's scores are read
// once into registers; longer caches re-read them from memory.
//  1. k = n - N tokens leave, chosen among the n - P oldest. A 4-pass radix
//     select over order-preserving uint32 images of the fp32 scores finds the
//     k-th smallest score T; every candidate below T leaves, plus the oldest
//     ties at T (a prefix count in position order), which makes the evicted
//     set unique: the k smallest (score, position) pairs.
//  2. One block scan gives each survivor its new logical index; the survivor
//     list (new index -> old index) is kept in LDS.
//  3. EMA / position metadata are rewritten densely in place.
//  4. K/V rows move inside their rings. Each region (INT8 ring, FP16 ring)
//     is packed toward the end that moves fewer rows: keep the base and
//     shift the survivors after the first hole down, or advance the base and
//     shift the survivors before the last hole up. Evictions mostly hit old
//     tokens, so usually only a few rows move. Moves go in rounds (read all
//     rows of a round, barrier, write them) in an order that never
//     overwrites an unread source.
//  5. The new token's K/V rows are written to the FP16 ring.
// Steps without eviction only append.
#include "confk_internal.h"

namespace confk {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kWin = 8192;                // survivor-list entries held in LDS at once
constexpr int kMetaPer = kWin / kThreads;  // metadata entries per thread per window
constexpr int kRegs = 8;                  // 16-byte row pieces per thread per move round
constexpr int kRegKeys = 8;               // scores per thread kept in registers

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t ord_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSmallK = 32;  // evictions up to this count use the minima select

struct Shared {
  int tmp[4][kWaves];
  uint32_t hist[256];
  uint32_t sel_digit, sel_before;
  uint64_t wk[kWaves][kSmallK];  // each wave's smallest keys
  uint64_t kth;
};

// Exclusive block scan of x[0..3] at once; totals in tot[0..3].
__device__ __forceinline__ void block_scan4(const int* x, int* excl, int* tot, Shared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    incl[q] = x[q];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl[q], o, 64);
      if (lane >= o) incl[q] += y;
    }
    if (lane == 63) sh.tmp[q][w] = incl[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int base = 0, t = 0;
#pragma unroll
    for (int z = 0; z < kWaves; ++z) {
      const int v = sh.tmp[q][z];
      base += (z < w) ? v : 0;
      t += v;
    }
    excl[q] = base + incl[q] - x[q];
    tot[q] = t;
  }
  __syncthreads();
}

// Block minimum of x[0..3] (maxima are passed negated).
__device__ __forceinline__ void block_min4(int* x, Shared& sh) {
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x[q] = min(x[q], __shfl_xor(x[q], o, 64));
    if ((threadIdx.x & 63) == 0) sh.tmp[q][w] = x[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int r = sh.tmp[q][0];
#pragma unroll
    for (int z = 1; z < kWaves; ++z) r = min(r, sh.tmp[q][z]);
    x[q] = r;
  }
  __syncthreads();
}

struct Region {
  int rs, m;     // first logical index, tokens before the step
  int e;         // evicted
  int first_ev;  // logical index of the first / last evicted token
  int last_ev;
  int js;        // new logical index of the region's first survivor
  bool left;     // pack toward the base (true) or toward the end (false)
  int movers;
};

__device__ __forceinline__ void plan_region(Region& r) {
  if (r.e == 0) {
    r.left = true;
    r.movers = 0;
    return;
  }
  const int mk = r.m - r.e;                           // survivors
  const int cost_l = mk - (r.first_ev - r.rs);        // survivors after the first hole
  const int cost_r = (r.last_ev - r.rs) - (r.e - 1);  // survivors before the last hole
  r.left = cost_l <= cost_r;
  r.movers = r.left ? cost_l : cost_r;
}

template <bool REG>
__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  const CacheView& c = a.c;
  const int lb = blockIdx.x;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  const int cap = c.cap;
  const int H = c.hkv, D = c.d;
  int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  const int n = meta[CONFK_META_N];
  const int n8 = meta[CONFK_META_N8];
  const int base8 = meta[CONFK_META_BASE8];
  const int base16 = meta[CONFK_META_BASE16];
  const int P = a.protect;
  const int N = max(a.budget[l * a.budget_stride + b], P);
  float* ema = c.ema + (size_t)lbc * cap;
  int32_t* pos = c.pos + (size_t)lbc * cap;
  const float* score = a.score + (size_t)lb * cap;

  extern __shared__ int lds_i[];
  int* S = lds_i;                                // [kWin] survivor list window
  uint32_t* evbits = (uint32_t*)(lds_i + kWin);  // [(cap + 31) / 32] eviction flags
  __shared__ Shared sh;

  const int nn = n + 1;  // tokens incl. the new one
  const int f = n - n8;
  if (!meta_ok(n, n8, base8, base16, cap, c.cap16)) {  // no room: flag, leave the cache as it is
    if (threadIdx.x == 0) {
      atomicOr(c.status, (uint32_t)CONFK_STATUS_CAPACITY);
      meta[CONFK_META_EVICTED] = 0;
      meta[CONFK_META_MOVED] = 0;
      meta[CONFK_META_MOVED16] = 0;
      if (a.evicted_out) a.evicted_out[lb] = 0;
    }
    return;
  }
  const int k = n > N ? n - N : 0;
  const int ncand = n - P;  // candidates: logical [0, ncand)

  // the new token's rows: 16-byte pieces over (K|V, head, d); each thread's
  // first piece is read now, the rest (large head counts only) at the append
  const int half_pieces = H * D / 8;
  auto app_src = [&](int e) {
    const int kv = e / half_pieces, r = e - kv * half_pieces;
    return reinterpret_cast<const u32x4*>((kv ? a.v_new : a.k_new) + (size_t)lb * H * D + r * 8);
  };
  u32x4 app = {0u, 0u, 0u, 0u};
  if ((int)threadIdx.x < 2 * half_pieces) app = *app_src(threadIdx.x);

  int n8n = n8, fn = f, b8 = base8, b16 = base16, nkeep = nn, moved8 = 0, moved16 = 0;
  if (k > 0) {
    const int chunk = (nn + kThreads - 1) / kThreads;
    const int lo = min(nn, (int)threadIdx.x * chunk);
    const int cnt = min(nn, lo + chunk) - lo;
    uint32_t kreg[REG ? kRegKeys : 1];
    if constexpr (REG) {
#pragma unroll
      for (int j = 0; j < kRegKeys; ++j) {
        const int i = lo + j;
        kreg[j] = (j < cnt && i < ncand) ? ord_bits(score[i]) : 0xFFFFFFFFu;
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
    for (int i = threadIdx.x; i < (nn + 31) / 32; i += kThreads) evbits[i] = 0u;

    // ------------------------------------------------------ 1. select
    // Small k (register path): the k smallest 64-bit keys (score bits, index)
    // are found exactly by k rounds of wave minima per wave, then k rounds
    // over the waves' candidates; no atomics. Otherwise a 4-pass radix select
    // on the score bits, with ties at the threshold resolved by index.
    const bool small = REG && k <= kSmallK;
    uint64_t T64 = 0;
    uint32_t T = 0;
    int kk = k;
    if (small) {
      uint64_t k64[REG ? kRegKeys : 1];
#pragma unroll
      for (int j = 0; j < (REG ? kRegKeys : 1); ++j) {
        const int i = lo + j;
        k64[j] = (j < cnt && i < ncand) ? (((uint64_t)key_at(j) << 32) | (uint32_t)i) : ~0ull;
      }
      const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
      for (int r = 0; r < k; ++r) {
        uint64_t m = ~0ull;
#pragma unroll
        for (int j = 0; j < (REG ? kRegKeys : 1); ++j) m = min(m, k64[j]);
        uint64_t wmin = m;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const uint64_t y = __shfl_xor(wmin, o, 64);
          wmin = min(wmin, y);
        }
        if (lane == 0) sh.wk[w][r] = wmin;
#pragma unroll
        for (int j = 0; j < (REG ? kRegKeys : 1); ++j)
          if (k64[j] == wmin) k64[j] = ~0ull;  // keys are unique: only the owner matches
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        // the waves' k smallest hold the block's k smallest
        uint64_t v[(kWaves * kSmallK + 63) / 64];
#pragma unroll
        for (int q = 0; q < (kWaves * kSmallK + 63) / 64; ++q) {
          const int e = lane + 64 * q;
          const int ww = e / kSmallK, rr = e - ww * kSmallK;
          v[q] = (ww < kWaves && rr < k) ? sh.wk[ww][rr] : ~0ull;
        }
        uint64_t kth = ~0ull;
        for (int r = 0; r < k; ++r) {
          uint64_t m = ~0ull;
#pragma unroll
          for (int q = 0; q < (kWaves * kSmallK + 63) / 64; ++q) m = min(m, v[q]);
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) {
            const uint64_t y = __shfl_xor(m, o, 64);
            m = min(m, y);
          }
          kth = m;
#pragma unroll
          for (int q = 0; q < (kWaves * kSmallK + 63) / 64; ++q)
            if (v[q] == m) v[q] = ~0ull;
        }
        if (lane == 0) sh.kth = kth;
      }
      __syncthreads();
      T64 = sh.kth;
    } else {
      uint32_t prefix = 0, mask = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0;
        __syncthreads();
        if constexpr (REG) {
#pragma unroll
          for (int j = 0; j < kRegKeys; ++j)
            if (j < cnt && lo + j < ncand && (kreg[j] & mask) == prefix)
              atomicAdd(&sh.hist[(kreg[j] >> shift) & 255u], 1u);
        } else {
          for (int j = 0; j < cnt; ++j) {
            const uint32_t key = key_at(j);
            if (lo + j < ncand && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
          }
        }
        __syncthreads();
        if (threadIdx.x < 64) {
          const int lane = threadIdx.x;
          const uint32_t h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1],
                         h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
          const int s = (int)(h0 + h1 + h2 + h3);
          int incl = s;
          for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
          }
          const int excl = incl - s;
          if (excl < kk && kk <= incl) {
            // first of the lane's 4 bins whose running count reaches kk
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
      T = prefix;  // the kk oldest ties at T leave
    }

    // ------------------------------------------- 2. flags, scans, regions
    const int jmax = REG ? kRegKeys : cnt;  // constant trip count keeps kreg in registers
    int x4[4] = {0, 0, 0, 0}, ex4[4], tot4[4];
    if (!small) {
#pragma unroll
      for (int j = 0; j < jmax; ++j)
        if (j < cnt) x4[0] += (lo + j < ncand && key_at(j) == T) ? 1 : 0;
      block_scan4(x4, ex4, tot4, sh);
    }
    int keeps = 0, e8 = 0, e16 = 0;
    int mm[4] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX};  // first8, -last8, first16, -last16
    {
      int tie_run = small ? 0 : ex4[0];
#pragma unroll
      for (int j = 0; j < jmax; ++j) {
        if (j >= cnt) break;
        const int i = lo + j;
        bool ev = false;
        if (i < ncand) {
          const uint32_t key = key_at(j);
          if (small) {
            ev = (((uint64_t)key << 32) | (uint32_t)i) <= T64;
          } else if (key < T) {
            ev = true;
          } else if (key == T) {
            ev = tie_run < kk;
            ++tie_run;
          }
        }
        if (ev) {
          atomicOr(&evbits[i >> 5], 1u << (i & 31));
          if (i < n8) {
            ++e8;
            mm[0] = min(mm[0], i);
            mm[1] = min(mm[1], -i);
          } else {
            ++e16;
            mm[2] = min(mm[2], i);
            mm[3] = min(mm[3], -i);
          }
        } else {
          ++keeps;
        }
      }
    }
    x4[0] = keeps;
    x4[1] = e8;
    x4[2] = e16;
    x4[3] = 0;
    block_scan4(x4, ex4, tot4, sh);  // its barriers also publish evbits
    const int keep_base = ex4[0];
    nkeep = tot4[0];
    block_min4(mm, sh);
    Region r8{0, n8, tot4[1], mm[0], -mm[1], 0, true, 0};
    Region r16{n8, f, tot4[2], mm[2], -mm[3], n8 - tot4[1], true, 0};
    plan_region(r8);
    plan_region(r16);

    // survivor list for new logical indices [w0, w0 + kWin)
    int have_w0 = -1;
    auto build_window = [&](int w0) {
      __syncthreads();
      int jn = keep_base;
      for (int j = 0; j < cnt; ++j) {
        const int i = lo + j;
        if (!((evbits[i >> 5] >> (i & 31)) & 1u)) {
          if (jn >= w0 && jn < w0 + kWin) S[jn - w0] = i;
          ++jn;
        }
      }
      __syncthreads();
      have_w0 = w0;
    };

    // ------------------------------------------------ 3. metadata, ascending
    for (int w0 = 0; w0 < nkeep; w0 += kWin) {
      build_window(w0);
      const int wend = min(nkeep, w0 + kWin);
      float ev_[kMetaPer];
      int pv_[kMetaPer];
#pragma unroll
      for (int r = 0; r < kMetaPer; ++r) {
        const int j = w0 + threadIdx.x + r * kThreads;
        if (j < wend) {
          const int i = S[j - w0];
          ev_[r] = ema[i];
          pv_[r] = pos[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kMetaPer; ++r) {
        const int j = w0 + threadIdx.x + r * kThreads;
        if (j < wend) {
          ema[j] = ev_[r];
          pos[j] = pv_[r];
        }
      }
    }

    // ------------------------------------------------------ 4. K/V rows
    auto move_region = [&](const Region& r, const bool is8) {
      if (r.movers == 0) return;
      const int C = is8 ? cap : c.cap16;
      const int base = is8 ? base8 : base16;
      const int rowbytes = is8 ? D : 2 * D;  // per head, K or V
      const int pieces_h = rowbytes / 16;    // 16-byte pieces per head row
      const int pieces = 2 * H * pieces_h;   // per token (K and V, all heads)
      const int per_round = max(1, (kRegs * kThreads) / pieces);
      unsigned char* kb = is8 ? (unsigned char*)c.k8 : (unsigned char*)c.k16;
      unsigned char* vb = is8 ? (unsigned char*)c.v8 : (unsigned char*)c.v16;
      const size_t head_stride = (size_t)C * rowbytes;  // bytes per (l, b, head) ring
      const size_t lb_off = (size_t)lbc * H * head_stride;
      const int mk = r.m - r.e;
      const int jlo = r.left ? (r.first_ev - r.rs) : 0;  // region-local new indices
      const int jhi = r.left ? mk : r.movers;            // exclusive
      const int nrounds = (jhi - jlo + per_round - 1) / per_round;
      // round rr covers region-local new indices [ja, jb): ascending when
      // packing toward the base, descending otherwise
      auto bounds = [&](int rr, int& ja, int& jb) {
        if (r.left) {
          ja = jlo + rr * per_round;
          jb = min(jhi, ja + per_round);
        } else {
          jb = jhi - rr * per_round;
          ja = max(jlo, jb - per_round);
        }
      };
      // row piece uu of round [ja, ...): pointer to its (l, b, head) ring and
      // the source / destination slots
      auto piece = [&](int uu, int ja, int& slot_src, int& slot_dst) -> unsigned char* {
        const int mv = uu / pieces;
        const int rem = uu - mv * pieces;
        const int kv = rem / (H * pieces_h);
        const int rem2 = rem - kv * H * pieces_h;
        const int hh = rem2 / pieces_h;
        const int pc = rem2 - hh * pieces_h;
        const int jl = ja + mv;
        int s0 = base + (S[r.js + jl - have_w0] - r.rs);
        if (s0 >= C) s0 -= C;
        int s1 = base + (r.left ? jl : jl + r.e);
        if (s1 >= C) s1 -= C;
        slot_src = s0;
        slot_dst = s1;
        return (kv ? vb : kb) + lb_off + hh * head_stride + pc * 16;
      };
      // Round rr+1 reads only slots that round rr does not write (its sources
      // lie beyond round rr's destinations in the packing direction), so the
      // loads of the next round are issued right after the stores of this
      // one; a wait plus barrier then orders them before the next stores.
      u32x4 buf[kRegs];
      int ja, jb;
      bounds(0, ja, jb);
      {
        const int ga = r.js + ja, gb = r.js + jb;
        if (have_w0 < 0 || ga < have_w0 || gb > have_w0 + kWin) build_window(max(0, min(ga, nkeep - kWin)));
      }
#pragma unroll
      for (int q = 0; q < kRegs; ++q) {
        const int uu = threadIdx.x + q * kThreads;
        if (uu < (jb - ja) * pieces) {
          int ss, sd;
          unsigned char* p = piece(uu, ja, ss, sd);
          buf[q] = *reinterpret_cast<const u32x4*>(p + (size_t)ss * rowbytes);
        }
      }
      for (int rr = 0; rr < nrounds; ++rr) {
        // stores of round rr (destinations from the current window)
#pragma unroll
        for (int q = 0; q < kRegs; ++q) {
          const int uu = threadIdx.x + q * kThreads;
          if (uu < (jb - ja) * pieces) {
            int ss, sd;
            unsigned char* p = piece(uu, ja, ss, sd);
            *reinterpret_cast<u32x4*>(p + (size_t)sd * rowbytes) = buf[q];
          }
        }
        if (rr + 1 < nrounds) {
          int na, nb;
          bounds(rr + 1, na, nb);
          const int ga = r.js + na, gb = r.js + nb;
          if (ga < have_w0 || gb > have_w0 + kWin) {
            // the survivor list moves on: finish this round first
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            build_window(max(0, min(ga, nkeep - kWin)));
          }
#pragma unroll
          for (int q = 0; q < kRegs; ++q) {
            const int uu = threadIdx.x + q * kThreads;
            if (uu < (nb - na) * pieces) {
              int ss, sd;
              unsigned char* p = piece(uu, na, ss, sd);
              buf[q] = *reinterpret_cast<const u32x4*>(p + (size_t)ss * rowbytes);
            }
          }
          ja = na;
          jb = nb;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    };
    move_region(r8, true);
    move_region(r16, false);
    moved8 = r8.movers;
    moved16 = r16.movers;

    n8n = n8 - r8.e;
    fn = f - r16.e;
    if (!r8.left) {
      b8 += r8.e;
      if (b8 >= cap) b8 -= cap;
    }
    if (!r16.left) {
      b16 += r16.e;
      if (b16 >= c.cap16) b16 -= c.cap16;
    }
  }

  // ------------------------------------------------- 5. append + header
  {
    int slot = b16 + fn;
    if (slot >= c.cap16) slot -= c.cap16;
    for (int e = threadIdx.x; e < 2 * half_pieces; e += kThreads) {
      const int kv = e / half_pieces, r = e - kv * half_pieces;
      const int hh = (r * 8) / D, ch = (r * 8) - hh * D;
      uint16_t* dst = (kv ? c.v16 : c.k16) + (((size_t)lbc * H + hh) * c.cap16 + slot) * D + ch;
      *reinterpret_cast<u32x4*>(dst) = e == (int)threadIdx.x ? app : *app_src(e);
    }
  }
  if (threadIdx.x == 0) {
    meta[CONFK_META_N] = nkeep;
    meta[CONFK_META_N8] = n8n;
    meta[CONFK_META_BASE8] = b8;
    meta[CONFK_META_BASE16] = b16;
    meta[CONFK_META_EVICTED] = k;
    meta[CONFK_META_MOVED] = moved8;
    meta[CONFK_META_MOVED16] = moved16;
    if (a.evicted_out) a.evicted_out[lb] = k;
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const int lds = (kWin + (a.c.cap + 32) / 32 + 1) * 4;
  const int blocks = a.nl * a.c.B;
  if (a.c.cap <= kRegKeys * kThreads) {
    hipLaunchKernelGGL(compact_kernel<true>, dim3(blocks), dim3(kThreads), lds, s, a);
  } else {
    hipLaunchKernelGGL(compact_kernel<false>, dim3(blocks), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace confk

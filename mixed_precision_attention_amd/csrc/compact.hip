// Budget eviction, stable compaction and append of the new token.
//
// CONF-KV summary, "Methodik: CONF-KV": tokens are ranked by the composite
// score, the newest P are never evicted (Token-Ranking und Eviktion), and
// the survivors are packed contiguously so attention reads a dense layout
// without indirection tables (Implementierung). Review "方法步骤详情"
// (Algorithm 1): if |C_l| > N evict the lowest-ranked unprotected tokens and
// compact the survivors; step 13 appends the new K/V in FP16.
//
// One workgroup per (layer, sequence):
//  1. k = n - N tokens leave, chosen among the n - P oldest. A 4-pass radix
//     select over order-preserving uint32 images of the fp32 scores finds the
//     k-th smallest score T; every candidate below T leaves, plus the oldest
//     ties at T (a prefix count in position order), which makes the evicted
//     set unique: the k smallest (score, position) pairs.
//  2. Block scans give each survivor its new logical index; the survivor
//     list (new index -> old index) is kept in LDS.
//  3. EMA / position metadata are rewritten densely (in place, ascending).
//  4. K/V rows move inside their rings. Each region (INT8 ring, FP16 ring)
//     is packed toward the end that moves fewer rows: keep the base and
//     shift the survivors after the first hole down, or advance the base and
//     shift the survivors before the last hole up. Evictions mostly hit old
//     tokens, so usually only a few rows move. Moves go in rounds (read all
//     rows of a round, barrier, write them) in an order that never
//     overwrites an unread source.
//  5. The new token's K/V rows are written to the FP16 ring.
#include "confk_internal.h"

namespace confk {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kWin = 8192;  // survivor-list entries held in LDS at once
constexpr int kRegs = 4;    // 16-byte row pieces per thread per move round

__device__ __forceinline__ uint32_t ord_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Scan {
  int tmp[kWaves];
};

// Exclusive block scan; also returns the block total.
__device__ __forceinline__ int block_excl_scan(int x, Scan& sh, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh.tmp[w] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    const int v = sh.tmp[q];
    base += (q < w) ? v : 0;
    total += v;
  }
  __syncthreads();
  return base + incl - x;
}

__device__ __forceinline__ int block_min(int x, Scan& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  if ((threadIdx.x & 63) == 0) sh.tmp[threadIdx.x >> 6] = x;
  __syncthreads();
  int r = sh.tmp[0];
#pragma unroll
  for (int q = 1; q < kWaves; ++q) r = min(r, sh.tmp[q]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_max(int x, Scan& sh) { return -block_min(-x, sh); }

struct Region {
  int rs, m;      // first logical index, tokens before the step
  int e;          // evicted
  int first_ev;   // logical index of the first / last evicted token
  int last_ev;
  int js;         // new logical index of the region's first survivor
  bool left;      // pack toward the base (true) or toward the end (false)
  int movers;
};

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  const CacheView& c = a.c;
  const int lb = blockIdx.x;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  const int cap = c.cap;
  int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  const int n = meta[CONFK_META_N];
  const int n8 = meta[CONFK_META_N8];
  const int base8 = meta[CONFK_META_BASE8];
  const int base16 = meta[CONFK_META_BASE16];
  const int P = a.protect;
  int N = a.budget[l * a.budget_stride + b];
  N = max(N, P);
  float* ema = c.ema + (size_t)lbc * cap;
  int32_t* pos = c.pos + (size_t)lbc * cap;
  const float* score = a.score + (size_t)lb * cap;

  extern __shared__ int lds_i[];
  int* S = lds_i;                                // [kWin] survivor list window
  uint32_t* evbits = (uint32_t*)(lds_i + kWin);  // [(cap + 31) / 32]
  __shared__ Scan sh;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_digit, sel_before;

  const int nn = n + 1;                   // tokens incl. the new one
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
  const int ncand = n - P;                // candidates: logical [0, ncand)

  // ---------------------------------------------------------- 1. select
  uint32_t T = 0;
  int kk = 0;
  if (k > 0) {
    uint32_t prefix = 0, mask = 0;
    kk = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < 256; i += kThreads) hist[i] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < ncand; i += kThreads) {
        const uint32_t key = ord_bits(score[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                       h3 = hist[4 * lane + 3];
        const int s = (int)(h0 + h1 + h2 + h3);
        int incl = s;
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (lane >= o) incl += y;
        }
        const int excl = incl - s;
        if (excl < kk && kk <= incl) {
          int before = excl, dg = 4 * lane;
          const uint32_t hh[4] = {h0, h1, h2, h3};
          for (int q = 0; q < 4; ++q) {
            if (before + (int)hh[q] >= kk) {
              dg = 4 * lane + q;
              break;
            }
            before += (int)hh[q];
          }
          sel_digit = (uint32_t)dg;
          sel_before = (uint32_t)before;
        }
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      mask |= 0xFFu << shift;
      kk -= (int)sel_before;
      __syncthreads();
    }
    T = prefix;
  }

  // per-thread contiguous chunk of logical indices [lo, hi) over [0, nn)
  const int chunk = (nn + kThreads - 1) / kThreads;
  const int lo = min(nn, (int)threadIdx.x * chunk);
  const int hi = min(nn, lo + chunk);
  const int nwords = (nn + 31) >> 5;

  for (int i = threadIdx.x; i < nwords; i += kThreads) evbits[i] = 0u;
  __syncthreads();

  // ---------------------------------------------------- 2. flags and scans
  int tie_base = 0;
  if (k > 0) {
    int ties = 0;
    for (int i = lo; i < hi; ++i)
      if (i < ncand && ord_bits(score[i]) == T) ++ties;
    int tot;
    tie_base = block_excl_scan(ties, sh, tot);
  }
  int keeps = 0;
  int e8 = 0, e16 = 0;
  int f8 = INT32_MAX, l8 = -1, f16 = INT32_MAX, l16 = -1;
  if (k > 0) {
    int tie_run = tie_base;
    for (int i = lo; i < hi; ++i) {
      bool ev = false;
      if (i < ncand) {
        const uint32_t key = ord_bits(score[i]);
        if (key < T) {
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
          f8 = min(f8, i);
          l8 = max(l8, i);
        } else {
          ++e16;
          f16 = min(f16, i);
          l16 = max(l16, i);
        }
      } else {
        ++keeps;
      }
    }
  } else {
    keeps = hi - lo;
  }
  int nkeep;
  const int keep_base = block_excl_scan(keeps, sh, nkeep);  // == nn - k
  Region r8, r16;
  r8.rs = 0;
  r8.m = n8;
  r16.rs = n8;
  r16.m = f;
  {
    int t8, t16;
    block_excl_scan(e8, sh, t8);
    block_excl_scan(e16, sh, t16);
    r8.e = t8;
    r16.e = t16;
  }
  r8.first_ev = block_min(f8, sh);
  r8.last_ev = block_max(l8, sh);
  r16.first_ev = block_min(f16, sh);
  r16.last_ev = block_max(l16, sh);
  r8.js = 0;
  r16.js = n8 - r8.e;
  auto plan = [](Region& r) {
    if (r.e == 0) {
      r.left = true;
      r.movers = 0;
    } else {
      const int mk = r.m - r.e;                            // survivors
      const int cost_l = mk - (r.first_ev - r.rs);         // survivors after the first hole
      const int cost_r = (r.last_ev - r.rs) - (r.e - 1);   // survivors before the last hole
      r.left = cost_l <= cost_r;
      r.movers = r.left ? cost_l : cost_r;
    }
  };
  plan(r8);
  plan(r16);

  // survivor list for new logical indices [w0, w0 + kWin)
  auto build_window = [&](int w0) {
    __syncthreads();
    int j = keep_base;
    for (int i = lo; i < hi; ++i) {
      const bool ev = (evbits[i >> 5] >> (i & 31)) & 1u;
      if (!ev) {
        if (j >= w0 && j < w0 + kWin) S[j - w0] = i;
        ++j;
      }
    }
    __syncthreads();
  };

  int moved8 = 0, moved16 = 0;
  if (k > 0) {
    // ------------------------------------------------- 3. metadata, ascending
    int have_w0 = -1;
    for (int w0 = 0; w0 < nkeep; w0 += kWin) {
      build_window(w0);
      have_w0 = w0;
      const int wend = min(nkeep, w0 + kWin);
      for (int j0 = w0; j0 < wend; j0 += kThreads) {
        const int j = j0 + threadIdx.x;
        float ev_ = 0.f;
        int pv = 0;
        if (j < wend) {
          const int i = S[j - w0];
          ev_ = ema[i];
          pv = pos[i];
        }
        __syncthreads();
        if (j < wend) {
          ema[j] = ev_;
          pos[j] = pv;
        }
        __syncthreads();
      }
    }

    // ------------------------------------------------------ 4. K/V rows
    const int H = c.hkv, D = c.d;
    for (int ri = 0; ri < 2; ++ri) {
      Region& r = ri == 0 ? r8 : r16;
      if (r.movers == 0) continue;
      const bool is8 = ri == 0;
      const int C = is8 ? cap : c.cap16;
      const int base = is8 ? base8 : base16;
      const int rowbytes = is8 ? D : 2 * D;               // per head, K or V
      const int pieces_h = rowbytes / 16;                 // 16-byte pieces per head row
      const int pieces = 2 * H * pieces_h;                // per token (K and V, all heads)
      const int per_round = max(1, (kRegs * kThreads) / pieces);
      unsigned char* kb = is8 ? (unsigned char*)c.k8 : (unsigned char*)c.k16;
      unsigned char* vb = is8 ? (unsigned char*)c.v8 : (unsigned char*)c.v16;
      const size_t head_stride = (size_t)C * rowbytes;    // bytes per (l, b, head) ring
      const size_t lb_off = (size_t)lbc * H * head_stride;
      // region-local new index range of the movers
      const int mk = r.m - r.e;
      const int jlo = r.left ? (r.first_ev - r.rs) : 0;
      const int jhi = r.left ? mk : r.movers;   // exclusive
      // rounds in the safe order: ascending when packing left, descending otherwise
      const int nrounds = (jhi - jlo + per_round - 1) / per_round;
      for (int rr = 0; rr < nrounds; ++rr) {
        int ja, jb;  // region-local new indices [ja, jb) of this round
        if (r.left) {
          ja = jlo + rr * per_round;
          jb = min(jhi, ja + per_round);
        } else {
          jb = jhi - rr * per_round;
          ja = max(jlo, jb - per_round);
        }
        // make sure the survivor list window covers [js+ja, js+jb)
        const int ga = r.js + ja, gb = r.js + jb;
        if (have_w0 < 0 || ga < have_w0 || gb > have_w0 + kWin) {
          const int w0 = max(0, min(ga, nkeep - kWin));
          build_window(w0);
          have_w0 = w0;
        }
        uint4 buf[kRegs];
        const int total = (jb - ja) * pieces;
#pragma unroll
        for (int q = 0; q < kRegs; ++q) {
          const int u = threadIdx.x + q * kThreads;
          if (u < total) {
            const int mv = u / pieces;
            const int rem = u - mv * pieces;
            const int kv = rem / (H * pieces_h);
            const int rem2 = rem - kv * H * pieces_h;
            const int hh = rem2 / pieces_h;
            const int pc = rem2 - hh * pieces_h;
            const int jl = ja + mv;
            const int src_local = S[r.js + jl - have_w0] - r.rs;
            int slot = base + src_local;
            if (slot >= C) slot -= C;
            const unsigned char* src =
                (kv ? vb : kb) + lb_off + hh * head_stride + (size_t)slot * rowbytes + pc * 16;
            buf[q] = *reinterpret_cast<const uint4*>(src);
          }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kRegs; ++q) {
          const int u = threadIdx.x + q * kThreads;
          if (u < total) {
            const int mv = u / pieces;
            const int rem = u - mv * pieces;
            const int kv = rem / (H * pieces_h);
            const int rem2 = rem - kv * H * pieces_h;
            const int hh = rem2 / pieces_h;
            const int pc = rem2 - hh * pieces_h;
            const int jl = ja + mv;
            const int dst_local = r.left ? jl : jl + r.e;
            int slot = base + dst_local;
            if (slot >= C) slot -= C;
            unsigned char* dst =
                (kv ? vb : kb) + lb_off + hh * head_stride + (size_t)slot * rowbytes + pc * 16;
            *reinterpret_cast<uint4*>(dst) = buf[q];
          }
        }
        __syncthreads();
      }
      (is8 ? moved8 : moved16) += r.movers;
    }
  }

  // ------------------------------------------------- 5. append + header
  const int n8n = n8 - r8.e;
  const int fn = f - r16.e;  // FP16 survivors before the append
  int b8 = base8, b16 = base16;
  if (!r8.left) {
    b8 += r8.e;
    if (b8 >= cap) b8 -= cap;
  }
  if (!r16.left) {
    b16 += r16.e;
    if (b16 >= c.cap16) b16 -= c.cap16;
  }
  {
    int slot = b16 + fn;
    if (slot >= c.cap16) slot -= c.cap16;
    const int H = c.hkv, D = c.d;
    const size_t ring = (size_t)c.cap16 * D;  // halves per (l, b, head)
    const uint16_t* kn = a.k_new + (size_t)lb * H * D;
    const uint16_t* vn = a.v_new + (size_t)lb * H * D;
    for (int e = threadIdx.x; e < H * D; e += kThreads) {
      const int hh = e / D, ch = e - hh * D;
      const size_t off = ((size_t)lbc * H + hh) * ring + (size_t)slot * D + ch;
      c.k16[off] = kn[e];
      c.v16[off] = vn[e];
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
  hipLaunchKernelGGL(compact_kernel, dim3(a.nl * a.c.B), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace confk

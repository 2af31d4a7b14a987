// Device code of the confidence pass, shared by the confidence call's
// kernels and by the fused calls that run it inside other launches.
// CONF-KV summary, "Methodik: CONF-KV" (Konfidenzschaetzung, adaptive
// Budgetauswahl) and the review's "核心方法": from the merged row state
// (M, S = sum e^(z-M), T = sum (z-M) e^(z-M), top1 >= top2) the confidence is
// c = w_H (1 - H/ln V) + w_m sigmoid(top1 - top2) + w_p / S with
// H = ln S - T/S, and the budget is N_high when c >= tau, else N_low. The
// review's Algorithm 1, step 13: the next token (greedy, or by inversion of
// the tempered softmax with the caller's uniform number).
//
//  conf_partial_block: one 256-thread workgroup reduces one 4096-logit chunk
//    of a row to a state record;
//  conf_row_c: one wave merges a row's records in a fixed order (every lane
//    ends with the same state), takes the next token and returns c;
//  conf_final_row: conf_row_c plus the outputs (c, token, status, budgets).
#pragma once

#include "confk_internal.h"

namespace confk {
namespace confm {

constexpr int kConfThreads = 256;       // workgroup of the pass
constexpr int kConfPerThread = 16;      // logits per thread
constexpr int kChunk = kConfThreads * kConfPerThread;  // logits per partial state
constexpr int kLanePer = kChunk / 64;  // elements per lane in the sampling scan
constexpr float kLog2e = 1.4426950408889634f;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// e^d for d <= 0 through the hardware base-2 exponential.
__device__ __forceinline__ float exp_neg(float d) { return exp2f(d * kLog2e); }

struct RowState {
  float M, S, T, t1, t2;
  uint32_t flag;  // bit 0: NaN or +inf seen
  float ST;       // sum e^((z-M)/temp), sampling only
  int32_t i1;     // index of t1 (smallest among equal maxima)
};
constexpr int kRec = 8;  // floats per partial record

// kind of next-token choice made in the pass
enum { kNoChoice = 0, kGreedy = 1, kSample = 2 };

// Inserts x into the two largest values t1 >= t2 of a multiset.
__device__ __forceinline__ void top2_insert(float& t1, float& t2, float x) {
  const float n2 = fmaxf(t2, fminf(t1, x));
  t1 = fmaxf(t1, x);
  t2 = n2;
}

// inv_t: 1 / temperature (sampling only)
template <int CH>
__device__ __forceinline__ RowState merge(const RowState& a, const RowState& b, float inv_t) {
  // no FMA contraction: the same arithmetic in every kernel that inlines it
#pragma clang fp contract(off)
  RowState r;
  r.M = fmaxf(a.M, b.M);
  r.flag = a.flag | b.flag;
  r.t1 = fmaxf(a.t1, b.t1);
  r.t2 = fmaxf(fminf(a.t1, b.t1), fmaxf(a.t2, b.t2));
  if constexpr (CH == kGreedy)
    r.i1 = a.t1 > b.t1 ? a.i1 : (b.t1 > a.t1 ? b.i1 : min(a.i1, b.i1));
  else
    r.i1 = INT32_MAX;
  r.S = 0.f;
  r.T = 0.f;
  r.ST = 0.f;
  if (a.S > 0.f) {
    const float d = a.M - r.M;
    const float e = exp_neg(d);
    r.S += a.S * e;
    r.T += (a.T + d * a.S) * e;
    if constexpr (CH == kSample) r.ST += a.ST * exp_neg(d * inv_t);
  }
  if (b.S > 0.f) {
    const float d = b.M - r.M;
    const float e = exp_neg(d);
    r.S += b.S * e;
    r.T += (b.T + d * b.S) * e;
    if constexpr (CH == kSample) r.ST += b.ST * exp_neg(d * inv_t);
  }
  return r;
}

template <int CH>
__device__ __forceinline__ RowState shfl_state(const RowState& s, int o) {
  RowState r;
  r.M = __shfl_xor(s.M, o, 64);
  r.S = __shfl_xor(s.S, o, 64);
  r.T = __shfl_xor(s.T, o, 64);
  r.t1 = __shfl_xor(s.t1, o, 64);
  r.t2 = __shfl_xor(s.t2, o, 64);
  r.flag = (uint32_t)__shfl_xor((int)s.flag, o, 64);
  r.ST = CH == kSample ? __shfl_xor(s.ST, o, 64) : 0.f;
  r.i1 = CH == kGreedy ? __shfl_xor(s.i1, o, 64) : INT32_MAX;
  return r;
}

// One 256-thread workgroup (tid = its thread index) reduces chunk `chunk`
// of row b to a state record in a.partial.
template <int CH>
__device__ __forceinline__ void conf_partial_block(const ConfArgs& a, const int chunk, const int b, const int tid) {
  // no FMA contraction: the same arithmetic in every kernel that inlines it
#pragma clang fp contract(off)
  const float* row = a.logits + (int64_t)b * a.ld;
  const int start = chunk * a.chunk;
  const int end = min(a.vocab, start + a.chunk);

  float x[kConfPerThread];
  if (a.vec4) {
    // 16-byte loads: thread t reads groups t, t+256, ... of 4 logits
#pragma unroll
    for (int k = 0; k < kConfPerThread / 4; ++k) {
      const int i = start + 4 * (tid + k * kConfThreads);
      if (i + 3 < end) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + i);
        x[4 * k] = v[0];
        x[4 * k + 1] = v[1];
        x[4 * k + 2] = v[2];
        x[4 * k + 3] = v[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * k + e] = (i + e < end) ? row[i + e] : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kConfPerThread; ++k) {
      const int i = start + tid + k * kConfThreads;
      x[k] = (i < end) ? row[i] : -INFINITY;
    }
  }
  // logical index of x[k], ascending in k
  auto idx = [&](int k) {
    return a.vec4 ? start + 4 * (tid + (k >> 2) * kConfThreads) + (k & 3) : start + tid + k * kConfThreads;
  };
  const float inv_t = a.inv_temp;
  RowState s;
  s.M = -INFINITY;
  s.t1 = -INFINITY;
  s.t2 = -INFINITY;
  s.flag = 0;
  s.i1 = INT32_MAX;
#pragma unroll
  for (int k = 0; k < kConfPerThread; ++k) {
    const float v = x[k];
    if (v != v || v == INFINITY) {
      s.flag = 1;
    } else {
      s.M = fmaxf(s.M, v);
      if constexpr (CH == kGreedy)
        if (v > s.t1) s.i1 = idx(k);  // strict: the first of equal maxima stays
      top2_insert(s.t1, s.t2, v);
    }
  }
  s.S = 0.f;
  s.T = 0.f;
  s.ST = 0.f;
  if (s.M > -INFINITY) {
#pragma unroll
    for (int k = 0; k < kConfPerThread; ++k) {
      const float v = x[k];
      if (v > -INFINITY && v < INFINITY) {  // finite (NaN fails both)
        const float d = v - s.M;
        const float e = exp_neg(d);
        s.S += e;
        s.T += d * e;
        if constexpr (CH == kSample) s.ST += exp_neg(d * inv_t);
      }
    }
  }
  // wave reduction
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s = merge<CH>(s, shfl_state<CH>(s, o), inv_t);
  __shared__ RowState red[kConfThreads / 64];
  const int w = tid >> 6;
  if ((tid & 63) == 0) red[w] = s;
  __syncthreads();
  if (tid == 0) {
    RowState r = red[0];
    for (int i = 1; i < kConfThreads / 64; ++i) r = merge<CH>(r, red[i], inv_t);
    float* p = a.partial + ((int64_t)b * a.nchunks + chunk) * kRec;
    const f32x4 lo = {r.M, r.S, r.T, r.t1};
    const f32x4 hi = {r.t2, __builtin_bit_cast(float, r.flag), r.ST, __builtin_bit_cast(float, r.i1)};
    if (a.vecrec) {
      reinterpret_cast<f32x4*>(p)[0] = lo;
      reinterpret_cast<f32x4*>(p)[1] = hi;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = lo[e];
        p[4 + e] = hi[e];
      }
    }
  }
}

// Row b, lane `lane` of one wave: lane i merges partials i, i+64, ... in
// order, then a butterfly merge (commutative, so every lane ends with the
// same state); then the next-token choice (into tok, every lane) and the
// confidence, returned to every lane (NaN for non-finite logits).
// Record i of row b (two 16-byte words when the records are aligned).
__device__ __forceinline__ RowState conf_record(const ConfArgs& a, const int b, const int i) {
  const float* p = a.partial + ((int64_t)b * a.nchunks + i) * kRec;
  f32x4 lo, hi;
  if (a.vecrec) {
    lo = reinterpret_cast<const f32x4*>(p)[0];
    hi = reinterpret_cast<const f32x4*>(p)[1];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = p[e];
      hi[e] = p[4 + e];
    }
  }
  RowState q;
  q.M = lo[0];
  q.S = lo[1];
  q.T = lo[2];
  q.t1 = lo[3];
  q.t2 = hi[0];
  // vector elements are copied to scalars before the bit casts (a bit cast
  // of the element expression itself reads element 0)
  const float flag_bits = hi[1], i1_bits = hi[3];
  q.flag = __builtin_bit_cast(uint32_t, flag_bits);
  q.ST = hi[2];
  q.i1 = __builtin_bit_cast(int32_t, i1_bits);
  return q;
}

template <int CH>
__device__ __forceinline__ RowState conf_lane_state(const ConfArgs& a, const int b, const int lane);
template <int CH>
__device__ __forceinline__ float conf_row_finish(const ConfArgs& a, const int b, const int lane, RowState r,
                                                 int& tok);

template <int CH>
__device__ __forceinline__ float conf_row_c(const ConfArgs& a, const int b, const int lane, int& tok) {
  return conf_row_finish<CH>(a, b, lane, conf_lane_state<CH>(a, b, lane), tok);
}

// The first part of conf_row_c: lane `lane`'s merge of records lane,
// lane + 64, ... (its loads can be issued early and the rest done later).
template <int CH>
__device__ __forceinline__ RowState conf_lane_state(const ConfArgs& a, const int b, const int lane) {
  const float inv_t = a.inv_temp;
  auto load = [&](int i) { return conf_record(a, b, i); };
  RowState r;
  r.M = -INFINITY;
  r.S = 0.f;
  r.T = 0.f;
  r.t1 = -INFINITY;
  r.t2 = -INFINITY;
  r.flag = 0;
  r.ST = 0.f;
  r.i1 = INT32_MAX;
  for (int i = lane; i < a.nchunks; i += 64) r = merge<CH>(r, load(i), inv_t);
  return r;
}

// The rest of conf_row_c: the butterfly merge of the lanes' states, the
// next-token choice and c.
template <int CH>
__device__ __forceinline__ float conf_row_finish(const ConfArgs& a, const int b, const int lane, RowState r,
                                                 int& tok) {
  // no FMA contraction: the same arithmetic in every kernel that inlines it
#pragma clang fp contract(off)
  const float inv_t = a.inv_temp;
  auto load = [&](int i) { return conf_record(a, b, i); };
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) r = merge<CH>(r, shfl_state<CH>(r, o), inv_t);
  const bool bad = r.flag != 0 || !(r.M > -INFINITY);

  tok = -1;
  if constexpr (CH != kNoChoice) {  // next-token choice (uniform per row)
    if constexpr (CH == kGreedy) {
      if (!bad) tok = r.i1;
    } else if (!bad) {
      // chunk weights e^((M_c - M)/T) S_T,c in chunk order; lane holds
      // chunks lane, lane+64, ... (ascending), the wave scans them in order
      const float target = a.uniform[b] * r.ST;
      float run = 0.f;  // weight of all chunks before this lane's current group
      int cstar = -1;
      float before = 0.f;
      for (int c0 = 0; c0 < a.nchunks && cstar < 0; c0 += 64) {
        const int ci = c0 + lane;
        float wgt = 0.f;
        if (ci < a.nchunks) {
          const RowState q = load(ci);
          if (q.S > 0.f) wgt = q.ST * exp_neg((q.M - r.M) * inv_t);
        }
        float incl = wgt;
        for (int o = 1; o < 64; o <<= 1) {
          const float yv = __shfl_up(incl, o, 64);
          if (lane >= o) incl += yv;
        }
        const bool cross = ci < a.nchunks && run + incl > target;
        const uint64_t m = __ballot(cross);
        if (m) {
          const int src = __ffsll((unsigned long long)m) - 1;
          cstar = c0 + src;
          before = run + __shfl(incl - wgt, src, 64);
        }
        run += __shfl(incl, 63, 64);
      }
      // rounding left the target at the total: the last chunk's last element
      const bool past_end = cstar < 0;
      if (past_end) cstar = a.nchunks - 1;
      // inside chunk cstar: lane L owns elements [start + L*kLanePer, +kLanePer)
      // in index order; their weights are read once and kept in registers
      static_assert(kChunk == 64 * kLanePer, "one chunk is 64 lanes' runs");
      const float* row = a.logits + (int64_t)b * a.ld;
      const int start = cstar * a.chunk;
      const int end = min(a.vocab, start + a.chunk);
      const int lo = start + lane * kLanePer, hi = min(end, lo + kLanePer);
      float wt[kLanePer];
#pragma unroll
      for (int k = 0; k < kLanePer / 4; ++k) {
        const int i = lo + 4 * k;
        f32x4 v;
        if (a.vec4 && i + 3 < hi) {
          v = *reinterpret_cast<const f32x4*>(row + i);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = i + e < hi ? row[i + e] : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) wt[4 * k + e] = v[e] > -INFINITY ? exp_neg((v[e] - r.M) * inv_t) : 0.f;
      }
      float wsum = 0.f;
#pragma unroll
      for (int j = 0; j < kLanePer; ++j) wsum += wt[j];
      float incl = wsum;
      for (int o = 1; o < 64; o <<= 1) {
        const float yv = __shfl_up(incl, o, 64);
        if (lane >= o) incl += yv;
      }
      const float t2 = past_end ? INFINITY : target - before;
      const uint64_t m = __ballot(lo < hi && incl > t2);
      const int src = m ? __ffsll((unsigned long long)m) - 1 : 63 - __clzll((long long)__ballot(lo < hi));
      float acc = __shfl(incl - wsum, src, 64);
      if (lane == src) {
        tok = hi - 1;  // rounding: the lane's last element
        bool found = false;
#pragma unroll
        for (int j = 0; j < kLanePer; ++j) {
          if (!found && lo + j < hi && wt[j] > 0.f) {
            acc += wt[j];
            if (acc > t2) {
              tok = lo + j;
              found = true;
            }
          }
        }
      }
      tok = __shfl(tok, src, 64);
    }
  }

  // every lane holds the merged state and computes c
  float c;
  if (bad) {
    c = __builtin_nanf("");
  } else {
    const float H = logf(r.S) - r.T / r.S;
    const float Hn = H / logf((float)a.vocab);
    const float m = r.t1 - r.t2;  // +inf when only one finite logit
    const float sig = 1.f / (1.f + expf(-m));
    const float p1 = 1.f / r.S;
    c = a.w_h * (1.f - Hn) + a.w_m * sig + a.w_p * p1;
  }
  return c;
}

// Budget of budget row l (per-layer budgets when given) for confidence c.
__device__ __forceinline__ int conf_budget(const ConfArgs& a, const int l, const float c) {
  const bool tight = c >= a.tau;  // false for NaN
  const int nh = a.layer_n_high ? a.layer_n_high[l] : a.n_high;
  const int nlo = a.layer_n_low ? a.layer_n_low[l] : a.n_low;
  return tight ? nh : nlo;
}

// The confidence call's final step for row b: c, the next token, the status
// bit for non-finite logits, and the budgets of all nbl rows (lane l writes
// rows l, l + 64, ...).
template <int CH>
__device__ __forceinline__ void conf_final_row(const ConfArgs& a, const int b, const int lane) {
  int tok;
  const float c = conf_row_c<CH>(a, b, lane, tok);
  if (lane == 0) {
    if (CH != kNoChoice) a.token_out[b] = tok;
    a.c_out[b] = c;
    if (c != c && a.status) atomicOr(a.status, (uint32_t)CONFK_STATUS_NONFINITE_LOGITS);
  }
  for (int l = lane; l < a.nbl; l += 64) a.budget_out[(int64_t)l * a.batch + b] = conf_budget(a, l, c);
}

}  // namespace confm
}  // namespace confk

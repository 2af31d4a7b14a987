// Merge of the per-chunk confidence states and the budget gate, one wave
// per row. CONF-KV summary, "Methodik: CONF-KV" (Konfidenzschaetzung,
// adaptive Budgetauswahl) and the review's "核心方法": from the merged row
// state (M, S = sum e^(z-M), T = sum (z-M) e^(z-M), top1 >= top2) the
// confidence is c = w_H (1 - H/ln V) + w_m sigmoid(top1 - top2) + w_p / S with
// H = ln S - T/S, and the budget is N_high when c >= tau, else N_low. The
// review's Algorithm 1, step 13: the next token (greedy, or by inversion of
// the tempered softmax with the caller's uniform number).
//
// Shared by the confidence call's final kernel and the fused confidence +
// attention call, which runs it in workgroups of the attention launch.
#pragma once

#include "confk_internal.h"

namespace confk {
namespace confm {

constexpr int kChunk = 4096;           // logits per partial state (one workgroup of the pass)
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

// Row b, lane `lane` of one wave: lane i merges partials i, i+64, ... in
// order, then a butterfly merge (commutative, so every lane ends with the
// same state); then the next-token choice, the confidence and the budgets.
template <int CH>
__device__ __forceinline__ void conf_final_row(const ConfArgs& a, const int b, const int lane) {
  const float* p = a.partial + (int64_t)b * a.nchunks * kRec;
  const float inv_t = a.inv_temp;
  auto load = [&](int i) {
    f32x4 lo, hi;
    if (a.vecrec) {
      lo = reinterpret_cast<const f32x4*>(p + kRec * i)[0];
      hi = reinterpret_cast<const f32x4*>(p + kRec * i)[1];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = p[kRec * i + e];
        hi[e] = p[kRec * i + 4 + e];
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
  };
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
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) r = merge<CH>(r, shfl_state<CH>(r, o), inv_t);
  const bool bad = r.flag != 0 || !(r.M > -INFINITY);

  if constexpr (CH != kNoChoice) {  // next-token choice (uniform per row)
    int tok = -1;
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
    if (lane == 0) a.token_out[b] = tok;
  }

  // every lane holds the merged state: each computes c, lane l writes the
  // budgets of layers l, l + 64, ... (per-layer budgets in parallel)
  float c;
  if (bad) {
    c = __builtin_nanf("");
    if (lane == 0 && a.status) atomicOr(a.status, (uint32_t)CONFK_STATUS_NONFINITE_LOGITS);
  } else {
    const float H = logf(r.S) - r.T / r.S;
    const float Hn = H / logf((float)a.vocab);
    const float m = r.t1 - r.t2;  // +inf when only one finite logit
    const float sig = 1.f / (1.f + expf(-m));
    const float p1 = 1.f / r.S;
    c = a.w_h * (1.f - Hn) + a.w_m * sig + a.w_p * p1;
  }
  if (lane == 0) a.c_out[b] = c;
  const bool tight = c >= a.tau;  // false for NaN
  for (int l = lane; l < a.nbl; l += 64) {
    const int nh = a.layer_n_high ? a.layer_n_high[l] : a.n_high;
    const int nlo = a.layer_n_low ? a.layer_n_low[l] : a.n_low;
    a.budget_out[(int64_t)l * a.batch + b] = tight ? nh : nlo;
  }
}

}  // namespace confm
}  // namespace confk

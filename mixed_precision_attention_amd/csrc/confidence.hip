// Confidence score and budget gate.
//
// CONF-KV summary, "Methodik: CONF-KV" (Konfidenzschaetzung, adaptive
// Budgetauswahl) and the review's "核心方法": each decode step reduces the
// vocab logits to c = w_H (1 - H/ln V) + w_m sigmoid(ln p1 - ln p2) + w_p p1
// and takes the tight budget N_high when c >= tau, the loose N_low otherwise.
//
// One pass over the logits. Every thread keeps, for its elements z,
//   M = max z,  S = sum e^(z-M),  T = sum (z-M) e^(z-M),  top1 >= top2,
// and the states merge associatively; from the merged row state
//   H = ln S - T/S,   p1 = 1/S,   ln p1 - ln p2 = top1 - top2.
// Rows are split over many workgroups (HBM-bound: each logit is read once);
// a second tiny kernel merges the per-chunk states in a fixed order, so the
// result does not depend on scheduling.
#include "confk_internal.h"

namespace confk {

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kThreads * kPerThread;
constexpr float kLog2e = 1.4426950408889634f;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// e^d for d <= 0 through the hardware base-2 exponential.
__device__ __forceinline__ float exp_neg(float d) { return exp2f(d * kLog2e); }

struct RowState {
  float M, S, T, t1, t2;
  uint32_t flag;  // bit 0: NaN or +inf seen
};

// Inserts x into the two largest values t1 >= t2 of a multiset.
__device__ __forceinline__ void top2_insert(float& t1, float& t2, float x) {
  const float n2 = fmaxf(t2, fminf(t1, x));
  t1 = fmaxf(t1, x);
  t2 = n2;
}

__device__ __forceinline__ RowState merge(const RowState& a, const RowState& b) {
  RowState r;
  r.M = fmaxf(a.M, b.M);
  r.flag = a.flag | b.flag;
  r.t1 = fmaxf(a.t1, b.t1);
  r.t2 = fmaxf(fminf(a.t1, b.t1), fmaxf(a.t2, b.t2));
  r.S = 0.f;
  r.T = 0.f;
  if (a.S > 0.f) {
    const float d = a.M - r.M;
    const float e = exp_neg(d);
    r.S += a.S * e;
    r.T += (a.T + d * a.S) * e;
  }
  if (b.S > 0.f) {
    const float d = b.M - r.M;
    const float e = exp_neg(d);
    r.S += b.S * e;
    r.T += (b.T + d * b.S) * e;
  }
  return r;
}

__device__ __forceinline__ RowState shfl_state(const RowState& s, int o) {
  RowState r;
  r.M = __shfl_xor(s.M, o, 64);
  r.S = __shfl_xor(s.S, o, 64);
  r.T = __shfl_xor(s.T, o, 64);
  r.t1 = __shfl_xor(s.t1, o, 64);
  r.t2 = __shfl_xor(s.t2, o, 64);
  r.flag = (uint32_t)__shfl_xor((int)s.flag, o, 64);
  return r;
}

__global__ __launch_bounds__(kThreads) void conf_partial_kernel(ConfArgs a) {
  const int b = blockIdx.y;
  const int chunk = blockIdx.x;
  const float* row = a.logits + (int64_t)b * a.ld;
  const int start = chunk * a.chunk;
  const int end = min(a.vocab, start + a.chunk);

  float x[kPerThread];
  if (a.vec4) {
    // 16-byte loads: thread t reads groups t, t+256, ... of 4 logits
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const int i = start + 4 * (threadIdx.x + k * kThreads);
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
    for (int k = 0; k < kPerThread; ++k) {
      const int i = start + threadIdx.x + k * kThreads;
      x[k] = (i < end) ? row[i] : -INFINITY;
    }
  }
  RowState s;
  s.M = -INFINITY;
  s.t1 = -INFINITY;
  s.t2 = -INFINITY;
  s.flag = 0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const float v = x[k];
    if (v != v || v == INFINITY) {
      s.flag = 1;
    } else {
      s.M = fmaxf(s.M, v);
      top2_insert(s.t1, s.t2, v);
    }
  }
  s.S = 0.f;
  s.T = 0.f;
  if (s.M > -INFINITY) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const float v = x[k];
      if (v > -INFINITY && v < INFINITY) {  // finite (NaN fails both)
        const float d = v - s.M;
        const float e = exp_neg(d);
        s.S += e;
        s.T += d * e;
      }
    }
  }
  // wave reduction
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s = merge(s, shfl_state(s, o));
  __shared__ RowState red[kThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = merge(r, red[i]);
    float* p = a.partial + ((int64_t)b * a.nchunks + chunk) * 6;
    p[0] = r.M;
    p[1] = r.S;
    p[2] = r.T;
    p[3] = r.t1;
    p[4] = r.t2;
    p[5] = __builtin_bit_cast(float, r.flag);
  }
}

// One wave per row: lane i merges partials i, i+64, ... in order, then a
// butterfly merge (commutative, so every lane ends with the same state).
__global__ __launch_bounds__(64) void conf_final_kernel(ConfArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float* p = a.partial + (int64_t)b * a.nchunks * 6;
  RowState r;
  r.M = -INFINITY;
  r.S = 0.f;
  r.T = 0.f;
  r.t1 = -INFINITY;
  r.t2 = -INFINITY;
  r.flag = 0;
  for (int i = lane; i < a.nchunks; i += 64) {
    RowState q;
    q.M = p[6 * i + 0];
    q.S = p[6 * i + 1];
    q.T = p[6 * i + 2];
    q.t1 = p[6 * i + 3];
    q.t2 = p[6 * i + 4];
    q.flag = __builtin_bit_cast(uint32_t, p[6 * i + 5]);
    r = merge(r, q);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) r = merge(r, shfl_state(r, o));
  if (lane != 0) return;
  float c;
  const bool bad = r.flag != 0 || !(r.M > -INFINITY);
  if (bad) {
    c = __builtin_nanf("");
    if (a.status) atomicOr(a.status, (uint32_t)CONFK_STATUS_NONFINITE_LOGITS);
  } else {
    const float H = logf(r.S) - r.T / r.S;
    const float Hn = H / logf((float)a.vocab);
    const float m = r.t1 - r.t2;  // +inf when only one finite logit
    const float sig = 1.f / (1.f + expf(-m));
    const float p1 = 1.f / r.S;
    c = a.w_h * (1.f - Hn) + a.w_m * sig + a.w_p * p1;
  }
  a.c_out[b] = c;
  const bool tight = c >= a.tau;  // false for NaN
  for (int l = 0; l < a.nbl; ++l) {
    const int nh = a.layer_n_high ? a.layer_n_high[l] : a.n_high;
    const int nlo = a.layer_n_low ? a.layer_n_low[l] : a.n_low;
    a.budget_out[(int64_t)l * a.batch + b] = tight ? nh : nlo;
  }
}

}  // namespace

size_t confidence_ws_bytes(int32_t batch, int32_t vocab) {
  const int nchunks = (vocab + kChunk - 1) / kChunk;
  return (size_t)batch * nchunks * 6 * sizeof(float);
}

hipError_t launch_confidence(const ConfArgs& in, hipStream_t s) {
  ConfArgs a = in;
  a.chunk = kChunk;
  a.nchunks = (a.vocab + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(conf_partial_kernel, dim3(a.nchunks, a.batch), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(conf_final_kernel, dim3(a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace confk

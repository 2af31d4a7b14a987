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
//
// Next-token choice (review Algorithm 1, step 13, the sampling of x_{t+1}),
// fused into the same pass: the state also carries the index of top1
// (greedy: the smallest index among equal maxima) and, for temperature
// sampling, S_T = sum e^((z-M)/T). The final kernel draws by inversion with
// the caller's uniform number u: the smallest index whose cumulative weight in
// index order exceeds u * S_T, found chunk by chunk and then inside the one
// chunk where the cumulative weight crosses. The kernels are instantiated per
// kind of choice (none, greedy, sampling), so each carries only the state it
// needs.
#include "confk_internal.h"

#include "confidence_merge.h"

namespace confk {

using namespace confm;

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
static_assert(kThreads * kPerThread == kChunk, "one workgroup reduces one chunk");

template <int CH>
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
  // logical index of x[k], ascending in k
  auto idx = [&](int k) {
    return a.vec4 ? start + 4 * (threadIdx.x + (k >> 2) * kThreads) + (k & 3) : start + threadIdx.x + k * kThreads;
  };
  const float inv_t = a.inv_temp;
  RowState s;
  s.M = -INFINITY;
  s.t1 = -INFINITY;
  s.t2 = -INFINITY;
  s.flag = 0;
  s.i1 = INT32_MAX;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
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
    for (int k = 0; k < kPerThread; ++k) {
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
  __shared__ RowState red[kThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = merge<CH>(r, red[i], inv_t);
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

template <int CH>
__global__ __launch_bounds__(64) void conf_final_kernel(ConfArgs a) {
  conf_final_row<CH>(a, blockIdx.x, threadIdx.x);
}

}  // namespace

size_t confidence_ws_bytes(int32_t batch, int32_t vocab) {
  const int nchunks = (vocab + kChunk - 1) / kChunk;
  return (size_t)batch * nchunks * kRec * sizeof(float);
}

namespace {
int choice_of(const ConfArgs& a) { return !a.token_out ? kNoChoice : (a.inv_temp > 0.f ? kSample : kGreedy); }
}  // namespace

hipError_t launch_confidence_partial(ConfArgs& a, hipStream_t s) {
  a.chunk = kChunk;
  a.nchunks = (a.vocab + kChunk - 1) / kChunk;
  a.choice = choice_of(a);
  const dim3 grid(a.nchunks, a.batch);
  if (a.choice == kNoChoice) hipLaunchKernelGGL(conf_partial_kernel<kNoChoice>, grid, dim3(kThreads), 0, s, a);
  else if (a.choice == kSample) hipLaunchKernelGGL(conf_partial_kernel<kSample>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(conf_partial_kernel<kGreedy>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_confidence(const ConfArgs& in, hipStream_t s) {
  ConfArgs a = in;
  const hipError_t e = launch_confidence_partial(a, s);
  if (e != hipSuccess) return e;
  if (a.choice == kNoChoice) hipLaunchKernelGGL(conf_final_kernel<kNoChoice>, dim3(a.batch), dim3(64), 0, s, a);
  else if (a.choice == kSample) hipLaunchKernelGGL(conf_final_kernel<kSample>, dim3(a.batch), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(conf_final_kernel<kGreedy>, dim3(a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace confk

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

#include "confidence_dev.h"

namespace confk {

using namespace confm;

namespace {


template <int CH>
__global__ __launch_bounds__(kConfThreads) void conf_partial_kernel(ConfArgs a) {
  conf_partial_block<CH>(a, blockIdx.x, blockIdx.y, threadIdx.x);
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

void confidence_prepare(ConfArgs& a) {
  a.chunk = kChunk;
  a.nchunks = (a.vocab + kChunk - 1) / kChunk;
  a.choice = choice_of(a);
}

hipError_t launch_confidence_partial(ConfArgs& a, hipStream_t s) {
  confidence_prepare(a);
  const dim3 grid(a.nchunks, a.batch);
  if (a.choice == kNoChoice) hipLaunchKernelGGL(conf_partial_kernel<kNoChoice>, grid, dim3(kConfThreads), 0, s, a);
  else if (a.choice == kSample) hipLaunchKernelGGL(conf_partial_kernel<kSample>, grid, dim3(kConfThreads), 0, s, a);
  else hipLaunchKernelGGL(conf_partial_kernel<kGreedy>, grid, dim3(kConfThreads), 0, s, a);
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

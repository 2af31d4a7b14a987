// EMA of the attention mass and composite rank score.
//
// Review "前置知识" (EMA prerequisite): a_i <- lambda a_i + (1 - lambda) Abar_i
// with Abar_i the current attention mass; review "核心方法": tokens are ranked
// by s_i = alpha a^_i + (1 - alpha) r^_i (normalised EMA mass and normalised
// recency). Abar_i is the mean over all query heads of the softmax weight of
// key i; a^ = a / max a and r^ = (pos - pos_min) / (pos_max - pos_min) over
// the cached tokens, which are stored in ascending position order.
//
// One workgroup per (layer, sequence); ~16 bytes per token, memory-bound.
#include "confk_internal.h"

namespace confk {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void ema_rank_kernel(EmaArgs a) {
  const CacheView& c = a.c;
  const int lb = blockIdx.x;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  const int cap = c.cap;
  const int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  const int n = meta[CONFK_META_N];
  float* ema = c.ema + (size_t)lbc * cap;
  int32_t* pos = c.pos + (size_t)lbc * cap;
  const float* mass = a.mass + (size_t)lb * c.hkv * cap;
  float* score = a.score + (size_t)lb * cap;
  const float inv_hq = 1.f / (float)c.hq;
  const float lam = a.lambda;
  const float oml = 1.f - lam;

  if (!meta_ok(n, meta[CONFK_META_N8], meta[CONFK_META_BASE8], meta[CONFK_META_BASE16], cap,
               c.cap16)) {  // no slot for the new token: flag, leave the state alone
    if (threadIdx.x == 0) atomicOr(c.status, (uint32_t)CONFK_STATUS_CAPACITY);
    return;
  }

  float amax = 0.f;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    float m = 0.f;
    for (int j = 0; j < c.hkv; ++j) m += mass[(size_t)j * cap + i];
    const float v = lam * ema[i] + oml * (m * inv_hq);
    ema[i] = v;
    amax = fmaxf(amax, v);
  }
  if (threadIdx.x == 0) {
    float m = 0.f;
    for (int j = 0; j < c.hkv; ++j) m += mass[(size_t)j * cap + n];
    ema[n] = oml * (m * inv_hq);
    pos[n] = a.t;
  }
  amax = wave_max(amax);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
  for (int q = 1; q < kThreads / 64; ++q) amax = fmaxf(amax, red[q]);
  if (n == 0) return;

  const int p0 = pos[0];
  const int p1 = pos[n - 1];
  const float inv_a = amax > 0.f ? 1.f / amax : 0.f;
  const float inv_r = p1 > p0 ? 1.f / (float)(p1 - p0) : 0.f;
  const float alpha = a.alpha;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const float ah = ema[i] * inv_a;
    const float rh = p1 > p0 ? (float)(pos[i] - p0) * inv_r : 1.f;
    score[i] = alpha * ah + (1.f - alpha) * rh;
  }
}

}  // namespace

hipError_t launch_ema_rank(const EmaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ema_rank_kernel, dim3(a.nl * a.c.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace confk

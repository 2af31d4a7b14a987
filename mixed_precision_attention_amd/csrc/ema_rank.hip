// EMA of the attention mass and composite rank score.
//
// Review "前置知识" (EMA prerequisite): a_i <- lambda a_i + (1 - lambda) Abar_i
// with Abar_i the current attention mass; review "核心方法": tokens are ranked
// by s_i = alpha a^_i + (1 - alpha) r^_i (normalised EMA mass and normalised
// recency). Abar_i is the mean over all query heads of the softmax weight of
// key i; a^ = a / max a and r^ = (pos - pos_min) / (pos_max - pos_min) over
// the cached tokens (position extremes reduced here: compaction may reorder
// the INT8 part).
//
// One workgroup per (layer, sequence); ~16 bytes per token, memory-bound.
// For up to kThreads * kPer tokens every thread issues all of its loads at
// once and keeps the updated EMA and positions in registers for the score
// pass, so the kernel costs one round trip to memory plus one barrier.
// Longer caches run the same code over blocks of kThreads * kPer tokens (a
// thread's loads of a block go out together), twice: the EMA pass, then,
// once the extremes are known, the score pass.
#include "confk_internal.h"

namespace confk {

namespace {

constexpr int kThreads = 512;
constexpr int kPer = 8;

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
  const float* mass = a.mass ? a.mass + (size_t)lb * c.hkv * cap : nullptr;
  float* score = a.score + (size_t)lb * cap;
  const float inv_hq = 1.f / (float)c.hq;
  const float lam = a.lambda;
  const float oml = 1.f - lam;
  const int H = mass_rows(meta, c.hkv);  // rows of partial mass sums

  if (!meta_ok(n, meta[CONFK_META_N8], meta[CONFK_META_BASE8], meta[CONFK_META_BASE16], cap,
               c.cap16)) {  // no slot for the new token: flag, leave the state alone
    if (threadIdx.x == 0) atomicOr(c.status, (uint32_t)CONFK_STATUS_CAPACITY);
    return;
  }
  if (a.mass == nullptr) {  // no attention mass this step: only the new token's slot
    if (threadIdx.x == 0) {
      ema[n] = 0.f;
      pos[n] = a.t;
    }
    return;
  }
  __shared__ float red[kThreads / 64];
  __shared__ int redp[2][kThreads / 64];

  const bool fast = n <= kThreads * kPer;
  float av[kPer];
  int pv[kPer];
  float amax = 0.f;
  int pmin = INT32_MAX, pmax = INT32_MIN;
  if (fast) {
    float ms[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = threadIdx.x + r * kThreads;
      ms[r] = 0.f;
      av[r] = 0.f;
      pv[r] = 0;
      if (i < n) {
        av[r] = ema[i];
        pv[r] = pos[i];
      }
    }
    // eight partial mass rows per round trip, summed in row order
    for (int j0 = 0; j0 < H; j0 += 8) {
      float t8[8][kPer];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
          const int i = threadIdx.x + r * kThreads;
          t8[q][r] = (j0 + q < H && i < n) ? mass[(size_t)(j0 + q) * cap + i] : 0.f;
        }
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int r = 0; r < kPer; ++r)
          if (j0 + q < H) ms[r] += t8[q][r];
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = threadIdx.x + r * kThreads;
      if (i < n) {
        av[r] = fmaf(lam, av[r], oml * (ms[r] * inv_hq));
        ema[i] = av[r];
        amax = fmaxf(amax, av[r]);
        pmin = min(pmin, pv[r]);
        pmax = max(pmax, pv[r]);
      }
    }
  } else {
    for (int base = 0; base < n; base += kThreads * kPer) {
      float ms[kPer], bv[kPer];
      int qv[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = base + threadIdx.x + r * kThreads;
        ms[r] = 0.f;
        bv[r] = i < n ? ema[i] : 0.f;
        qv[r] = i < n ? pos[i] : 0;
      }
      for (int j0 = 0; j0 < H; j0 += 8) {  // rows summed in row order, as above
        float t8[8][kPer];
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int r = 0; r < kPer; ++r) {
            const int i = base + threadIdx.x + r * kThreads;
            t8[q][r] = (j0 + q < H && i < n) ? mass[(size_t)(j0 + q) * cap + i] : 0.f;
          }
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int r = 0; r < kPer; ++r)
            if (j0 + q < H) ms[r] += t8[q][r];
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = base + threadIdx.x + r * kThreads;
        if (i < n) {
          const float v = fmaf(lam, bv[r], oml * (ms[r] * inv_hq));
          ema[i] = v;
          amax = fmaxf(amax, v);
          pmin = min(pmin, qv[r]);
          pmax = max(pmax, qv[r]);
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    float m = 0.f;
    for (int j = 0; j < H; ++j) m += mass[(size_t)j * cap + n];
    ema[n] = oml * (m * inv_hq);
  }
  amax = wave_max(amax);
  for (int o = 32; o > 0; o >>= 1) {
    pmin = min(pmin, __shfl_xor(pmin, o, 64));
    pmax = max(pmax, __shfl_xor(pmax, o, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = amax;
    redp[0][threadIdx.x >> 6] = pmin;
    redp[1][threadIdx.x >> 6] = pmax;
  }
  __syncthreads();  // also orders every read of pos[] before the write of pos[n]
  if (threadIdx.x == 0) pos[n] = a.t;
  amax = red[0];
  int p0 = redp[0][0], p1 = redp[1][0];
#pragma unroll
  for (int q = 1; q < kThreads / 64; ++q) {
    amax = fmaxf(amax, red[q]);
    p0 = min(p0, redp[0][q]);
    p1 = max(p1, redp[1][q]);
  }
  if (n == 0) return;

  const float inv_a = amax > 0.f ? 1.f / amax : 0.f;
  const float inv_r = p1 > p0 ? 1.f / (float)(p1 - p0) : 0.f;
  const float alpha = a.alpha;
  if (fast) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = threadIdx.x + r * kThreads;
      if (i < n) {
        const float rh = p1 > p0 ? (float)(pv[r] - p0) * inv_r : 1.f;
        score[i] = fmaf(alpha, av[r] * inv_a, (1.f - alpha) * rh);
      }
    }
  } else {  // each thread re-reads the EMA it wrote above
    for (int base = 0; base < n; base += kThreads * kPer) {
      float ev[kPer];
      int qv[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = base + threadIdx.x + r * kThreads;
        ev[r] = i < n ? ema[i] : 0.f;
        qv[r] = i < n ? pos[i] : 0;
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = base + threadIdx.x + r * kThreads;
        if (i < n) {
          const float rh = p1 > p0 ? (float)(qv[r] - p0) * inv_r : 1.f;
          score[i] = fmaf(alpha, ev[r] * inv_a, (1.f - alpha) * rh);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_ema_rank(const EmaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ema_rank_kernel, dim3(a.nl * a.c.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace confk

// FP16 -> INT8 storage of tokens that leave the FP16 window, and cache
// construction from a prefill.
//
// CONF-KV summary, "Methodik: CONF-KV" (gemischte Praezisionsspeicherung):
// the newest W tokens stay FP16 and older retained tokens are INT8 per head
// and per channel; review "方法步骤详情" (Algorithm 1 step 10) quantises the
// retained positions outside the newest W. Scales are symmetric absmax,
// scale = fp32(absmax) / 127 (IEEE quotient), set once when a sequence's INT8
// region is first populated and frozen afterwards; a code is
// clamp(rint(fp32(x) / scale), -127, 127) with the IEEE fp32 quotient
// (0 when the scale is 0), so codes are reproducible bit for bit.
#include "confk_internal.h"

namespace confk {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int8_t quant_code(float x, float s, int& sat) {
  if (!(s > 0.f)) return 0;
  const float r = rintf(__fdiv_rn(x, s));
  if (r > 127.f) {
    ++sat;
    return 127;
  }
  if (r < -127.f) {
    ++sat;
    return -127;
  }
  return (int8_t)r;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Codes of 8 consecutive channels (fp16 bits in h) under 8 scales.
__device__ __forceinline__ u32x2 quant8(u32x4 h, const float* s, int& sat) {
  u32x2 out = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t bits = (uint16_t)(h[e >> 1] >> (16 * (e & 1)));
    const int8_t q = quant_code(half_bits_to_float(bits), s[e], sat);
    out[e >> 2] |= (uint32_t)(uint8_t)q << (8 * (e & 3));
  }
  return out;
}

// One workgroup per (layer, sequence); thread e handles 8 consecutive
// channels of one (K|V, head) row. The oldest FP16 row and its scales are
// fetched together with its position, so the common case costs two round
// trips to memory.
__global__ __launch_bounds__(kThreads) void quantize_step_kernel(QuantArgs a) {
  const CacheView& c = a.c;
  const int lb = blockIdx.x;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  const int n = meta[CONFK_META_N];
  int n8 = meta[CONFK_META_N8];
  const int base8 = meta[CONFK_META_BASE8];
  int base16 = meta[CONFK_META_BASE16];
  int calib = meta[CONFK_META_CALIB];
  const int32_t* pos = c.pos + (size_t)lbc * c.cap;
  const int H = c.hkv, D = c.d;
  const int groups = 2 * H * D / 8;  // 8-channel groups over (K|V, head)
  // after the append the FP16 ring may hold cap16 tokens, so only check the
  // INT8 side and the ring bases here
  if (n < 0 || n8 < 0 || n8 > n || n > c.cap || n - n8 > c.cap16 || base8 < 0 || base8 >= c.cap ||
      base16 < 0 || base16 >= c.cap16) {
    if (threadIdx.x == 0) atomicOr(c.status, (uint32_t)CONFK_STATUS_CAPACITY);
    return;
  }
  const int limit = a.t - a.window;
  int sat = 0;

  while (n8 < n) {
    // the oldest FP16 token's position, the next one's, and (speculatively)
    // the row and its scales: one round trip in the common case
    const int p_first = pos[n8];
    const int p_next = n8 + 1 < n ? pos[n8 + 1] : INT32_MAX;
    u32x4 hv[4];
    f32x4 sv[4][2];
    int hq_[4];
    int cnt = 0;
    for (int e = threadIdx.x; e < groups; e += kThreads, ++cnt) {
      const int kv = e / (groups / 2);
      const int r = e - kv * (groups / 2);
      const int hh = (8 * r) / D;
      const size_t hrow = (size_t)lbc * H + hh;
      if (cnt < 4) {
        hv[cnt] = *reinterpret_cast<const u32x4*>((kv ? c.v16 : c.k16) + (hrow * c.cap16 + base16) * D +
                                                  (8 * r - hh * D));
        const float* sp = (kv ? c.vs : c.ks) + hrow * D + (8 * r - hh * D);
        sv[cnt][0] = *reinterpret_cast<const f32x4*>(sp);
        sv[cnt][1] = *reinterpret_cast<const f32x4*>(sp + 4);
        hq_[cnt] = e;
      }
    }
    if (p_first > limit) break;  // uniform: every thread reads the same word
    const int f = n - n8;
    const bool fresh_scales = !calib;
    if (!calib) {
      // scales over every cached token (all FP16 while uncalibrated)
      for (int e = threadIdx.x; e < 2 * H * D; e += kThreads) {
        const int kv = e / (H * D);
        const int hd = e - kv * H * D;
        const int hh = hd / D, ch = hd - hh * D;
        const uint16_t* ring = (kv ? c.v16 : c.k16) + ((size_t)lbc * H + hh) * c.cap16 * D;
        float amax = 0.f;
        for (int j = 0; j < f; ++j) {
          int slot = base16 + j;
          if (slot >= c.cap16) slot -= c.cap16;
          amax = fmaxf(amax, fabsf(half_bits_to_float(ring[(size_t)slot * D + ch])));
        }
        (kv ? c.vs : c.ks)[((size_t)lbc * H + hh) * D + ch] = __fdiv_rn(amax, 127.f);
      }
      __syncthreads();  // scales written by other threads are read below
      calib = 1;
    }
    int dst = base8 + n8;
    if (dst >= c.cap) dst -= c.cap;
    int q = 0;
    for (int e = threadIdx.x; e < groups; e += kThreads, ++q) {
      const int kv = e / (groups / 2);
      const int r = e - kv * (groups / 2);
      const int hh = (8 * r) / D;
      const int ch = 8 * r - hh * D;
      const size_t hrow = (size_t)lbc * H + hh;
      const bool pre = q < 4 && hq_[q] == e;
      float s8[8];
      if (pre && !fresh_scales) {
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          s8[z] = sv[q][0][z];
          s8[4 + z] = sv[q][1][z];
        }
      } else {
        const float* sp = (kv ? c.vs : c.ks) + hrow * D + ch;
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(sp);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(sp + 4);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          s8[z] = s0[z];
          s8[4 + z] = s1[z];
        }
      }
      const u32x4 h = pre ? hv[q]
                          : *reinterpret_cast<const u32x4*>((kv ? c.v16 : c.k16) +
                                                            (hrow * c.cap16 + base16) * D + ch);
      *reinterpret_cast<u32x2*>((kv ? c.v8 : c.k8) + (hrow * c.cap + dst) * D + ch) = quant8(h, s8, sat);
    }
    base16 = base16 + 1 == c.cap16 ? 0 : base16 + 1;
    ++n8;
    if (p_next > limit) break;  // the next FP16 token stays FP16 (uniform)
  }
  sat = wave_sum_i(sat);
  __shared__ int red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sat;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int q = 0; q < kThreads / 64; ++q) tot += red[q];
    meta[CONFK_META_N8] = n8;
    meta[CONFK_META_BASE16] = base16;
    meta[CONFK_META_CALIB] = calib;
    meta[CONFK_META_SAT] += tot;
  }
}

// One workgroup per (layer, sequence, kv head); threads over (K|V, channel).
__global__ __launch_bounds__(kThreads) void prefill_kernel(QuantArgs a) {
  const CacheView& c = a.c;
  const int u = blockIdx.x;
  const int H = c.hkv, D = c.d;
  const int hh = u % H;
  const int lb = u / H;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  const int L0 = a.n_src;
  const int W = a.window;
  const int nq = L0 > W ? L0 - W : 0;  // tokens stored INT8
  const size_t hrow = (size_t)lbc * H + hh;
  const size_t srow = (size_t)lb * H + hh;

  for (int e = threadIdx.x; e < 2 * D; e += kThreads) {
    const int kv = e / D, ch = e - kv * D;
    const uint16_t* src = (kv ? a.v_src : a.k_src) + srow * (size_t)L0 * D + ch;
    float s = 0.f;
    if (nq > 0) {
      float amax = 0.f;
      for (int i = 0; i < L0; ++i) amax = fmaxf(amax, fabsf(half_bits_to_float(src[(size_t)i * D])));
      s = __fdiv_rn(amax, 127.f);
    }
    (kv ? c.vs : c.ks)[hrow * D + ch] = s;
    int sat = 0;
    int8_t* q8 = (kv ? c.v8 : c.k8) + hrow * c.cap * D + ch;
    for (int i = 0; i < nq; ++i) q8[(size_t)i * D] = quant_code(half_bits_to_float(src[(size_t)i * D]), s, sat);
    uint16_t* r16 = (kv ? c.v16 : c.k16) + hrow * c.cap16 * D + ch;
    for (int i = nq; i < L0; ++i) r16[(size_t)(i - nq) * D] = src[(size_t)i * D];
  }
  if (hh == 0) {
    float* ema = c.ema + (size_t)lbc * c.cap;
    int32_t* pos = c.pos + (size_t)lbc * c.cap;
    for (int i = threadIdx.x; i < c.cap; i += kThreads) {
      ema[i] = 0.f;
      pos[i] = i < L0 ? i : 0;
    }
    if (threadIdx.x == 0) {
      int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
      meta[CONFK_META_N] = L0;
      meta[CONFK_META_N8] = nq;
      meta[CONFK_META_BASE8] = 0;
      meta[CONFK_META_BASE16] = 0;
      meta[CONFK_META_CALIB] = nq > 0 ? 1 : 0;
      meta[CONFK_META_SAT] = 0;
      meta[CONFK_META_EVICTED] = 0;
      meta[CONFK_META_MOVED] = 0;
      meta[CONFK_META_MOVED16] = 0;
      if (lb == 0) *c.status = 0u;
    }
  }
}

}  // namespace

hipError_t launch_quantize_step(const QuantArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(quantize_step_kernel, dim3(a.nl * a.c.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const QuantArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prefill_kernel, dim3(a.nl * a.c.B * a.c.hkv), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace confk

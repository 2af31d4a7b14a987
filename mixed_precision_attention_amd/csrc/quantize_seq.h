// The FP16 -> INT8 window step of one (layer, sequence), shared by the
// quantisation kernel and the fused EMA + compaction kernel.
//
// CONF-KV summary, "Methodik: CONF-KV" (gemischte Praezisionsspeicherung):
// the newest W tokens stay FP16, older retained tokens are INT8 per head and
// per channel; review "方法步骤详情" (Algorithm 1 step 10). Scales are symmetric
// absmax, scale = fp32(absmax) / 127 (IEEE quotient), set once when the
// sequence's INT8 region is first populated and frozen afterwards; a code is
// clamp(rint(fp32(x) / scale), -127, 127) with the IEEE fp32 quotient (0 when
// the scale is 0).
#pragma once
#include "confk_internal.h"

namespace confk {

typedef uint32_t qu32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t qu32x2 __attribute__((ext_vector_type(2)));
typedef float qf32x4 __attribute__((ext_vector_type(4)));

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

// Codes of 8 consecutive channels (fp16 bits in h) under 8 scales.
__device__ __forceinline__ qu32x2 quant8(qu32x4 h, const float* s, int& sat) {
  qu32x2 out = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t bits = (uint16_t)(h[e >> 1] >> (16 * (e & 1)));
    const int8_t q = quant_code(half_bits_to_float(bits), s[e], sat);
    out[e >> 2] |= (uint32_t)(uint8_t)q << (8 * (e & 3));
  }
  return out;
}

// Every FP16 token of the sequence whose position is at most t - window
// moves to INT8 (calibrating the scales first if the sequence has none),
// oldest first; thread e of the NT threads handles 8 consecutive channels of
// one (K|V, head) row. The oldest FP16 row and its scales are fetched
// together with its position, so the common case costs two round trips.
// All NT threads of the workgroup call it with the sequence's metadata
// (uniform, valid); thread 0 writes N8, BASE16, CALIB and adds to SAT.
template <int NT>
__device__ __forceinline__ void quantize_window(const CacheView& c, int lbc, int t, int window, int n, int n8,
                                                int base8, int base16, int calib) {
  int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  const int32_t* pos = c.pos + (size_t)lbc * c.cap;
  const int H = c.hkv, D = c.d;
  const int groups = 2 * H * D / 8;  // 8-channel groups over (K|V, head)
  const int limit = t - window;
  // groups a thread prefetches with the position (further ones load later)
  constexpr int SPEC = NT >= 512 ? 1 : 4;
  int sat = 0;

  while (n8 < n) {
    // the oldest FP16 token's position, the next one's, and (speculatively)
    // the row and its scales: one round trip in the common case
    const int p_first = pos[n8];
    const int p_next = n8 + 1 < n ? pos[n8 + 1] : INT32_MAX;
    qu32x4 hv[SPEC];
    qf32x4 sv[SPEC][2];
    int hq_[SPEC];
    int cnt = 0;
    for (int e = threadIdx.x; e < groups; e += NT, ++cnt) {
      const int kv = e / (groups / 2);
      const int r = e - kv * (groups / 2);
      const int hh = (8 * r) / D;
      const size_t hrow = (size_t)lbc * H + hh;
      if (cnt < SPEC) {
        hv[cnt] = *reinterpret_cast<const qu32x4*>((kv ? c.v16 : c.k16) + (hrow * c.cap16 + base16) * D +
                                                  (8 * r - hh * D));
        const float* sp = (kv ? c.vs : c.ks) + hrow * D + (8 * r - hh * D);
        sv[cnt][0] = *reinterpret_cast<const qf32x4*>(sp);
        sv[cnt][1] = *reinterpret_cast<const qf32x4*>(sp + 4);
        hq_[cnt] = e;
      }
    }
    if (p_first > limit) break;  // uniform: every thread reads the same word
    const int f = n - n8;
    const bool fresh_scales = !calib;
    if (!calib) {
      // scales over every cached token (all FP16 while uncalibrated)
      for (int e = threadIdx.x; e < 2 * H * D; e += NT) {
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
    for (int e = threadIdx.x; e < groups; e += NT, ++q) {
      const int kv = e / (groups / 2);
      const int r = e - kv * (groups / 2);
      const int hh = (8 * r) / D;
      const int ch = 8 * r - hh * D;
      const size_t hrow = (size_t)lbc * H + hh;
      const bool pre = q < SPEC && hq_[q] == e;
      float s8[8];
      if (pre && !fresh_scales) {
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          s8[z] = sv[q][0][z];
          s8[4 + z] = sv[q][1][z];
        }
      } else {
        const float* sp = (kv ? c.vs : c.ks) + hrow * D + ch;
        const qf32x4 s0 = *reinterpret_cast<const qf32x4*>(sp);
        const qf32x4 s1 = *reinterpret_cast<const qf32x4*>(sp + 4);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          s8[z] = s0[z];
          s8[4 + z] = s1[z];
        }
      }
      const qu32x4 h = pre ? hv[q]
                          : *reinterpret_cast<const qu32x4*>((kv ? c.v16 : c.k16) +
                                                            (hrow * c.cap16 + base16) * D + ch);
      *reinterpret_cast<qu32x2*>((kv ? c.v8 : c.k8) + (hrow * c.cap + dst) * D + ch) = quant8(h, s8, sat);
    }
    base16 = base16 + 1 == c.cap16 ? 0 : base16 + 1;
    ++n8;
    if (p_next > limit) break;  // the next FP16 token stays FP16 (uniform)
  }
  sat = wave_sum_i(sat);
  __shared__ int red[NT / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sat;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int q = 0; q < NT / 64; ++q) tot += red[q];
    meta[CONFK_META_N8] = n8;
    meta[CONFK_META_BASE16] = base16;
    meta[CONFK_META_CALIB] = calib;
    meta[CONFK_META_SAT] += tot;
  }
}

}  // namespace confk

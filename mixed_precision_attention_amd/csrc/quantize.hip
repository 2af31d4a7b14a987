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
#include "quantize_seq.h"

namespace confk {

namespace {

constexpr int kThreads = 256;

// One workgroup per (layer, sequence).
__global__ __launch_bounds__(kThreads) void quantize_step_kernel(QuantArgs a) {
  const CacheView& c = a.c;
  const int lb = blockIdx.x;
  const int l = lb / c.B;
  const int b = lb - l * c.B;
  const int lbc = (a.layer0 + l) * c.B + b;
  const int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  const int n = meta[CONFK_META_N];
  const int n8 = meta[CONFK_META_N8];
  const int base8 = meta[CONFK_META_BASE8];
  const int base16 = meta[CONFK_META_BASE16];
  const int calib = meta[CONFK_META_CALIB];
  // after the append the FP16 ring may hold cap16 tokens, so only check the
  // INT8 side and the ring bases here
  if (n < 0 || n8 < 0 || n8 > n || n > c.cap || n - n8 > c.cap16 || base8 < 0 || base8 >= c.cap ||
      base16 < 0 || base16 >= c.cap16) {
    if (threadIdx.x == 0) atomicOr(c.status, (uint32_t)CONFK_STATUS_CAPACITY);
    return;
  }
  quantize_window<kThreads>(c, lbc, a.t, a.window, n, n8, base8, base16, calib);
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

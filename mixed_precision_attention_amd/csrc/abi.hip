// Host side of the C ABI: argument validation, launch planning, error codes.
// Every entry point validates all arguments before enqueuing anything.
#include <string.h>

#include "confk_internal.h"

using namespace confk;

namespace {

bool cache_ok(const confk_cache* c) {
  if (!c) return false;
  if (c->layers < 1 || c->batch < 1 || c->hkv < 1 || c->hq < c->hkv || c->hq % c->hkv) return false;
  if (c->d < 16 || c->cap < 2 || c->cap16 < 2) return false;
  if (!c->k8 || !c->v8 || !c->k16 || !c->v16 || !c->kscale || !c->vscale || !c->ema ||
      !c->pos || !c->meta || !c->status)
    return false;
  return true;
}

bool layers_ok(const confk_cache* c, int32_t layer0, int32_t nlayers) {
  return layer0 >= 0 && nlayers >= 1 && layer0 + nlayers <= c->layers;
}

bool policy_ok(const confk_policy* p) {
  if (!p) return false;
  if (p->n_high < 1 || p->n_low < 1 || p->protect < 0 || p->window < 1) return false;
  if (!(p->lambda >= 0.f && p->lambda <= 1.f) || !(p->alpha >= 0.f && p->alpha <= 1.f)) return false;
  if (p->block != 0 && p->block < 16) return false;
  if (p->order != CONFK_ORDER_FILL && p->order != CONFK_ORDER_STABLE) return false;
  return true;
}

int launch_status(hipError_t e) { return e == hipSuccess ? CONFK_OK : CONFK_ERR_LAUNCH; }

}  // namespace

extern "C" {

int confk_version(void) { return 107; }

const char* confk_strerror(int code) {
  switch (code) {
    case CONFK_OK: return "ok";
    case CONFK_ERR_INVALID_ARG: return "invalid argument";
    case CONFK_ERR_BUDGET: return "budget below the protected window or above capacity";
    case CONFK_ERR_WORKSPACE: return "workspace missing or too small";
    case CONFK_ERR_UNSUPPORTED: return "unsupported head dimension or group size";
    case CONFK_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

namespace {
// Byte offset of the split exchange area in the attention workspace: after
// the score spill area, 256-byte aligned.
size_t xchg_offset(size_t spill) { return (spill + 255) / 256 * 256; }

}  // namespace

size_t confk_workspace_size(int32_t which, const confk_cache* cache, int32_t nlayers, int32_t batch,
                            int32_t vocab) {
  if (which == CONFK_WS_CONFIDENCE) {
    if (batch < 1 || vocab < 1) return 0;
    return confidence_ws_bytes(batch, vocab);
  }
  if (which == CONFK_WS_COMPACT) {
    if (!cache || nlayers < 1 || cache->cap < 2) return 0;
    return compact_ws_bytes(nlayers, cache->batch, cache->cap);
  }
  if (which == CONFK_WS_ATTENTION || which == CONFK_WS_ATTENTION_NOSPLIT) {
    if (!cache || nlayers < 1 || cache->hkv < 1 || cache->hq % cache->hkv) return 0;
    const int g = cache->hq / cache->hkv;
    int stride = 0;
    attention_plan_n_lds(cache->d, g, cache->cap, &stride);
    const int64_t units = (int64_t)nlayers * cache->batch * cache->hkv;
    const size_t spill = (size_t)units * g * (size_t)stride * sizeof(float);
    const size_t xchg = which == CONFK_WS_ATTENTION ? attention_xchg_bytes(units, g, cache->d) : 0;
    return xchg ? xchg_offset(spill) + xchg : spill;
  }
  return 0;
}

namespace {
// Validation and argument set-up of the confidence call (shared by the fused
// confidence + attention call).
int conf_args(const float* logits, int64_t ld, int32_t batch, int32_t vocab, const confk_policy* pol,
              const int32_t* layer_n_high, const int32_t* layer_n_low, int32_t nbl, float* c_out,
              int32_t* budget_out, uint32_t* status, const float* uniform, float temperature,
              int32_t* token_out, void* ws, size_t ws_bytes, ConfArgs* out) {
  if (!logits || !c_out || !budget_out || !pol) return CONFK_ERR_INVALID_ARG;
  if (!(temperature >= 0.f) || temperature == INFINITY) return CONFK_ERR_INVALID_ARG;
  if (token_out && temperature > 0.f && !uniform) return CONFK_ERR_INVALID_ARG;
  if (batch < 1 || vocab < 2 || ld < vocab || nbl < 1) return CONFK_ERR_INVALID_ARG;
  if ((layer_n_high == nullptr) != (layer_n_low == nullptr)) return CONFK_ERR_INVALID_ARG;
  if (!layer_n_high && nbl != 1) return CONFK_ERR_INVALID_ARG;
  if (pol->n_high < 1 || pol->n_low < 1) return CONFK_ERR_INVALID_ARG;
  const size_t need = confidence_ws_bytes(batch, vocab);
  if (!ws || ws_bytes < need) return CONFK_ERR_WORKSPACE;
  ConfArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.batch = batch;
  a.vocab = vocab;
  a.nbl = nbl;
  a.vec4 = (ld % 4 == 0) && (((uintptr_t)logits & 15) == 0);
  a.tau = pol->tau;
  a.w_h = pol->w_h;
  a.w_m = pol->w_m;
  a.w_p = pol->w_p;
  a.n_high = pol->n_high;
  a.n_low = pol->n_low;
  a.layer_n_high = layer_n_high;
  a.layer_n_low = layer_n_low;
  a.partial = (float*)ws;
  a.vecrec = ((uintptr_t)ws & 31) == 0;
  a.c_out = c_out;
  a.budget_out = budget_out;
  a.token_out = token_out;
  a.uniform = uniform;
  a.inv_temp = (token_out && temperature > 0.f) ? 1.f / temperature : 0.f;
  a.status = status;
  *out = a;
  return CONFK_OK;
}

// Validation and argument set-up of the attention call; *lds_bytes is the
// launch's shared memory for the default plan.
int attn_args(const confk_cache* cache, int32_t layer0, int32_t nlayers, const uint16_t* q,
              const uint16_t* k_new, const uint16_t* v_new, uint16_t* out, float* mass, void* ws,
              size_t ws_bytes, AttnArgs* res, int* lds_bytes) {
  if (!cache_ok(cache) || !layers_ok(cache, layer0, nlayers)) return CONFK_ERR_INVALID_ARG;
  if (!q || !k_new || !v_new || !out) return CONFK_ERR_INVALID_ARG;
  const int g = cache->hq / cache->hkv;
  if ((cache->d != 64 && cache->d != 128) || g > 16) return CONFK_ERR_UNSUPPORTED;
  int stride = 0;
  const int n_lds = mass ? attention_plan_n_lds(cache->d, g, cache->cap, &stride) : 0;
  const size_t need = (size_t)nlayers * cache->batch * cache->hkv * g * (size_t)stride * sizeof(float);
  if (need && (!ws || ws_bytes < need)) return CONFK_ERR_WORKSPACE;
  AttnArgs a{};
  a.c = view_of(cache);
  a.layer0 = layer0;
  a.nl = nlayers;
  a.g = g;
  a.n_lds = n_lds;
  a.spill_stride = stride;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  a.mass = mass;
  a.spill = need ? (float*)ws : nullptr;
  // the split exchange area, when the workspace holds it (otherwise the
  // launch does not split keys)
  const size_t xchg = mass ? attention_xchg_bytes((int64_t)nlayers * cache->batch * cache->hkv, g, cache->d) : 0;
  if (xchg && ws && ((uintptr_t)ws & 7) == 0 && ws_bytes >= xchg_offset(need) + xchg)
    a.xchg = reinterpret_cast<uint64_t*>(static_cast<unsigned char*>(ws) + xchg_offset(need));
  *res = a;
  *lds_bytes = attention_lds_bytes(cache->d, g, n_lds);
  return CONFK_OK;
}
}  // namespace

int confk_confidence(const float* logits, int64_t ld, int32_t batch, int32_t vocab,
                     const confk_policy* pol, const int32_t* layer_n_high,
                     const int32_t* layer_n_low, int32_t nbl, float* c_out, int32_t* budget_out,
                     uint32_t* status, const float* uniform, float temperature, int32_t* token_out,
                     void* ws, size_t ws_bytes, void* stream) {
  ConfArgs a;
  const int rc = conf_args(logits, ld, batch, vocab, pol, layer_n_high, layer_n_low, nbl, c_out, budget_out,
                           status, uniform, temperature, token_out, ws, ws_bytes, &a);
  if (rc != CONFK_OK) return rc;
  return launch_status(launch_confidence(a, (hipStream_t)stream));
}

int confk_attn_decode(const confk_cache* cache, int32_t layer0, int32_t nlayers, const uint16_t* q,
                      const uint16_t* k_new, const uint16_t* v_new, uint16_t* out, float* mass,
                      void* ws, size_t ws_bytes, void* stream) {
  AttnArgs a;
  int lds = 0;
  const int rc = attn_args(cache, layer0, nlayers, q, k_new, v_new, out, mass, ws, ws_bytes, &a, &lds);
  if (rc != CONFK_OK) return rc;
  return launch_status(launch_attention(a, lds, (hipStream_t)stream));
}

int confk_confidence_attn_decode(const float* logits, int64_t ld, int32_t batch, int32_t vocab,
                                 const confk_policy* pol, const int32_t* layer_n_high,
                                 const int32_t* layer_n_low, int32_t nbl, float* c_out,
                                 int32_t* budget_out, uint32_t* status, const float* uniform,
                                 float temperature, int32_t* token_out, void* conf_ws,
                                 size_t conf_ws_bytes, const confk_cache* cache, int32_t layer0,
                                 int32_t nlayers, const uint16_t* q, const uint16_t* k_new,
                                 const uint16_t* v_new, uint16_t* out, float* mass, void* attn_ws,
                                 size_t attn_ws_bytes, void* stream) {
  ConfArgs ca;
  int rc = conf_args(logits, ld, batch, vocab, pol, layer_n_high, layer_n_low, nbl, c_out, budget_out, status,
                     uniform, temperature, token_out, conf_ws, conf_ws_bytes, &ca);
  if (rc != CONFK_OK) return rc;
  AttnArgs a;
  int lds = 0;
  rc = attn_args(cache, layer0, nlayers, q, k_new, v_new, out, mass, attn_ws, attn_ws_bytes, &a, &lds);
  if (rc != CONFK_OK) return rc;
  if (token_out && temperature > 0.f) {  // sampling: the confidence call's own two kernels
    const hipError_t e = launch_confidence(ca, (hipStream_t)stream);
    if (e != hipSuccess) return launch_status(e);
    return launch_status(launch_attention(a, lds, (hipStream_t)stream));
  }
  const hipError_t e = launch_confidence_partial(ca, (hipStream_t)stream);
  if (e != hipSuccess) return launch_status(e);
  a.conf = ca;  // with the chunking the partial pass used
  a.conf_mode = kConfMerge;
  return launch_status(launch_attention(a, lds, (hipStream_t)stream));
}

int confk_ema_rank(const confk_cache* cache, int32_t layer0, int32_t nlayers, const float* mass,
                   const confk_policy* pol, int32_t t, float* score, void* stream) {
  if (!cache_ok(cache) || !layers_ok(cache, layer0, nlayers)) return CONFK_ERR_INVALID_ARG;
  if (!score || !policy_ok(pol) || t < 0) return CONFK_ERR_INVALID_ARG;
  EmaArgs a{};
  a.c = view_of(cache);
  a.layer0 = layer0;
  a.nl = nlayers;
  a.t = t;
  a.lambda = pol->lambda;
  a.alpha = pol->alpha;
  a.mass = mass;
  a.score = score;
  return launch_status(launch_ema_rank(a, (hipStream_t)stream));
}

namespace {
// Validation and argument set-up shared by the split and the fused entry.
int compact_args(const confk_cache* cache, int32_t layer0, int32_t nlayers, const int32_t* budget,
                 int32_t budget_layer_stride, const float* score, const confk_policy* pol,
                 const uint16_t* k_new, const uint16_t* v_new, int32_t* evicted_out, void* ws,
                 size_t ws_bytes, confk::CompactArgs& a) {
  if (!cache_ok(cache) || !layers_ok(cache, layer0, nlayers)) return CONFK_ERR_INVALID_ARG;
  if (!budget || !score || !k_new || !v_new || !policy_ok(pol)) return CONFK_ERR_INVALID_ARG;
  if (budget_layer_stride != 0 && budget_layer_stride != cache->batch) return CONFK_ERR_INVALID_ARG;
  if (cache->d % 16) return CONFK_ERR_UNSUPPORTED;
  if (pol->protect > pol->n_high || pol->protect > pol->n_low) return CONFK_ERR_BUDGET;
  if (pol->n_low + 1 > cache->cap - 1 || pol->n_high + 1 > cache->cap - 1) return CONFK_ERR_BUDGET;
  if (pol->window + 1 > cache->cap16) return CONFK_ERR_BUDGET;
  // token eviction reorders the INT8 part: the newest P tokens must be FP16
  if (pol->block == 0 && pol->order == CONFK_ORDER_FILL && pol->protect > pol->window) return CONFK_ERR_BUDGET;
  if (pol->block > 0 && cache->cap / pol->block > kMaxEvictBlocks) return CONFK_ERR_UNSUPPORTED;
  // stable packing moves rows in a kernel that holds a head's scales on chip
  const bool packs = pol->block > 0 || pol->order == CONFK_ORDER_STABLE;
  if (packs && (cache->d > kMaxMoveHeadDim || nlayers * cache->batch > kMaxMovePairs)) return CONFK_ERR_UNSUPPORTED;
  const size_t need = compact_ws_bytes(nlayers, cache->batch, cache->cap);
  if (!ws || ws_bytes < need) return CONFK_ERR_WORKSPACE;
  a = CompactArgs{};
  a.plan = (int32_t*)ws;
  a.jobs = (int32_t*)((char*)ws + compact_jobs_offset(nlayers, cache->batch, cache->cap));
  a.stage = (int32_t*)((char*)ws + compact_plan_bytes(nlayers, cache->batch, cache->cap));
  a.c = view_of(cache);
  a.layer0 = layer0;
  a.nl = nlayers;
  a.budget_stride = budget_layer_stride;
  a.protect = pol->protect;
  a.block = pol->block;
  a.stable = pol->block == 0 && pol->order == CONFK_ORDER_STABLE;
  a.budget = budget;
  a.score = score;
  a.k_new = k_new;
  a.v_new = v_new;
  a.evicted_out = evicted_out;
  return CONFK_OK;
}
}  // namespace

int confk_compact(const confk_cache* cache, int32_t layer0, int32_t nlayers, const int32_t* budget,
                  int32_t budget_layer_stride, const float* score, const confk_policy* pol,
                  const uint16_t* k_new, const uint16_t* v_new, int32_t* evicted_out, void* ws,
                  size_t ws_bytes, void* stream) {
  CompactArgs a;
  const int e = compact_args(cache, layer0, nlayers, budget, budget_layer_stride, score, pol, k_new, v_new,
                             evicted_out, ws, ws_bytes, a);
  if (e != CONFK_OK) return e;
  return launch_status(launch_compact(a, (hipStream_t)stream));
}

int confk_ema_compact(const confk_cache* cache, int32_t layer0, int32_t nlayers, const float* mass,
                      const confk_policy* pol, int32_t t, float* score, const int32_t* budget,
                      int32_t budget_layer_stride, const uint16_t* k_new, const uint16_t* v_new,
                      int32_t* evicted_out, int32_t flags, void* ws, size_t ws_bytes, void* stream) {
  if (!mass || t < 0 || (flags & ~CONFK_FUSE_QUANTIZE) != 0) return CONFK_ERR_INVALID_ARG;
  CompactArgs a;
  const int e = compact_args(cache, layer0, nlayers, budget, budget_layer_stride, score, pol, k_new, v_new,
                             evicted_out, ws, ws_bytes, a);
  if (e != CONFK_OK) return e;
  a.fuse = 1;
  a.t = t;
  a.lambda = pol->lambda;
  a.alpha = pol->alpha;
  a.mass = mass;
  a.score_out = score;
  a.quantize = (flags & CONFK_FUSE_QUANTIZE) ? 1 : 0;
  a.window = pol->window;
  return launch_status(launch_compact(a, (hipStream_t)stream));
}

int confk_decode_step(const float* logits, int64_t ld, int32_t vocab, const confk_policy* pol,
                      const int32_t* layer_n_high, const int32_t* layer_n_low, int32_t nbl, float* c_out,
                      int32_t* budget_out, const float* uniform, float temperature, int32_t* token_out,
                      const confk_cache* cache, int32_t layer0, int32_t nlayers, int32_t t, const uint16_t* q,
                      const uint16_t* k_new, const uint16_t* v_new, uint16_t* out, float* mass, float* score,
                      int32_t* evicted_out, int32_t flags, void* conf_ws, size_t conf_ws_bytes, void* attn_ws,
                      size_t attn_ws_bytes, void* compact_ws, size_t compact_ws_bytes, void* stream) {
  if (!cache_ok(cache)) return CONFK_ERR_INVALID_ARG;
  if (!mass || t < 0 || (flags & ~CONFK_FUSE_QUANTIZE) != 0) return CONFK_ERR_INVALID_ARG;
  if (nbl != 1 && nbl != nlayers) return CONFK_ERR_INVALID_ARG;
  ConfArgs ca;
  int rc = conf_args(logits, ld, cache->batch, vocab, pol, layer_n_high, layer_n_low, nbl, c_out, budget_out,
                     cache->status, uniform, temperature, token_out, conf_ws, conf_ws_bytes, &ca);
  if (rc != CONFK_OK) return rc;
  AttnArgs aa;
  int lds = 0;
  rc = attn_args(cache, layer0, nlayers, q, k_new, v_new, out, mass, attn_ws, attn_ws_bytes, &aa, &lds);
  if (rc != CONFK_OK) return rc;
  CompactArgs cp;
  rc = compact_args(cache, layer0, nlayers, budget_out, nbl > 1 ? cache->batch : 0, score, pol, k_new, v_new,
                    evicted_out, compact_ws, compact_ws_bytes, cp);
  if (rc != CONFK_OK) return rc;
  cp.fuse = 1;
  cp.t = t;
  cp.lambda = pol->lambda;
  cp.alpha = pol->alpha;
  cp.mass = mass;
  cp.score_out = score;
  cp.quantize = (flags & CONFK_FUSE_QUANTIZE) ? 1 : 0;
  cp.window = pol->window;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (token_out && temperature > 0.f) {  // sampling: the confidence call's own two kernels first
    e = launch_confidence(ca, s);
    if (e == hipSuccess) e = launch_attention(aa, lds, s);
  } else {
    confidence_prepare(ca);
    aa.conf = ca;
    aa.conf_mode = kConfPass;  // the pass in the attention launch
    e = launch_attention(aa, lds, s);
    cp.conf = ca;
    cp.conf_merge = 1;  // the merge and the budgets in the plan kernel
  }
  if (e != hipSuccess) return launch_status(e);
  return launch_status(launch_compact(cp, s));
}

int confk_quantize(const confk_cache* cache, int32_t layer0, int32_t nlayers, int32_t t,
                   const confk_policy* pol, int32_t mode, const uint16_t* k_src,
                   const uint16_t* v_src, int32_t n_src, void* stream) {
  if (!cache_ok(cache) || !layers_ok(cache, layer0, nlayers)) return CONFK_ERR_INVALID_ARG;
  if (!policy_ok(pol)) return CONFK_ERR_INVALID_ARG;
  if (pol->window + 1 > cache->cap16) return CONFK_ERR_BUDGET;
  QuantArgs a{};
  a.c = view_of(cache);
  a.layer0 = layer0;
  a.nl = nlayers;
  a.t = t;
  a.window = pol->window;
  if (mode == CONFK_QUANT_STEP) {
    return launch_status(launch_quantize_step(a, (hipStream_t)stream));
  }
  if (mode == CONFK_QUANT_PREFILL) {
    if (n_src < 0) return CONFK_ERR_INVALID_ARG;
    if (n_src > 0 && (!k_src || !v_src)) return CONFK_ERR_INVALID_ARG;
    if (n_src > cache->cap - 1) return CONFK_ERR_BUDGET;
    a.n_src = n_src;
    a.k_src = k_src;
    a.v_src = v_src;
    return launch_status(launch_prefill(a, (hipStream_t)stream));
  }
  return CONFK_ERR_INVALID_ARG;
}

}  // extern "C"

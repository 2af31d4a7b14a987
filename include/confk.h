/*
 * confk.h -- C ABI of libconfk, the CONF-KV decode-step library for AMD
 * MI355X (gfx950).
 *
 * CONF-KV ("CONF-KV: Confidence-Aware KV Cache Eviction with Mixed-Precision
 * Storage for Long-Horizon LLM"; gist.science technical summary, section
 * "Methodik: CONF-KV"; paper.rainbus.top review, sections "核心方法" and
 * "方法步骤详情" (Algorithm 1)) turns each decode step's logits into a
 * confidence score, picks a tight or loose KV budget from it, attends over a
 * densely packed cache whose newest W tokens are FP16 and older tokens INT8
 * per (head, channel), tracks an EMA of each token's attention mass, and
 * evicts the lowest-ranked tokens outside a protected recent window.
 *
 * One decode step at position t is, in this order (each call enqueues work
 * on `stream` and returns without waiting):
 *   confk_confidence   logits -> c[B], budget[.][B]            (steps 3-4)
 *   confk_attn_decode  q, cache, new k/v -> o, per-key mass    (steps 1-2)
 *   confk_ema_rank     mass -> EMA update, new-token metadata, rank scores
 *   confk_compact      scores, budget -> evict, compact, append new token
 *   confk_quantize     FP16 token that left the window -> INT8   (step 10)
 * confk_ema_compact runs confk_ema_rank and confk_compact (and, with
 * CONFK_FUSE_QUANTIZE, confk_quantize's window step) as one launch with the
 * same results; confk_confidence_attn_decode runs confk_confidence and
 * confk_attn_decode in two launches instead of three, and confk_decode_step
 * runs the whole step (all five) in three. The streaming-read probe that measurements compare the
 * attention kernel with is a separate library (confk_probe.h).
 *
 * Conventions for every entry point:
 *  - Pointers named in a confk_cache and every tensor argument are DEVICE
 *    pointers owned by the caller, which keeps them alive until the stream
 *    work finishes. confk_policy and confk_cache structs are HOST memory,
 *    read during the call only. The library allocates nothing and keeps no
 *    state between calls.
 *  - fp16 tensors are passed as uint16_t holding IEEE binary16 bits.
 *  - `stream` is a hipStream_t (NULL = default stream).
 *  - Return value: CONFK_OK (0) or a negative CONFK_ERR_* code. Arguments are
 *    validated before anything is launched; on an error nothing is enqueued.
 *    Conditions only the device can see set bits in cache->status (sticky,
 *    cleared by the caller), readable after the stream synchronises.
 *  - Calls on one cache must be stream-ordered; concurrent calls on the same
 *    cache race.
 */
#ifndef CONFK_H
#define CONFK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------- */
#define CONFK_OK 0
#define CONFK_ERR_INVALID_ARG -1 /* null pointer, bad dimension, bad mode    */
#define CONFK_ERR_BUDGET -2      /* N < P, budget or prefill above capacity  */
#define CONFK_ERR_WORKSPACE -3   /* workspace missing or too small           */
#define CONFK_ERR_UNSUPPORTED -4 /* head dim / group size not built          */
#define CONFK_ERR_LAUNCH -5      /* the HIP runtime rejected a launch        */

/* ---- device status bits (cache->status[0] / status argument) ---------- */
#define CONFK_STATUS_NONFINITE_LOGITS 1u /* NaN, +inf, all -inf logits      */
#define CONFK_STATUS_CAPACITY 2u         /* a (layer, seq) ran out of slots */
#define CONFK_STATUS_SPLIT_WAIT 4u       /* a split-key attention workgroup gave up
                                            waiting for another split's values */

/* ---- per-(layer, sequence) header words (cache->meta) ------------------ */
#define CONFK_META_N 0       /* tokens retained                                 */
#define CONFK_META_N8 1      /* of which INT8 (the oldest ones)                 */
#define CONFK_META_BASE8 2   /* INT8 ring slot of the oldest token              */
#define CONFK_META_BASE16 3  /* FP16 ring slot of the oldest FP16 token         */
#define CONFK_META_CALIB 4   /* 1 once the INT8 scales are set                  */
#define CONFK_META_SAT 5     /* INT8 codes clamped at +-127 so far              */
#define CONFK_META_EVICTED 6 /* tokens evicted by the last confk_compact        */
#define CONFK_META_MOVED 7   /* INT8 tokens moved by the last confk_compact     */
#define CONFK_META_MOVED16 8 /* FP16 tokens moved by the last confk_compact     */
#define CONFK_META_MASSROWS 9 /* mass rows written by the last confk_attn_decode
                                 (0, as in a fresh cache, reads as hkv)          */
#define CONFK_META_WORDS 16

/* ---- confk_quantize modes ---------------------------------------------- */
#define CONFK_QUANT_STEP 0    /* move the token that left the FP16 window     */
#define CONFK_QUANT_PREFILL 1 /* build the cache from L0 prefill tokens       */

/* ---- confk_workspace_size selectors ------------------------------------ */
#define CONFK_WS_CONFIDENCE 0
#define CONFK_WS_ATTENTION 1
#define CONFK_WS_COMPACT 2
#define CONFK_WS_ATTENTION_NOSPLIT 3 /* the score spill part alone */

/*
 * Policy (hyper-parameters of the review's "复现评估" section and the
 * summary's "Methodik" section): tau is the confidence threshold, n_high the
 * tight budget taken when c >= tau, n_low the loose budget, protect (P) the
 * newest tokens never evicted, window (W) the FP16 window, alpha the rank
 * mix, lambda the EMA decay, (w_h, w_m, w_p) the confidence weights.
 * block: 0 for the method's token eviction; B >= 16 evicts whole blocks of B
 * consecutive cached tokens instead (the coarse, block-level eviction the
 * review's "局限与改进" and "独立分析的弱点" sections name as the way to fit
 * paged serving layouts; block score and grouping are this library's
 * reading, the pages fix neither): the candidates are
 * grouped into blocks of B from the oldest (a trailing partial block is kept),
 * a block ranks by the largest score of its tokens, and the ceil((n-N)/B)
 * lowest-ranked blocks leave (the older block first among equals).
 * order: the order of the survivors inside the compacted cache under token
 * eviction. CONFK_ORDER_STABLE (0, the default): the survivors keep position
 * order in both parts, a stable gather (the review's Algorithm 1 compacts the
 * survivors in place; the summary's "Implementierung" asks for a dense
 * layout without indirection tables), each ring packed toward whichever end
 * moves fewer rows. CONFK_ORDER_FILL (1), an option: the surviving INT8
 * tokens at or beyond the new INT8 length fill the INT8 holes below it, in
 * slot order (fewer row moves; the INT8 part then leaves position order;
 * needs protect <= window). Block eviction always packs stably and ignores
 * this field.
 */
#define CONFK_ORDER_STABLE 0
#define CONFK_ORDER_FILL 1
typedef struct confk_policy {
  float tau, alpha, lambda, w_h, w_m, w_p;
  int32_t n_high, n_low, protect, window, block, order;
} confk_policy;

/*
 * Cache of L layers x B sequences with Hkv kv heads of dimension d.
 * Per (layer l, sequence b) the first meta[N8] logical tokens are INT8 (the
 * oldest; in position order until token eviction fills holes, see
 * confk_compact) and the rest FP16, in position order. Logical token i < n8 lives in
 * INT8 ring slot (base8 + i) % cap, logical token i >= n8 in FP16 ring slot
 * (base16 + i - n8) % cap16. ema and pos are dense in logical order.
 * Layouts (row-major):
 *   k8, v8       int8   [L][B][Hkv][cap][d]      INT8 codes
 *   k16, v16     fp16   [L][B][Hkv][cap16][d]    FP16 window
 *   kscale,vscale fp32  [L][B][Hkv][d]           per-(head, channel) scales
 *   ema          fp32   [L][B][cap]              EMA attention mass
 *   pos          int32  [L][B][cap]              token positions
 *   meta         int32  [L][B][CONFK_META_WORDS]
 *   status       uint32 [1]
 * cap must be at least max(L0, N_low + 1) + 1 (the largest cache before a
 * step plus the new token); cap16 at least window + 1.
 */
typedef struct confk_cache {
  int32_t layers, batch, hq, hkv, d, cap, cap16;
  int8_t *k8, *v8;
  uint16_t *k16, *v16;
  float *kscale, *vscale;
  float *ema;
  int32_t *pos;
  int32_t *meta;
  uint32_t *status;
} confk_cache;

/*
 * confk_confidence -- confidence score and budget per sequence.
 * Summary "Methodik: CONF-KV" (Konfidenzschaetzung, adaptive Budgetauswahl);
 * review "核心方法": c = w_h(1 - H/ln V) + w_m*sigmoid(ln p1 - ln p2) + w_p*p1
 * with p = softmax(logits[b]); budget = n_high if c >= tau else n_low.
 *   logits        fp32 [batch][ld] device, first `vocab` entries used
 *   layer_n_high, layer_n_low  int32 [nbl] device, or both NULL with nbl = 1
 *                 to use pol->n_high / pol->n_low (per-layer budgets give the
 *                 pyramid variant)
 *   c_out         fp32 [batch]
 *   budget_out    int32 [nbl][batch]
 *   status        uint32 [1] device or NULL; NaN / +inf / all -inf logits
 *                 set CONFK_STATUS_NONFINITE_LOGITS, give c = NaN and the
 *                 loose budget
 *   token_out     int32 [batch] device or NULL: the next token x_{t+1}
 *                 (review Algorithm 1, step 13), chosen in the same pass.
 *                 temperature = 0: greedy, the smallest index among the
 *                 largest logits. temperature > 0: the smallest index i whose
 *                 cumulative weight sum_{j<=i} e^(z_j/temperature) (index
 *                 order) exceeds uniform[b] times the total, i.e. sampling
 *                 from softmax(z / temperature) by inversion. -1 for flagged
 *                 rows.
 *   uniform       fp32 [batch] device, each in [0, 1): the caller's random
 *                 draw per row (read only when temperature > 0)
 *   ws            >= confk_workspace_size(CONFK_WS_CONFIDENCE, ...) bytes
 *                 (per-chunk partial reductions; no initialisation needed)
 * Errors: INVALID_ARG (null, batch < 1, vocab < 2, ld < vocab, nbl < 1,
 * only one of the layer arrays given, temperature negative, NaN or +inf,
 * token_out with temperature > 0 but no uniform), WORKSPACE.
 */
int confk_confidence(const float* logits, int64_t ld, int32_t batch, int32_t vocab,
                     const confk_policy* pol, const int32_t* layer_n_high,
                     const int32_t* layer_n_low, int32_t nbl, float* c_out,
                     int32_t* budget_out, uint32_t* status, const float* uniform,
                     float temperature, int32_t* token_out, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * confk_attn_decode -- decode attention over the cache plus the new token,
 * with INT8 dequantisation fused into the tile reads, and the per-key
 * attention mass. Summary "Methodik" (Implementierung: compact layout,
 * dequantisation fused into blockwise attention reads); review "前置知识"
 * (blockwise online softmax gives the exact softmax) and Algorithm 1 steps
 * 1-2. For query head h (kv head j = h / (hq/hkv)) over keys i = 0..n
 * (i = n the new token): u = q_h . k_i / sqrt(d), P_h = softmax(u),
 * o_h = sum_i P_h,i v_i.
 *   q             fp16 [nlayers][B][hq][d]
 *   k_new, v_new  fp16 [nlayers][B][hkv][d]
 *   out           fp16 [nlayers][B][hq][d]
 *   mass          fp32 [nlayers][B][hkv][cap], rows of partial sums: the
 *                 first R rows of a (layer, sequence), R = its meta word
 *                 CONFK_META_MASSROWS (1 <= R <= hkv, written by this call),
 *                 hold sums over disjoint runs of its kv heads of P_h,i
 *                 summed over each kv head's query heads, i = 0..n, so that
 *                 sum over rows r < R of mass[..][r][i] = sum over all query
 *                 heads of P_h,i (the per-key mean is that sum / hq). Rows
 *                 r >= R are left as they were. R = hkv (row j = kv head j)
 *                 unless the launch's units (layer, sequence, kv head) fill
 *                 at least two rounds of the GPU's resident workgroups; then
 *                 the workgroups run two consecutive units each (kv heads
 *                 fastest), except the last round of dispatch, whose
 *                 workgroups run one, and each writes one row per (layer,
 *                 sequence) it touches: R = hkv / 2 for an even hkv, hkv in
 *                 the last round, and in between where the two meet (pairs
 *                 of kv heads first, then single heads). NULL
 *                 when the caller needs only the output (no workspace then;
 *                 the meta word is not touched)
 *   ws            >= confk_workspace_size(CONFK_WS_ATTENTION_NOSPLIT, ...)
 *                 bytes (score spill for caches too long for on-chip
 *                 memory); with confk_workspace_size(CONFK_WS_ATTENTION,
 *                 ...) bytes it also holds the split exchange area (below).
 *                 The exchange area must be zero before its first use (the
 *                 library keeps it consistent from then on); the spill part
 *                 needs no initialisation
 * Split keys: a launch of few units (at most 64 and at most 1/32 of the
 * GPU's resident workgroup slots; e.g. one layer at batch 1), given the
 * exchange area and a capacity that allows long units, runs each unit of
 * more than 512 keys as several workgroups, each over one range of its
 * keys (blockwise online softmax, review "前置知识"): they exchange each
 * query head's running max and normaliser and their output partials through
 * the exchange area with device-scope atomics, so the output and the
 * per-key mass are those of the whole unit (up to rounding). A workgroup
 * that waits too long for another's values sets CONFK_STATUS_SPLIT_WAIT and
 * goes on. Two launches that share a workspace must not overlap in time.
 * Layers layer0 .. layer0+nlayers-1 of the cache are processed; tensor
 * arguments are indexed from layer0. Supported: d in {64, 128},
 * hq/hkv in 1..16.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, LAUNCH.
 */
int confk_attn_decode(const confk_cache* cache, int32_t layer0, int32_t nlayers,
                      const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                      uint16_t* out, float* mass, void* ws, size_t ws_bytes, void* stream);

/*
 * confk_confidence_attn_decode -- confk_confidence followed by
 * confk_attn_decode on the same stream, with the same results bit for bit,
 * in two launches instead of three: the confidence pass over the logits,
 * then the attention launch, whose first workgroups merge the per-chunk
 * confidence states, take the next token (greedy or none) and write c and
 * the budgets while the others run attention. Summary "Methodik"
 * (Konfidenzschaetzung, Implementierung); review Algorithm 1 steps 1-4.
 * Arguments: those of confk_confidence (conf_ws as its ws), then those of
 * confk_attn_decode (attn_ws as its ws); each set is validated as there,
 * and an error enqueues nothing. With temperature sampling (token_out and
 * temperature > 0) the confidence call's own final kernel runs instead (its
 * draw holds a chunk of weights in registers), so the call is three launches.
 * Errors: those of the two calls.
 */
int confk_confidence_attn_decode(const float* logits, int64_t ld, int32_t batch, int32_t vocab,
                                 const confk_policy* pol, const int32_t* layer_n_high,
                                 const int32_t* layer_n_low, int32_t nbl, float* c_out,
                                 int32_t* budget_out, uint32_t* status, const float* uniform,
                                 float temperature, int32_t* token_out, void* conf_ws,
                                 size_t conf_ws_bytes, const confk_cache* cache, int32_t layer0,
                                 int32_t nlayers, const uint16_t* q, const uint16_t* k_new,
                                 const uint16_t* v_new, uint16_t* out, float* mass, void* attn_ws,
                                 size_t attn_ws_bytes, void* stream);

/*
 * confk_ema_rank -- EMA update of the attention mass and rank scores.
 * Review "前置知识" (EMA: a_i <- lambda a_i + (1-lambda) Abar_i) and "核心方法"
 * (s_i = alpha a^_i + (1-alpha) r^_i). Abar_i = sum_{r<R} mass[r][i] / hq,
 * R the (layer, sequence)'s CONFK_META_MASSROWS word (0 reads as hkv; a
 * value above hkv is taken as hkv), rows summed in order.
 * For cached tokens i < n: ema[i] is updated in place, then
 * score[i] = alpha * ema[i] / max(ema) + (1 - alpha) * (pos[i] - pmin) /
 * (pmax - pmin), with pmin and pmax the smallest and largest position among
 * the n cached tokens (first term 0 when max(ema) = 0, second 1 when
 * pmax = pmin, e.g. n = 1). The positions are reduced, not read at the ends,
 * because the hole-filling order leaves the INT8 part out of position order.
 * The new token's metadata is written to slot n: ema[n] = (1-lambda) Abar_n,
 * pos[n] = t.
 *   mass   fp32 [nlayers][B][hkv][cap] as confk_attn_decode writes it
 *          (any per-kv-head mass with CONFK_META_MASSROWS = 0), or NULL for a
 *          step without attention mass (a run that never evicts, e.g. the
 *          full-cache comparison): then only slot n is written (ema[n] = 0,
 *          pos[n] = t) and the cached tokens' EMA and the scores are left as
 *          they are
 *   score  fp32 [nlayers][B][cap]
 * Errors: INVALID_ARG.
 */
int confk_ema_rank(const confk_cache* cache, int32_t layer0, int32_t nlayers, const float* mass,
                   const confk_policy* pol, int32_t t, float* score, void* stream);

/*
 * confk_compact -- budget eviction, compaction and append.
 * Summary "Methodik" (Token-Ranking und Eviktion; zusammenhaengende
 * Komprimierung without indirection tables); review Algorithm 1 steps 5-11
 * and 13. Per (layer, sequence) with n tokens and budget N: if n > N, the
 * k = n - N tokens with the smallest (score, position) among all but the
 * newest `protect` tokens are evicted and the survivors are packed densely;
 * the new token (slot n metadata from confk_ema_rank, K/V from k_new/v_new)
 * is appended as FP16. Each part (INT8, FP16) keeps position order, packed
 * toward whichever end of its ring moves fewer rows, except that with token
 * eviction and pol->order = CONFK_ORDER_FILL the surviving INT8 tokens at or
 * beyond the INT8 part's new length fill the holes below it, in slot order
 * (the INT8 part is then no longer in position order).
 *   budget       int32, entry for (l, b) at budget[l * budget_layer_stride + b]
 *                (stride 0: one budget per sequence; stride B: per layer)
 *   score        fp32 [nlayers][B][cap] from confk_ema_rank
 *   k_new,v_new  fp16 [nlayers][B][hkv][d]
 *   evicted_out  int32 [nlayers][B] device or NULL: tokens evicted
 *   ws           >= confk_workspace_size(CONFK_WS_COMPACT, ...) bytes: the
 *                move plans (and, above 4096 tokens per sequence, metadata
 *                staging); contents need no initialisation
 * With pol->block = B > 0, whole blocks of B tokens leave (see confk_policy).
 * Sets CONFK_STATUS_CAPACITY (and skips the append) if a sequence has no
 * free slot. Errors: INVALID_ARG, BUDGET (protect > n_low or > n_high,
 * capacity below n_low + 2, FP16 ring below window + 1, protect > window
 * with token eviction in the fill order), UNSUPPORTED (more than 512 blocks per sequence;
 * d above 512 with stable packing, i.e. the stable order or block eviction), WORKSPACE.
 */
int confk_compact(const confk_cache* cache, int32_t layer0, int32_t nlayers, const int32_t* budget,
                  int32_t budget_layer_stride, const float* score, const confk_policy* pol,
                  const uint16_t* k_new, const uint16_t* v_new, int32_t* evicted_out, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * confk_ema_compact -- confk_ema_rank followed by confk_compact in one launch
 * (one workgroup per (layer, sequence) updates the EMA, forms the rank scores
 * and evicts / compacts / appends, without a second pass over the metadata).
 * Same arguments, results and errors as the two calls in sequence (the score
 * buffer receives the rank scores), bit for bit; the split calls stay for
 * callers that inspect or replace the scores in between.
 *   mass   as for confk_ema_rank; t >= 0 the new token's position
 *   score  fp32 [nlayers][B][cap], written
 *   flags  0, or CONFK_FUSE_QUANTIZE: then confk_quantize's window step
 *          (CONFK_QUANT_STEP, same t and layers) follows the append, bit for
 *          bit as the separate call would do it: in the same kernel under
 *          token eviction, as one more launch under block eviction (whose
 *          rows move in a second kernel). Other bits: CONFK_ERR_INVALID_ARG.
 *   other arguments as for confk_compact
 */
#define CONFK_FUSE_QUANTIZE 1
int confk_ema_compact(const confk_cache* cache, int32_t layer0, int32_t nlayers, const float* mass,
                      const confk_policy* pol, int32_t t, float* score, const int32_t* budget,
                      int32_t budget_layer_stride, const uint16_t* k_new, const uint16_t* v_new,
                      int32_t* evicted_out, int32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * confk_ema_compact_static -- confk_ema_compact for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same call, results and errors, with
 * the compaction scratch in a static device array of the library instead of
 * a caller workspace. Nothing is allocated and no allocating routine is
 * called (the array's address is looked up once per device, on the first
 * call with that device current).
 *   Limit: confk_workspace_size(CONFK_WS_COMPACT, cache, nlayers, ...) must
 *   not exceed CONFK_STATIC_SCRATCH_BYTES (64 MiB; e.g. 64 layers x 8
 *   sequences at 2050 slots need 8.4 MB); larger calls return
 *   CONFK_ERR_WORKSPACE and enqueue nothing.
 *   Each GPU holds one array for the life of the process, shared by every
 *   call on that GPU: calls that overlap on one GPU (other streams, other
 *   threads) race and must be serialised by the caller.
 * Other errors: as confk_ema_compact; CONFK_ERR_LAUNCH if the device or the
 * array's address cannot be obtained.
 */
#define CONFK_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int confk_ema_compact_static(const confk_cache* cache, int32_t layer0, int32_t nlayers,
                             const float* mass, const confk_policy* pol, int32_t t, float* score,
                             const int32_t* budget, int32_t budget_layer_stride, const uint16_t* k_new,
                             const uint16_t* v_new, int32_t* evicted_out, int32_t flags, void* stream);

/*
 * confk_decode_step -- one whole decode step in three launches:
 * confk_confidence, confk_attn_decode and confk_ema_compact on the same
 * stream, with the same results bit for bit. The confidence pass over the
 * logits runs as the last workgroups of the attention launch (they fill the
 * slots its last round of dispatch leaves idle); each workgroup of the
 * compaction's plan kernel merges its sequence's confidence states, takes
 * its budget from them and, for the call's first layer, writes c, the token
 * and the budgets. Review Algorithm 1 (the whole step); summary "Methodik".
 * Arguments are those of the three calls: batch is cache->batch, the status
 * word is cache->status, the budget rows are budget_out (nbl = 1: shared,
 * nbl = nlayers: one row per layer of the call), q/k_new/v_new are shared
 * by attention and the append, flags as for confk_ema_compact. conf_ws,
 * attn_ws and compact_ws are the three calls' workspaces. With temperature
 * sampling the confidence call's own two kernels run first (four launches).
 * Errors: those of the three calls; INVALID_ARG also for a NULL mass or nbl
 * other than 1 or nlayers.
 */
int confk_decode_step(const float* logits, int64_t ld, int32_t vocab, const confk_policy* pol,
                      const int32_t* layer_n_high, const int32_t* layer_n_low, int32_t nbl, float* c_out,
                      int32_t* budget_out, const float* uniform, float temperature, int32_t* token_out,
                      const confk_cache* cache, int32_t layer0, int32_t nlayers, int32_t t, const uint16_t* q,
                      const uint16_t* k_new, const uint16_t* v_new, uint16_t* out, float* mass, float* score,
                      int32_t* evicted_out, int32_t flags, void* conf_ws, size_t conf_ws_bytes, void* attn_ws,
                      size_t attn_ws_bytes, void* compact_ws, size_t compact_ws_bytes, void* stream);

/*
 * confk_quantize -- FP16 -> INT8 storage per (head, channel).
 * Summary "Methodik" (gemischte Praezisionsspeicherung: newest W tokens FP16,
 * older retained tokens INT8 per head and channel); review Algorithm 1
 * step 10. Symmetric absmax scales, scale = fp32(absmax)/127, set once per
 * (layer, sequence) when the INT8 region is first populated (over every
 * token then cached) and frozen; code = clamp(rint(fp32(x) / scale), -127,
 * 127) with the IEEE fp32 quotient (0 when the scale is 0).
 *   CONFK_QUANT_STEP: every FP16 token with position <= t - window moves to
 *     the INT8 region (one per step in steady state). k_src/v_src unused.
 *   CONFK_QUANT_PREFILL: (re)initialise layers layer0.. from n_src prefill
 *     tokens k_src/v_src fp16 [nlayers][B][hkv][n_src][d] at positions
 *     0..n_src-1: EMA 0, INT8 for positions <= n_src-1-window, FP16 for the
 *     rest, scales over all n_src tokens when any token is INT8. n_src = 0
 *     gives an empty cache. Also clears the status word.
 * Errors: INVALID_ARG, BUDGET (n_src > cap - 1).
 */
int confk_quantize(const confk_cache* cache, int32_t layer0, int32_t nlayers, int32_t t,
                   const confk_policy* pol, int32_t mode, const uint16_t* k_src,
                   const uint16_t* v_src, int32_t n_src, void* stream);

/* Workspace bytes needed by confk_confidence (which = CONFK_WS_CONFIDENCE;
 * uses batch, vocab), confk_attn_decode (CONFK_WS_ATTENTION) or confk_compact
 * (CONFK_WS_COMPACT; both use the cache dims and nlayers). Returns 0 when
 * none is needed. CONFK_WS_ATTENTION_NOSPLIT gives the part of the attention
 * workspace without the split exchange area: a workspace of that size (or
 * none, when it is 0) makes every launch run one workgroup per unit. */
size_t confk_workspace_size(int32_t which, const confk_cache* cache, int32_t nlayers,
                            int32_t batch, int32_t vocab);

/* Static text for an error code. */
const char* confk_strerror(int code);

/* ABI version (major * 100 + minor). 101: confk_policy.order and the flags
 * argument of confk_ema_compact. 102: the stable survivor order is order 0
 * (the default) and the hole-filling order is 1. 103: confk_ema_compact_static.
 * 104: mass rows are partial sums over runs of kv heads (CONFK_META_MASSROWS).
 * 105: confk_confidence_attn_decode. 106: confk_decode_step. 107: split keys
 * (the attention workspace's exchange area, CONFK_WS_ATTENTION_NOSPLIT,
 * CONFK_STATUS_SPLIT_WAIT). */
int confk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONFK_H */

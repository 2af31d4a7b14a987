// Internal declarations shared by the libconfk HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "confk.h"

namespace confk {

// ---------------------------------------------------------------------------
// Kernel argument blocks (passed by value).
// ---------------------------------------------------------------------------

struct CacheView {
  int32_t L, B, hq, hkv, d, cap, cap16;
  int8_t* k8;
  int8_t* v8;
  uint16_t* k16;
  uint16_t* v16;
  float* ks;
  float* vs;
  float* ema;
  int32_t* pos;
  int32_t* meta;
  uint32_t* status;
};

inline CacheView view_of(const confk_cache* c) {
  return CacheView{c->layers, c->batch, c->hq, c->hkv, c->d, c->cap, c->cap16,
                   c->k8,     c->v8,    c->k16, c->v16, c->kscale, c->vscale,
                   c->ema,    c->pos,   c->meta, c->status};
}

struct ConfArgs {
  const float* logits;
  int64_t ld;
  int32_t batch, vocab, chunk, nchunks, nbl;
  int32_t vec4;  // rows are 16-byte aligned: vector loads
  int32_t vecrec;  // partial records are 32-byte aligned: vector loads/stores
  float tau, w_h, w_m, w_p;
  int32_t n_high, n_low;
  const int32_t* layer_n_high;
  const int32_t* layer_n_low;
  float* partial;  // [batch][nchunks][8]
  float* c_out;
  int32_t* budget_out;
  uint32_t* status;
  const float* uniform;  // [batch] in [0, 1): temperature sampling
  float inv_temp;        // 1 / temperature, 0 for greedy or no choice
  int32_t* token_out;    // [batch] or null
  int32_t choice;        // next-token choice of the pass (set by the launch)
};

struct AttnArgs {
  CacheView c;
  int32_t layer0, nl, g;
  int32_t n_lds;  // score slots (padded key positions) held in LDS per head
  int32_t spill_stride;  // score slots per head in the global spill area
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* out;
  float* mass;
  float* spill;  // [nl*B*hkv][g][spill_stride] or null
  // Fused confidence work on `conf` (conf_mode, set by the caller):
  //  kConfMerge: the launch's first conf_groups workgroups merge the
  //    confidence rows (one wave per row) before the units start;
  //  kConfPass: its last conf_tail workgroups run the confidence pass (one
  //    chunk of one row each). The launcher sets the two counts.
  ConfArgs conf;
  int32_t conf_mode;
  int32_t conf_groups, conf_tail;
  // two kv heads per workgroup (set by the launcher): workgroups
  // [0, acc_pairs) run two units each, the later ones one each
  int32_t acc_pairs;
  // Split keys (launches that leave most resident workgroup slots idle):
  // xchg is the exchange area of the workspace (null: no split), laid out
  // per unit as split_words() words (see attention.hip); split (set by the
  // launcher) is the number of workgroups per unit, split_tiles the INT8
  // tile weight one of them takes at most before a unit is split further.
  uint64_t* xchg;
  int32_t split, split_tiles;
};
// Split-key launches: at most this many workgroups per unit, and only for
// launches of at most kSplitMaxUnits units (the workspace holds an exchange
// area for that many units, whatever the layer count it is sized for, so
// that a workspace sized for every layer also serves one-layer calls).
constexpr int kMaxSplit = 16;
constexpr int64_t kSplitMaxUnits = 64;
// 64-bit words of the exchange area per unit: the epoch word (and a spare),
// each split's (max, normaliser) per query head, each split's output partial.
__host__ __device__ constexpr int64_t split_words(int g, int d) {
  return 2 + (int64_t)kMaxSplit * 32 + (int64_t)kMaxSplit * g * d;
}
enum { kConfNone = 0, kConfMerge = 1, kConfPass = 2 };

struct EmaArgs {
  CacheView c;
  int32_t layer0, nl, t;
  float lambda, alpha;
  const float* mass;
  float* score;
};

constexpr int kMaxEvictBlocks = 512;  // blocks per sequence in block eviction
constexpr int kMaxMoveHeadDim = 512;  // head dimension limit of stable packing (move kernel)
constexpr int kMaxMovePairs = 16384;  // (layer, sequence) pairs per stable-packing call (move kernel)

struct CompactArgs {
  CacheView c;
  int32_t layer0, nl, budget_stride, protect;
  int32_t block;  // 0: token eviction; B: whole blocks of B tokens
  int32_t stable; // token eviction with stable packing (the move kernel moves the rows)
  int32_t* plan;   // workspace: per-(layer, sequence) move plans
  int32_t* jobs;   // workspace: per (layer, sequence), 1 if the move kernel has work there
  int32_t* stage;  // workspace: metadata staging (caches above 4096 tokens)
  const int32_t* budget;
  const float* score;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int32_t* evicted_out;
  // fused form (EMA + rank in the same kernel): mass in, scores out to
  // score_out (the buffer `score` also points at)
  int32_t fuse, t;
  float lambda, alpha;
  const float* mass;
  float* score_out;
  // fused form with the window step (token eviction: in the same kernel)
  int32_t quantize, window;
  // whole-step call: each plan workgroup merges its sequence's confidence
  // states (written by the attention launch) and takes its budget from them
  ConfArgs conf;
  int32_t conf_merge;
  // stable packing of a small launch (set by the launcher): the plan kernel
  // moves the rows itself and no move kernel follows
  int32_t plan_moves;
};

struct QuantArgs {
  CacheView c;
  int32_t layer0, nl, t, window, n_src;
  const uint16_t* k_src;
  const uint16_t* v_src;
};

// ---------------------------------------------------------------------------
// Launchers (defined next to their kernels). Return hipError_t of the launch.
// ---------------------------------------------------------------------------
hipError_t launch_confidence(const ConfArgs& a, hipStream_t s);
size_t confidence_ws_bytes(int32_t batch, int32_t vocab);
hipError_t launch_attention(const AttnArgs& a, int lds_bytes, hipStream_t s);
// Chunking and next-token choice of the confidence pass, set in a.
void confidence_prepare(ConfArgs& a);
// The confidence pass without the final merge (prepares a first).
hipError_t launch_confidence_partial(ConfArgs& a, hipStream_t s);
int attention_lds_bytes(int d, int g, int n_lds);
int attention_plan_n_lds(int d, int g, int cap, int* spill_stride);
// Bytes of the split exchange area for a launch of `units` units (0 when
// such a launch never splits).
size_t attention_xchg_bytes(int64_t units, int g, int d);
hipError_t launch_ema_rank(const EmaArgs& a, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
size_t compact_ws_bytes(int nlayers, int batch, int cap);
size_t compact_plan_bytes(int nlayers, int batch, int cap);
size_t compact_jobs_offset(int nlayers, int batch, int cap);
hipError_t launch_quantize_step(const QuantArgs& a, hipStream_t s);
hipError_t launch_prefill(const QuantArgs& a, hipStream_t s);


// ---------------------------------------------------------------------------
// Small device helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Mass rows of a (layer, sequence): its CONFK_META_MASSROWS word, where 0
// (a fresh cache) or a value outside 1..hkv reads as hkv (one row per kv head).
__device__ __forceinline__ int mass_rows(const int32_t* meta, int hkv) {
  const int r = meta[CONFK_META_MASSROWS];
  return (r >= 1 && r <= hkv) ? r : hkv;
}

// A (layer, sequence) header the kernels can act on: room for the new token
// in the metadata and in the FP16 ring, ring bases inside their rings.
__device__ __forceinline__ bool meta_ok(int n, int n8, int base8, int base16, int cap, int cap16) {
  return n >= 0 && n8 >= 0 && n8 <= n && n + 1 <= cap && n - n8 + 1 <= cap16 && base8 >= 0 &&
         base8 < cap && base16 >= 0 && base16 < cap16;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace confk

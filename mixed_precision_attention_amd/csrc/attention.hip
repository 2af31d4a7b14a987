// Decode attention over the mixed FP16/INT8 cache with fused dequantisation,
// plus the per-key attention mass.
//
// CONF-KV summary, "Methodik: CONF-KV" (Implementierung): survivors sit in a
// dense layout without indirection tables and dequantisation is fused into
// the blockwise attention reads; the review's "前置知识" section: blockwise
// online softmax keeps a running max and normaliser and is exact. The mass
// feeds the EMA of the review's "前置知识"/"核心方法" sections.
//
// One workgroup (4 waves) per (layer, sequence, kv head), or, when the units
// fill two or more rounds of resident workgroups, two consecutive kv heads of
// one (layer, sequence) per workgroup (their mass summed in LDS) except in
// the launch's last round, which runs one per workgroup. The g query heads
// sharing the kv head form the N side of the matrix-core tiles, keys the M
// side, so every K/V byte is read from HBM once per step:
//   scores  S^T[16 keys x 16 heads] = K_tile[16 x d] . Q^T      (16x16x32 f16)
//   output  O^T[16 ch x 16 heads]  += V^T[16 ch x 16 keys] . P^T (16x16x16 f16)
// The score accumulator layout (lane = head + 16*key-group, 4 keys per lane)
// is exactly the B-operand layout of the second product, so P^T goes from
// registers to the matrix core with one fp16 conversion.
//
// Dequantisation: per-channel K scales are folded into the query once
// (q' = q * s_K * log2(e)/sqrt(d)); INT8 codes become fp16 exactly through a
// byte permute (0x64 exponent byte) and one packed subtract; per-channel V
// scales multiply the INT8 part of the accumulator once, when the wave moves
// from the INT8 region to the FP16 region.
//
// Score accuracy: q' is split into fp16 hi + lo parts (after scaling by a
// power of two into fp16's normal range), so the fp32 scores carry ~22 bits;
// the probabilities fed to the second product are fp16.
//
// Memory pipeline: each wave walks every 4th 16-key tile of a region. In the
// INT8 region it holds three tiles of raw codes in registers (two loads in
// flight while one tile is converted and multiplied), in the FP16 region two.
// The query, K scales and V scales are staged once in LDS, so switching
// regions costs no memory round trip, and the first FP16 tiles are requested
// before the FP16 query operands are built. Tail rows are clamped to a valid
// row (their scores are masked), so loads carry no branches.
//
// Mass: the log2-domain scores are kept in LDS (or, in a separate kernel
// instance chosen by the capacity, partly in a global spill area for a unit
// whose scores exceed the LDS budget; its other units run the spill-free
// form); once the waves' running maxima and normalisers are merged, each
// key's mass sum_h 2^(s_h - M_h) / L_h is formed exactly. A two-unit
// workgroup issues its second unit's first loads before its first unit's
// merge, mass pass and output.
#include <mutex>
#include <type_traits>

#include "confidence_dev.h"
#include "confk_internal.h"

namespace confk {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Waves per workgroup (one workgroup per (layer, sequence, kv head)) and the
// target waves per SIMD; the register budget follows from the latter.
#ifndef CONFK_ATTN_WAVES
#define CONFK_ATTN_WAVES 4
#endif
#ifndef CONFK_ATTN_OCCUPANCY
#define CONFK_ATTN_OCCUPANCY 3
#endif
constexpr int kWaves = CONFK_ATTN_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kScoreLdsBytes = 48 * 1024;  // LDS budget for the score store (3 groups per CU)

// Two INT8 codes (bytes b0/b1 or b2/b3 of x = codes ^ 0x80808080) -> two fp16.
// perm places each biased code under an 0x64 exponent byte: fp16 value
// 1024 + (code + 128); subtracting 1152 leaves the code, exactly.
__device__ __forceinline__ uint32_t codes_to_h2(uint32_t x, uint32_t sel) {
  const uint32_t p = __builtin_amdgcn_perm(0x64646464u, x, sel);
  half2_t h = __builtin_bit_cast(half2_t, p);
  h = h - (half2_t){(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, h);
}
constexpr uint32_t kSelLo = 0x04010400u;  // [b0, 0x64, b1, 0x64]
constexpr uint32_t kSelHi = 0x04030402u;  // [b2, 0x64, b3, 0x64]

// Byte bb of row0 and of row1 -> fp16 pair (row0, row1).
__device__ __forceinline__ uint32_t code_pair_rows(uint32_t row0w, uint32_t row1w, int bb) {
  const uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + bb) << 16) | (uint32_t)bb;
  uint32_t p = __builtin_amdgcn_perm(row1w, row0w, sel) ^ 0x64806480u;
  half2_t h = __builtin_bit_cast(half2_t, p);
  h = h - (half2_t){(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, h);
}

// Half hf (0/1) of row0w and of row1w -> fp16 pair (row0, row1).
__device__ __forceinline__ uint32_t half_pair_rows(uint32_t row0w, uint32_t row1w, int hf) {
  return __builtin_amdgcn_perm(row1w, row0w, hf ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ half8_t as_half8(u32x4 v) { return __builtin_bit_cast(half8_t, v); }
__device__ __forceinline__ half4_t as_half4(u32x2 v) { return __builtin_bit_cast(half4_t, v); }

// INT8 K and all V rows are read with non-temporal (streaming) loads, each
// instruction covering whole 128-byte lines (INT8 K rows through lane pairs,
// see unpair); the INT8 K change took the kernel from 241 to 233 us on the
// Qwen-32B-shape batch-8 cache. FP16 K rows stay on plain loads (one
// instruction reads half a line of each of 16 rows, the next the other half,
// which then hits): paired
// streaming loads there were measured 2-3% slower, also with a 1 GiB read
// between launches. Streaming the mass stores was measured slower.
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) { return __builtin_nontemporal_load(p); }

// Paired K-row loads: the lanes of key rows r and r ^ 8 (r of the 16 rows of
// the operand layout) read the two 64-byte halves of one 128-byte row in one
// instruction, a = the rows r & 7, b = the rows (r & 7) + 8. Afterwards lane r < 8 holds its own first
// half (a) and row r + 8's first half (b), lane r >= 8 row r - 8's second half
// (a) and its own second half (b). One row rotation by 8 lanes swaps the
// foreign halves, leaving each lane its row's first and second half.
__device__ __forceinline__ void unpair(const u32x4& a, const u32x4& b, bool lo, u32x4& first,
                                       u32x4& second) {
  const u32x4 x = lo ? b : a;
  u32x4 y;
#pragma unroll
  for (int z = 0; z < 4; ++z) y[z] = (uint32_t)__builtin_amdgcn_mov_dpp((int)x[z], 0x128, 0xF, 0xF, false);
  first = lo ? a : y;
  second = lo ? y : b;
}

template <int D>
struct Tile {
  static constexpr int KC = D / 32;  // 16x16x32 chunks along d
  static constexpr int CB = D / 16;  // 16-channel blocks of the output
  static constexpr int KU = D / 64;  // 16-byte loads per INT8 K row per lane
};

// Physical d of element j of chunk kc in the query/key operands of lane
// group kg. INT8 rows: each lane reads 16 contiguous bytes per 64-byte half
// of the row; FP16 rows: 8 contiguous halves per chunk.
__device__ __forceinline__ int d_int8(int kc, int kg) {
  return (kc >> 1) * 64 + 16 * kg + 8 * (kc & 1);
}
__device__ __forceinline__ int d_fp16(int kc, int kg) { return 32 * kc + 8 * kg; }

// Builds the hi/lo fp16 query operands of this lane (head hh, group kg) for
// one key region from the LDS copy of the query (and K scales); returns the
// power-of-two factor that undoes the scaling.
template <int D, bool INT8>
__device__ __forceinline__ float build_q(const uint16_t* qrow, const float* kscale, bool active,
                                         int kg, half8_t* qhi, half8_t* qlo) {
  constexpr int KC = Tile<D>::KC;
  const float cq = kLog2e / sqrtf((float)D);
  float x[KC][8];
  float mx = 0.f;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int d0 = INT8 ? d_int8(kc, kg) : d_fp16(kc, kg);
    if (active) {
      const half8_t h = as_half8(*reinterpret_cast<const u32x4*>(qrow + d0));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = (float)h[j] * cq;
        if (INT8) v *= kscale[d0 + j];
        x[kc][j] = v;
        mx = fmaxf(mx, fabsf(v));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[kc][j] = 0.f;
    }
  }
  mx = wave_max(mx);
  int e = 0;
  if (mx > 0.f) {
    frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
  }
  int sh = 12 - e;  // scaled max in [2^11, 2^12)
  sh = max(-100, min(100, sh));
  const float up = ldexpf(1.f, sh);
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = x[kc][j] * up;
      const _Float16 hi = (_Float16)v;
      qhi[kc][j] = hi;
      qlo[kc][j] = (_Float16)(v - (float)hi);
    }
  }
  return ldexpf(1.f, -sh);
}

struct SoftState {
  float m;  // running max of this lane's head (log2 units)
  float l;  // partial normaliser over this lane's keys
};

// max without NaN canonicalisation (operands are finite scores or -inf)
__device__ __forceinline__ float fmax_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max over the four lanes {l, l^16, l^32, l^48} (the 16 keys of a tile for
// one head): two cross-row swaps, no LDS round trip.
__device__ __forceinline__ float tile_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = fmax_raw(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmax_raw(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Online-softmax update for one 16-key tile of raw scores s (true score =
// s * unscale, log2 units); returns the P^T operand.
template <int CB>
__device__ __forceinline__ half4_t softmax_tile(float4_t s, float unscale, SoftState& st,
                                                float4_t* acc) {
  const float tmax = tile_max(fmax_raw(fmax_raw(s[0], s[1]), fmax_raw(s[2], s[3]))) * unscale;
  const float mnew = fmaxf(st.m, tmax);
  if (__any(mnew > st.m)) {
    const float corr = __builtin_amdgcn_exp2f(st.m - mnew);
    st.l *= corr;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] *= corr;
  }
  st.m = mnew;
  half4_t p;
  float lsum = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float e = __builtin_amdgcn_exp2f(fmaf(s[v], unscale, -mnew));
    lsum += e;
    p[v] = (_Float16)e;
  }
  st.l += lsum;
  return p;
}

// Raw registers of one 16-key INT8 tile of this lane.
template <int D>
struct Raw8 {
  u32x4 k[Tile<D>::KU];            // K rows: 16 bytes per 64-byte half (lane pairs when KU = 2)
  uint32_t v[4][Tile<D>::CB / 4];  // V rows 4kg+j: D/16 bytes at channel (D/16)*r16
};

// Raw registers of one 16-key FP16 tile of this lane.
template <int D>
struct Raw16 {
  u32x4 k[Tile<D>::KC];            // K row r16: 8 halves per chunk
  uint32_t v[4][Tile<D>::CB / 2];  // V rows 4kg+j: D/16 halves at channel (D/16)*r16
};

// Output reduction rows: lane (head r16, group kg) holds d/4 consecutive
// channels; each such block is padded by 4 floats and a head's row spans
// 4 blocks, so the 64 lanes of a wave spread over all LDS banks.
__host__ __device__ constexpr int red_block(int d) { return d / 4 + 4; }
__host__ __device__ constexpr int red_row(int d) { return 4 * red_block(d); }

// LDS layout: scores [g][n_lds] fp32 (n_lds = 4 mod 32, so the heads' rows
// fall on different banks; later the per-wave output reduction
// [kWaves][g][red_row] fp32), then the query [g][D] fp16, K scales [D],
// V scales [D].
__host__ __device__ __forceinline__ int score_area_floats(int d, int g, int n_lds) {
  const int sc = g * n_lds;
  const int red = kWaves * g * red_row(d);
  return sc > red ? sc : red;
}

// Units (layer, sequence, kv head) per workgroup with the LDS mass sum.
// Two kv heads per workgroup halve the mass rows written; more would leave
// a long last round of dispatch (e.g. 4 per workgroup: 4096 units of the
// 64-layer, batch-8 shape become 1024 workgroups, 1.33 rounds of 768).
constexpr int kAccUnits = 2;

// The unit ranges: workgroup w < P (P = acc_pairs) runs units [2w, 2w + 2),
// a later one the single unit P + w, so the last workgroups dispatched are
// one-unit ones and the launch's last round drains sooner.
__device__ __forceinline__ int unit_owner(uint32_t x, uint32_t P) {
  return (int)(x < 2 * P ? x >> 1 : x - P);
}

// Split keys: the INT8 tiles [t8a, t8b) of one of ns workgroups sharing a
// unit, the last of which also takes the FP16 region with the new token.
// The unit weighs nt8 + 2 nt16 INT8 tiles (an FP16 tile reads twice the
// bytes) and is cut into ns = floor(weight / wtile) pieces of equal weight
// (at least one, at most S), so a piece weighs at least wtile tiles; fewer
// when a piece but the last would start past the INT8 region, so every
// piece holds keys.
struct SplitRange {
  int ns, t8a, t8b;
  bool fp;
};
__device__ __forceinline__ SplitRange split_range(int n, int n8, int S, int wtile, int sj) {
  const int nt8 = (n8 + 15) >> 4, nt16 = (n - n8 + 1 + 15) >> 4;
  const int wt = nt8 + 2 * nt16;
  int ns = min(S, wt / wtile);
  while (ns > 1 && (int)((int64_t)(ns - 2) * wt / ns) >= nt8) --ns;
  ns = max(ns, 1);
  SplitRange r;
  r.ns = ns;
  r.t8a = min(nt8, (int)((int64_t)sj * wt / ns));
  r.t8b = sj >= ns - 1 ? nt8 : min(nt8, (int)((int64_t)(sj + 1) * wt / ns));
  r.fp = sj == ns - 1;
  return r;
}

// Split-key exchange words are (fp32 bits << 32 | tag) with tag = 2 e + 1
// for the unit's epoch word e: a word written in an earlier launch (or a
// zeroed one) never carries the current tag, so a reader waits until the
// writer of this launch has stored it. Relaxed device-scope atomics keep
// each word coherent across the chip's L2 caches without fences.
constexpr int kSpinMax = 1 << 14;  // waits give up (and flag the status word) after this many polls
__device__ __forceinline__ void xput(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)__builtin_bit_cast(uint32_t, v) << 32) | tag, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float xget(const uint64_t* p, uint32_t tag, uint32_t* status) {
  uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0; (uint32_t)v != tag && it < kSpinMax; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if ((uint32_t)v != tag) {
    atomicOr(status, (uint32_t)CONFK_STATUS_SPLIT_WAIT);
    return 0.f;
  }
  return __builtin_bit_cast(float, (uint32_t)(v >> 32));
}

// SPILL: scores past the LDS budget go to global memory. Kept out of the
// common instance because global stores in the tile loop make the load
// counter unusable for partial waits (stores complete out of order); the
// instance runs each unit whose scores fit the LDS budget in the form
// without them.
// MASS = false: no per-key mass (no score store; for callers that only need
// the attention output, e.g. a full-cache baseline).
// ACC (an even hkv): workgroup w runs the unit range of unit_owner (kv heads
// fastest, at most kAccUnits units) and sums the mass of the
// consecutive kv heads of one (layer, sequence) in LDS, so it writes one
// partial mass row per (layer, sequence) it touches instead of one per kv
// head. Row r of a (layer, sequence) is the r-th workgroup that covers it;
// the row count goes to its metadata.
// SPLIT (launches that fill few of the resident workgroup slots): a.split
// consecutive workgroups per unit, each taking a range of the unit's keys
// (split_range). They run the tile loops on their keys, publish each
// head's running max and normaliser, take the unit's merged values from
// every split's, write the mass of their own keys and (the later ones)
// publish their output partial, which the first sums in split order. The
// per-key mass stays exact without any score leaving the workgroup.
template <int D, bool SPILL, bool MASS, bool ACC, bool SPLIT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(CONFK_ATTN_OCCUPANCY)))
void attn_decode_kernel(AttnArgs a) {
  constexpr int KC = Tile<D>::KC;
  constexpr int CB = Tile<D>::CB;
  constexpr int KU = Tile<D>::KU;
  static_assert(!ACC || (MASS && !SPILL), "mass rows are summed in LDS only with the LDS score store");
  static_assert(!SPLIT || (MASS && !ACC), "split keys: one unit per workgroup group, with the mass");
  static_assert(kMaxSplit * 16 <= kThreads, "one thread per (split, head) pair of the exchange");
  extern __shared__ float lds[];

  // Fused confidence call: the launch's first conf_groups workgroups merge
  // the confidence rows (one wave per row, the confidence call's final
  // step) while the others run the units.
  if (a.conf_groups > 0 && (int)blockIdx.x < a.conf_groups) {  // uniform per workgroup
    const int row = (int)blockIdx.x * kWaves + (int)(threadIdx.x >> 6);
    if (row < a.conf.batch) {  // uniform per wave
      const int lane = threadIdx.x & 63;
      // (a pass with temperature sampling keeps its own final kernel: the
      // draw holds a chunk of weights in registers)
      if (a.conf.choice == confm::kGreedy) confm::conf_final_row<confm::kGreedy>(a.conf, row, lane);
      else confm::conf_final_row<confm::kNoChoice>(a.conf, row, lane);
    }
    return;
  }
  // Whole-step call: the launch's last conf_tail workgroups run the
  // confidence pass, one chunk of one row each; dispatched last, they fill
  // the slots the units' last round leaves idle.
  if (a.conf_tail > 0 && (int)blockIdx.x >= (int)gridDim.x - a.conf_tail) {  // uniform per workgroup
    const int p = (int)blockIdx.x - ((int)gridDim.x - a.conf_tail);
    const int row = p / a.conf.nchunks, chunk = p - row * a.conf.nchunks;
    static_assert(kThreads == confm::kConfThreads, "a pass workgroup is an attention workgroup");
    if (a.conf.choice == confm::kGreedy) confm::conf_partial_block<confm::kGreedy>(a.conf, chunk, row, threadIdx.x);
    else confm::conf_partial_block<confm::kNoChoice>(a.conf, chunk, row, threadIdx.x);
    return;
  }

  const CacheView& c = a.c;
  const int H = c.hkv;
  const int g = a.g;
  const uint32_t P = (uint32_t)a.acc_pairs;
  const int wg = blockIdx.x - a.conf_groups;
  // SPLIT: a.split consecutive workgroups per unit, split sj of it
  const int u_split = SPLIT ? wg / a.split : 0;
  const int sj = SPLIT ? wg - u_split * a.split : 0;
  const int u_begin = ACC ? ((uint32_t)wg < P ? 2 * wg : (int)P + wg) : SPLIT ? u_split : wg;
  const int u_end = ACC ? ((uint32_t)wg < P ? 2 * wg + 2 : (int)P + wg + 1) : u_begin + 1;
  // (layer, sequence, kv head) of the current unit, advanced without
  // divisions; a (layer, sequence) that starts inside this range has its
  // first unit here, so this workgroup writes its row 0
  int h = u_begin % H;
  int lb = u_begin / H;  // local (layer, sequence)
  int b = lb % c.B;
  int l = lb / c.B;
  const int lb_first = lb;
  const int mrow_first = ACC ? wg - unit_owner((uint32_t)(lb * H), P) : h;

  // ACC: the next unit of a workgroup is the next kv head of the same
  // (layer, sequence) (same cache header, same ring slots); its first loads
  // (the query and scale pieces, each wave's first two INT8 tiles) go out
  // when this unit's tiles are done, and arrive during its merge, mass pass
  // and output.
  u32x4 nx_piece[2];
  Raw8<D> nx_a, nx_b;  // set before any read (no initial value: no copies where they are set)
  bool nx_ok = false;
  // The second unit of a range also takes the first one's cache header (the
  // same (layer, sequence)), and the first unit's output waits in registers
  // until the second unit's tile loops are done: a store still in flight
  // would turn the second unit's first wait for its early loads into a wait
  // for every memory operation (loads and stores share one counter and
  // complete out of order with respect to each other).
  int hd_n, hd_n8, hd_b8, hd_b16;
  uint32_t oh[2];
  bool oh_ok = false;
  const int h_first = h;  // kv head of the range's first unit

  // the work of one unit; ACC runs it for each unit of the range in turn.
  // Compile-time flags: NEXT, the first of a workgroup's two units, which
  // issues the second one's first loads at its end; SPL, scores past the
  // LDS budget go to the spill area (a unit whose scores fit runs the form
  // without global stores in its tile loops).
  auto unit_body = [&](int u, auto NEXT, auto SPL) __attribute__((always_inline)) {
  constexpr bool next = decltype(NEXT)::value;
  constexpr bool spl = SPILL && decltype(SPL)::value;
  if (u != u_begin) {
    if (++h == H) {
      h = 0;
      ++lb;
      if (++b == c.B) {
        b = 0;
        ++l;
      }
    }
  }
  // the thread index, opaque per unit: values derived from it are formed
  // again in each unit instead of being held in registers across units
  int tid = threadIdx.x;
  if constexpr (ACC) asm volatile("" : "+v"(tid));
  const int lbc = (a.layer0 + l) * c.B + b;
  // mass row of this unit; its (layer, sequence)'s first workgroup writes
  // the row count
  const int mrow = !ACC ? h : (lb == lb_first ? mrow_first : 0);
  const bool acc_first = !ACC || h == 0 || u == u_begin;    // first of this row's heads
  const bool acc_last = !ACC || h == H - 1 || u == u_end - 1;  // last: write the row

  int32_t* meta = c.meta + lbc * CONFK_META_WORDS;
  int n, n8, base8, base16;
  if (ACC && !next && nx_ok) {  // uniform
    n = hd_n;
    n8 = hd_n8;
    base8 = hd_b8;
    base16 = hd_b16;
  } else {
    n = meta[CONFK_META_N];
    n8 = meta[CONFK_META_N8];
    base8 = meta[CONFK_META_BASE8];
    base16 = meta[CONFK_META_BASE16];
  }
  if constexpr (ACC && next) {
    hd_n = n;
    hd_n8 = n8;
    hd_b8 = base8;
    hd_b16 = base16;
  }
  const int f = n - n8;
  const int nk = n + 1;
  if (!meta_ok(n, n8, base8, base16, c.cap, c.cap16)) {  // uniform per workgroup
    if (tid == 0) atomicOr(c.status, (uint32_t)CONFK_STATUS_CAPACITY);
    return;
  }
  const int nt8 = (n8 + 15) >> 4;
  const int nt16 = (f + 1 + 15) >> 4;
  // SPLIT: this workgroup's INT8 tiles [t8a, t8b), and the FP16 region if
  // it is the unit's last split (fp); score slot 0 is key so8. Otherwise
  // the whole unit.
  int t8a = 0, t8b = nt8, ns = 1;
  bool fp = true;
  if constexpr (SPLIT) {
    const SplitRange sr = split_range(n, n8, a.split, a.split_tiles, sj);
    if (sj >= sr.ns) return;  // uniform: the unit needs fewer workgroups
    ns = sr.ns;
    t8a = sr.t8a;
    t8b = sr.t8b;
    fp = sr.fp;
  }
  const int so8 = 16 * t8a;
  const int p16 = (t8b - t8a) * 16;  // first score slot of the FP16 region
  // split exchange: the unit's words and this launch's tag
  uint64_t* xw = SPLIT ? a.xchg + (size_t)u * split_words(g, D) : nullptr;
  uint32_t xtag = 0;
  if (SPLIT && ns > 1) xtag = 2u * (uint32_t)__hip_atomic_load(xw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  const size_t hrow = (size_t)lbc * H + h;
  const int8_t* k8 = c.k8 + hrow * c.cap * D;
  const int8_t* v8 = c.v8 + hrow * c.cap * D;
  const uint16_t* k16 = c.k16 + hrow * c.cap16 * D;
  const uint16_t* v16 = c.v16 + hrow * c.cap16 * D;
  const size_t qoff = ((size_t)lb * c.hq + (size_t)h * g) * D;
  const uint16_t* kn = a.k_new + ((size_t)lb * H + h) * D;
  const uint16_t* vn = a.v_new + ((size_t)lb * H + h) * D;
  float* spill = spl ? a.spill + (size_t)u * g * a.spill_stride + so8 : nullptr;

  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const bool head_ok = r16 < g;

  const int n_lds = a.n_lds;
  float* sc = lds;  // [g][n_lds]
  uint16_t* q_lds = reinterpret_cast<uint16_t*>(lds + score_area_floats(D, g, n_lds));  // [g][D]
  float* ks_lds = reinterpret_cast<float*>(q_lds + g * D);                               // [D]
  float* vs_lds = ks_lds + D;                                                            // [D]
  float* acc_lds = vs_lds + D;  // [cap] mass of this row's earlier kv heads (ACC)
  const uint16_t* qrow = q_lds + (size_t)(head_ok ? r16 : 0) * D;

  float4_t acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = (float4_t){0.f, 0.f, 0.f, 0.f};
  SoftState st{-INFINITY, 0.f};
  // Stored scores are raw products; usc[0] / usc[1] turn INT8 / FP16 region
  // scores into log2 units.
  __shared__ float usc[2];

  auto store_scores = [&](int p0, float4_t s) {
    if (!MASS || !head_ok) return;
    const int p = p0 + 4 * kg;
    if (!spl || p0 + 16 <= n_lds) {  // whole tiles stay in LDS (n_lds is not a multiple of 16)
      *reinterpret_cast<float4_t*>(sc + (size_t)r16 * n_lds + p) = s;
    } else {
      *reinterpret_cast<float4_t*>(spill + (size_t)r16 * a.spill_stride + p) = s;
    }
  };

  // ------------------------------------------------------------ tile loads
  // INT8 rows: running ring slots of this lane's first K row and first V
  // row in the next tile this wave loads (tiles w, w+kWaves, ... in order;
  // the slot stops advancing at the wave's last tile). 32-bit byte offsets
  // from the uniform ring base.
  const int last8 = max(t8b - 1, t8a);
  const uint32_t cap = (uint32_t)c.cap;
  auto wrap = [&](uint32_t x) { return min(x, x - cap); };  // x < 2 cap
  const uint32_t step8 = (uint32_t)(16 * kWaves) % cap;
  uint32_t vinc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vinc[j] = (uint32_t)j % cap;
  int tnext = min(t8a + w, last8);  // tile of the next load (uniform)
  // 128-byte INT8 K rows are read in lane pairs (see unpair): each
  // instruction covers whole rows.
  constexpr bool kpair = KU == 2;
  const int krow0 = kpair ? (r16 & 7) : r16;
  const uint32_t kcol = 16 * kg + (kpair ? 64 * (r16 >> 3) : 0);
  const uint32_t kinc8 = 8u % cap;
  const uint32_t sk0 = (uint32_t)((base8 + 16 * tnext + krow0) % c.cap);
  const uint32_t sv0 = (uint32_t)((base8 + 16 * tnext + 4 * kg) % c.cap);
  uint32_t sk = sk0, sv = sv0;
  // one tile of the rings at kb / vb from ring slots s_k (K) and s_v (V)
  auto ld8 = [&](Raw8<D>& r, const int8_t* kb, const int8_t* vb, uint32_t s_k, uint32_t s_v) {
    if constexpr (kpair) {
      r.k[0] = stream_load(reinterpret_cast<const u32x4*>(kb + s_k * D + kcol));
      r.k[1] = stream_load(reinterpret_cast<const u32x4*>(kb + wrap(s_k + kinc8) * D + kcol));
    } else {  // 64-byte rows: one instruction covers 16 consecutive rows
      r.k[0] = stream_load(reinterpret_cast<const u32x4*>(kb + s_k * D + kcol));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t vo = wrap(s_v + vinc[j]) * D + (D / 16) * r16;
      if constexpr (CB == 8) {
        const u32x2 t2 = stream_load(reinterpret_cast<const u32x2*>(vb + vo));
        r.v[j][0] = t2[0];
        r.v[j][1] = t2[1];
      } else {
        r.v[j][0] = stream_load(reinterpret_cast<const uint32_t*>(vb + vo));
      }
    }
  };
  auto adv8 = [&]() {  // the slots of this wave's next tile
    const bool adv = tnext + kWaves <= last8;
    const uint32_t by = adv ? step8 : 0u;
    tnext += adv ? kWaves : 0;
    sk = wrap(sk + by);
    sv = wrap(sv + by);
  };
  auto load8 = [&](Raw8<D>& r) {
    ld8(r, k8, v8, sk, sv);
    adv8();
  };
  auto row16 = [&](const uint16_t* ring, const uint16_t* nw, int jj) {  // FP16-local index jj
    if (jj >= f) return nw;  // the new token (also the clamp target of tail rows)
    int s = base16 + jj;
    s = s >= c.cap16 ? s - c.cap16 : s;
    return ring + (size_t)s * D;
  };
  auto load16 = [&](Raw16<D>& r, int t) {
    const int j0 = t * 16;
    const uint16_t* krow = row16(k16, kn, j0 + r16);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) r.k[kc] = *reinterpret_cast<const u32x4*>(krow + d_fp16(kc, kg));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* vrow = row16(v16, vn, j0 + 4 * kg + j) + (D / 16) * r16;
      if constexpr (CB == 8) {
        const u32x4 t4 = stream_load(reinterpret_cast<const u32x4*>(vrow));
#pragma unroll
        for (int z = 0; z < 4; ++z) r.v[j][z] = t4[z];
      } else {
        const u32x2 t2 = stream_load(reinterpret_cast<const u32x2*>(vrow));
        r.v[j][0] = t2[0];
        r.v[j][1] = t2[1];
      }
    }
  };

  // ------------------------------------------------------------ prologue
  // The query and the K/V scales (at most 2 x 256 16-byte pieces) are fetched
  // first, then this wave's first INT8 tiles, then the pieces go to LDS: the
  // tile loads stay in flight across the barrier.
  const int qp = g * D / 8;          // 16-byte pieces of the query block
  const int npieces = qp + D / 2;    // + K scales, V scales
  const u32x4* qsrc4 = reinterpret_cast<const u32x4*>(a.q + qoff);
  const u32x4* ks4 = reinterpret_cast<const u32x4*>(c.ks + hrow * D);
  const u32x4* vs4 = reinterpret_cast<const u32x4*>(c.vs + hrow * D);
  // the pieces of query block qs, K scales kss and V scales vss
  auto load_pieces = [&](u32x4* pc, const u32x4* qs, const u32x4* kss, const u32x4* vss) {
#pragma unroll
    for (int z = 0; z < 2; ++z) {  // unconditional loads (spare threads re-read piece 0)
      const int e = tid + z * kThreads;
      const u32x4* src = e < qp             ? qs + e
                         : e < qp + D / 4   ? kss + (e - qp)
                         : e < npieces      ? vss + (e - qp - D / 4)
                                            : qs;
      pc[z] = *src;
    }
  };
  // (uniform) this unit's first loads were issued by the previous unit
  const bool pre = ACC && !next && nx_ok;
  u32x4 piece[2];
  if (pre) {
    piece[0] = nx_piece[0];
    piece[1] = nx_piece[1];
  } else {
    load_pieces(piece, qsrc4, ks4, vs4);
  }
  const bool has8 = t8b - t8a > w;  // this wave has INT8 tiles (uniform per wave)
  // This wave's INT8 tiles are t_j = w + 4j, j < m8. Each is loaded exactly
  // once: the loops below are peeled so that no load reaches past the last
  // tile, and the loads inside a loop body are unconditional, so the load
  // counter allows partial waits there.
  const int m8 = (t8b - t8a - w + kWaves - 1) / kWaves;
  Raw8<D> ra8{}, rb8{}, rc8{};  // defined on every path (the unit loop carries no undefined values)
  if (pre) {
    ra8 = nx_a;
    rb8 = nx_b;
    if (m8 >= 1) adv8();
    if (m8 >= 2) adv8();
  } else {
    if (m8 >= 1) load8(ra8);
    if (m8 >= 2) load8(rb8);
  }
#pragma unroll
  for (int z = 0; z < 2; ++z) {
    const int e = tid + z * kThreads;
    if (e < qp) {
      reinterpret_cast<u32x4*>(q_lds)[e] = piece[z];
    } else if (e < npieces) {
      reinterpret_cast<u32x4*>(ks_lds)[e - qp] = piece[z];
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ INT8 region
  if (has8) {
    half8_t qhi[KC], qlo[KC];
    const float unscale = build_q<D, true>(qrow, ks_lds, head_ok, kg, qhi, qlo);
    if (w == 0) usc[0] = unscale;  // every wave computes the same factor
    auto tile8 = [&](const Raw8<D>& r, int t) {
      const int i0 = t * 16;
      float4_t s = {0.f, 0.f, 0.f, 0.f};
      u32x4 kk[KU];
      if constexpr (kpair) {
        unpair(r.k[0], r.k[1], r16 < 8, kk[0], kk[1]);
      } else {
#pragma unroll
        for (int uu = 0; uu < KU; ++uu) kk[uu] = r.k[uu];
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const u32x4 xw = kk[kc >> 1] ^ 0x80808080u;
        const int o = 2 * (kc & 1);
        u32x4 hv;
        hv[0] = codes_to_h2(xw[o], kSelLo);
        hv[1] = codes_to_h2(xw[o], kSelHi);
        hv[2] = codes_to_h2(xw[o + 1], kSelLo);
        hv[3] = codes_to_h2(xw[o + 1], kSelHi);
        const half8_t ak = as_half8(hv);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qhi[kc], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qlo[kc], s, 0, 0, 0);
      }
      if (i0 + 16 > n8) {  // tail tile (uniform)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (head_ok && i0 + 4 * kg + v >= n8) s[v] = -INFINITY;
      }
      store_scores(i0 - so8, s);
      const half4_t pT = softmax_tile<CB>(s, unscale, st, acc);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int wd = cb >> 2, bb = cb & 3;
        u32x2 av;
        av[0] = code_pair_rows(r.v[0][wd], r.v[1][wd], bb);
        av[1] = code_pair_rows(r.v[2][wd], r.v[3][wd], bb);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(av), pT, acc[cb], 0, 0, 0);
      }
    };
    // three tiles in registers: two loads in flight while one is computed.
    // ra8 / rb8 hold tiles j, j+1 at the top of the loop, which runs while
    // tiles j+2..j+4 exist; the last 0-4 tiles follow it.
    int j = 0;
    for (; j + 5 <= m8; j += 3) {
      const int t = t8a + w + kWaves * j;
      load8(rc8);
      tile8(ra8, t);
      load8(ra8);
      tile8(rb8, t + kWaves);
      load8(rb8);
      tile8(rc8, t + 2 * kWaves);
    }
    const int rest = m8 - j, t = t8a + w + kWaves * j;
    if (rest >= 3) {
      load8(rc8);
      tile8(ra8, t);
      if (rest == 4) load8(ra8);
      tile8(rb8, t + kWaves);
      tile8(rc8, t + 2 * kWaves);
      if (rest == 4) tile8(ra8, t + 3 * kWaves);
    } else {
      tile8(ra8, t);
      if (rest == 2) tile8(rb8, t + kWaves);
    }
  }

  // ------------------------------------------------------ FP16 region + new
  const bool has16 = fp && nt16 > w;
  Raw16<D> ra{}, rb{};
  if (has16) load16(ra, w);
  if (has8) {
    // V scales of the INT8 part: channel of acc[cb][v] is CB*(4kg+v)+cb
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[cb][v] *= vs_lds[CB * (4 * kg + v) + cb];
  }
  if (has16) {
    half8_t qhi[KC], qlo[KC];
    const float unscale = build_q<D, false>(qrow, nullptr, head_ok, kg, qhi, qlo);
    if (w == 0) usc[1] = unscale;
    auto tile16 = [&](const Raw16<D>& r, int t) {
      const int j0 = t * 16;
      float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const half8_t ak = as_half8(r.k[kc]);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qhi[kc], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qlo[kc], s, 0, 0, 0);
      }
      if (j0 + 16 > f + 1) {  // tail tile (uniform)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (head_ok && j0 + 4 * kg + v > f) s[v] = -INFINITY;
      }
      store_scores(p16 + j0, s);
      const half4_t pT = softmax_tile<CB>(s, unscale, st, acc);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int wd = cb >> 1, hf = cb & 1;
        u32x2 av;
        av[0] = half_pair_rows(r.v[0][wd], r.v[1][wd], hf);
        av[1] = half_pair_rows(r.v[2][wd], r.v[3][wd], hf);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(av), pT, acc[cb], 0, 0, 0);
      }
    };
    // two tiles in registers; the loop runs while a third tile remains, so
    // no load reaches past this wave's last tile
    const int m16 = (nt16 - w + kWaves - 1) / kWaves;
    int j = 0;
    for (; j + 2 < m16; j += 2) {
      const int t = w + kWaves * j;
      load16(rb, t + kWaves);
      tile16(ra, t);
      load16(ra, t + 2 * kWaves);
      tile16(rb, t + kWaves);
    }
    if (j + 1 < m16) {
      load16(rb, w + kWaves * (j + 1));
      tile16(ra, w + kWaves * j);
      tile16(rb, w + kWaves * (j + 1));
    } else {
      tile16(ra, w + kWaves * j);
    }
  }

  if constexpr (ACC && next) {
    {  // the next unit is kv head h + 1 of this (layer, sequence) (hkv is even)
      const size_t hn = hrow + 1;
      load_pieces(nx_piece, reinterpret_cast<const u32x4*>(a.q + qoff + (size_t)g * D),
                  reinterpret_cast<const u32x4*>(c.ks + hn * D), reinterpret_cast<const u32x4*>(c.vs + hn * D));
      // this wave's first two tiles in the next kv head's rings (the slots
      // are ring slots whatever the tile count, so the loads need no test;
      // the second is the first again when the wave has one tile)
      const int8_t* k8n = k8 + (size_t)c.cap * D;
      const int8_t* v8n = v8 + (size_t)c.cap * D;
      // the first slots again, from an opaque thread index (nothing of
      // the tile loops' state is held for this)
      int t2 = threadIdx.x;
      asm volatile("" : "+v"(t2));
      const int l2 = t2 & 63, r2 = l2 & 15, g2 = l2 >> 4;
      const int tn = min(w, last8);
      const uint32_t s_k = (uint32_t)((base8 + 16 * tn + (kpair ? (r2 & 7) : r2)) % c.cap);
      const uint32_t s_v = (uint32_t)((base8 + 16 * tn + 4 * g2) % c.cap);
      const uint32_t by = tn + kWaves <= last8 ? step8 : 0u;
      ld8(nx_a, k8n, v8n, s_k, s_v);
      ld8(nx_b, k8n, v8n, wrap(s_k + by), wrap(s_v + by));
      nx_ok = true;
    }
  }

  if constexpr (ACC && !next) {
    if (oh_ok) {  // uniform: the previous unit's output (the query block before this one's)
      uint16_t* op = a.out + qoff - (size_t)g * D;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = tid + k * kThreads;
        if (idx < g * D) op[idx] = (uint16_t)(oh[k >> 1] >> (16 * (k & 1)));
      }
    }
  }

  // -------------------------------------------------------------- merge
  __shared__ float wm[kWaves][16], wl[kWaves][16], Mh[16], iL[16];
  float lt = st.l + __shfl_xor(st.l, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (kg == 0) {
    wm[w][r16] = st.m;
    wl[w][r16] = lt;
  }
  __syncthreads();
  if ((int)tid < g) {
    const int hh = tid;
    float M = -INFINITY;
    for (int q = 0; q < kWaves; ++q) M = fmaxf(M, wm[q][hh]);
    float L = 0.f;
    for (int q = 0; q < kWaves; ++q)
      if (wl[q][hh] > 0.f) L += wl[q][hh] * exp2f(wm[q][hh] - M);
    if (SPLIT && ns > 1) {  // publish this split's pair (uniform)
      uint64_t* xs = xw + 2;  // [kMaxSplit][16 heads][max, normaliser]
      xput(xs + sj * 32 + 2 * hh, M, xtag);
      xput(xs + sj * 32 + 2 * hh + 1, L, xtag);
    }
    Mh[hh] = M;
    iL[hh] = 1.f / L;
  }
  if (SPLIT && ns > 1) {  // uniform
    // every split's pairs (thread j * g + h reads split j's pair of head h,
    // both words requested at once), then each head merges them in split
    // order, so every split forms the same values
    __shared__ float xm[kMaxSplit][16], xl[kMaxSplit][16];
    const uint64_t* xs = xw + 2;
    if ((int)tid < ns * g) {
      const int j = (int)tid / g, hh = (int)tid - j * g;
      const uint64_t* pw = xs + j * 32 + 2 * hh;
      const uint64_t v0 = __hip_atomic_load(pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t v1 = __hip_atomic_load(pw + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      xm[j][hh] = (uint32_t)v0 == xtag ? __builtin_bit_cast(float, (uint32_t)(v0 >> 32)) : xget(pw, xtag, c.status);
      xl[j][hh] = (uint32_t)v1 == xtag ? __builtin_bit_cast(float, (uint32_t)(v1 >> 32)) : xget(pw + 1, xtag, c.status);
    }
    __syncthreads();
    if ((int)tid < g) {
      const int hh = tid;
      float M = -INFINITY;
      for (int j = 0; j < ns; ++j) M = fmaxf(M, xm[j][hh]);
      float L = 0.f;
      for (int j = 0; j < ns; ++j)
        if (xl[j][hh] > 0.f) L += xl[j][hh] * exp2f(xm[j][hh] - M);
      Mh[hh] = M;
      iL[hh] = 1.f / L;
    }
    // every split has read the epoch (its pairs carry the tag): the unit's
    // next launch takes the next one; this launch's words keep this tag
    if (sj == 0 && tid == 0)
      __hip_atomic_store(xw, (uint64_t)(((xtag - 1u) >> 1) + 1u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // per-key mass (summed over this kv head's query heads, and with ACC
  // over this row's earlier kv heads)
  float* mout = a.mass + ((size_t)lb * H + mrow) * c.cap;
  if constexpr (MASS && !spl) {
    // groups of 4 slots (both regions start 16-aligned; slots past a region
    // hold masked scores and are not written out); all heads' scores of a
    // group are fetched before the exponentials
    // end of this workgroup's INT8 keys; an empty range (a last split with
    // FP16 tiles only) starts past n8 at the padded tile boundary
    const int lim8 = min(16 * t8b, n8);
    const int q8 = max(0, (lim8 - so8 + 3) >> 2), q16 = fp ? (f + 1 + 3) >> 2 : 0;
    for (int gi = tid; gi < q8 + q16; gi += kThreads) {
      const bool r8 = gi < q8;
      const int slot = r8 ? 4 * gi : p16 + 4 * (gi - q8);
      const int i0 = r8 ? so8 + 4 * gi : n8 + 4 * (gi - q8);
      const int lim = r8 ? lim8 : nk;
      const float u = usc[r8 ? 0 : 1];
      float4_t sum = {0.f, 0.f, 0.f, 0.f};
      for (int h0 = 0; h0 < g; h0 += 4) {  // four heads' scores fetched before their exponentials
        float4_t sv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (h0 + j < g) sv[j] = *reinterpret_cast<const float4_t*>(sc + (size_t)(h0 + j) * n_lds + slot);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (h0 + j < g) {
            const float m = Mh[h0 + j], il = iL[h0 + j];
#pragma unroll
            for (int v = 0; v < 4; ++v) sum[v] += __builtin_amdgcn_exp2f(fmaf(sv[j][v], u, -m)) * il;
          }
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (i0 + v < lim) {
          float m = sum[v];
          if constexpr (ACC) {  // each thread owns the same keys in every unit of a row
            if (!acc_first) m += acc_lds[i0 + v];
            if (!acc_last) acc_lds[i0 + v] = m;
          }
          if (acc_last) mout[i0 + v] = m;
        }
      }
    }
  } else if constexpr (MASS) {
    // the same groups of 4 slots. A 16-slot tile's scores are all in LDS or
    // all in the spill area, and slots grow with the group index, so the
    // groups in LDS come first: [0, gs) (the spill area is written and read
    // by this workgroup only)
    // end of this workgroup's INT8 keys; an empty range (a last split with
    // FP16 tiles only) starts past n8 at the padded tile boundary
    const int lim8 = min(16 * t8b, n8);
    const int q8 = max(0, (lim8 - so8 + 3) >> 2), q16 = fp ? (f + 1 + 3) >> 2 : 0;
    const int t_lds = n_lds >> 4;  // tiles wholly in LDS
    const int a8 = min(q8, 4 * t_lds);
    const int gs = a8 < q8 ? a8 : q8 + min(q16, max(0, 4 * t_lds - (p16 >> 2)));
    auto group = [&](int gi, const float* src, size_t stride) __attribute__((always_inline)) {
      const bool r8 = gi < q8;
      const int slot = r8 ? 4 * gi : p16 + 4 * (gi - q8);
      const int i0 = r8 ? so8 + 4 * gi : n8 + 4 * (gi - q8);
      const int lim = r8 ? lim8 : nk;
      const float u = usc[r8 ? 0 : 1];
      float4_t sum = {0.f, 0.f, 0.f, 0.f};
      for (int h0 = 0; h0 < g; h0 += 4) {
        float4_t sv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (h0 + j < g) sv[j] = *reinterpret_cast<const float4_t*>(src + (size_t)(h0 + j) * stride + slot);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (h0 + j < g) {
            const float m = Mh[h0 + j], il = iL[h0 + j];
#pragma unroll
            for (int v = 0; v < 4; ++v) sum[v] += __builtin_amdgcn_exp2f(fmaf(sv[j][v], u, -m)) * il;
          }
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (i0 + v < lim) mout[i0 + v] = sum[v];
    };
    for (int gi = tid; gi < gs; gi += kThreads) group(gi, sc, (size_t)n_lds);
    for (int gi = gs + tid; gi < q8 + q16; gi += kThreads) group(gi, spill, (size_t)a.spill_stride);
  }
  __syncthreads();

  // output: scale each wave's accumulator to the merged normaliser, sum waves.
  // Channel of acc[cb][v] is CB*(4kg+v)+cb: lane block kg, offset CB*v+cb.
  constexpr int RB = red_block(D), RR = red_row(D);
  float* red = lds;  // [kWaves][g][RR], aliases the score area
  if (head_ok) {
    const float fct = (wl[w][r16] > 0.f) ? exp2f(st.m - Mh[r16]) * iL[r16] : 0.f;
    float* dst = red + ((size_t)w * g + r16) * RR + kg * RB;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int hf = 0; hf < CB / 4; ++hf) {
        const float4_t x = {acc[4 * hf][v] * fct, acc[4 * hf + 1][v] * fct, acc[4 * hf + 2][v] * fct,
                            acc[4 * hf + 3][v] * fct};
        *reinterpret_cast<float4_t*>(dst + CB * v + 4 * hf) = x;
      }
  }
  __syncthreads();
  uint16_t* ob = a.out + qoff;
  auto out_sum = [&](int idx) {
    const int hh = idx / D, ch = idx - hh * D;
    const int off = hh * RR + (ch / (D / 4)) * RB + ch % (D / 4);
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) o += red[(size_t)q * g * RR + off];
    return o;
  };
  auto out_at = [&](int idx) { return float_to_half_bits(out_sum(idx)); };
  if (SPLIT && ns > 1) {  // uniform
    // every split publishes its output partial; split j then adds all
    // partials of its share of the output elements, in split order, and
    // writes them (one round trip: a thread's loads go out together)
    uint64_t* xo = xw + 2 + kMaxSplit * 32;  // [kMaxSplit][g][D]
    const int gD = g * D;
    for (int idx = tid; idx < gD; idx += kThreads) xput(xo + (size_t)sj * gD + idx, out_sum(idx), xtag);
    const int e0 = (int)((int64_t)sj * gD / ns), e1 = (int)((int64_t)(sj + 1) * gD / ns);
    for (int e = e0 + tid; e < e1; e += kThreads) {
      uint64_t v[kMaxSplit];
#pragma unroll
      for (int j = 0; j < kMaxSplit; ++j)
        v[j] = j < ns ? __hip_atomic_load(xo + (size_t)j * gD + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
      float o = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxSplit; ++j)
        if (j < ns)
          o += (uint32_t)v[j] == xtag ? __builtin_bit_cast(float, (uint32_t)(v[j] >> 32))
                                      : xget(xo + (size_t)j * gD + e, xtag, c.status);
      ob[e] = float_to_half_bits(o);
    }
  } else if (ACC && next && g * D <= 4 * kThreads) {  // uniform: held until the next unit's tile loops are done
    oh[0] = oh[1] = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = tid + k * kThreads;
      if (idx < g * D) oh[k >> 1] |= (uint32_t)out_at(idx) << (16 * (k & 1));
    }
    oh_ok = true;
  } else {
    for (int idx = tid; idx < g * D; idx += kThreads) ob[idx] = out_at(idx);
  }
  // the row count of the range's (layer, sequence), once its first kv head
  // is done (written last: no store in flight at the next unit's start)
  if (MASS && tid == 0 && u == u_end - 1 && h_first == 0 && sj == 0)
    meta[CONFK_META_MASSROWS] = ACC ? unit_owner((uint32_t)(lb * H + H - 1), P) - wg + 1 : H;
  if constexpr (ACC) __syncthreads();  // the next unit reuses the LDS
  };
  if constexpr (ACC) {
    // written out once per unit rather than as a loop: a loop keeps values
    // live across its back edge and spills registers in the tile loops
    // a two-unit range starts at an even kv head (hkv is even, ranges
    // start at even units), so both units share the (layer, sequence)
    static_assert(kAccUnits == 2, "the units are written out below");
    if (u_end - u_begin == 2) unit_body(u_begin, std::true_type{}, std::false_type{});  // uniform
    unit_body(u_end - 1, std::false_type{}, std::false_type{});
  } else if constexpr (SPILL) {
    // the spill form only for a unit whose score slots (INT8 tiles, then
    // FP16 tiles with the new token) pass the LDS budget: a capacity that
    // needs the spill area says nothing of the current length
    const int32_t* mt = c.meta + ((a.layer0 + l) * c.B + b) * CONFK_META_WORDS;
    const int n0 = mt[CONFK_META_N], n80 = mt[CONFK_META_N8];
    int64_t slots = (int64_t)((n80 + 15) >> 4) * 16 + (int64_t)((n0 - n80 + 1 + 15) >> 4) * 16;
    if (SPLIT && n80 >= 0 && n80 <= n0 && n0 < c.cap) {  // this split's slots (a bad header fails in the body)
      const SplitRange sr = split_range(n0, n80, a.split, a.split_tiles, sj);
      slots = (int64_t)(sr.t8b - sr.t8a) * 16 + (sr.fp ? (int64_t)((n0 - n80 + 1 + 15) >> 4) * 16 : 0);
    }
    if (slots <= a.n_lds)  // uniform
      unit_body(u_begin, std::false_type{}, std::false_type{});
    else
      unit_body(u_begin, std::false_type{}, std::true_type{});
  } else {
    unit_body(u_begin, std::false_type{}, std::false_type{});
  }
}

}  // namespace

size_t attention_xchg_bytes(int64_t units, int g, int d) {
  return units >= 1 ? (size_t)std::min<int64_t>(units, kSplitMaxUnits) * split_words(g, d) * 8 : 0;
}

int attention_lds_bytes(int d, int g, int n_lds) {
  // scores / output reduction, the query, K and V scales
  return 4 * score_area_floats(d, g, n_lds) + 2 * g * d + 8 * d;
}

// Score slots per head: padded INT8 tiles + padded FP16 tiles (incl. new).
static int score_slots(int cap) { return ((cap + 30 + 15) / 16) * 16; }

// Row length of the LDS score store: a multiple of 4 floats that is 4 mod 32
// (bank spread across heads).
static int bank_pad(int x) { return (x + 31) / 32 * 32 + 4; }

int attention_plan_n_lds(int d, int g, int cap, int* spill_stride) {
  const int need = score_slots(cap);
  int fit = bank_pad(kScoreLdsBytes / (4 * g) - 36);
  const int min_slots = bank_pad(kWaves * red_row(d));  // room for the output reduction
  if (fit < min_slots) fit = min_slots;
  if (bank_pad(need) <= fit) {
    *spill_stride = 0;
    return bank_pad(need);
  }
  *spill_stride = need;
  return fit;
}

namespace {

// Compute units of the current device, read once per device.
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && cus[dev]) return cus[dev];
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = 0;
  if (dev < 64) cus[dev] = v;
  return v;
}

// Resident workgroups per compute unit of a kernel at a dynamic LDS size,
// remembered per (kernel, size).
int resident_per_cu(const void* fn, int lds_bytes) {
  struct Entry {
    const void* fn;
    int lds, dev, occ;
  };
  static std::mutex mu;
  static Entry seen[32];
  static int nseen = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < nseen; ++i)
    if (seen[i].fn == fn && seen[i].lds == lds_bytes && seen[i].dev == dev) return seen[i].occ;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kThreads, (size_t)lds_bytes) != hipSuccess) occ = 0;
  seen[nseen % 32] = Entry{fn, lds_bytes, dev, occ};
  ++nseen;
  return occ;
}

#ifndef CONFK_ACC_TAIL
#define CONFK_ACC_TAIL 8
#endif
// Split keys, for launches whose units fill at most 1/32 of the resident
// workgroup slots: a unit weighing at least twice split_tiles INT8 tiles
// (an FP16 tile counts twice) is cut into pieces of at least that weight, at
// most min(kMaxSplit, 2 * slots / units) of them, and no more than the
// capacity's largest unit needs. A piece weighs at least kMinSplitTiles
// tiles (512 keys): the exchange costs two device-wide round trips, which
// shorter pieces do not repay. Measured on one-layer launches of the
// 64-layer GQA-5 shape, back to back: eight units over 32001 keys took 37
// against 460 us (unsplit, those units take the score-spill form, whose
// stores in the tile loop serialise the loads); eight units over 500-2000
// keys take about 16.5 us split or not (latency-bound); 64 units over 1966
// keys ran slower in 5 pieces (49.7 against 39.4 us), where most of the
// launch's workgroups find no piece to run and exit.
#ifndef CONFK_SPLIT_MIN_TILES
#define CONFK_SPLIT_MIN_TILES 32
#endif
constexpr int kMinSplitTiles = CONFK_SPLIT_MIN_TILES;
constexpr int kSplitTileScale = 160;

template <int D>
hipError_t launch_d(const AttnArgs& a, int lds_bytes, hipStream_t s) {
  const int64_t units = (int64_t)a.nl * a.c.B * a.c.hkv;
  const int64_t cg = a.conf_groups + a.conf_tail;  // workgroups of the fused confidence work
  const dim3 block(kThreads);
  if (a.mass && a.xchg && units <= kSplitMaxUnits) {
    // a launch that leaves resident workgroup slots idle splits its units'
    // keys over several workgroups each
    const void* fn = a.spill ? reinterpret_cast<const void*>(&attn_decode_kernel<D, true, true, false, true>)
                             : reinterpret_cast<const void*>(&attn_decode_kernel<D, false, true, false, true>);
    const int64_t slots = (int64_t)resident_per_cu(fn, lds_bytes) * device_cus();
    const int64_t tiles = std::max<int64_t>(kMinSplitTiles, kSplitTileScale * units / std::max<int64_t>(slots, 1));
    // the weight of the largest unit the capacity allows
    const int64_t wmax = (a.c.cap + 15) / 16 + 2 * ((a.c.cap16 + 15) / 16);
    const int64_t S = std::min<int64_t>({kMaxSplit, (2 * slots + units - 1) / units, (wmax + tiles - 1) / tiles});
    // (a capacity whose largest unit makes fewer than three pieces gains too
    // little to pay for the workgroups that find no piece once the cache is
    // short: the 12-unit, 1026-slot launch ran 1 us slower split)
    if (32 * units <= slots && wmax >= 3 * tiles && S >= 2) {
      AttnArgs b = a;
      b.split = (int32_t)S;
      b.split_tiles = (int32_t)tiles;
      if (a.spill)
        hipLaunchKernelGGL((attn_decode_kernel<D, true, true, false, true>), dim3(units * S + cg), block, lds_bytes, s, b);
      else
        hipLaunchKernelGGL((attn_decode_kernel<D, false, true, false, true>), dim3(units * S + cg), block, lds_bytes, s, b);
      return hipGetLastError();
    }
  }
  if (!a.mass) {
    hipLaunchKernelGGL((attn_decode_kernel<D, false, false, false>), dim3(units + cg), block, lds_bytes, s, a);
  } else if (a.spill) {
    hipLaunchKernelGGL((attn_decode_kernel<D, true, true, false>), dim3(units + cg), block, lds_bytes, s, a);
  } else {
    // At least two rounds of resident workgroups: kAccUnits kv heads per
    // workgroup with the mass summed in LDS, if the accumulator costs no
    // residency (the launch keeps at least one round).
    const int acc_bytes = lds_bytes + 4 * ((a.c.cap + 3) / 4 * 4);
    const void* plain = reinterpret_cast<const void*>(&attn_decode_kernel<D, false, true, false>);
    const void* acc = reinterpret_cast<const void*>(&attn_decode_kernel<D, false, true, true>);
    const int occ_acc = resident_per_cu(acc, acc_bytes);
    const int64_t slots = (int64_t)occ_acc * device_cus();
    const int64_t groups = (units + kAccUnits - 1) / kAccUnits;
    if (occ_acc > 0 && slots > 0 && groups >= slots && units < ((int64_t)1 << 31) && a.c.hkv % 2 == 0 &&
        occ_acc >= resident_per_cu(plain, lds_bytes)) {
      // single-unit workgroups for the last CONFK_ACC_TAIL / 8 of a round
      const int64_t tail = std::min<int64_t>(units, slots * CONFK_ACC_TAIL / 8);
      AttnArgs b = a;
      b.acc_pairs = (int32_t)((units - tail) / 2);
      const int64_t g2 = b.acc_pairs + (units - 2 * (int64_t)b.acc_pairs);
      hipLaunchKernelGGL((attn_decode_kernel<D, false, true, true>), dim3(g2 + cg), block, acc_bytes, s, b);
    } else {
      hipLaunchKernelGGL((attn_decode_kernel<D, false, true, false>), dim3(units + cg), block, lds_bytes, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& in, int lds_bytes, hipStream_t s) {
  AttnArgs a = in;
  // the fused confidence work: the merge in leading workgroups (the pass ran
  // before), or the pass in trailing ones (the merge runs after)
  a.conf_groups = a.conf_mode == kConfMerge ? (a.conf.batch + kWaves - 1) / kWaves : 0;
  a.conf_tail = a.conf_mode == kConfPass ? a.conf.nchunks * a.conf.batch : 0;
  return a.c.d == 128 ? launch_d<128>(a, lds_bytes, s) : launch_d<64>(a, lds_bytes, s);
}

}  // namespace confk

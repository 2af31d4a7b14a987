// Streaming-read probe: reads a buffer once with the load form the attention
// kernel streams its K/V tiles with (16-byte non-temporal loads, whole lines
// per instruction), so a timed launch gives the read rate HBM sustains for
// that form on this part. A measurement aid beside the decode step, not a
// step of it. The words read are folded into one XOR so that the loads stay
// live and the result can be checked exactly.
//
// Launch shape: a sweep over 1-16 loads in flight per thread and 256-16384
// workgroups (2 GiB of random data) read fastest with two four-wave
// workgroups per compute unit and four loads per thread, 7.2 TB/s; more
// bytes in flight read slower (6.3 TB/s at eight workgroups per unit, 5.4
// with 16384 one-load workgroups), and contiguous per-workgroup runs read
// as fast as interleaved blocks.
#include <hip/hip_runtime.h>

#include "confk_probe.h"

namespace confk {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // independent 16-byte loads in flight per thread
constexpr int kGrid = 512;   // two four-wave workgroups per compute unit

// Block b of the buffer is kBlock contiguous bytes (one load per thread and
// unrolled step); workgroup g reads blocks g, g + grid, g + 2 grid, ...
constexpr uint64_t kBlock = (uint64_t)kThreads * kUnroll * 16;
constexpr uint64_t kProbeBlock = 65536;  // the size granule of the entry point
static_assert(kProbeBlock % kBlock == 0, "the size granule must be whole blocks");
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* p, uint64_t nblocks,
                                                              uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    const u32x4* q = p + blk * (kThreads * kUnroll) + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(q + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t ^= red[w];
    atomicXor(sink, t);
  }
}

}  // namespace

}  // namespace confk

extern "C" int confk_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  using namespace confk;
  if (!buf || !sink || bytes == 0 || bytes % kProbeBlock != 0) return CONFK_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return CONFK_ERR_INVALID_ARG;
  const uint64_t nblocks = bytes / kBlock;
  const unsigned grid = (unsigned)(nblocks < kGrid ? nblocks : kGrid);
  read_probe_kernel<<<grid, kThreads, 0, (hipStream_t)stream>>>(reinterpret_cast<const u32x4*>(buf), nblocks,
                                                                 sink);
  return hipGetLastError() == hipSuccess ? CONFK_OK : CONFK_ERR_LAUNCH;
}

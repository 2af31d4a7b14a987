// confk_ema_compact_static: the fused EMA + compaction entry point with its
// scratch memory in a static device array instead of a caller workspace, for
// callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid device allocation).
//
// The array is a file-scope __device__ object: its name in host code is a
// host-side stand-in, not a device address. Its device address is taken once
// per device with hipGetSymbolAddress (each GPU holds its own copy at its own
// address) and only that address is passed to the kernels. Every call on a
// device shares the device's array, which keeps the last call's contents;
// the compaction kernels write every scratch word they read within the same
// call (plans, job flags, staging), so nothing has to start at zero. Calls
// that overlap on one device race on the array.
#include <mutex>

#include "confk_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // CONFK_STATIC_SCRATCH_BYTES
static_assert(kScratchBytes == CONFK_STATIC_SCRATCH_BYTES, "header and library agree on the limit");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array (set up on the first call on
// the device, with the device current).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CONFK_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CONFK_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CONFK_OK;
}

}  // namespace

extern "C" int confk_ema_compact_static(const confk_cache* cache, int32_t layer0, int32_t nlayers,
                                        const float* mass, const confk_policy* pol, int32_t t, float* score,
                                        const int32_t* budget, int32_t budget_layer_stride,
                                        const uint16_t* k_new, const uint16_t* v_new, int32_t* evicted_out,
                                        int32_t flags, void* stream) {
  if (!cache || nlayers < 1) return CONFK_ERR_INVALID_ARG;
  const size_t need = confk_workspace_size(CONFK_WS_COMPACT, cache, nlayers, 0, 0);
  if (need > kScratchBytes) return CONFK_ERR_WORKSPACE;
  void* p = nullptr;
  const int e = scratch_address(&p);
  if (e != CONFK_OK) return e;
  return confk_ema_compact(cache, layer0, nlayers, mass, pol, t, score, budget, budget_layer_stride, k_new,
                           v_new, evicted_out, flags, p, kScratchBytes, stream);
}

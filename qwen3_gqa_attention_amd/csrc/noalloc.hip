// Allocation-free decode: qwen3_attn_forward_decode with its scratch memory
// in a static device array instead of a caller-supplied workspace, for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array lives in the library's code object, so every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In host
// code the array's name is not a device address: the address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// only that pointer is handed to the kernels.  The decode kernels write every
// scratch word they later read (partial sums of the projections, per-chunk
// softmax partials), so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qwen3_attn.h"

namespace {

constexpr size_t kScratchBytes = QWEN3_ATTN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// The scratch memory of qwen3_attn_forward_decode_noalloc (one copy per GPU).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of the current device's copy of `scratch`.
qwen3_attn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QWEN3_ATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return QWEN3_ATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return QWEN3_ATTN_EHIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return QWEN3_ATTN_OK;
}

}  // namespace

extern "C" qwen3_attn_status qwen3_attn_forward_decode_noalloc(qwen3_attn_t* h,
                                                               const void* hidden,
                                                               const int32_t* positions,
                                                               void* k_cache, void* v_cache,
                                                               int64_t cache_cap, void* out,
                                                               int32_t N, void* stream) {
  if (!h) return QWEN3_ATTN_EINVAL;
  void* ws = nullptr;
  const qwen3_attn_status st = scratch_address(&ws);
  if (st != QWEN3_ATTN_OK) return st;
  // Same validation, kernels and launch order as the workspace call; a call
  // needing more than kScratchBytes is rejected there with EWORKSPACE before
  // anything is enqueued.
  return qwen3_attn_forward_decode(h, hidden, positions, k_cache, v_cache, cache_cap, out, N, ws,
                                   kScratchBytes, stream);
}

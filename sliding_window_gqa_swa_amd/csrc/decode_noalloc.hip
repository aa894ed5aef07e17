// decode_noalloc.hip -- swa_decode_step_noalloc: the fused decode step with
// its split-K scratch in a static device array instead of a caller
// workspace, for callers that cannot allocate (code under HIP graph
// capture, serving loops, harnesses that forbid allocation).
//
// The scratch array holds, at fixed offsets, the split counters
// (kNaCounterBytes) and the fp32 split partials after them.  The counters
// live in a region of their own that no partial ever overwrites, and every
// launch returns the counters it used to zero (the decode kernel's own
// reset), so they start at zero on the next call whatever its sizes.  At
// set-up (the first call on a device, once per device) the host resolves
// the array's device address with hipGetSymbolAddress and clears the
// counter region with a fill kernel on the caller's stream, ordered before
// that call's decode.  Calls that overlap on one GPU (different streams)
// share the array and race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/swa.h"
#include "swa_internal.h"

namespace {

constexpr size_t kNaScratchBytes = SWA_NOALLOC_SCRATCH_BYTES;
constexpr size_t kNaCounterBytes = 65536;  // up to 16384 split counters
static_assert(kNaScratchBytes % 256 == 0 && kNaCounterBytes % 256 == 0, "aligned regions");

// The scratch.  In host code this name is a host-side stand-in, not a
// device address: only the pointer that hipGetSymbolAddress returns (kept
// per device below) is ever handed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[kNaScratchBytes];

__global__ void na_zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kNaMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kNaMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch, resolved once per device (its
// counter region cleared on `stream` the first time); nullptr on failure.
void* scratch_ptr(hipStream_t stream, int* rc) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNaMaxDevices) {
    *rc = SWA_ELAUNCH;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p != nullptr) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
    *rc = SWA_ELAUNCH;
    return nullptr;
  }
  const int words = (int)(kNaCounterBytes / 4);
  hipLaunchKernelGGL(na_zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                     (uint32_t*)q, words);
  if (hipGetLastError() != hipSuccess) {
    *rc = SWA_ELAUNCH;
    return nullptr;
  }
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

bool ok16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

SWA_API int swa_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                    void* k_ring, void* v_ring, int32_t* ring_meta,
                                    int32_t window, void* out, int32_t batch, int32_t ring_rows,
                                    int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                                    float scale, void* stream) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return SWA_EINVAL;
  if (batch < 0 || window < 1 || ring_rows <= window) return SWA_EINVAL;
  if (ring_rows > SWA_MAX_RING_ROWS) return SWA_EUNSUPPORTED;
  if (!swa::head_dim_supported(d)) return SWA_EUNSUPPORTED;
  if (dtype != SWA_BF16 && dtype != SWA_F32) return SWA_EUNSUPPORTED;
  if (batch == 0) return SWA_OK;
  if (!ok16(q) || !ok16(k_new) || !ok16(v_new) || !ok16(k_ring) || !ok16(v_ring) ||
      !ok16(ring_meta) || !ok16(out))
    return SWA_EINVAL;
  swa::DecodePlan plan = swa::plan_decode(batch, hq, hkv, d, ring_rows);
  // the same kernels as swa_decode_step; only the counter region is fixed
  if (plan.counter_bytes > kNaCounterBytes ||
      plan.workspace_bytes - plan.counter_bytes > kNaScratchBytes - kNaCounterBytes)
    return SWA_ESCRATCH;
  plan.workspace_bytes = plan.workspace_bytes - plan.counter_bytes + kNaCounterBytes;
  plan.counter_bytes = kNaCounterBytes;
  if (!(scale > 0.f)) scale = 1.0f / __builtin_sqrtf((float)d);
  int rc = SWA_OK;
  void* ws = scratch_ptr((hipStream_t)stream, &rc);
  if (ws == nullptr) return rc;
  return swa::launch_decode(q, k_new, v_new, k_ring, v_ring, ring_meta, window, out, batch,
                            ring_rows, hq, hkv, d, dtype, scale, ws, plan, (hipStream_t)stream);
}

}  // extern "C"

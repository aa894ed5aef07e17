// capi.cpp -- the extern "C" entry points of libswa (declared in swa.h).
//
// Every entry point validates its arguments on the host first and returns a
// negative code before touching the HIP runtime when one is wrong, so the
// checks are testable on a machine without a GPU.  The library allocates
// nothing and keeps no state; all buffers belong to the caller.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/swa.h"
#include "swa_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// head dimensions of every entry point (swa::head_dim_supported)
bool supported_d(int32_t d) { return swa::head_dim_supported(d); }
bool supported_prefill_d(int32_t d) { return supported_d(d); }

size_t elem_size(int32_t dtype) { return dtype == SWA_BF16 ? 2 : 4; }

// Shared checks of the head geometry and element type.
int check_heads(int32_t hq, int32_t hkv, int32_t d, int32_t dtype, bool prefill = false) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return SWA_EINVAL;
  if (!(prefill ? supported_prefill_d(d) : supported_d(d))) return SWA_EUNSUPPORTED;
  if (dtype != SWA_BF16 && dtype != SWA_F32) return SWA_EUNSUPPORTED;
  return SWA_OK;
}

int check_ring(int32_t window, int32_t batch, int32_t ring_rows, int32_t hkv,
               int32_t d, int32_t dtype) {
  if (batch < 0 || hkv <= 0 || window < 1) return SWA_EINVAL;
  if (ring_rows <= window) return SWA_EINVAL;
  if (ring_rows > SWA_MAX_RING_ROWS) return SWA_EUNSUPPORTED;
  if (!supported_d(d)) return SWA_EUNSUPPORTED;
  if (dtype != SWA_BF16 && dtype != SWA_F32) return SWA_EUNSUPPORTED;
  return SWA_OK;
}

bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }

}  // namespace

namespace swa {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace swa

extern "C" {

SWA_API const char* swa_strerror(int code) {
  switch (code) {
    case SWA_OK:
      return "ok";
    case SWA_EINVAL:
      return "invalid argument (null or misaligned pointer, or bad size)";
    case SWA_EUNSUPPORTED:
      return "unsupported head dimension, element type, mode or size";
    case SWA_ELAUNCH:
      return "the HIP runtime refused a kernel launch";
    case SWA_EWORKSPACE:
      return "workspace missing or smaller than swa_decode_workspace_bytes()";
    case SWA_ESCRATCH:
      return "sizes need more split-K scratch than the static array of "
             "swa_decode_step_noalloc holds (use swa_decode_step with a workspace)";
    default:
      return "unknown error code";
  }
}

SWA_API int swa_prefill(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens,
                        const int32_t* doc_or_block_ids, int32_t window,
                        int32_t causal_mode, void* out, int32_t total_tokens,
                        int32_t num_docs, int32_t hq, int32_t hkv, int32_t d,
                        int32_t dtype, float scale, void* stream) {
  // a whole prompt is the chunk that covers every key of its document
  return swa_prefill_chunk(q, k, v, cu_seqlens, cu_seqlens, doc_or_block_ids, window,
                           causal_mode, out, total_tokens, total_tokens, num_docs, hq, hkv, d,
                           dtype, scale, stream);
}

}  // extern "C"

namespace {

// swa_prefill_chunk with an optional per-row log-sum-exp output
int prefill_impl(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                 const int32_t* cu_seqlens_k, const int32_t* doc_or_block_ids, int32_t window,
                 int32_t causal_mode, void* out, float* lse, int32_t total_q, int32_t total_k,
                 int32_t num_docs, int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                 float scale, void* stream) {
  int rc = check_heads(hq, hkv, d, dtype, true);
  if (rc) return rc;
  if (total_q < 0 || total_k < 0 || num_docs < 0) return SWA_EINVAL;
  if (causal_mode != SWA_CAUSAL && causal_mode != SWA_BLOCKWISE) return SWA_EUNSUPPORTED;
  if (total_q == 0) return SWA_OK;  // nothing to compute
  if (num_docs < 1 || total_k < 1) return SWA_EINVAL;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out)) return SWA_EINVAL;
  if (cu_seqlens_q == nullptr || ((uintptr_t)cu_seqlens_q & 3u)) return SWA_EINVAL;
  if (cu_seqlens_k == nullptr || ((uintptr_t)cu_seqlens_k & 3u)) return SWA_EINVAL;
  if (causal_mode == SWA_BLOCKWISE &&
      (doc_or_block_ids == nullptr || ((uintptr_t)doc_or_block_ids & 3u)))
    return SWA_EINVAL;
  // element offsets stay below 2^63; token indices below 2^31
  if ((int64_t)total_q * hq * d >= (int64_t)1 << 62 ||
      (int64_t)total_k * hkv * d >= (int64_t)1 << 62)
    return SWA_EUNSUPPORTED;
  if (!(scale > 0.f)) scale = 1.0f / __builtin_sqrtf((float)d);
  swa::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.ids = causal_mode == SWA_BLOCKWISE ? doc_or_block_ids : nullptr;
  a.window = window;
  a.mode = causal_mode;
  a.out = out;
  a.lse = lse;
  a.total_q = total_q;
  a.total_k = total_k;
  a.num_docs = num_docs;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.dtype = dtype;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  return swa::launch_prefill(a);
}

}  // namespace

extern "C" {

SWA_API int swa_prefill_chunk(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              const int32_t* doc_or_block_ids, int32_t window,
                              int32_t causal_mode, void* out, int32_t total_q,
                              int32_t total_k, int32_t num_docs, int32_t hq, int32_t hkv,
                              int32_t d, int32_t dtype, float scale, void* stream) {
  return prefill_impl(q, k, v, cu_seqlens_q, cu_seqlens_k, doc_or_block_ids, window,
                      causal_mode, out, nullptr, total_q, total_k, num_docs, hq, hkv, d, dtype,
                      scale, stream);
}

SWA_API int swa_prefill_lse(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, const int32_t* doc_or_block_ids,
                            int32_t window, int32_t causal_mode, void* out, float* lse,
                            int32_t total_tokens, int32_t num_docs, int32_t hq, int32_t hkv,
                            int32_t d, int32_t dtype, float scale, void* stream) {
  if (total_tokens > 0 && (lse == nullptr || ((uintptr_t)lse & 3u))) return SWA_EINVAL;
  return prefill_impl(q, k, v, cu_seqlens, cu_seqlens, doc_or_block_ids, window, causal_mode,
                      out, lse, total_tokens, total_tokens, num_docs, hq, hkv, d, dtype, scale,
                      stream);
}

SWA_API size_t swa_prefill_backward_workspace_bytes(int32_t total_tokens, int32_t hq) {
  if (total_tokens < 0 || hq <= 0) return 0;
  return swa::bwd_workspace_bytes(total_tokens, hq);
}

SWA_API int swa_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                                 const void* dout, const int32_t* cu_seqlens,
                                 const int32_t* doc_or_block_ids, int32_t window,
                                 int32_t causal_mode, const float* lse, void* dq, void* dk,
                                 void* dv, int32_t total_tokens, int32_t num_docs, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t dtype, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(hq, hkv, d, dtype, true);
  if (rc) return rc;
  if (!swa::bwd_supported(d, dtype)) return SWA_EUNSUPPORTED;
  if (total_tokens < 0 || num_docs < 0) return SWA_EINVAL;
  if (causal_mode != SWA_CAUSAL && causal_mode != SWA_BLOCKWISE) return SWA_EUNSUPPORTED;
  if (total_tokens == 0) return SWA_OK;  // nothing to compute
  if (num_docs < 1) return SWA_EINVAL;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out) || !ptr_ok(dout) || !ptr_ok(dq) ||
      !ptr_ok(dk) || !ptr_ok(dv))
    return SWA_EINVAL;
  if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3u)) return SWA_EINVAL;
  if (causal_mode == SWA_BLOCKWISE &&
      (doc_or_block_ids == nullptr || ((uintptr_t)doc_or_block_ids & 3u)))
    return SWA_EINVAL;
  if ((uintptr_t)lse & 3u) return SWA_EINVAL;
  // tile offsets (64 rows of hq * d elements) stay below 2^31 bytes
  if ((int64_t)hq * d >= ((int64_t)1 << 22) ||
      (int64_t)total_tokens * hq * d >= (int64_t)1 << 62)
    return SWA_EUNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < swa::bwd_workspace_bytes(total_tokens, hq))
    return SWA_EWORKSPACE;
  if (!(scale > 0.f)) scale = 1.0f / __builtin_sqrtf((float)d);
  swa::PrefillBwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.cu = cu_seqlens;
  a.ids = causal_mode == SWA_BLOCKWISE ? doc_or_block_ids : nullptr;
  a.window = window;
  a.mode = causal_mode;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.total = total_tokens;
  a.num_docs = num_docs;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.dtype = dtype;
  a.scale = scale;
  a.lse = lse;
  a.workspace = workspace;
  a.stream = (hipStream_t)stream;
  return swa::launch_prefill_bwd(a);
}

SWA_API size_t swa_decode_workspace_bytes(int32_t batch, int32_t hq,
                                          int32_t hkv, int32_t d,
                                          int32_t ring_rows) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || !supported_d(d) ||
      ring_rows <= 0 || ring_rows > SWA_MAX_RING_ROWS)
    return 0;
  return swa::plan_decode(batch, hq, hkv, d, ring_rows).workspace_bytes;
}

SWA_API int swa_decode(const void* q, const void* k_ring, const void* v_ring,
                       const int32_t* ring_meta, int32_t window, void* out,
                       int32_t batch, int32_t ring_rows, int32_t hq,
                       int32_t hkv, int32_t d, int32_t dtype, float scale,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(hq, hkv, d, dtype);
  if (rc) return rc;
  rc = check_ring(window, batch, ring_rows, hkv, d, dtype);
  if (rc) return rc;
  if (batch == 0) return SWA_OK;
  if (!ptr_ok(q) || !ptr_ok(k_ring) || !ptr_ok(v_ring) || !ptr_ok(ring_meta) || !ptr_ok(out))
    return SWA_EINVAL;
  const swa::DecodePlan plan = swa::plan_decode(batch, hq, hkv, d, ring_rows);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < plan.workspace_bytes)
    return SWA_EWORKSPACE;
  if (!(scale > 0.f)) scale = 1.0f / __builtin_sqrtf((float)d);
  // (decode only: the kernel reads the rings and ring_meta and writes neither)
  return swa::launch_decode(q, nullptr, nullptr, const_cast<void*>(k_ring),
                            const_cast<void*>(v_ring), const_cast<int32_t*>(ring_meta), window,
                            out, batch, ring_rows, hq, hkv, d, dtype, scale, workspace, plan,
                            (hipStream_t)stream);
}

SWA_API int swa_decode_step(const void* q, const void* k_new, const void* v_new,
                            void* k_ring, void* v_ring, int32_t* ring_meta, int32_t window,
                            void* out, int32_t batch, int32_t ring_rows, int32_t hq,
                            int32_t hkv, int32_t d, int32_t dtype, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_heads(hq, hkv, d, dtype);
  if (rc) return rc;
  rc = check_ring(window, batch, ring_rows, hkv, d, dtype);
  if (rc) return rc;
  if (batch == 0) return SWA_OK;
  if (!ptr_ok(q) || !ptr_ok(k_new) || !ptr_ok(v_new) || !ptr_ok(k_ring) || !ptr_ok(v_ring) ||
      !ptr_ok(ring_meta) || !ptr_ok(out))
    return SWA_EINVAL;
  const swa::DecodePlan plan = swa::plan_decode(batch, hq, hkv, d, ring_rows);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < plan.workspace_bytes)
    return SWA_EWORKSPACE;
  if (!(scale > 0.f)) scale = 1.0f / __builtin_sqrtf((float)d);
  return swa::launch_decode(q, k_new, v_new, k_ring, v_ring, ring_meta, window, out, batch,
                            ring_rows, hq, hkv, d, dtype, scale, workspace, plan,
                            (hipStream_t)stream);
}

SWA_API int swa_cache_append(const void* k_new, const void* v_new,
                             void* k_ring, void* v_ring, int32_t* ring_meta,
                             int32_t batch, int32_t ring_rows, int32_t hkv,
                             int32_t d, int32_t dtype, void* stream) {
  if (batch < 0 || hkv <= 0 || ring_rows < 1 || ring_rows > SWA_MAX_RING_ROWS)
    return batch < 0 || hkv <= 0 || ring_rows < 1 ? SWA_EINVAL : SWA_EUNSUPPORTED;
  if (!supported_d(d)) return SWA_EUNSUPPORTED;
  if (dtype != SWA_BF16 && dtype != SWA_F32) return SWA_EUNSUPPORTED;
  if (batch == 0) return SWA_OK;
  if (!ptr_ok(k_new) || !ptr_ok(v_new) || !ptr_ok(k_ring) || !ptr_ok(v_ring) ||
      !ptr_ok(ring_meta))
    return SWA_EINVAL;
  return swa::launch_ring_append(k_new, v_new, k_ring, v_ring, ring_meta, batch, ring_rows,
                                 hkv, d * (int)elem_size(dtype), (hipStream_t)stream);
}

SWA_API int swa_cache_compact(const void* k_src, const void* v_src,
                              const int32_t* cu_seqlens,
                              const int32_t* prompt_lens,
                              const int32_t* left_pad, int32_t src_rows,
                              void* k_ring, void* v_ring, int32_t* ring_meta,
                              int32_t window, int32_t batch, int32_t ring_rows,
                              int32_t hkv, int32_t d, int32_t dtype,
                              void* stream) {
  int rc = check_ring(window, batch, ring_rows, hkv, d, dtype);
  if (rc) return rc;
  if (src_rows < 0) return SWA_EINVAL;
  if (batch == 0) return SWA_OK;
  if (!ptr_ok(k_ring) || !ptr_ok(v_ring) || !ptr_ok(ring_meta)) return SWA_EINVAL;
  if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3u)) return SWA_EINVAL;
  if (src_rows > 0 && (!ptr_ok(k_src) || !ptr_ok(v_src))) return SWA_EINVAL;
  if (((uintptr_t)prompt_lens & 3u) || ((uintptr_t)left_pad & 3u)) return SWA_EINVAL;
  return swa::launch_ring_compact(k_src, v_src, cu_seqlens, prompt_lens, left_pad, src_rows,
                                  k_ring, v_ring, ring_meta, window, batch, ring_rows, hkv,
                                  d * (int)elem_size(dtype), (hipStream_t)stream);
}

SWA_API int swa_cache_roll(void* k_ring, void* v_ring, int32_t* ring_meta,
                           int32_t window, int32_t batch, int32_t ring_rows,
                           int32_t hkv, int32_t d, int32_t dtype, void* stream) {
  int rc = check_ring(window, batch, ring_rows, hkv, d, dtype);
  if (rc) return rc;
  if (batch == 0) return SWA_OK;
  if (!ptr_ok(k_ring) || !ptr_ok(v_ring) || !ptr_ok(ring_meta)) return SWA_EINVAL;
  return swa::launch_ring_roll(k_ring, v_ring, ring_meta, window, batch, ring_rows, hkv,
                               d * (int)elem_size(dtype), (hipStream_t)stream);
}

}  // extern "C"

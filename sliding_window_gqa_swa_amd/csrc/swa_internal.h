// swa_internal.h -- launchers behind the C ABI (host side, C++).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

// Head sizes of every entry point: the multiples of 64 up to 512.  (Rows of
// 64 elements are whole 16-byte chunks in a count the LDS tile layout takes
// at every element size; a size with no schedule of its own runs on the
// pipelined prefill loop of the next multiple of 128, with no products over
// the padding.)
inline bool head_dim_supported(int d) { return d >= 64 && d <= 512 && d % 64 == 0; }

// Ring cache (byte copies; row_bytes = d * element size, a multiple of 16).
int launch_ring_append(const void* k_new, const void* v_new, void* k_ring,
                       void* v_ring, int32_t* meta, int batch, int ring_rows,
                       int hkv, int row_bytes, hipStream_t stream);
int launch_ring_compact(const void* k_src, const void* v_src,
                        const int32_t* cu, const int32_t* prompt_lens,
                        const int32_t* left_pad, int src_rows, void* k_ring,
                        void* v_ring, int32_t* meta, int window, int batch,
                        int ring_rows, int hkv, int row_bytes,
                        hipStream_t stream);
int launch_ring_roll(void* k_ring, void* v_ring, int32_t* meta, int window,
                     int batch, int ring_rows, int hkv, int row_bytes,
                     hipStream_t stream);

// Decode: split-K partials then a fixed-order combine.
struct DecodePlan {
  int heads_per_block;  // query heads of one kv group handled per block
  int head_blocks;      // ceil(g / heads_per_block)
  int splits;           // ring row ranges per (sequence, kv head)
  int rows_per_split;   // multiple of 32
  bool load_all;        // rows loaded before the ring state is known (small grids)
  size_t counter_bytes;  // leading region of the workspace: split counters
  size_t workspace_bytes;
};
DecodePlan plan_decode(int batch, int hq, int hkv, int d, int ring_rows);
// k_new == NULL: decode only (the rings and ring_meta are read, not
// written); otherwise a decode step (metadata roll + append + decode).
int launch_decode(const void* q, const void* k_new, const void* v_new, void* k_ring,
                  void* v_ring, int32_t* meta, int window, void* out, int batch,
                  int ring_rows, int hq, int hkv, int d, int dtype,
                  float scale, void* workspace, const DecodePlan& plan,
                  hipStream_t stream);

// Compute units of the current device (queried once per device).
int device_cu_count();

// Prefill.  Query rows are the last rows of each document's keys: cu_k ==
// cu_q (and total_k == total_q) for whole prompts, per-document longer key
// ranges for a chunk of each prompt.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* ids;  // key-indexed block ids (SWA_BLOCKWISE), else NULL
  int window, mode;
  void* out;
  float* lse;  // [hq, total_q] row log-sum-exp (natural log), or NULL
  int total_q, total_k, num_docs, hq, hkv, d, dtype;
  float scale;
  hipStream_t stream;
};
int launch_prefill(const PrefillArgs& a);

// Prefill backward (whole prompts): dq, dk, dv from q, k, v, the forward
// output and its gradient dout.
struct PrefillBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const int32_t* cu;
  const int32_t* ids;  // block ids (SWA_BLOCKWISE), else NULL
  int window, mode;
  void* dq;
  void* dk;
  void* dv;
  int total, num_docs, hq, hkv, d, dtype;
  float scale;
  const float* lse;  // [hq, T] forward row log-sum-exp, or NULL (recomputed)
  void* workspace;
  hipStream_t stream;
};
// regions of the backward's workspace
struct BwdWorkspace {
  float* lse;    // [hq, T] log2-sum-exp2 of each row's scaled scores
  float* delta;  // [hq, T] <dout, out> of each row
  int32_t* lo;   // [T] first admitted key of each row
  int32_t* hi;   // [T] last admitted key of each row
};
size_t bwd_workspace_bytes(int total, int hq);
BwdWorkspace bwd_workspace(void* base, int total, int hq);
bool bwd_supported(int d, int dtype);
int launch_prefill_bwd(const PrefillBwdArgs& a);

}  // namespace swa

// ring.hip -- compact sliding-window ring cache: append, compaction, roll.
//
// Pages cited (title; section):
//   [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
//            variants" (torch-spyre/hf-adapters pull request 496)
//   [BONSAI] "Gemma3 Local Attention Cache" (jax-ml/bonsai issue 124)
//
// State per sequence b: ring_meta[b] = {pos, anchor, start, lo}; position p
// (anchor <= p < anchor + R) lives at physical row (start + p - anchor) mod R.
// All three operations are byte copies of whole rows (16-byte chunks), so
// one kernel serves every element type.  Every row index is derived as a
// remainder modulo R or checked against the host-given sizes, so malformed
// device-resident metadata cannot send an access outside the buffers.
#include "swa_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kRingThreads = 256;

// Append: one block per sequence so that every kv head reads the old pos
// before thread 0 advances it ([SPYRE] Summary: writes go through the
// compact cache index; [BONSAI] Step 2: the index wraps modulo the ring).
__global__ __launch_bounds__(kRingThreads) void ring_append_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    u32x4* __restrict__ k_ring, u32x4* __restrict__ v_ring,
    int32_t* __restrict__ meta, int R, int hkv, int cpr) {
  const int b = blockIdx.x;
  int32_t* m = meta + 4 * (size_t)b;
  const int64_t pos = m[0], anchor = m[1], start = m[2];
  const int64_t p = pos + 1;
  const int64_t off = p - anchor;
  const bool refuse = off >= R || off < 0;  // full ring, or inconsistent state
  if (!refuse) {
    const int64_t slot = pos_mod(start + off, R);
    const int per = hkv * cpr;
    for (int c = threadIdx.x; c < 2 * per; c += kRingThreads) {
      const bool isv = c >= per;
      const int cc = isv ? c - per : c;
      const int h = cc / cpr, q = cc - h * cpr;
      const size_t src = ((size_t)b * hkv + h) * cpr + q;
      const size_t dst = (((size_t)b * hkv + h) * R + slot) * cpr + q;
      if (isv)
        v_ring[dst] = v_new[src];
      else
        k_ring[dst] = k_new[src];
    }
  }
  __syncthreads();  // all reads of m[] above happen before the update below
  if (threadIdx.x == 0) {
    if (refuse)
      m[3] = m[3] | SWA_META_ERR;
    else
      m[0] = (int32_t)p;
  }
}

// Compaction ([SPYRE] Summary: prompt-sized cache -> window + slack rows at
// the first decode; short prompts handled).  Grid: (row blocks, kv head, b).
// Every block derives the sequence's state from the inputs alone (never
// from ring_meta), so blocks need no ordering; block (0, 0, b) writes meta.
__global__ __launch_bounds__(kRingThreads) void ring_compact_kernel(
    const u32x4* __restrict__ k_src, const u32x4* __restrict__ v_src,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ prompt_lens,
    const int32_t* __restrict__ left_pad, int src_rows,
    u32x4* __restrict__ k_ring, u32x4* __restrict__ v_ring,
    int32_t* __restrict__ meta, int W, int R, int hkv, int cpr,
    int rows_per_block) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int r0 = blockIdx.x * rows_per_block;
  const int64_t c0 = cu[b], c1 = cu[b + 1];
  const int64_t n = c1 - c0;
  const int64_t L = prompt_lens ? (int64_t)prompt_lens[b] : n;
  const int64_t lo = left_pad ? (int64_t)left_pad[b] : 0;
  const int64_t need = max(lo, max(L - W + 1, (int64_t)0));
  const bool ok = c0 >= 0 && c1 >= c0 && c1 <= src_rows && L >= 1 && n <= L &&
                  lo >= 0 && lo < L && L - n <= need;
  const int64_t anchor = L - W;
  const int64_t start = pos_mod(anchor, R);
  const int64_t first = max(anchor, max((int64_t)0, L - n));
  if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0) {
    int32_t* m = meta + 4 * (size_t)b;
    m[0] = (int32_t)(L - 1);
    m[1] = (int32_t)anchor;
    m[2] = (int32_t)start;
    m[3] = (int32_t)lo | (ok ? 0 : SWA_META_ERR);
  }
  const int per = rows_per_block * cpr;
  for (int c = threadIdx.x; c < 2 * per; c += kRingThreads) {
    const bool isv = c >= per;
    const int cc = isv ? c - per : c;
    const int r = r0 + cc / cpr, q = cc % cpr;
    if (r >= R) continue;
    const int64_t a = anchor + pos_mod((int64_t)r - start, R);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (ok && a >= first && a <= L - 1) {
      const int64_t srow = c0 + (a - (L - n));  // in [c0, c1) by construction
      const size_t si = ((size_t)srow * hkv + h) * cpr + q;
      val = isv ? v_src[si] : k_src[si];
    }
    const size_t di = (((size_t)b * hkv + h) * R + r) * cpr + q;
    if (isv)
      v_ring[di] = val;
    else
      k_ring[di] = val;
  }
}

// Roll ([SPYRE] Summary: every slack-count decode tokens the compact caches
// are rolled with offset-aware device copies).  In place rotation left by
// A rows: new[r] = old[(r + A) mod R].  The permutation splits into
// gcd(A, R) cycles; one thread owns one (cycle, 16-byte column chunk) of one
// (sequence, kv head, K or V) ring and walks it, so no two threads touch
// the same bytes.  Lanes run along the chunks of a row: coalesced rows.
constexpr int kRollBatch = 16;

__global__ __launch_bounds__(kRingThreads) void ring_roll_kernel(
    u32x4* k_ring, u32x4* v_ring,  // read and written in place: no restrict
    const int32_t* __restrict__ meta, int R, int A, int ncycles, int cyc_len,
    int hkv, int cpr, int64_t total) {
  const int64_t t = (int64_t)blockIdx.x * kRingThreads + threadIdx.x;
  if (t >= total) return;
  const int q = (int)(t % cpr);
  int64_t rest = t / cpr;
  const int cyc = (int)(rest % ncycles);
  rest /= ncycles;
  const int isv = (int)(rest % 2);
  rest /= 2;
  const int h = (int)(rest % hkv);
  const int b = (int)(rest / hkv);
  const int32_t* m = meta + 4 * (size_t)b;
  if ((int64_t)m[0] + 1 - (int64_t)m[1] < R) return;  // ring not full
  u32x4* base = (isv ? v_ring : k_ring) + ((size_t)b * hkv + h) * (size_t)R * cpr + q;
  // cycle rows: r_k = (cyc + k * A) mod R, k = 0 .. cyc_len - 1
  const u32x4 save = base[(size_t)cyc * cpr];
  int r_cur = cyc;
  int k = 0;
  while (k < cyc_len - 1) {
    const int nb = min(kRollBatch, cyc_len - 1 - k);
    u32x4 vals[kRollBatch];
    int rows[kRollBatch + 1];
    rows[0] = r_cur;
    int r = r_cur;
#pragma unroll
    for (int i = 0; i < kRollBatch; ++i) {
      if (i < nb) {
        r += A;
        if (r >= R) r -= R;
        rows[i + 1] = r;
        vals[i] = base[(size_t)r * cpr];  // old[r_{k+i+1}], not yet overwritten
      }
    }
#pragma unroll
    for (int i = 0; i < kRollBatch; ++i)
      if (i < nb) base[(size_t)rows[i] * cpr] = vals[i];  // new[r_{k+i}]
    r_cur = r;  // == r_{k+nb}
    k += nb;
  }
  base[(size_t)r_cur * cpr] = save;  // new[r_{len-1}] = old[r_0]
}

// Second half of the roll: advance the anchor of every rolled sequence.
// A separate launch, so every roll thread has read the old anchor first.
__global__ __launch_bounds__(kRingThreads) void ring_roll_commit_kernel(
    int32_t* __restrict__ meta, int batch, int R, int A) {
  const int b = blockIdx.x * kRingThreads + threadIdx.x;
  if (b >= batch) return;
  int32_t* m = meta + 4 * (size_t)b;
  if ((int64_t)m[0] + 1 - (int64_t)m[1] >= R) m[1] = m[1] + A;
}

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

}  // namespace

int launch_ring_append(const void* k_new, const void* v_new, void* k_ring,
                       void* v_ring, int32_t* meta, int batch, int ring_rows,
                       int hkv, int row_bytes, hipStream_t stream) {
  const int cpr = row_bytes / 16;
  hipLaunchKernelGGL(ring_append_kernel, dim3(batch), dim3(kRingThreads), 0,
                     stream, (const u32x4*)k_new, (const u32x4*)v_new,
                     (u32x4*)k_ring, (u32x4*)v_ring, meta, ring_rows, hkv, cpr);
  return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ELAUNCH;
}

int launch_ring_compact(const void* k_src, const void* v_src,
                        const int32_t* cu, const int32_t* prompt_lens,
                        const int32_t* left_pad, int src_rows, void* k_ring,
                        void* v_ring, int32_t* meta, int window, int batch,
                        int ring_rows, int hkv, int row_bytes,
                        hipStream_t stream) {
  const int cpr = row_bytes / 16;
  // ~4 KB of each of K and V per block
  int rows_per_block = 4096 / row_bytes;
  if (rows_per_block < 1) rows_per_block = 1;
  dim3 grid((ring_rows + rows_per_block - 1) / rows_per_block, hkv, batch);
  hipLaunchKernelGGL(ring_compact_kernel, grid, dim3(kRingThreads), 0, stream,
                     (const u32x4*)k_src, (const u32x4*)v_src, cu, prompt_lens,
                     left_pad, src_rows, (u32x4*)k_ring, (u32x4*)v_ring, meta,
                     window, ring_rows, hkv, cpr, rows_per_block);
  return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ELAUNCH;
}

int launch_ring_roll(void* k_ring, void* v_ring, int32_t* meta, int window,
                     int batch, int ring_rows, int hkv, int row_bytes,
                     hipStream_t stream) {
  const int cpr = row_bytes / 16;
  const int A = ring_rows - window;
  const int ncycles = gcd_int(A, ring_rows);
  const int cyc_len = ring_rows / ncycles;
  const int64_t total = (int64_t)batch * hkv * 2 * ncycles * cpr;
  const int64_t blocks = (total + kRingThreads - 1) / kRingThreads;
  if (blocks > 0x7fffffffLL) return SWA_EUNSUPPORTED;
  hipLaunchKernelGGL(ring_roll_kernel, dim3((unsigned)blocks),
                     dim3(kRingThreads), 0, stream, (u32x4*)k_ring,
                     (u32x4*)v_ring, (const int32_t*)meta, ring_rows, A,
                     ncycles, cyc_len, hkv, cpr, total);
  if (hipGetLastError() != hipSuccess) return SWA_ELAUNCH;
  hipLaunchKernelGGL(ring_roll_commit_kernel,
                     dim3((batch + kRingThreads - 1) / kRingThreads),
                     dim3(kRingThreads), 0, stream, meta, batch, ring_rows, A);
  return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ELAUNCH;
}

}  // namespace swa

// prefill_bwd.hip -- host launchers of the prefill backward (bwd_kernel.h).
#include "prefill_bwd_launch.h"

namespace swa {

namespace {

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Per-row key intervals: lo[i] = max(doc start, i - W + 1) (doc start when
// W <= 0); hi[i] = i, or the last token of i's image run when i is an image
// token in blockwise mode (a run: consecutive tokens of one document with
// the same non-negative id).  One wave per 64 rows; a run that continues
// past the wave's rows is followed 64 tokens per step.
__global__ __launch_bounds__(256) void bwd_rows_kernel(const int32_t* __restrict__ cu, int ndocs,
                                                       const int32_t* __restrict__ ids, int W,
                                                       int mode, int T, int32_t* __restrict__ lo_out,
                                                       int32_t* __restrict__ hi_out) {
  const int lane = threadIdx.x & 63;
  const int base = ((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * 64;
  if (base >= T) return;  // uniform per wave
  const int i = base + lane;
  const bool valid = i < T;
  int ds = i, de = i + 1;
  if (valid) {
    int a = 0, b = ndocs + 1;  // first d with cu[d] > i
    while (a < b) {
      const int m = (a + b) >> 1;
      if (cu[m] > i) b = m; else a = m + 1;
    }
    const int d = a - 1;
    if (d >= 0 && d < ndocs) {
      ds = cu[d];
      de = cu[d + 1];
    }
    ds = min(max(ds, 0), i);  // clamps against malformed offsets
    de = max(min(de, T), i + 1);
  }
  const int lo = W > 0 ? max(ds, i - W + 1) : ds;
  int hi = i;
  if (mode == SWA_BLOCKWISE) {
    const int id = valid ? ids[i] : -1;
    const bool last = !valid || i + 1 >= de || ids[i + 1] != id;
    const unsigned long long bal = __ballot(last);
    const unsigned long long mine = bal & (~0ull << lane);
    int end = mine ? base + __builtin_ctzll(mine) : -1;
    // lanes with no run end at or after them share lane 63's open run
    if (__ballot(valid && id >= 0 && end < 0)) {
      const int rid = __builtin_amdgcn_readlane(id, 63);
      const int rde = __builtin_amdgcn_readlane(de, 63);
      int t0 = base + 64, found = -1;
      while (found < 0) {  // ends: t >= rde stops the run
        const int t = t0 + lane;
        const bool stop = t >= rde || ids[t] != rid;
        const unsigned long long m = __ballot(stop);
        if (m) found = t0 + __builtin_ctzll(m) - 1;
        t0 += 64;
      }
      if (end < 0) end = found;
    }
    if (valid && id >= 0) hi = end;
  }
  if (valid) {
    lo_out[i] = lo;
    hi_out[i] = hi;
  }
}


size_t bwd_workspace_bytes(int total, int hq) {
  const size_t t = (size_t)(total > 0 ? total : 0);
  // lse2 and delta [hq, T] fp32, lo and hi [T] int32, each padded for the
  // 16-byte metadata loads that read a few entries past the end
  return 2 * round256((size_t)hq * t * 4 + 16) + 2 * round256(t * 4 + 16);
}

BwdWorkspace bwd_workspace(void* base, int total, int hq) {
  const size_t t = (size_t)total;
  unsigned char* p = (unsigned char*)base;
  BwdWorkspace w;
  w.lse = (float*)p;
  p += round256((size_t)hq * t * 4 + 16);
  w.delta = (float*)p;
  p += round256((size_t)hq * t * 4 + 16);
  w.lo = (int32_t*)p;
  p += round256(t * 4 + 16);
  w.hi = (int32_t*)p;
  return w;
}

bool bwd_supported(int d, int dtype) {
  (void)dtype;  // (fp32 at D = 512: the dq kernel spills 27 registers, correct but slow)
  return head_dim_supported(d);
}

int launch_prefill_bwd(const PrefillBwdArgs& a) {
  const BwdWorkspace w = bwd_workspace(a.workspace, a.total, a.hq);
  const int T_ = a.total;
  hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)((T_ + 255) / 256)), dim3(256), 0, a.stream,
                     a.cu, a.num_docs, a.ids, a.window, a.mode, T_, w.lo, w.hi);
  switch (a.d) {
    case 64:
      return launch_bwd_d64(a, w);
    case 128:
      return launch_bwd_d128(a, w);
    case 192:
      return launch_bwd_d192(a, w);
    case 256:
      return launch_bwd_d256(a, w);
    case 320:
      return launch_bwd_d320(a, w);
    case 384:
      return launch_bwd_d384(a, w);
    case 448:
      return launch_bwd_d448(a, w);
    case 512:
      return launch_bwd_d512(a, w);
    default:
      return SWA_EUNSUPPORTED;
  }
}

}  // namespace swa

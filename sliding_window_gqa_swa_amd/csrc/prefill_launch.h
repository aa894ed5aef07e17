// prefill_launch.h -- host launcher template for prefill_fwd_kernel.
#pragma once

#include "prefill_kernel.h"
#include "swa_internal.h"

#include <algorithm>

namespace swa {

// DM: the head size in memory (D > DM: computed zero-padded to D, see the
// kernel)
template <int D, typename T, int MB, int BN, int NW, int GH, bool PL = false, int DM = D>
int launch_prefill_cfg(const PrefillArgs& a) {
  using G = PfGeom<D, T, MB, BN, NW, GH, PL>;
  const int ntiles = (a.total_q + G::BM - 1) / G::BM;
  const int hq = a.hq, hkv = a.hkv;
  const int g = hq / hkv;
  const long long nwork = (long long)ntiles * hkv * (g / GH);
  const long long per_xcd = (nwork + 7) / 8;  // 8 XCDs, blocks round-robin over them
  if (8 * per_xcd > 0x7fffffffLL) return SWA_EUNSUPPORTED;
  // the pipelined kernel runs up to two items per work-group: as many
  // work-groups per XCD as its CUs hold at once (the kernel's occupancy), or
  // half the items when there are more
  int slots = (int)per_xcd, colocated = 0;
  // A window shorter than the average document makes most work items cost
  // the same (a full window of key tiles): then every work-group takes one
  // item, so that the items of an XCD start and end in cohorts that stream
  // the same key tiles through its L2 (the rotated visit order in the
  // kernel aligns them); pairing a long and a short item would stagger the
  // cohorts.
  const bool window_bound = a.window > 0 && (long long)a.window * a.num_docs < a.total_k;
  if (PL && !window_bound) {
    constexpr int kWgPerCu = (NW == 4 && D <= 128 && !std::is_same<T, float>::value) ? 2 : 1;
    const long long fill = (long long)kWgPerCu * (device_cu_count() / 8);
    slots = (int)std::min<long long>(per_xcd, std::max<long long>(fill, (per_xcd + 1) / 2));
    slots = std::max(slots, 1);
    colocated = kWgPerCu == 2 && slots == fill;  // two work-groups on every CU
  }
  // (the variant that stores the row log-sum-exp is a separate kernel, so
  // that its extra live values cost the plain forward no registers)
  auto kern = a.lse != nullptr ? prefill_fwd_kernel<D, T, MB, BN, NW, GH, PL, true, DM>
                               : prefill_fwd_kernel<D, T, MB, BN, NW, GH, PL, false, DM>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(8 * slots)), dim3(G::NT), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, a.cu_q, a.cu_k, a.num_docs,
                     a.ids, a.window, a.mode, (T*)a.out, a.lse, a.total_q, a.total_k, hq, hkv,
                     a.scale * kPrefillLog2e, ntiles, (int)nwork, (int)per_xcd, slots,
                     colocated);
  return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ELAUNCH;
}

// One translation unit per head dimension keeps compile times parallel.
int launch_prefill_d64(const PrefillArgs& a);
int launch_prefill_d128(const PrefillArgs& a);
int launch_prefill_d192(const PrefillArgs& a);
int launch_prefill_d256(const PrefillArgs& a);
int launch_prefill_d320(const PrefillArgs& a);
int launch_prefill_d384(const PrefillArgs& a);
int launch_prefill_d448(const PrefillArgs& a);
int launch_prefill_d512(const PrefillArgs& a);

}  // namespace swa

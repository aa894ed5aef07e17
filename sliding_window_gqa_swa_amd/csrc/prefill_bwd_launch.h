// prefill_bwd_launch.h -- host launcher template of the prefill backward
// (bwd_kernel.h); one translation unit per head size instantiates it.
#pragma once

#include "bwd_kernel.h"
#include "swa_internal.h"

#include <algorithm>

namespace swa {

// 16-row blocks per dq wave: one at every head size (at D = 128 the 16-row
// wave lets two work-groups share each CU: 147 us against 187 us for
// 32-row waves with one work-group per CU, measured; larger D have no
// registers for 32 rows)
template <int D, typename T>
constexpr int dq_mb() {
  return 1;
}

// dk/dv kernel shape per head size: DS waves per key block (each one part
// of d), KB 16-key blocks per wave, BQ query rows per tile; chosen so that
// one wave's fragments and accumulators fit its registers and the stages
// plus the partial-sum exchange fit the LDS
template <int D, typename T>
struct DkdvCfg {
  static constexpr bool F = std::is_same<T, float>::value;
  static constexpr int DS = F ? (D >= 256 ? 2 : 1) : (D >= 384 || D == 256 ? 2 : 1);
  // (two key blocks per wave halve the LDS reads per product but cost the
  // second wave per SIMD: 241 vs 197 us at D = 128, measured)
  static constexpr int KB = 1;
  static constexpr int BQ = (!F && D <= 256) ? 32 : 0;  // 0: the default tile
  static constexpr int NW = (!F && D == 256) ? 8 : 4;   // waves per work-group
};

template <int D, typename T>
inline int launch_bwd_cfg(const PrefillBwdArgs& a, const BwdWorkspace& w) {
  constexpr int MB = dq_mb<D, T>();
  constexpr int BM = 64 * MB;
  // dq key tile: 32 keys at bf16 D = 256 (a 64 KB ring: two work-groups
  // per CU), else the default
  constexpr int DQBN = (!std::is_same<T, float>::value && D <= 256) ? 32 : 0;
  const int T_ = a.total;
  // (bwd_rows_kernel, launched first by launch_prefill_bwd, has filled
  // w.lo and w.hi)
  const float c = a.scale * kPrefillLog2e;
  {
    const int ntiles = (T_ + BM - 1) / BM;
    const long long nwork = (long long)ntiles * a.hq;
    const long long per_xcd = (nwork + 7) / 8;
    if (8 * per_xcd > 0x7fffffffLL) return SWA_EUNSUPPORTED;
    hipLaunchKernelGGL((bwd_dq_kernel<D, T, MB, DQBN>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.out,
                       (const T*)a.dout, w.lo, w.hi, a.lse, T_, a.hq, a.hkv, a.window, c, a.scale, ntiles,
                       (int)nwork, (int)per_xcd, (T*)a.dq, w.lse, w.delta);
  }
  {
    using C = DkdvCfg<D, T>;
    constexpr int BK = 16 * C::KB * C::NW / C::DS;  // keys per work-group
    const int nkt = (T_ + BK - 1) / BK;
    const long long nwork = (long long)nkt * a.hkv;
    const long long per_xcd = (nwork + 7) / 8;
    if (8 * per_xcd > 0x7fffffffLL) return SWA_EUNSUPPORTED;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, C::DS, C::KB, C::BQ, C::NW>), dim3((unsigned)(8 * per_xcd)),
                       dim3(64 * C::NW), 0,
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
                       w.lse, w.delta, w.lo, w.hi, T_, a.hq, a.hkv, a.window, c, a.scale, nkt, (int)nwork,
                       (int)per_xcd, (T*)a.dk, (T*)a.dv);
  }
  return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ELAUNCH;
}


// per head size: both element types (prefill_bwd_d*.hip)
int launch_bwd_d64(const PrefillBwdArgs& a, const BwdWorkspace& w);
int launch_bwd_d128(const PrefillBwdArgs& a, const BwdWorkspace& w);
int launch_bwd_d192(const PrefillBwdArgs& a, const BwdWorkspace& w);
int launch_bwd_d256(const PrefillBwdArgs& a, const BwdWorkspace& w);
int launch_bwd_d320(const PrefillBwdArgs& a, const BwdWorkspace& w);
int launch_bwd_d384(const PrefillBwdArgs& a, const BwdWorkspace& w);
int launch_bwd_d448(const PrefillBwdArgs& a, const BwdWorkspace& w);
int launch_bwd_d512(const PrefillBwdArgs& a, const BwdWorkspace& w);

}  // namespace swa

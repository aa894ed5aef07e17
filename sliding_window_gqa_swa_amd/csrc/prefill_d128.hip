// prefill_d128.hip -- prefill instantiations for head dimension 128.
// Template arguments: <D, element, q-blocks of 16 rows per wave, key tile,
// waves, query heads per work-group sharing the K/V tiles, pipelined loop>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d128(const PrefillArgs& a) {
  const int g = a.hq / a.hkv;
  if (a.dtype == SWA_BF16) {
    // every wave of a work-group reads the same K/V tiles: 4 heads of a
    // group of 4 or 8 share them (32 rows each), else 2 heads (64 rows)
    if (g % 4 == 0)
      return launch_prefill_cfg<128, __bf16, 2, 64, 4, 4, true>(a);
    if (g % 2 == 0)
      return launch_prefill_cfg<128, __bf16, 2, 64, 4, 2, true>(a);
    return launch_prefill_cfg<128, __bf16, 2, 64, 4, 1, true>(a);
  }
  return launch_prefill_cfg<128, float, 1, 32, 4, 1>(a);
}

}  // namespace swa

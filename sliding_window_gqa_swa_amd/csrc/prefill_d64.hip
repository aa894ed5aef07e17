// prefill_d64.hip -- prefill instantiations for head dimension 64.
// Template arguments: <D, element, q-blocks of 16 rows per wave, key tile,
// waves, query heads per work-group sharing the K/V tiles>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d64(const PrefillArgs& a) {
  const int g = a.hq / a.hkv;
  if (a.dtype == SWA_BF16) {
    if (g % 4 == 0)
      return launch_prefill_cfg<64, __bf16, 2, 64, 4, 4>(a);
    if (g % 2 == 0)
      return launch_prefill_cfg<64, __bf16, 2, 64, 4, 2>(a);
    return launch_prefill_cfg<64, __bf16, 2, 64, 4, 1>(a);
  }
  return launch_prefill_cfg<64, float, 2, 32, 4, 1>(a);
}

}  // namespace swa

// prefill_d256.hip -- prefill instantiations for head dimension 256.
// Template arguments: <D, element, q-blocks of 16 rows per wave, key tile,
// waves, query heads per work-group sharing the K/V tiles, pipelined loop>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d256(const PrefillArgs& a) {
  const int g = a.hq / a.hkv;
  if (a.dtype == SWA_BF16) {
    if (g % 4 == 0)
      return launch_prefill_cfg<256, __bf16, 2, 64, 4, 4, true>(a);
    if (g % 2 == 0)
      return launch_prefill_cfg<256, __bf16, 2, 64, 4, 2, true>(a);
    return launch_prefill_cfg<256, __bf16, 2, 64, 4, 1, true>(a);
  }
  return launch_prefill_cfg<256, float, 1, 32, 4, 1>(a);
}

}  // namespace swa

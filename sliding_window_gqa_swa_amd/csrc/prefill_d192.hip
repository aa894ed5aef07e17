// prefill_d192.hip -- prefill instantiations for head dimension 192.
// Template arguments: <D computed, element, q-blocks of 16 rows per wave, key
// tile, waves, query heads per work-group sharing the K/V tiles, pipelined
// loop, D in memory>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d192(const PrefillArgs& a) {
  const int g = a.hq / a.hkv;
  if (a.dtype == SWA_BF16) {
    // computed as head size 256 on its pipelined loop, with no products over
    // the 64 padding columns
    if (g % 4 == 0)
      return launch_prefill_cfg<256, __bf16, 2, 64, 4, 4, true, 192>(a);
    if (g % 2 == 0)
      return launch_prefill_cfg<256, __bf16, 2, 64, 4, 2, true, 192>(a);
    return launch_prefill_cfg<256, __bf16, 2, 64, 4, 1, true, 192>(a);
  }
  return launch_prefill_cfg<192, float, 1, 32, 4, 1>(a);
}

}  // namespace swa

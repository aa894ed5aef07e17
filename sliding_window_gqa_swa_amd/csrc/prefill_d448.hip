// prefill_d448.hip -- prefill instantiations for head dimension 448.
// Template arguments: <D computed, element, q-blocks of 16 rows per wave, key
// tile, waves, query heads per work-group sharing the K/V tiles, pipelined
// loop, D in memory>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d448(const PrefillArgs& a) {
  const int g = a.hq / a.hkv;
  if (a.dtype == SWA_BF16) {
    // computed as head size 512 on its pipelined loop, with no products over
    // the 64 padding columns
    if (g % 4 == 0)
      return launch_prefill_cfg<512, __bf16, 2, 32, 4, 4, true, 448>(a);
    if (g % 2 == 0)
      return launch_prefill_cfg<512, __bf16, 2, 32, 4, 2, true, 448>(a);
    return launch_prefill_cfg<512, __bf16, 2, 32, 4, 1, true, 448>(a);
  }
  return launch_prefill_cfg<448, float, 1, 16, 4, 1>(a);
}

}  // namespace swa

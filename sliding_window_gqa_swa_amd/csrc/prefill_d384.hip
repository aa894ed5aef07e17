// prefill_d384.hip -- prefill instantiations for head dimension 384 (the
// loop that head size 320 also runs, here with no padding).
// Template arguments: <D, element, q-blocks of 16 rows per wave, key tile,
// waves, query heads per work-group sharing the K/V tiles, pipelined loop>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d384(const PrefillArgs& a) {
  const int g = a.hq / a.hkv;
  if (a.dtype == SWA_BF16) {
    if (g % 4 == 0)
      return launch_prefill_cfg<384, __bf16, 2, 32, 4, 4, true>(a);
    if (g % 2 == 0)
      return launch_prefill_cfg<384, __bf16, 2, 32, 4, 2, true>(a);
    return launch_prefill_cfg<384, __bf16, 2, 32, 4, 1, true>(a);
  }
  return launch_prefill_cfg<384, float, 1, 16, 4, 1>(a);
}

}  // namespace swa

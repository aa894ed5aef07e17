// prefill_d320.hip -- prefill instantiations for head dimension 320 (the
// non-power-of-two head size that [SDPA] Test plan exercises).
// Template arguments: <D, element, q-blocks of 16 rows per wave, key tile,
// waves, query heads per work-group sharing the K/V tiles>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d320(const PrefillArgs& a) {
  const int g = a.hq / a.hkv;
  if (a.dtype == SWA_BF16) {
    // computed as head size 384 with zero padding on the pipelined loop
    if (g % 4 == 0)
      return launch_prefill_cfg<384, __bf16, 2, 32, 4, 4, true, 320>(a);
    if (g % 2 == 0)
      return launch_prefill_cfg<384, __bf16, 2, 32, 4, 2, true, 320>(a);
    return launch_prefill_cfg<384, __bf16, 2, 32, 4, 1, true, 320>(a);
  }
  return launch_prefill_cfg<320, float, 1, 16, 4, 1>(a);
}

}  // namespace swa

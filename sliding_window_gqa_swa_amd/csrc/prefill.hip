// prefill.hip -- head-dimension dispatch of the prefill kernel.
#include "prefill_launch.h"

namespace swa {

int launch_prefill(const PrefillArgs& a) {
  switch (a.d) {
    case 64:
      return launch_prefill_d64(a);
    case 128:
      return launch_prefill_d128(a);
    case 192:
      return launch_prefill_d192(a);
    case 256:
      return launch_prefill_d256(a);
    case 320:
      return launch_prefill_d320(a);
    case 384:
      return launch_prefill_d384(a);
    case 448:
      return launch_prefill_d448(a);
    case 512:
      return launch_prefill_d512(a);
    default:
      return SWA_EUNSUPPORTED;
  }
}

}  // namespace swa

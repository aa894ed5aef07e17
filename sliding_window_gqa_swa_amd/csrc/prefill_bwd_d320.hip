// prefill_bwd_d320.hip -- prefill backward instantiations for head dimension 320.
#include "prefill_bwd_launch.h"

namespace swa {

int launch_bwd_d320(const PrefillBwdArgs& a, const BwdWorkspace& w) {
  return a.dtype == SWA_BF16 ? launch_bwd_cfg<320, __bf16>(a, w) : launch_bwd_cfg<320, float>(a, w);
}

}  // namespace swa

// prefill_bwd_d512.hip -- prefill backward instantiations for head dimension 512.
#include "prefill_bwd_launch.h"

namespace swa {

int launch_bwd_d512(const PrefillBwdArgs& a, const BwdWorkspace& w) {
  return a.dtype == SWA_BF16 ? launch_bwd_cfg<512, __bf16>(a, w) : launch_bwd_cfg<512, float>(a, w);
}

}  // namespace swa

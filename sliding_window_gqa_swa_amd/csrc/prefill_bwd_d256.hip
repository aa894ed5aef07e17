// prefill_bwd_d256.hip -- prefill backward instantiations for head dimension 256.
#include "prefill_bwd_launch.h"

namespace swa {

int launch_bwd_d256(const PrefillBwdArgs& a, const BwdWorkspace& w) {
  return a.dtype == SWA_BF16 ? launch_bwd_cfg<256, __bf16>(a, w) : launch_bwd_cfg<256, float>(a, w);
}

}  // namespace swa

// prefill_bwd_d64.hip -- prefill backward instantiations for head dimension 64.
#include "prefill_bwd_launch.h"

namespace swa {

int launch_bwd_d64(const PrefillBwdArgs& a, const BwdWorkspace& w) {
  return a.dtype == SWA_BF16 ? launch_bwd_cfg<64, __bf16>(a, w) : launch_bwd_cfg<64, float>(a, w);
}

}  // namespace swa

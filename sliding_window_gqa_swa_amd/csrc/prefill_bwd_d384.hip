// prefill_bwd_d384.hip -- prefill backward instantiations for head dimension 384.
#include "prefill_bwd_launch.h"

namespace swa {

int launch_bwd_d384(const PrefillBwdArgs& a, const BwdWorkspace& w) {
  return a.dtype == SWA_BF16 ? launch_bwd_cfg<384, __bf16>(a, w) : launch_bwd_cfg<384, float>(a, w);
}

}  // namespace swa

// prefill_bwd_d128.hip -- prefill backward instantiations for head dimension 128.
#include "prefill_bwd_launch.h"

namespace swa {

int launch_bwd_d128(const PrefillBwdArgs& a, const BwdWorkspace& w) {
  return a.dtype == SWA_BF16 ? launch_bwd_cfg<128, __bf16>(a, w) : launch_bwd_cfg<128, float>(a, w);
}

}  // namespace swa

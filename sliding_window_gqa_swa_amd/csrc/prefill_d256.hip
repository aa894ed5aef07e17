// prefill_d256.hip -- prefill instantiations for head dimension 256.
// Template arguments: <D, element, q-blocks of 16 rows per wave, key tile,
// waves, query heads per work-group sharing the K/V tiles, pipelined loop>.
#include "prefill_launch.h"

namespace swa {

int launch_prefill_d256(const void* q, const void* k, const void* v, const int32_t* cu,
                       const int32_t* ids, int window, int mode, void* out, int total_tokens,
                       int num_docs, int hq, int hkv, int dtype, float scale, hipStream_t s) {
  const int g = hq / hkv;
  if (dtype == SWA_BF16) {
    if (g % 2 == 0)
      return launch_prefill_cfg<256, __bf16, 2, 64, 4, 2, true>(q, k, v, cu, ids, window, mode, out,
                                                       total_tokens, num_docs, hq, hkv, scale, s);
    return launch_prefill_cfg<256, __bf16, 2, 64, 4, 1, true>(q, k, v, cu, ids, window, mode, out,
                                                     total_tokens, num_docs, hq, hkv, scale, s);
  }
  return launch_prefill_cfg<256, float, 1, 32, 4, 1>(q, k, v, cu, ids, window, mode, out,
                                                  total_tokens, num_docs, hq, hkv, scale, s);
}

}  // namespace swa

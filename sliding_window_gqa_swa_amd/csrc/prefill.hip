// prefill.hip -- head-dimension dispatch of the prefill kernel.
#include "prefill_launch.h"

namespace swa {

int launch_prefill(const void* q, const void* k, const void* v, const int32_t* cu,
                   const int32_t* ids, int window, int mode, void* out, int total_tokens,
                   int num_docs, int hq, int hkv, int d, int dtype, float scale,
                   hipStream_t stream) {
  switch (d) {
    case 64:
      return launch_prefill_d64(q, k, v, cu, ids, window, mode, out, total_tokens, num_docs,
                                hq, hkv, dtype, scale, stream);
    case 128:
      return launch_prefill_d128(q, k, v, cu, ids, window, mode, out, total_tokens, num_docs,
                                 hq, hkv, dtype, scale, stream);
    case 256:
      return launch_prefill_d256(q, k, v, cu, ids, window, mode, out, total_tokens, num_docs,
                                 hq, hkv, dtype, scale, stream);
    case 512:
      return launch_prefill_d512(q, k, v, cu, ids, window, mode, out, total_tokens, num_docs,
                                 hq, hkv, dtype, scale, stream);
    default:
      return SWA_EUNSUPPORTED;
  }
}

}  // namespace swa

// head_dim 128 instantiation of the prefill kernel in prefill_kernel.h.
#include "prefill_kernel.h"

namespace sinkattn {

hipError_t launch_prefill_d128(const PrefillArgs& a, int heads_per_wg, int64_t num_blocks,
                               hipStream_t stream) {
  return launch_d<128>(a, heads_per_wg, num_blocks, stream);
}

}  // namespace sinkattn

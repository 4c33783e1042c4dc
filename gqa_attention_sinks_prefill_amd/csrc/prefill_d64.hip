// head_dim 64 instantiation of the prefill kernel in prefill_kernel.h (built
// with its own scheduler flag: build_native.py, SOURCE_FLAGS).
#include "prefill_kernel.h"

namespace sinkattn {

hipError_t launch_prefill_d64(const PrefillArgs& a, int heads_per_wg, int64_t num_blocks,
                              hipStream_t stream) {
  return launch_d<64>(a, heads_per_wg, num_blocks, stream);
}

}  // namespace sinkattn

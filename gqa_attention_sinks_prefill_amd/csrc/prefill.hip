// Host side of the prefill: work shape and dispatch to the per-head_dim
// instantiations of the kernel in prefill_kernel.h.
#include "prefill_kernel.h"

namespace sinkattn {

int prefill_heads_per_workgroup(int group) {
  return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

int prefill_rows_per_workgroup(int group, int head_dim) {
  return 32 * query_blocks(head_dim) * 4 / prefill_heads_per_workgroup(group);
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int64_t num_blocks,
                          hipStream_t stream) {
  const int hpw = prefill_heads_per_workgroup(a.group);
  return head_dim == 64 ? launch_prefill_d64(a, hpw, num_blocks, stream)
                        : launch_prefill_d128(a, hpw, num_blocks, stream);
}

}  // namespace sinkattn

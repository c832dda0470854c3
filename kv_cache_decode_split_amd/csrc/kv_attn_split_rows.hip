// Instantiations of the split kernel for rows mode (variant 2: several query tokens, or one
// token with a bf16 group of 4 or more heads; scores and P.V on the matrix cores), head dims 64
// and 128.
#include "kv_attn_split.h"

namespace kvattn {

int launch_split_rows(const SplitArgs& a, const Plan& plan, int head_dim, bool paged, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (head_dim == 64) return launch_rows<64>(a, plan, paged, s);
  if (head_dim == 128) return launch_rows<128>(a, plan, paged, s);
  return int(hipErrorInvalidValue);
}

}  // namespace kvattn

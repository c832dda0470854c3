// Instantiations of the split kernel for bf16 q and KV with matrix-core scores (variant 1), head dim 64.
#include "kv_attn_split.h"

namespace kvattn {

int launch_split_mfma_d64(const SplitArgs& a, const Plan& plan, bool paged, void* stream) {
  return launch_mfma<64>(a, plan, paged, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace kvattn

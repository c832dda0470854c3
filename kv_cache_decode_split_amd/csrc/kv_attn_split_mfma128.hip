// Instantiations of the split kernel for bf16 q and KV with matrix-core scores (variant 1), head dim 128.
#include "kv_attn_split.h"

namespace kvattn {

int launch_split_mfma_d128(const SplitArgs& a, const Plan& plan, bool paged, void* stream) {
  return launch_mfma<128>(a, plan, paged, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace kvattn

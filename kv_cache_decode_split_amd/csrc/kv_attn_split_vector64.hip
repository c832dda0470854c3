// Instantiations of the split kernel for the vector path (variant 0: fp32 or mixed q/KV dtypes), head dim 64.
#include "kv_attn_split.h"

namespace kvattn {

int launch_split_vector_d64(const SplitArgs& a, const Plan& plan, bool q_bf16, bool kv_bf16,
                            void* stream) {
  return launch_vector<64>(a, plan, q_bf16, kv_bf16, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace kvattn

// Forward-kernel instances for head dim 64 (bf16/fp16 x causal x varlen x bias x split).
#include "fwd_kernel.hpp"

namespace mi355attn {

hipError_t launch_fwd_d64(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                          bool split, bool dsplit, hipStream_t s) {
    return launch_fwd_any<64>(p, bf16, causal, varlen, bias, split, dsplit, s);
}

}  // namespace mi355attn

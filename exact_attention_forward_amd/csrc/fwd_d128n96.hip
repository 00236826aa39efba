// Forward-kernel instances of class 128 narrowed to 96 columns (head dims 72..96:
// bf16/fp16 x causal x varlen x bias x split).
#include "fwd_kernel.hpp"

namespace mi355attn {

hipError_t launch_fwd_d128_n96(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                               bool split, bool dsplit, hipStream_t s) {
    return launch_fwd_any<128, 96>(p, bf16, causal, varlen, bias, split, dsplit, s);
}

}  // namespace mi355attn

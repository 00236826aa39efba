// Forward-kernel instances of class 256 narrowed to 192 columns (head dims 136..192 outside
// the decode form: bf16/fp16 x causal x varlen x bias x split).
#include "fwd_kernel.hpp"

namespace mi355attn {

hipError_t launch_fwd_d256_n192(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                                bool split, bool dsplit, hipStream_t s) {
    return launch_fwd_any<256, 192>(p, bf16, causal, varlen, bias, split, dsplit, s);
}

}  // namespace mi355attn

// Forward-kernel instances of class 64 narrowed to 48 columns (head dims 40..48:
// bf16/fp16 x causal x varlen x bias x split).
#include "fwd_kernel.hpp"

namespace mi355attn {

hipError_t launch_fwd_d64_n48(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                              bool split, bool dsplit, hipStream_t s) {
    return launch_fwd_any<64, 48>(p, bf16, causal, varlen, bias, split, dsplit, s);
}

}  // namespace mi355attn

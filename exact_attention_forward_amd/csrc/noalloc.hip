// noalloc.hip -- attn_fwd for callers that cannot allocate device memory.
//
// The split-KV partials (fp32 O and LSE of every split) live in a file-scope device
// array instead of a caller workspace. Each GPU the library runs on holds its own copy
// until the process ends; its address on a device is taken once, with that device
// current, through hipGetSymbolAddress. Calls on one GPU share the array: calls that
// overlap in time on the same GPU (different streams, or threads) race on it.
// Nothing in it needs to start at zero: every partial the combine kernel reads is
// written by the forward kernel of the same call (an empty split writes O = 0 and
// LSE = -inf).
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>

#include "../../include/attn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)ATTN_SCRATCH_BYTES;

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

// The array's device address on the current device (taken once per device).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" attn_status_t attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                          int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale,
                                          int causal, const int* cu_seqlens_q, const int* cu_seqlens_k,
                                          int max_seqlen_q, int max_seqlen_k, const int* seqused_k,
                                          const void* rel_bias, int rel_extent, int num_splits, int pack_gqa,
                                          attn_dtype_t dtype, void* stream) {
    // attn_fwd's own checks first, with no workspace: every error but the missing
    // workspace (the last check, reached only when the split count is above one) is
    // returned as attn_fwd would, before any HIP call
    const attn_status_t st = attn_check_args(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal,
                                             cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, seqused_k,
                                             rel_bias, rel_extent, num_splits, pack_gqa, dtype, nullptr, 0);
    if (st != ATTN_OK && st != ATTN_ERR_WORKSPACE) return st;
    size_t bytes = 0;
    void* ws = nullptr;
    if (st == ATTN_ERR_WORKSPACE) {
        const int varlen = cu_seqlens_q != nullptr;
        const int ns = attn_num_splits(B, Sq, Sk, Hq, Hkv, D, Dv, causal, varlen, max_seqlen_q, max_seqlen_k,
                                       pack_gqa, num_splits);
        bytes = attn_fwd_workspace_size(B, Sq, Hq, Dv, varlen, ns);
        if (bytes > kScratchBytes) return ATTN_ERR_SCRATCH;
        if (scratch_address(&ws) != hipSuccess) return ATTN_ERR_HIP;
    }
    return attn_fwd(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal, cu_seqlens_q, cu_seqlens_k,
                    max_seqlen_q, max_seqlen_k, seqused_k, rel_bias, rel_extent, num_splits, pack_gqa, dtype, ws,
                    bytes, stream);
}

// combine.hip -- LSE-weighted merge of split-KV partials (gfx950).
//
// Each split s of the key range produced O_s (normalised within the split) and
// LSE_s; the exact result over the union of the key ranges is
//   M = max_s LSE_s,  LSE = M + ln sum_s exp(LSE_s - M),  O = sum_s exp(LSE_s - LSE) O_s.
// This is the merge that the returned LSE makes possible outside the kernel
// (TabPFN issue #1235, closing comment; tml-fa4 "split-KV combine").
// One wave per (query row, head); lanes split the Dv columns. HBM-bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mi355attn {

namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <bool BF>
__device__ __forceinline__ uint16_t narrow(float x) {
    if (BF) return __builtin_bit_cast(uint16_t, (__bf16)x);
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int DV, bool BF>
__global__ void __launch_bounds__(256) attn_combine_kernel(const CombineParams p) {
    constexpr int PER = DV >= 64 ? DV / 64 : 1;  // columns per lane
    const int lane = threadIdx.x & 63;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long n_items = p.rows_q * p.Hq;
    if (item >= n_items) return;
    const long long t = item / p.Hq;
    const int h = (int)(item % p.Hq);
    long long lidx;
    if (p.is_varlen) {
        lidx = (long long)h * p.rows_q + t;
    } else {
        const long long bb = t / p.Sq;
        const long long i = t % p.Sq;
        lidx = (bb * p.Hq + h) * p.Sq + i;
    }
    const long long lse_stride = p.rows_q * p.Hq;  // per split
    const float* lp = p.lse_part + lidx;

    float M = -INFINITY;
    for (int s = lane; s < p.ns; s += 64) M = fmaxf(M, lp[(long long)s * lse_stride]);
    M = wave_max(M);

    const int dv0 = lane * PER;
    const bool active = dv0 < DV;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; e++) acc[e] = 0.f;
    float L = -INFINITY;
    if (M != -INFINITY) {
        float sum = 0.f;
        for (int s = lane; s < p.ns; s += 64) sum += expf(lp[(long long)s * lse_stride] - M);
        sum = wave_sum(sum);
        L = M + logf(sum);
        const float* op = p.o_part + item * DV + dv0;
        for (int s = 0; s < p.ns; s++) {
            const float ls = lp[(long long)s * lse_stride];
            const float w = expf(ls - L);  // 0 for an empty split (ls = -inf)
            if (active && w != 0.f) {
                const float* src = op + (long long)s * lse_stride * DV;
#pragma unroll
                for (int e = 0; e < PER; e++) acc[e] += w * src[e];
            }
        }
    }
    if (active) {
        uint16_t* dst = p.out + item * DV + dv0;
#pragma unroll
        for (int e = 0; e < PER; e++) dst[e] = narrow<BF>(acc[e]);
    }
    if (p.lse && lane == 0) p.lse[lidx] = L;
}

template <int DV, bool BF>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t s) {
    const long long n_items = p.rows_q * p.Hq;
    const long long blocks = (n_items + 3) / 4;
    if (blocks <= 0) return hipSuccess;
    CombineParams pp = p;
    void* args[] = {(void*)&pp};
    return hipLaunchKernel((const void*)attn_combine_kernel<DV, BF>, dim3((unsigned)blocks), dim3(256), args,
                           0, s);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, int Dv, bool bf16, hipStream_t s) {
    switch (Dv) {
        case 16: return bf16 ? launch_combine_t<16, true>(p, s) : launch_combine_t<16, false>(p, s);
        case 64: return bf16 ? launch_combine_t<64, true>(p, s) : launch_combine_t<64, false>(p, s);
        case 128: return bf16 ? launch_combine_t<128, true>(p, s) : launch_combine_t<128, false>(p, s);
        case 256: return bf16 ? launch_combine_t<256, true>(p, s) : launch_combine_t<256, false>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mi355attn

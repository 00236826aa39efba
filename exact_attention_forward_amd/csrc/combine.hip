// combine.hip -- LSE-weighted merge of split-KV partials (gfx950).
//
// Each split s of the key range produced O_s (normalised within the split) and
// LSE_s; the exact result over the union of the key ranges is
//   M = max_s LSE_s,  LSE = M + ln sum_s exp(LSE_s - M),  O = sum_s exp(LSE_s - LSE) O_s.
// This is the merge that the returned LSE makes possible outside the kernel
// (TabPFN issue #1235, closing comment; tml-fa4 "split-KV combine").
// HBM-bound.
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

// One work-group of 4 waves per (query row, head). The split-wise max and sum
// run over all 256 threads; then wave w accumulates the splits s = w, w+4, ...
// with its lanes over the Dv columns (several partial rows in flight per lane),
// and the four partial sums meet in LDS.
template <int DV, bool BF>
__global__ void __launch_bounds__(256) attn_combine_kernel(const CombineParams p) {
    constexpr int PER = DV >= 64 ? DV / 64 : 1;  // columns per lane
    constexpr int UNROLL = 16 / PER;              // splits per wave in flight (16 loads per lane)
    __shared__ float red[4];
    __shared__ float part[4][DV];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const long long item = blockIdx.x;
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

    // M = max_s LSE_s over the work-group
    float M = -INFINITY;
    for (int s = tid; s < p.ns; s += 256) M = fmaxf(M, lp[(long long)s * lse_stride]);
    M = wave_max(M);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();

    float L = -INFINITY;
    if (M != -INFINITY) {  // uniform over the work-group
        float sum = 0.f;
        for (int s = tid; s < p.ns; s += 256) sum += expf(lp[(long long)s * lse_stride] - M);
        sum = wave_sum(sum);
        if (lane == 0) red[wave] = sum;
        __syncthreads();
        L = M + logf((red[0] + red[1]) + (red[2] + red[3]));
    }

    const int dv0 = lane * PER;
    const bool active = dv0 < p.Dv;  // Dv <= DV, a multiple of 8 (whole PER-column groups)
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; e++) acc[e] = 0.f;
    if (L != -INFINITY && active) {
        const float* op = p.o_part + item * p.Dv + dv0;
        const long long ostride = lse_stride * p.Dv;  // floats between splits
        int s = wave;
        for (; s + 4 * (UNROLL - 1) < p.ns; s += 4 * UNROLL) {
            float w[UNROLL], x[UNROLL][PER];
#pragma unroll
            for (int u = 0; u < UNROLL; u++) {
                const long long su = s + 4 * u;
                w[u] = lp[su * lse_stride];
#pragma unroll
                for (int e = 0; e < PER; e++) x[u][e] = op[su * ostride + e];
            }
#pragma unroll
            for (int u = 0; u < UNROLL; u++) {
                const float wu = expf(w[u] - L);  // 0 for an empty split (LSE_s = -inf)
                if (wu != 0.f)
#pragma unroll
                    for (int e = 0; e < PER; e++) acc[e] += wu * x[u][e];
            }
        }
        for (; s < p.ns; s += 4) {
            const float wu = expf(lp[(long long)s * lse_stride] - L);
            if (wu != 0.f)
#pragma unroll
                for (int e = 0; e < PER; e++) acc[e] += wu * op[(long long)s * ostride + e];
        }
    }
    if (active)
#pragma unroll
        for (int e = 0; e < PER; e++) part[wave][dv0 + e] = acc[e];
    __syncthreads();
    if (wave == 0 && active) {
        uint16_t* dst = p.out + item * p.Dv + dv0;
#pragma unroll
        for (int e = 0; e < PER; e++) {
            const int c = dv0 + e;
            dst[e] = narrow<BF>((part[0][c] + part[1][c]) + (part[2][c] + part[3][c]));
        }
    }
    if (p.lse && tid == 0) p.lse[lidx] = L;
}

template <int DV, bool BF>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t s) {
    const long long blocks = p.rows_q * p.Hq;  // one work-group per (query row, head)
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    CombineParams pp = p;
    void* args[] = {(void*)&pp};
    return hipLaunchKernel((const void*)attn_combine_kernel<DV, BF>, dim3((unsigned)blocks), dim3(256), args,
                           0, s);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, int Dv, bool bf16, hipStream_t s) {
    switch (head_dim_class(Dv)) {
        case 16: return bf16 ? launch_combine_t<16, true>(p, s) : launch_combine_t<16, false>(p, s);
        case 64: return bf16 ? launch_combine_t<64, true>(p, s) : launch_combine_t<64, false>(p, s);
        case 128: return bf16 ? launch_combine_t<128, true>(p, s) : launch_combine_t<128, false>(p, s);
        case 256: return bf16 ? launch_combine_t<256, true>(p, s) : launch_combine_t<256, false>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mi355attn

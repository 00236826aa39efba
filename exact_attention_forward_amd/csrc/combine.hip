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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One work-group of 256 threads per (query row, head). Thread s holds split s's LSE
// (num_splits <= 256): the max, the sum and the weights exp(LSE_s - LSE) come from one
// read each, and the weights go to LDS. Then the threads take 16-byte column chunks of
// the partial rows, SP splits side by side (thread = split slot x chunk), each with
// UNROLL rows in flight (the first UNROLL issued before the LSE reduction), and the SP
// partial sums of a chunk meet in LDS in a fixed order.
// Splits with weight 0 (empty key ranges) are skipped, whatever their partial holds.
template <int DV, bool BF>
__global__ void __launch_bounds__(256) attn_combine_kernel(const CombineParams p) {
    constexpr int CH = DV / 4;     // 16-byte chunks of a row
    constexpr int SP = 256 / CH;   // splits read side by side
    constexpr int UNROLL = 16;     // partial rows in flight per thread
    static_assert(CH * SP == 256, "a row's chunks tile the work-group");
    __shared__ float red[4];
    __shared__ float wts[256];
    __shared__ f32x4 part[SP][CH];
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
    const float ls = tid < p.ns ? p.lse_part[lidx + (long long)tid * lse_stride] : -INFINITY;

    // The first UNROLL partial rows of this thread's chunk go out before the LSE reduction
    // (they do not depend on the weights), so their latency and the reduction's overlap.
    const int c = tid % CH, sg = tid / CH;
    const bool active = 4 * c < p.Dv;  // Dv <= DV, a multiple of 8: whole chunks
    const float* op = p.o_part + item * p.Dv + 4 * c;
    const long long ostride = lse_stride * p.Dv;  // floats between splits
    f32x4 x0[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; u++)
        x0[u] = active && sg + SP * u < p.ns ? *(const f32x4*)(op + (long long)(sg + SP * u) * ostride)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};

    // M = max_s LSE_s, LSE = M + ln sum_s exp(LSE_s - M)
    float M = wave_max(ls);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float L = -INFINITY;
    if (M != -INFINITY) {  // uniform over the work-group
        const float e = wave_sum(expf(ls - M));  // exp(-inf) = 0 past the last split
        if (lane == 0) red[wave] = e;
        __syncthreads();
        L = M + logf((red[0] + red[1]) + (red[2] + red[3]));
    }
    wts[tid] = expf(ls - L);  // (unused when L = -inf)
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (L != -INFINITY && active) {
#pragma unroll
        for (int u = 0; u < UNROLL; u++) {
            const int s0 = sg + SP * u;
            const float w = s0 < p.ns ? wts[s0] : 0.f;
            if (w != 0.f) acc += w * x0[u];
        }
        int s = sg + SP * UNROLL;
        for (; s + SP * (UNROLL - 1) < p.ns; s += SP * UNROLL) {
            f32x4 x[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; u++) x[u] = *(const f32x4*)(op + (long long)(s + SP * u) * ostride);
#pragma unroll
            for (int u = 0; u < UNROLL; u++) {
                const float w = wts[s + SP * u];
                if (w != 0.f) acc += w * x[u];
            }
        }
        for (; s < p.ns; s += SP) {
            const float w = wts[s];
            if (w != 0.f) acc += w * *(const f32x4*)(op + (long long)s * ostride);
        }
    }
    part[sg][c] = acc;
    __syncthreads();
    if (tid < CH && active) {
        f32x4 o = part[0][tid];
#pragma unroll
        for (int g = 1; g < SP; g++) o += part[g][tid];
        uint16_t* dst = p.out + item * p.Dv + 4 * tid;
        const unsigned lo = (unsigned)narrow<BF>(o[0]) | ((unsigned)narrow<BF>(o[1]) << 16);
        const unsigned hi = (unsigned)narrow<BF>(o[2]) | ((unsigned)narrow<BF>(o[3]) << 16);
        *(uint2*)dst = make_uint2(lo, hi);
    }
    if (p.lse && tid == 0) p.lse[lidx] = L;
}

// One wave per (query row, head), four per work-group, for calls with many rows, at most
// 64 splits (use_rows_combine below): lane s holds split s's LSE, so the max, the sum and the weights stay in
// registers (no LDS, no barrier), and the wave's lanes take 16-byte column chunks, SPW
// splits side by side, U partial rows in flight per lane. The per-work-group fixed cost
// of the kernel above (three barriers and an LDS round trip per row) is what bounds it
// when a row has only a few partials to read.
template <int DV, bool BF>
__global__ void __launch_bounds__(256) attn_combine_rows_kernel(const CombineParams p) {
    constexpr int CH = DV / 4;   // 16-byte chunks of a row
    constexpr int SPW = 64 / CH; // splits read side by side
    constexpr int U = 8;         // partial rows in flight per lane
    static_assert(CH * SPW == 64, "a row's chunks tile the wave");
    const int lane = threadIdx.x & 63;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= p.rows_q * p.Hq) return;  // uniform over the wave
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
    const float ls = lane < p.ns ? p.lse_part[lidx + (long long)lane * lse_stride] : -INFINITY;

    // M = max_s LSE_s, LSE = M + ln sum_s exp(LSE_s - M); both uniform over the wave
    const float M = wave_max(ls);
    float L = -INFINITY;
    if (M != -INFINITY) L = M + logf(wave_sum(expf(ls - M)));
    const float wl = expf(ls - L);  // split `lane`'s weight (unused when L = -inf)

    const int c = lane % CH, sg = lane / CH;
    const bool active = 4 * c < p.Dv;  // Dv <= DV, a multiple of 8: whole chunks
    const float* op = p.o_part + item * p.Dv + 4 * c;
    const long long ostride = lse_stride * p.Dv;  // floats between splits
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (L != -INFINITY) {  // every lane of the wave takes part in the shuffles below
        for (int s0 = 0; s0 < p.ns; s0 += SPW * U) {
            f32x4 x[U];
            float w[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int sp = s0 + sg + SPW * u;
                const float wu = __shfl(wl, sp < 64 ? sp : 0, 64);
                w[u] = sp < p.ns ? wu : 0.f;
                // splits with weight 0 (empty key ranges) are neither read nor added
                x[u] = active && w[u] != 0.f ? *(const f32x4*)(op + (long long)sp * ostride)
                                             : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < U; u++)
                if (w[u] != 0.f) acc += w[u] * x[u];
        }
    }
    // the SPW partial sums of a chunk, added in slot order
    f32x4 o = acc;
#pragma unroll
    for (int g = 1; g < SPW; g++) {
        const int src = c + g * CH;
        o[0] += __shfl(acc[0], src, 64);
        o[1] += __shfl(acc[1], src, 64);
        o[2] += __shfl(acc[2], src, 64);
        o[3] += __shfl(acc[3], src, 64);
    }
    if (sg == 0 && active) {
        uint16_t* dst = p.out + item * p.Dv + 4 * c;
        const unsigned lo = (unsigned)narrow<BF>(o[0]) | ((unsigned)narrow<BF>(o[1]) << 16);
        const unsigned hi = (unsigned)narrow<BF>(o[2]) | ((unsigned)narrow<BF>(o[3]) << 16);
        *(uint2*)dst = make_uint2(lo, hi);
    }
    if (p.lse && lane == 0) p.lse[lidx] = L;
}

// Calls with at most 64 splits take the wave-per-row kernel when they have at least
// kRowsCombineMinItems (row, head) items (enough waves to fill the chip several times over,
// so the merge is bound by its reads, not by a work-group's fixed cost), or at least
// kRowsCombineFewItems items whose lanes each read at most two rounds of U partial rows:
// a lane of the class-DV kernel reads ns / (256 / DV) of them, so ns * DV <= 2 * 8 * 256
// (the short-query split calls: 64 splits at class 64).
constexpr long long kRowsCombineMinItems = 8192;
constexpr long long kRowsCombineFewItems = 2048;

template <int DV>
bool use_rows_combine(const CombineParams& p, long long items) {
    if (p.ns > 64) return false;
    if (items >= kRowsCombineMinItems) return true;
    return items >= kRowsCombineFewItems && (long long)p.ns * DV <= 16 * 256;
}

template <int DV, bool BF>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t s) {
    const long long items = p.rows_q * p.Hq;
    if (items <= 0) return hipSuccess;
    CombineParams pp = p;
    void* args[] = {(void*)&pp};
    if (use_rows_combine<DV>(p, items)) {
        const long long blocks = (items + 3) / 4;  // four waves, four items per work-group
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        return hipLaunchKernel((const void*)attn_combine_rows_kernel<DV, BF>, dim3((unsigned)blocks), dim3(256),
                               args, 0, s);
    }
    if (items > 0x7fffffffLL) return hipErrorInvalidValue;  // one work-group per (query row, head)
    return hipLaunchKernel((const void*)attn_combine_kernel<DV, BF>, dim3((unsigned)items), dim3(256), args,
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

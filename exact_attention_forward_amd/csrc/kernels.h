// kernels.h -- parameters and launchers shared by the host planner and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355attn {

// Head-dim class: the kernels are compiled for D, Dv up to 16, 64, 128 and 256;
// a call with any D, Dv in 8..256 (multiples of 8) runs the smallest class that
// holds both, with the K / V / Q columns past D (Dv) zero in registers and LDS.
__host__ __device__ constexpr int head_dim_class(int d) {
    return d <= 16 ? 16 : d <= 64 ? 64 : d <= 128 ? 128 : 256;
}

// Work-group geometry of the forward kernel for head-dim class D: NW waves of 64
// lanes; each wave owns NQB blocks of 32 query rows (one MFMA 32x32 output column
// block per row block); BN keys per K/V tile.

__host__ __device__ constexpr int tile_nqb(int /*D*/) { return 1; }
// Waves per work-group: eight at head-dim class 128 without the causal mask, so a 256-row
// work-group shares each K / V tile it brings into LDS (half the L2 -> LDS traffic per FLOP
// of four waves: [1,20480,56,128] bf16 forward -3.9% time with the pipelined key loop);
// four elsewhere. Causal row tiles keep 128 rows: the diagonal stays finer and unequal
// varlen sequences balance better (the varlen causal GQA + rel_bias workload measured +4.9%
// time with 256-row tiles).
__host__ __device__ constexpr int tile_nw(int D, bool causal) { return D == 128 && !causal ? 8 : 4; }
__host__ __device__ constexpr int tile_bm(int D, bool causal) { return tile_nw(D, causal) * 32 * tile_nqb(D); }
// Keys per K/V tile: 64; 128 at head-dim class 16, where a tile's MFMA work is smallest
// (measured c4b -6% time against 64; at class 64 the same measured +3% on c4a).
__host__ __device__ constexpr int tile_bn(int D) { return D <= 16 ? 128 : 64; }
// Work-groups resident per CU: two of four waves up to head dim 128; one of eight waves
// at 128 without the causal mask; one at 256, where a wave needs more than 256 registers.
__host__ __device__ constexpr int tile_wg_per_cu(int D, bool causal) {
    return D <= 64 || (D == 128 && causal) ? 2 : D == 128 ? 1 : 1;
}
// K/V tiles loaded ahead of the one being consumed (the LDS ring has one more stage):
// one, in a ring of at most 64 KB up to head dim 64 and 128 KB at 256 (measured at 256
// against 32-key tiles three ahead: prefill c5a -16%, decode c5b -10% time). At 128
// (eight waves, 64 KB) three tiles ahead in a 128 KB ring measured 2% slower on the
// [1,20480,56,128] bf16 forward.
__host__ __device__ constexpr int tile_prefetch(int /*D*/) { return 1; }
// LDS of the K/V ring: (PREFETCH + 1) stages, each a K and a V tile of BN x D 16-bit values
__host__ __device__ constexpr int tile_ring_bytes(int D) { return (tile_prefetch(D) + 1) * 2 * tile_bn(D) * D * 2; }
constexpr int kLdsBytesPerCU = 160 * 1024;

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    float* lse;            // may be null
    const uint16_t* bias;  // rel_bias or null
    // fused rel_bias producer (bias instances, bias == null): r [rows_q, Hq, d_rel] and
    // rel_proj [d_rel, E]; the work-group's bias rows are built in LDS past the K/V ring
    const uint16_t* rel_r;
    const uint16_t* rel_proj;
    int d_rel;
    int lds_extra;         // bytes of that LDS region (0 without the fused producer)
    float* o_part;         // split partials (split mode)
    float* lse_part;
    const int* cu_q;       // varlen offsets (varlen mode)
    const int* cu_k;
    const int* seqused_k;  // may be null
    int B, Sq, Sk, Hq, Hkv;
    int D, Dv;             // head dims of q/k and of v / out (at most the class)
    int G;                 // Hq / Hkv
    int gp;                // query heads packed per tile row group (G with pack-GQA, else 1)
    int n_hg;              // head groups: Hkv when packed, else Hq
    int n_tiles;           // row tiles per (batch, head group)
    int ns;                // key-range splits (1 = none)
    int E;                 // rel_extent (0 without bias)
    int nblocks;           // grid size
    float c2;              // scale * log2(e)
    long long rows_q;      // rows of q's flattened order: B*Sq (dense) or total_q (varlen)
};

struct CombineParams {
    const float* o_part;
    const float* lse_part;
    uint16_t* out;
    float* lse;            // may be null
    long long rows_q;      // rows of q's flattened order
    int Hq, Sq, ns, is_varlen;
    int Dv;                // columns of a row (at most the class the kernel is compiled for)
};

hipError_t launch_fwd_d16(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                          bool split, bool dsplit, hipStream_t s);
hipError_t launch_fwd_d64(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                          bool split, bool dsplit, hipStream_t s);
hipError_t launch_fwd_d64_n48(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                          bool split, bool dsplit, hipStream_t s);
hipError_t launch_fwd_d128(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                           bool split, bool dsplit, hipStream_t s);
hipError_t launch_fwd_d128_n96(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                           bool split, bool dsplit, hipStream_t s);
hipError_t launch_fwd_d256(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                           bool split, bool dsplit, hipStream_t s);
hipError_t launch_fwd_d256_n192(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias,
                           bool split, bool dsplit, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, int Dv, bool bf16, hipStream_t s);

}  // namespace mi355attn

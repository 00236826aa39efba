// fwd_kernel.hpp -- fused exact attention forward for gfx950 (MI355X).
//
// What is computed (per batch b, query head h, query row i): the scaled dot
// products with K, the bottom-right causal mask and the relative-bias band of
// the tml-fa4 "Argument contract" (score += rel_bias[q_off + i, h, d] for
// d = i + (k_len - q_len) - j in [0, rel_extent)), an online softmax with a
// running max and normaliser, P*V, and O plus the fp32 log-sum-exp that the
// FA4 forward returns (fa4-cute-runtime card, Functions). The tiling, running
// max, normaliser and PV steps leave the plain softmax result unchanged up to
// rounding (ATFlash-Kernel-FA4 page, the online-softmax figure).
//
// gfx950 mapping (one work-group = 4 waves; a wave owns NQB blocks of 32 rows):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}: A = a K row per lane
//     (read from LDS, 16 bytes), B = the wave's Q rows, kept in registers.
//     Per 32-key block, lane l then holds 16 keys of query row l%32; lanes l
//     and l^32 share a row, so a row max is an in-lane max plus one
//     permlane32_swap.
//   * O^T = V^T P^T on the same MFMA: B = P^T comes straight from the S^T
//     accumulators (same lane = same query), A = V^T is read from LDS with
//     ds_read_b64_tr_b16 out of a 4x4-blocked V layout, so each 16-lane group
//     reads 128 contiguous bytes. Every O^T register of a lane belongs to one
//     query, so the online-softmax rescale is a per-lane scalar multiply.
//   * K/V tiles of BN keys (64; 128 at head-dim class 16) sit in an LDS ring of
//     PREFETCH + 1 = 2 stages; the loads of the next tile are in flight while a
//     tile is computed; one barrier per tile.
//   * Only tiles that cross the key bound, the causal diagonal or the bias band
//     run the per-element mask / bias code (band tiles and the other masked
//     tiles in passes of their own).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <atomic>
#include <utility>

#include "kernels.h"

namespace mi355attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
typedef short s16x4v __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4v lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// bfloat16 P: a row whose uncorrected weights may have fewer effective keys than this
// ((sum p)^2 / sum p^2, from a bound on the squares) gets the P remainder MFMA for the tile
constexpr float kLoThresh = 64.f;
constexpr float kTau = 8.f;  // O / l are rescaled only when the row max grows by more than 2^kTau
// a buffer offset past every range the kernel builds (row bytes x 64 keys stay below it:
// the host bounds heads x head dim)
constexpr int kOobOffset = 0x40000000;

template <bool BF>
struct Elem;

template <>
struct Elem<true> {  // bfloat16
    typedef bf16x8 v8;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float widen(uint16_t x) {
        return __uint_as_float(((unsigned)x) << 16);
    }
    static __device__ __forceinline__ uint16_t narrow(float x) {  // round to nearest even
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
    static __device__ __forceinline__ __bf16 to_elem(float x) { return (__bf16)x; }
    static constexpr uint16_t kNegInfBits = 0xFF80;
    static constexpr uint32_t kOnePairBits = 0x3F803F80u;  // (1, 1)
};

template <>
struct Elem<false> {  // IEEE half
    typedef f16x8 v8;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float widen(uint16_t x) {
        return (float)__builtin_bit_cast(_Float16, x);
    }
    static __device__ __forceinline__ uint16_t narrow(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    static __device__ __forceinline__ _Float16 to_elem(float x) { return (_Float16)x; }
    static constexpr uint16_t kNegInfBits = 0xFC00;
    static constexpr uint32_t kOnePairBits = 0x3C003C00u;  // (1, 1)
};

template <int D, bool CAUSAL = false>
struct Tile {
    static constexpr int NW = tile_nw(D, CAUSAL); // waves per work-group
    static constexpr int NT = NW * 64;            // threads
    static constexpr int NQB = tile_nqb(D);       // 32-row blocks per wave
    static constexpr int BM = tile_bm(D, CAUSAL); // rows per work-group
    static constexpr int BN = tile_bn(D);         // keys per tile
    static constexpr int NC = D / 16;             // 16-wide steps of the QK contraction
    static constexpr int NDT = (D + 31) / 32;     // 32-wide dv blocks of O^T
    static constexpr int NKB = BN / 32;           // 32-key blocks of S^T
    static constexpr int NG = D / 8;              // 16-byte granules per K / V row
    static constexpr int SWZ_DIV = NG >= 16 ? 1 : 16 / NG;
    static constexpr int TILE_BYTES = BN * D * 2; // one K or V tile in LDS
    static constexpr int PREFETCH = tile_prefetch(D);  // tiles loaded ahead of the one being consumed
    static constexpr int NB = PREFETCH + 1;       // LDS ring stages, each a K tile and a V tile
    static constexpr int WG_PER_CU = tile_wg_per_cu(D, CAUSAL);
    // load offsets and K read addresses formed per tile instead of held in registers
    // across the key loop: fewer live registers for a few more VALU operations
    // (measured: faster at head-dim classes 16 and 256, slower at 64 and 128)
    static constexpr bool LEAN = D == 16 || D == 256;
    static constexpr int LDS = NB * 2 * TILE_BYTES;
    static_assert(LDS == tile_ring_bytes(D), "host and kernel agree on the ring size");
    static constexpr int GRANULES = BN * NG;      // 16-byte granules per tile
    static constexpr int LOADS = (GRANULES + NT - 1) / NT;  // per thread, per K (or V) tile
    static constexpr int VM_PER_TILE = 2 * LOADS;           // buffer loads a wave issues per tile
    static_assert(D == 16 || D == 64 || D == 128 || D == 256, "head dim");
    static_assert(LDS * WG_PER_CU <= 160 * 1024, "LDS budget");
    static_assert(NB <= 5, "tile loop unrolled over at most five ring stages");
    static_assert(GRANULES % NT == 0 || LOADS == 1, "a wave issues all of its loads of a tile or none");
    static_assert(GRANULES % 64 == 0, "whole waves per load instruction");
};

// Position of element r (0..15) of a 32x32 MFMA accumulator in lane half hf:
// row offset within the 32-row block (the "M" index).
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// K tile in LDS: granule (key, c) of 8 elements sits at key * NG + (c ^ swizzle(key)),
// so the 16 rows read by one ds_read_b128 pass fall in 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_granule(int key, int c) {
    using T = Tile<D>;
    return key * T::NG + (c ^ ((key / T::SWZ_DIV) % T::NG));
}

// V tile in LDS, 4-key blocks: granule (key, 8-wide dv chunk q8) sits at
// ((key / 4) * NG + q8) * 4 + key % 4. A ds_read_b64_tr_b16 group then reads
// 4 keys x 16 dv = 128 contiguous bytes.
template <int D>
__device__ __forceinline__ int v_granule(int key, int q8) {
    return ((key >> 2) * Tile<D>::NG + q8) * 4 + (key & 3);
}

typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b64_tr_b16 through a restrict pointer: once inlined, the read carries
// alias-scope information, which lets the wait-count insertion tell it apart
// from the buffer-to-LDS loads in flight (ordering against those is explicit:
// each wave waits for its own loads and a barrier follows).
__device__ __forceinline__ s16x4v lds_read_tr16(const lds_s16x4* __restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left unconstrained
template <int N>
__device__ __forceinline__ void wait_vm_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vm_all() { wait_vm_loads<0>(); }


// DSPLIT (class 256, every tile at most 32 rows: decode): the four waves take the
// same rows; each computes S and the softmax for all of them (identical values)
// and accumulates a quarter of the V columns, so the PV MFMAs of a tile are shared
// out instead of all falling to the one wave that holds rows.
// W (a multiple of 16 up to D) narrows the arithmetic to the first W columns of the class: a
// call whose head dims fit W runs the class's tile geometry and LDS layout but only the QK
// steps and O^T blocks that can hold data (head dims 72..96 on class 128, 40..48 on 64,
// 136..192 on 256 outside decode).
template <int D, bool BF, bool CAUSAL, bool VARLEN, bool BIAS, bool SPLIT, bool DSPLIT, int W>
__global__ void __launch_bounds__((Tile<D, CAUSAL>::NT), (Tile<D, CAUSAL>::WG_PER_CU)) attn_fwd_kernel(const FwdParams p) {
    using T = Tile<D, CAUSAL>;
    static_assert(!DSPLIT || (D == 256 && T::NQB == 1 && T::NW == 4 && W == D), "dv split: class 256, one row block, four waves");
    static_assert(W == D || (W < D && W % 16 == 0), "narrowed width: a multiple of 16 below the class");
    constexpr int NCK = W / 16;  // 16-wide steps of the QK contraction that can hold data
    constexpr int ODT = DSPLIT ? T::NDT / 4 : (W + 31) / 32;  // dv blocks of O^T this wave accumulates
    using E = Elem<BF>;
    typedef typename E::v8 v8;
    typedef f32x16 STile[T::NQB][T::NKB];
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // ---- work-group -> (batch, head group, split, row tile), XCD-aware ----
    // Work-groups are handed to the 8 XCDs round-robin. The row tiles of one
    // (batch, head group, split) read the same K/V and should share an L2.
    // Dense: each XCD gets a contiguous eighth of the logical ids. Varlen: the
    // work of a (batch, head group) follows its sequence length, so whole chunks
    // of row tiles are dealt to the XCDs in turn (chunk c to XCD c % 8), which
    // spreads unequal sequences over all eight; the last, incomplete round of
    // eight chunks stays round-robin.
    int lid;
    {
        const int nb = p.nblocks, bid = blockIdx.x;
        if (!VARLEN) {
            const int q8 = nb >> 3, r8 = nb & 7, x = bid & 7, slot = bid >> 3;
            lid = (x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8) + slot;
        } else {
            const int C = p.n_tiles;
            const long long full = (long long)(nb / (8LL * C)) * 8 * C;
            if (bid < full) {
                const int x = bid & 7, slot = bid >> 3;
                lid = ((slot / C) * 8 + x) * C + slot % C;
            } else {
                lid = bid;
            }
        }
    }
    int tile = lid % p.n_tiles;
    int rest = lid / p.n_tiles;
    const int split = rest % p.ns;
    rest /= p.ns;
    const int hg = rest % p.n_hg;
    const int b = rest / p.n_hg;
    if (CAUSAL) tile = p.n_tiles - 1 - tile;  // longest key ranges first

    // ---- sequence geometry ----
    long long q_off, k_off;
    int q_len, k_len;
    if (VARLEN) {
        const int a0 = p.cu_q[b], a1 = p.cu_q[b + 1];
        q_off = a0;
        q_len = a1 - a0;
        const int c0 = p.cu_k[b], c1 = p.cu_k[b + 1];
        k_off = c0;
        k_len = c1 - c0;
    } else {
        q_off = (long long)b * p.Sq;
        q_len = p.Sq;
        k_off = (long long)b * p.Sk;
        k_len = p.Sk;
    }
    if (p.seqused_k) k_len = p.seqused_k[b];
    const int delta = k_len - q_len;
    const int gp = p.gp;
    const int n_rows = q_len * gp;
    const int row0 = tile * T::BM;
    if (row0 >= n_rows) return;  // uniform: this tile lies past the sequence

    int hk, h_base;
    if (gp > 1) {
        hk = hg;
        h_base = hg * p.G;
    } else {
        h_base = hg;
        hk = hg / p.G;
    }
    const int r_last = min(row0 + T::BM, n_rows) - 1;
    const int i_hi = r_last / gp;
    // query rows of this wave (a wave past the last row repeats the last one)
    const int w_row = row0 + (DSPLIT ? 0 : wave * T::NQB * 32);
    const int dt0 = DSPLIT ? wave * ODT : 0;  // first dv block of this wave
    const int wi_lo = min(w_row, r_last) / gp;
    const int wi_hi = min(w_row + T::NQB * 32 - 1, r_last) / gp;
    const bool wave_live = w_row < n_rows;

    int kv_end = k_len;
    if (CAUSAL) kv_end = min(k_len, i_hi + delta + 1);
    kv_end = max(kv_end, 0);
    const int nkb = (kv_end + T::BN - 1) / T::BN;
    int kb_begin = 0, kb_end = nkb;
    if (SPLIT) {
        kb_begin = (int)(((long long)nkb * split) / p.ns);
        kb_end = (int)(((long long)nkb * (split + 1)) / p.ns);
    }

    // ---- this lane's rows ----
    int qi[T::NQB], qh[T::NQB];
    bool qvalid[T::NQB];
#pragma unroll
    for (int qb = 0; qb < T::NQB; qb++) {
        const int row = row0 + ((DSPLIT ? 0 : wave * T::NQB) + qb) * 32 + l32;
        qvalid[qb] = row < n_rows;
        const int rr = qvalid[qb] ? row : r_last;
        qi[qb] = rr / gp;
        qh[qb] = h_base + rr % gp;
    }

    // ---- Q fragments (B operand of S^T = K Q^T): lane holds q[row][16c + 8hf .. +7] ----
    v8 qf[T::NQB][NCK];
#pragma unroll
    for (int qb = 0; qb < T::NQB; qb++) {
        const uint16_t* qrow = p.q + ((q_off + qi[qb]) * p.Hq + qh[qb]) * (long long)p.D;
#pragma unroll
        for (int c = 0; c < NCK; c++) {
            u32x4 x = {0u, 0u, 0u, 0u};  // columns past D stay zero
            if (qvalid[qb] && 16 * c + 8 * hf < p.D) x = *(const u32x4*)(qrow + 16 * c + 8 * hf);
            qf[qb][c] = __builtin_bit_cast(v8, x);
        }
    }

    // Online-softmax state per row, log2 domain. m_run is the running row max;
    // m_used is the max the exponentials and O are currently referred to. O and
    // l are only rescaled when m_run exceeds m_used by more than kTau, so
    // p = 2^(t - m_used) <= 2^kTau and the rescale is rare after the first tiles.
    f32x16 o[T::NQB][ODT];
    float m_run[T::NQB], m_used[T::NQB], l_run[T::NQB];
    // bfloat16 P: q_run bounds the sum of squares of the weights O holds without the
    // remainder correction (scaled with l); l_stop is l when that bookkeeping last paused;
    // m_tile is the current tile's row max (log2 domain, scaled)
    float q_run[T::NQB], l_stop[T::NQB], m_tile[T::NQB];
#pragma unroll
    for (int qb = 0; qb < T::NQB; qb++) {
        m_run[qb] = -INFINITY;
        m_used[qb] = -INFINITY;
        l_run[qb] = 0.f;
        q_run[qb] = 0.f;
        l_stop[qb] = 0.f;
        m_tile[qb] = -INFINITY;
#pragma unroll
        for (int dt = 0; dt < ODT; dt++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[qb][dt][r] = 0.f;
    }

    // ---- K/V tiles: buffer loads straight into LDS (no register staging) ----
    // Rows past k_len lie outside the buffer range, so the hardware writes zeros
    // for them: padding (even NaN) never reaches the MFMAs.
    const uint16_t* kbase = p.k + (k_off * p.Hkv + hk) * (long long)p.D;
    const uint16_t* vbase = p.v + (k_off * p.Hkv + hk) * (long long)p.Dv;
    const int krow_bytes = p.Hkv * p.D * 2;   // bytes between consecutive keys of K
    const int vrow_bytes = p.Hkv * p.Dv * 2;  // and of V
    auto kstage = [&](int st) __attribute__((always_inline)) { return smem + st * 2 * T::TILE_BYTES; };
    auto vstage = [&](int st) __attribute__((always_inline)) { return smem + st * 2 * T::TILE_BYTES + T::TILE_BYTES; };

    auto issue_tile = [&](const uint16_t* base, int kb, char* dst, bool is_v) __attribute__((always_inline)) {
        const int j0 = kb * T::BN;
        // every field of the descriptor is wave-uniform; saying so keeps the loads
        // free of the per-lane "waterfall" the compiler would otherwise wrap them in
        const int row_bytes = is_v ? vrow_bytes : krow_bytes;
        const int ng = (is_v ? p.Dv : p.D) >> 3;  // granules of a row that hold data
        const int nrec = __builtin_amdgcn_readfirstlane(max(0, min(T::BN, k_len - j0)) * row_bytes);
        const uint64_t addr = (uint64_t)((const char*)base + (long long)j0 * row_bytes);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(((uint64_t)hi << 32) | lo), (short)0, nrec, 0x00020000);
        // this lane's offset for the first load instruction; where later ones only
        // add whole rows (the swizzle repeats every key step), they add a scalar
        constexpr int KSTEP = T::NT / T::NG;  // keys between consecutive instructions of a tile
        constexpr bool K_ADD = (KSTEP % (T::SWZ_DIV * T::NG)) == 0;
        int off0;
        {
            const int g = 64 * wave + lane;
            int key, c;
            if (!is_v) {
                key = g / T::NG;
                c = (g % T::NG) ^ ((key / T::SWZ_DIV) % T::NG);
            } else {
                key = (g / (4 * T::NG)) * 4 + (g & 3);
                c = (g >> 2) % T::NG;
            }
            // columns past D (Dv): an offset past any range, so the load writes zeros
            off0 = c < ng ? key * row_bytes + c * 16 : kOobOffset;
        }
        if (T::LEAN) asm volatile("" : "+v"(off0));  // formed per tile, not held across the loop
#pragma unroll
        for (int u = 0; u < T::LOADS; u++) {
            const int g0 = T::NT * u + 64 * wave;  // first granule of this wave's instruction
            if (T::GRANULES % T::NT == 0 || g0 < T::GRANULES) {
                int off;
                if (T::LEAN && (is_v || K_ADD)) {
                    off = off0 + u * KSTEP * row_bytes;
                } else {
                    const int g = g0 + lane;
                    int key, c;
                    if (!is_v) {
                        key = g / T::NG;
                        c = (g % T::NG) ^ ((key / T::SWZ_DIV) % T::NG);
                    } else {
                        key = (g / (4 * T::NG)) * 4 + (g & 3);
                        c = (g >> 2) % T::NG;
                    }
                    off = c < ng ? key * row_bytes + c * 16 : kOobOffset;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + g0 * 16), 16, off, 0, 0, 0);
            }
        }
    };

    // S^T = K Q^T for one key tile
    auto qk = [&](const char* kl, STile& s) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) s[qb][kb2][r] = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < T::NKB; kb2++) {
            // the swizzle puts granule 2c + hf of a key at (granule hf) ^ 2c, so the
            // byte offsets of a lane's reads differ by an XOR with 32c from the first
            int a0 = k_granule<D>(l32, hf) * 16;
            if (T::LEAN) asm volatile("" : "+v"(a0));  // formed per tile, not held across the loop
            const char* base = kl + kb2 * 32 * T::NG * 16;
            // all reads of a 32-key block go out before its MFMAs (the compiler
            // barrier keeps them from being sunk back to their uses), so each MFMA
            // finds its operand landed instead of waiting out the LDS latency
            v8 ka[NCK];
#pragma unroll
            for (int c = 0; c < NCK; c++)
                ka[c] = T::LEAN ? *(const v8*)(base + (a0 ^ (32 * c)))
                                : *(const v8*)(kl + k_granule<D>(kb2 * 32 + l32, 2 * c + hf) * 16);
#pragma unroll
            for (int c = 0; c < NCK; c++)
#pragma unroll
                for (int qb = 0; qb < T::NQB; qb++) s[qb][kb2] = E::mma(ka[c], qf[qb][c], s[qb][kb2]);
        }
        // Order: the first block's reads, then each MFMA followed by one read of the
        // next block (into the registers it just freed), then the last block's MFMAs
        // (left alone, the compiler read the second block one fragment at a time, each
        // read waited for just before its MFMA; measured c5a -5%, c5b -3% time).
        __builtin_amdgcn_sched_group_barrier(0x100, NCK, 0);
#pragma unroll
        for (int g = 0; g < (T::NKB - 1) * NCK; g++) {
            __builtin_amdgcn_sched_group_barrier(0x008, T::NQB, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, T::NQB * NCK, 0);
    };

    auto partner_max = [](float x) __attribute__((always_inline)) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    auto partner_sum = [](float x) __attribute__((always_inline)) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    };
    // Head-dim class 16: columns 16..31 of the one 32-column block of O^T are padding, so
    // the V^T fragment feeds ones into column 16 and the PV MFMA accumulates there each
    // row's sum of the rounded weights it multiplies V by: the normaliser takes no VALU
    // adds, and a rescale of O rescales it too. Lane half 0 holds column 16 (o[qb][0][8]);
    // in half 1 that register is column 20, which stays 0, so the partner sum broadcasts it.
    // Elsewhere each lane half holds half of a row's sum in l_run.
    constexpr bool LSUM = D == 16;
    auto row_l = [&](int qb) __attribute__((always_inline)) {
        if constexpr (LSUM) return partner_sum(o[qb][0][8]);
        else return partner_sum(l_run[qb]);
    };

    // Raise m_used to m_run in the rows where it fell more than kTau behind; l is
    // rescaled here, O later (once, just before PV) by alpha. The decision is per
    // row, so a row's arithmetic never depends on the other rows of its wave; the
    // O multiply runs when any row of the wave needs it (alpha = 1 elsewhere).
    float alpha[T::NQB];
    bool rescale_o = false;
    auto update_used_max = [&]() __attribute__((always_inline)) {
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            alpha[qb] = 1.f;
            if (m_run[qb] > m_used[qb] + kTau) {  // false while nothing is visible (m_run = -inf)
                alpha[qb] = __builtin_amdgcn_exp2f(m_used[qb] - m_run[qb]);
                m_used[qb] = m_run[qb];
                l_run[qb] *= alpha[qb];
                q_run[qb] *= alpha[qb] * alpha[qb];
                l_stop[qb] *= alpha[qb];
                need = true;
            }
        }
        rescale_o = __any(need);
    };
    auto rescale_acc = [&]() __attribute__((always_inline)) {
        if (rescale_o) {
            // keeps this rare block a real branch (not speculated into every tile)
            asm volatile("; O rescale" ::: "memory");
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
                for (int dt = 0; dt < ODT; dt++) {
                    // At class 256 (O in AGPRs, more than 256 registers a wave) the block is
                    // pinned to AGPRs on both sides of its multiply: without the first pin the
                    // compiler copied all of O to VGPRs at the top of every key-loop iteration
                    // for this rare block (c5a -7.5% time with it, 443 -> 328 registers a wave)
                    f32x16 x = o[qb][dt];
                    if (D == 256) asm volatile("" : "+a"(x));
                    x *= alpha[qb];
                    if (D == 256) asm volatile("" : "+a"(x));
                    o[qb][dt] = x;
                }
        }
    };

    // Each tile's softmax runs in two phases around the (rare) O rescale:
    // phase 1 updates the row maxima and decides the rescale, phase 2 turns the
    // scores into p = 2^(s * c2 + b - m_used) and adds them to l.
    //
    // Unmasked tile, positive scale: the max of s * c2 is max(s) * c2 exactly
    // (rounding is monotonic), and p is one FMA + exp2.
    auto max_fast = [&](STile& s) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[qb][kb2][r]);
            m_tile[qb] = partner_max(mx) * p.c2;
            m_run[qb] = fmaxf(m_run[qb], m_tile[qb]);
        }
    };
    auto exp_fast = [&](STile& s) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            const float mu = m_used[qb];
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    s[qb][kb2][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb2][r], p.c2, -mu));
        }
    };

    // Tiles that cross the key bound, the causal diagonal or the bias band (or scale <= 0).
    // Per element the arithmetic is the fast path's (one FMA into exp2, with the
    // bias term folded into the addend), so the result of a row does not depend on
    // which path a tile takes; masked keys get p = 0. Band tiles and the other
    // masked tiles take separate passes, so no per-element test of the tile's kind.
    // The bias of a band tile is read once, at the start of the tile step and
    // before that step's K/V prefetch goes out (waiting for these loads then does
    // not wait for the prefetch), into 16-bit pairs, with the mask folded in:
    // visible elements outside the band hold 0, masked ones the dtype's -inf.
    typedef uint32_t BiasBits[T::NQB][T::NKB][8];
    // Visibility without per-element index arithmetic: key j = j0 + 32 kb2 + acc_row(r, hf)
    // of row i is visible iff j < k_len and (causal) j <= i + delta, i.e. iff its
    // offset 8 (r >> 2) + (r & 3) (the lane's 4 hf moved to the other side) is at most
    // one per-lane limit per 32-key block; the offsets are immediates, so each test is
    // one compare.
    typedef int VisLim[T::NQB][T::NKB];
    auto vis_limits = [&](VisLim& lim, int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            const int last = CAUSAL ? min(k_len - 1, qi[qb] + delta) : k_len - 1;  // last visible key
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++) lim[qb][kb2] = last - (j0 + kb2 * 32) - 4 * hf;
        }
    };
    auto lim_vis = [](const VisLim& lim, int qb, int kb2, int r) __attribute__((always_inline)) {
        return 8 * (r >> 2) + (r & 3) <= lim[qb][kb2];
    };
    auto bias_row = [&](int qb) __attribute__((always_inline)) {
        return BIAS ? p.bias + ((q_off + qi[qb]) * p.Hq + qh[qb]) * (long long)p.E : nullptr;
    };
    // fused producer: per band tile, each wave's bias values in LDS past the ring (32 rows x BN)
    const bool fused_bias = BIAS && p.rel_r != nullptr;
    uint16_t* bias_lds = (uint16_t*)(smem + T::LDS);
    // Every element reads its bias at a clamped index (inside the row) and the band
    // test selects with bit masks, so each read is used whatever the test gives:
    // the reads need no branches and go out together.
    auto load_bias_from = [&](BiasBits& bb, int j0, auto row_of) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            const auto brow = row_of(qb);
            const int i = qi[qb];
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r2 = 0; r2 < 8; r2++) {
                    uint32_t w = 0;
#pragma unroll
                    for (int e = 0; e < 2; e++) {
                        const int j = j0 + kb2 * 32 + acc_row(2 * r2 + e, hf);
                        const int d = i + delta - j;
                        const uint32_t v = brow[min(max(d, 0), p.E - 1)];
                        const bool vis = (j < k_len) && (!CAUSAL || j <= i + delta);
                        const bool keep = vis && qvalid[qb] && d >= 0 && d < p.E;
                        // masked: the -inf of the dtype; visible outside the band: 0
                        const uint32_t h = (v & (keep ? 0xFFFFu : 0u)) | (vis ? 0u : (uint32_t)E::kNegInfBits);
                        w |= h << (16 * e);
                    }
                    bb[qb][kb2][r2] = w;
                }
        }
    };
    // From HBM. A lane's elements come in groups of four consecutive keys (r = 4g ..
    // 4g + 3), whose d are four consecutive values of one bias row, highest d first;
    // each group is one 12-byte read from the dword boundary at or below its lowest d
    // (all of a lane's groups share that d's parity, so one funnel shift per word pair
    // puts the four values in place), all at one per-lane offset plus an immediate.
    // Within a lane the d of a tile's elements fall in a window of CMAX + 1 values
    // below d0, and over the lanes of a band tile d0 >= -35, so with the descriptor
    // starting one bias row before the wave's first row (first >= 1) every offset is
    // positive; a read reaches at most two values past a group, which stay inside the
    // tensor unless the wave holds its last row (then, as when the wave holds the first
    // row or its rows span more than 2^31 bytes of bias, the reads take clamped
    // indices). Values outside the band are masked whatever they hold.
    auto load_bias_global = [&](BiasBits& bb, int j0, long long base_row) __attribute__((always_inline)) {
        constexpr int CMAX = (T::NKB - 1) * 32 + 27;  // largest key offset within the tile, less 4hf
        constexpr int CG = CMAX - 3;                  // offset of the last group's first key
        const char* base = (const char*)p.bias + base_row * p.E * 2;
        const long long left = ((long long)p.rows_q * p.Hq - base_row) * p.E * 2;
        const int nrec = __builtin_amdgcn_readfirstlane((int)min(left, (long long)INT32_MAX));
        const uint64_t addr = (uint64_t)base;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(((uint64_t)hi << 32) | lo), (short)0, nrec, 0x00020000);
        VisLim lim;
        vis_limits(lim, j0);
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            const int i = qi[qb];
            const long long row = (q_off + i) * p.Hq + qh[qb];
            const int d0 = i + delta - j0 - 4 * hf;  // d of element (kb2, r) is d0 - c(kb2, r)
            // in the band (0 <= d < E, valid row) iff blo <= c <= bhi
            const int bhi = qvalid[qb] ? d0 : -1, blo = d0 - p.E + 1;
            // byte offset of d0 - CMAX, the lowest d of the last group; group (kb2, g) starts
            // 2 (CG - c_g) bytes above it, c_g = 32 kb2 + 8 g (a multiple of 16 bytes)
            const int vo = (int)((row - base_row) * p.E + d0 - CMAX) * 2;
            const int v4 = vo & ~3;
            const int sh = (vo & 2) * 8;  // 16: the group's lowest d is the upper half of a word
            u32x3 raw[T::NKB][4];
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int g = 0; g < 4; g++)
                    raw[kb2][g] = __builtin_bit_cast(
                        u32x3, __builtin_amdgcn_raw_buffer_load_b96(rsrc, v4 + 2 * (CG - kb2 * 32 - 8 * g), 0, 0));
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    // the group's four values in ascending d: (a0, a1) in w_lo, (a2, a3) in w_hi;
                    // element e = r & 3 has d = d0 - c_g - e, i.e. value a(3 - e)
                    const u32x3 x = raw[kb2][g];
                    const uint32_t w_lo = __builtin_amdgcn_alignbit(x[1], x[0], sh);
                    const uint32_t w_hi = __builtin_amdgcn_alignbit(x[2], x[1], sh);
                    const uint32_t pr[2] = {__builtin_amdgcn_alignbit(w_hi, w_hi, 16),   // elements 4g, 4g + 1
                                            __builtin_amdgcn_alignbit(w_lo, w_lo, 16)};  // elements 4g + 2, 4g + 3
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        uint32_t keepm = 0, neg = 0;
#pragma unroll
                        for (int e = 0; e < 2; e++) {
                            const int r = 4 * g + 2 * h2 + e;
                            const int c = kb2 * 32 + 8 * g + 2 * h2 + e;
                            const bool vis = lim_vis(lim, qb, kb2, r);
                            const bool keep = vis && c <= bhi && c >= blo;
                            // masked: the -inf of the dtype; visible outside the band: 0
                            keepm |= (keep ? 0xFFFFu : 0u) << (16 * e);
                            neg |= (vis ? 0u : (uint32_t)E::kNegInfBits) << (16 * e);
                        }
                        bb[qb][kb2][2 * g + h2] = (pr[h2] & keepm) | neg;
                    }
                }
        }
    };
    // the wave's first bias row (a lower bound over its lanes; uniform)
    long long bias_first_row = (q_off + min(w_row, r_last) / gp) * p.Hq + h_base;
    bias_first_row = (long long)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)bias_first_row >> 32)) << 32) |
                                 __builtin_amdgcn_readfirstlane((uint32_t)bias_first_row));
    // and its last (an upper bound: the wave's last query, its last packed head)
    long long bias_last_row = (q_off + wi_hi) * p.Hq + h_base + gp - 1;
    bias_last_row = (long long)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)bias_last_row >> 32)) << 32) |
                                __builtin_amdgcn_readfirstlane((uint32_t)bias_last_row));
    // Fused producer (tml-fa4 page: rel_bias = r . rel_proj, the einsum over d_rel), per
    // band tile, wave and 32-row block. Over the block's rows the tile needs d in
    // [dbase, dbase + BN + 31) with dbase = (block's first query) + delta - j0 - (BN - 1);
    // the MFMA forms C[d][row] = rel_proj^T r^T
    // for that range in 32-d blocks (A = a rel_proj column per lane, zero outside [0, E);
    // B = the lane's r row), so each lane ends up holding values of its own row. Rounded
    // to the dtype (as a materialised rel_bias is), they go to the row's LDS slot of BN
    // values, slot u holding d = dbase + (query - first query) + u: the first and the last block
    // share the slots (u = (m - off) mod BN takes the first block's value for m >= off,
    // the last one's below), the blocks between fill theirs whole, so every write is
    // unconditional. The tile's elements then read their d at a fixed u per element.
    auto produce_bias = [&](BiasBits& bb, int j0) __attribute__((always_inline)) {
        constexpr int NBLK = T::NKB + 1;  // 32-d blocks covering BN + 31 values
        // opaque copies: the addresses below are formed per tile instead of being
        // hoisted out of the key loop into registers held across it
        int E_ = p.E, drel = p.d_rel;
        asm volatile("" : "+s"(E_), "+s"(drel));
        const uint16_t* proj = p.rel_proj;
        VisLim lim;
        vis_limits(lim, j0);
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            // this row block's first query (rows past the last one repeat it)
            const int blo = min(w_row + 32 * qb, r_last) / gp;
            const int dbase = blo + delta - j0 - (T::BN - 1);
            const int i = qi[qb];
            const int off = i - blo;  // 0 .. 31
            uint16_t* slot = bias_lds + ((wave * T::NQB + qb) * 32 + l32) * T::BN;
            const uint16_t* rrow = p.rel_r + ((q_off + i) * p.Hq + qh[qb]) * (long long)drel;
            auto block = [&](int b) __attribute__((always_inline)) {
                f32x16 c = {};
                const int dcol = dbase + 32 * b + l32;  // the A row (d) this lane provides
                const bool din = dcol >= 0 && dcol < E_;
                const uint16_t* pcol = proj + min(max(dcol, 0), E_ - 1);
                for (int k0 = 0; k0 < drel; k0 += 16) {
                    const int ka = k0 + 8 * hf;  // this lane's 8 contraction indices
                    u32x4 bw = {0u, 0u, 0u, 0u};
                    if (ka < drel) bw = *(const u32x4*)(rrow + ka);
                    u32x4 aw = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const int k1 = min(ka + e, drel - 1), k2 = min(ka + e + 1, drel - 1);
                        const uint32_t v1 = pcol[k1 * E_];
                        const uint32_t v2 = pcol[k2 * E_];
                        const uint32_t keep1 = din && ka + e < drel ? 0xFFFFu : 0u;
                        const uint32_t keep2 = din && ka + e + 1 < drel ? 0xFFFFu : 0u;
                        aw[e >> 1] = (v1 & keep1) | ((v2 & keep2) << 16);
                    }
                    c = E::mma(__builtin_bit_cast(v8, aw), __builtin_bit_cast(v8, bw), c);
                }
                return c;
            };
            {
                const f32x16 cf = block(0), cl = block(NBLK - 1);
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = acc_row(r, hf);
                    slot[(m - off) & (T::BN - 1)] = E::narrow(m >= off ? cf[r] : cl[r]);
                }
            }
#pragma unroll
            for (int b = 1; b < NBLK - 1; b++) {
                const f32x16 c = block(b);
#pragma unroll
                for (int r = 0; r < 16; r++) slot[32 * b + acc_row(r, hf) - off] = E::narrow(c[r]);
            }
            // element (kb2, r) of the lane: u = BN - 1 - kb2 * 32 - acc_row(r, hf); a group of
            // four (r = 4g .. 4g + 3) is one aligned 8-byte read, its values in reverse order
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int u_lo = T::BN - 4 - kb2 * 32 - 8 * g - 4 * hf;
                    const u32x2 x = *(const u32x2*)(slot + u_lo);
                    const uint32_t pr[2] = {__builtin_amdgcn_alignbit(x[1], x[1], 16),  // elements 4g, 4g + 1
                                            __builtin_amdgcn_alignbit(x[0], x[0], 16)}; // elements 4g + 2, 4g + 3
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        uint32_t w = 0;
#pragma unroll
                        for (int e = 0; e < 2; e++) {
                            const int r = 4 * g + 2 * h2 + e;
                            const bool vis = lim_vis(lim, qb, kb2, r);
                            const uint32_t v = (pr[h2] >> (16 * e)) & 0xFFFFu;
                            // masked: the -inf of the dtype; values outside [0, E) came out 0
                            w |= (vis ? v : (uint32_t)E::kNegInfBits) << (16 * e);
                        }
                        bb[qb][kb2][2 * g + h2] = w;
                    }
                }
        }
    };
    auto load_bias = [&](BiasBits& bb, int j0) __attribute__((always_inline)) {
        if (fused_bias)
            produce_bias(bb, j0);
        else if (bias_first_row >= 1 && bias_last_row + 1 < p.rows_q * p.Hq &&
                 p.E > (T::NKB - 1) * 32 + 27 + 35 && (long long)(T::BM + 2) * p.Hq * p.E * 2 < INT32_MAX)
            load_bias_global(bb, j0, bias_first_row - 1);  // (offsets fit 31 bits)
        else
            load_bias_from(bb, j0, [&](int qb) { return bias_row(qb); });
    };
    // A band tile's terms were formed with the mask folded in (masked keys hold -inf).
    auto band_term = [&](int qb, int kb2, int r, const BiasBits& bb) __attribute__((always_inline)) {
        return E::widen((uint16_t)(bb[qb][kb2][r >> 1] >> (16 * (r & 1)))) * kLog2e;
    };
    auto max_band = [&](STile& s, const BiasBits& bb) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    // a masked key's term is -inf, and so is the FMA (scores are finite)
                    mx = fmaxf(mx, __builtin_fmaf(s[qb][kb2][r], p.c2, band_term(qb, kb2, r, bb)));
                }
            m_tile[qb] = partner_max(mx);
            m_run[qb] = fmaxf(m_run[qb], m_tile[qb]);
        }
    };
    auto exp_band = [&](STile& s, const BiasBits& bb) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            const float mu = m_used[qb] == -INFINITY ? 0.f : m_used[qb];
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++)  // exp2(-inf) = 0 for a masked key
                    s[qb][kb2][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb2][r], p.c2, band_term(qb, kb2, r, bb) - mu));
        }
    };
    // (a visible key's term is 0: the same FMA as the fast path, s * c2 - mu)
    // Each masked pass takes its own copy of the limits through an empty asm: otherwise the
    // compiler may form the 32 visibility compares per lane once, ahead of the tile-kind
    // branch, and keep the masks in scalar register pairs for both passes -- at head-dim
    // class 16 that spilled 144 scalar registers to vector lanes and ran the compares and
    // the spills on every tile (c4b +27% time).
    auto pin_limits = [](VisLim& lm, const VisLim& lim) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++) {
                lm[qb][kb2] = lim[qb][kb2];
                asm volatile("" : "+v"(lm[qb][kb2]));
            }
    };
    auto max_mask = [&](STile& s, const VisLim& lim_in) __attribute__((always_inline)) {
        VisLim lim;
        pin_limits(lim, lim_in);
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    mx = fmaxf(mx, lim_vis(lim, qb, kb2, r) ? __builtin_fmaf(s[qb][kb2][r], p.c2, 0.f) : -INFINITY);
            m_tile[qb] = partner_max(mx);
            m_run[qb] = fmaxf(m_run[qb], m_tile[qb]);
        }
    };
    auto exp_mask = [&](STile& s, const VisLim& lim_in) __attribute__((always_inline)) {
        VisLim lim;
        pin_limits(lim, lim_in);
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            const float mu = m_used[qb] == -INFINITY ? 0.f : m_used[qb];
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    s[qb][kb2][r] = lim_vis(lim, qb, kb2, r)
                                        ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb2][r], p.c2, -mu)) : 0.f;
        }
    };

    // P in the dtype, as the B operand of O^T += V^T P^T: step t (16 keys) of row block
    // qb holds the exponentials of S^T registers [t / 2][8 (t % 2) .. + 7]
    auto p_step = [&](const STile& s, int qb, int t) __attribute__((always_inline)) {
        v8 x;
#pragma unroll
        for (int e = 0; e < 8; e++) x[e] = E::to_elem(s[qb][t >> 1][8 * (t & 1) + e]);
        return x;
    };
    // Row sums of a tile's weights, one fixed order whatever the path: per 32-key block a
    // chain over the block's two steps, pairs in order, then a tree over the blocks into l.
    // bfloat16: the sum of the rounded weights the PV MFMA uses (one v_dot2 with (1, 1)
    // per pair), so l normalises exactly the weights O was built from. IEEE half: the
    // fp32 exponentials (pair sums of half values would lose those below the half
    // normal range).
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    auto sum_pair = [&](float acc, const STile& s, const v8& pt, int qb, int t, int i) __attribute__((always_inline)) {
        if constexpr (BF) {
            // (the pair is built from its two elements: taking it as a 32-bit word of the
            // bit-cast vector has compiled to the first pair for every i)
            const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
            const bf16x2 x = {pt[2 * i], pt[2 * i + 1]};
            return __builtin_amdgcn_fdot2_f32_bf16(x, one2, acc, false);
        } else {
            acc += s[qb][t >> 1][8 * (t & 1) + 2 * i];
            return acc + s[qb][t >> 1][8 * (t & 1) + 2 * i + 1];
        }
    };
    auto sums_into_l = [&](float (&rs)[T::NKB], int qb) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 1; w < T::NKB; w *= 2)
#pragma unroll
            for (int kb2 = 0; kb2 + w < T::NKB; kb2 += 2 * w) rs[kb2] += rs[kb2 + w];
        l_run[qb] += rs[0];
    };

    // which rows take the remainder MFMA for the tile whose exponentials were just added to l
    bool need_lo[T::NQB];
    bool any_lo = false;
    // the remainder test and its bookkeeping run while lo_check holds (wave-uniform)
    bool lo_check = true;
    // this lane's share of a row's l (the lane halves hold disjoint keys of the row)
    auto l_part = [&](int qb) __attribute__((always_inline)) {
        if constexpr (LSUM) return o[qb][0][8];
        else return l_run[qb];
    };
    // The pause test of one row (l and q: row totals relative to m_used): taken to the row
    // max, (l + x)^2 >= (q + x) kLoThresh must hold for every x >= 0, i.e. further weights
    // at or below the max (x: their sum, their squares at most x) cannot bring the row's
    // effective key count below the threshold. Rows without weight pass.
    auto pause_ok = [&](int qb, float lt, float qt) __attribute__((always_inline)) {
        const float f = __builtin_amdgcn_exp2f(m_used[qb] - m_run[qb]);
        const float l1 = lt * f, q1 = qt * f * f;
        const float slack = l1 * l1 - q1 * kLoThresh, b = kLoThresh - 2.f * l1;
        return !(lt > 0.f) || (slack >= 0.f && (b <= 0.f || 4.f * slack >= b * b));
    };
    // Some row max grew (m_prev: the maxima before, m_run: after) while the test was
    // paused. If every row's l, taken to the new max, is still at least kLoThresh, the
    // pause holds as it is: any q is at most l there (no weight exceeds the max), which
    // passes pause_ok, and the weights added since the pause stay covered by the bound
    // below, taken at a later resume with a larger max. Otherwise the weights added since
    // the pause, each at most 2^(m_prev - m_used), add at most that times their sum to the
    // squares: q_run takes that bound, and the pause test runs against the new max; the
    // test resumes if a row fails it or has just seen its first keys. (A rescale scales
    // l_stop with l.)
    auto lo_resume = [&](const float (&m_prev)[T::NQB]) __attribute__((always_inline)) {
        if (BF && !lo_check) {
            bool low = false;
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++)
                low = low || row_l(qb) * __builtin_amdgcn_exp2f(m_used[qb] - m_run[qb]) < kLoThresh;
            if (__any(low)) {
                bool stay = false;
#pragma unroll
                for (int qb = 0; qb < T::NQB; qb++) {
                    const bool had = m_prev[qb] > -INFINITY;
                    if (had) q_run[qb] += __builtin_amdgcn_exp2f(m_prev[qb] - m_used[qb]) * (l_part(qb) - l_stop[qb]);
                    l_stop[qb] = l_part(qb);
                    stay = stay || (!had && m_run[qb] > -INFINITY) || !pause_ok(qb, row_l(qb), partner_sum(q_run[qb]));
                }
                lo_check = __any(stay);
            }
        }
    };
    // V^T fragment (A operand of O^T += V^T P^T) for keys 16t.. and dv block dt:
    // lanes of group g = lane / 16 receive dv = 32dt + 16(g&1) + lane%16, keys
    // 16t + 4hf (+8), via two ds_read_b64_tr_b16 of the 4-key-blocked V tile.
    const int vg = lane >> 4, vj = lane & 15;
    auto vfrag = [&](const char* vl, int t, int dt) __attribute__((always_inline)) {
        int dv0 = 32 * dt + 16 * (vg & 1);
        const bool dv_ok = dv0 < D;
        if (!dv_ok) dv0 = 0;  // D = 16: the upper half of the dv block is padding
        const int kq = 4 * t + hf;  // (16t + 4hf) / 4
        const char* pa = vl + v_granule<D>(4 * kq + (vj >> 2), (dv0 >> 3) + ((vj & 3) >> 1)) * 16 + (vj & 1) * 8;
        const char* pb = pa + 2 * T::NG * 4 * 16;  // keys + 8 = two 4-key blocks later
        const s16x4v ra = lds_read_tr16((const lds_s16x4*)pa);
        const s16x4v rb = lds_read_tr16((const lds_s16x4*)pb);
        u32x4 w;
        w[0] = __builtin_bit_cast(u32x2, ra)[0];
        w[1] = __builtin_bit_cast(u32x2, ra)[1];
        w[2] = __builtin_bit_cast(u32x2, rb)[0];
        w[3] = __builtin_bit_cast(u32x2, rb)[1];
        if (!dv_ok) {
            // class 16: ones in column 16 (the row sums), zeros in 17..31
            const uint32_t f = LSUM && vj == 0 ? E::kOnePairBits : 0u;
            w = u32x4{f, f, f, f};
        }
        return __builtin_bit_cast(v8, w);
    };
    // bf16 P carries a relative rounding error of up to 2^-8 per weight; where few keys
    // hold a row's weight that error can reach the output tolerance, so such rows also
    // feed the remainder P - bf16(P) through the MFMA (after the tile's main product; its
    // rounded weights join l).
    auto pv_rem = [&](const char* vl, const STile& s) __attribute__((always_inline)) {
        if constexpr (BF) {
            // rare: only while some row of the wave has a small normaliser
            asm volatile("; P remainder" ::: "memory");
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) {
                float rs[T::NKB];
#pragma unroll
                for (int kb2 = 0; kb2 < T::NKB; kb2++) rs[kb2] = 0.f;
#pragma unroll
                for (int t = 0; t < T::BN / 16; t++) {
                    const v8 pt = p_step(s, qb, t);
                    v8 ptl;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const float pvv = s[qb][t >> 1][8 * (t & 1) + e];
                        ptl[e] = E::to_elem(need_lo[qb] ? pvv - (float)pt[e] : 0.f);
                    }
#pragma unroll
                    for (int dt = 0; dt < ODT; dt++) o[qb][dt] = E::mma(vfrag(vl, t, dt0 + dt), ptl, o[qb][dt]);
                    if constexpr (!LSUM)
#pragma unroll
                        for (int i = 0; i < 4; i++) rs[t >> 1] = sum_pair(rs[t >> 1], s, ptl, qb, t, i);
                }
                if constexpr (!LSUM) sums_into_l(rs, qb);  // (zero for the rows that skip it)
            }
        }
    };
    // The remainder test, after a tile's weights have joined l (l0: this lane's share of l
    // before). The rounding errors of the weights O holds uncorrected add up to a relative
    // error in O with a spread of at most about 2^-8 / sqrt(3 n), n = l^2 / q their
    // effective key count (q: the sum of their squares; no rescale changes the ratio). q is
    // kept as a bound: a tile adds at most its row max weight times its row sum. A row
    // whose bound on n would fall below kLoThresh with this tile takes the remainder for
    // the tile; the others add the tile's term to q_run. The bookkeeping pauses once every
    // row passes pause_ok; a new row max tests again (lo_resume).
    auto lo_step = [&](const char* vl, const STile& s, const float (&l0)[T::NQB]) __attribute__((always_inline)) {
        if (BF && lo_check) {
            float lt[T::NQB], qt[T::NQB];
            bool any = false;
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) {
                const float ts = l_part(qb) - l0[qb];  // this lane's share of the tile's row sum
                const float t2 = ts > 0.f ? __builtin_amdgcn_exp2f(m_tile[qb] - m_used[qb]) * ts : 0.f;
                const float qn = q_run[qb] + t2;
                lt[qb] = row_l(qb);
                qt[qb] = partner_sum(qn);
                need_lo[qb] = qt[qb] * kLoThresh > lt[qb] * lt[qb];
                if (!need_lo[qb]) q_run[qb] = qn;
                any = any || need_lo[qb];
            }
            any_lo = __any(any);
            // (the pause test is evaluated either way: O stays out of the branches)
            bool stay = any;
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) stay = stay || !pause_ok(qb, lt[qb], qt[qb]);
            lo_check = __any(stay);
            // pausing: no row took the remainder, so l is final for the tile
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) l_stop[qb] = lo_check ? l_stop[qb] : l_part(qb);
            if (any_lo) pv_rem(vl, s);
        }
    };
    // O^T += V^T P^T, 16 keys per MFMA step, with P formed and summed into l step by
    // step; then the remainder test on the updated l
    auto pv = [&](const char* vl, const STile& s) __attribute__((always_inline)) {
        float l0[T::NQB];
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) l0[qb] = BF ? l_part(qb) : 0.f;
        float rs[T::NQB][T::NKB];
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++) rs[qb][kb2] = 0.f;
#pragma unroll
        for (int t = 0; t < T::BN / 16; t++) {
            v8 pt[T::NQB];
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) pt[qb] = p_step(s, qb, t);
#pragma unroll
            for (int dt = 0; dt < ODT; dt++) {
                const v8 a = vfrag(vl, t, dt0 + dt);
#pragma unroll
                for (int qb = 0; qb < T::NQB; qb++) o[qb][dt] = E::mma(a, pt[qb], o[qb][dt]);
            }
            if constexpr (!LSUM)
#pragma unroll
                for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
                    for (int i = 0; i < 4; i++) rs[qb][t >> 1] = sum_pair(rs[qb][t >> 1], s, pt[qb], qb, t, i);
        }
        if constexpr (D != 16) {
            // Order: the reads of two V^T fragments ahead of the MFMA that uses the first
            // (two transposing reads per fragment), one fragment's reads after each MFMA
            // (measured: c5a -7%, n1a -3%, c2 -1% time; at head-dim class 16, where the
            // softmax dominates, +2.5% on c4b, so not there)
            constexpr int NF = T::BN / 16 * ODT, AHEAD = NF < 2 ? NF : 2;
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 1);
#pragma unroll
            for (int n = 0; n < NF - AHEAD; n++) {
                __builtin_amdgcn_sched_group_barrier(0x008, T::NQB, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, T::NQB * AHEAD, 1);
        }
        if constexpr (!LSUM)
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) sums_into_l(rs[qb], qb);
        lo_step(vl, s, l0);
    };

    // ---- main loop over key tiles ----
    // Tile j (its K and V) lives in ring stage (j - kb_begin) % NB and is loaded
    // PREFETCH iterations before it is used. Iteration j: loads of tile
    // j + PREFETCH go out; S^T = K Q^T; softmax; O^T += V^T P^T; then each wave
    // waits until tile j+1 has landed (vmcnt counts this wave's buffer loads,
    // which complete in order) and the work-group meets at one barrier.
    auto wait_tiles_after_next = [&](int n_after) __attribute__((always_inline)) {
        // s_waitcnt vmcnt(n_after * VM_PER_TILE), n_after <= PREFETCH - 1
        constexpr int L = T::VM_PER_TILE;
        static_assert((T::PREFETCH - 1) * L < 64, "vmcnt field");
        if (T::PREFETCH <= 1 || n_after <= 0) wait_vm_loads<0>();
        else if (T::PREFETCH == 2 || n_after == 1) wait_vm_loads<L>();
        else if (T::PREFETCH == 3 || n_after == 2) wait_vm_loads<2 * L>();
        else wait_vm_loads<3 * L>();
    };
    static_assert(T::PREFETCH >= 1 && T::PREFETCH <= 4, "wait_tiles_after_next covers up to three later tiles");
    auto issue = [&](int j, int st) __attribute__((always_inline)) {
        issue_tile(kbase, j, kstage(st), false);
        issue_tile(vbase, j, vstage(st), true);
    };
    // one key tile; st = (kb - kb_begin) % NB is a literal at every call site, so all
    // LDS addresses are a per-lane base plus an immediate offset
    auto tile_step = [&](int kb, int st) __attribute__((always_inline)) {
        if (!BIAS && kb + T::PREFETCH < kb_end) issue(kb + T::PREFETCH, (st + T::PREFETCH) % T::NB);
        const int j0 = kb * T::BN;
        const bool need_mask = (j0 + T::BN > k_len) || (CAUSAL && (j0 + T::BN - 1 > wi_lo + delta));
        const bool band = BIAS && (wi_hi + delta - j0 >= 0) && (wi_lo + delta - (j0 + T::BN - 1) < p.E);
        BiasBits bb;
        if (BIAS) {
            if (band) load_bias(bb, j0);
            if (kb + T::PREFETCH < kb_end) issue(kb + T::PREFETCH, (st + T::PREFETCH) % T::NB);
        }
        // At D = 256 (decode, 8:1 pack-GQA) a wave with no rows in this tile, or
        // whose rows see none of its keys (below the causal diagonal), only loads.
        // (At smaller head dims the branch around the accumulators costs more
        // than it saves.)
        if (D != 256 || (wave_live && (!CAUSAL || j0 <= wi_hi + delta))) {
            STile s;
            // Class 128: the waves raise their priority while issuing the tile's MFMAs, so
            // a wave with MFMAs ready goes before the other wave's softmax on the SIMD
            // (two independent work-groups per CU on this loop; varlen causal GQA + bias
            // -1.7%, its fused-producer form -2.9% time; at class 16 +1.8%, so not there)
            constexpr bool PRIO = D == 128;
            if (PRIO) __builtin_amdgcn_s_setprio(1);
            qk(kstage(st), s);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
            // Three kinds of tile (unmasked, band, other masked), each softmax pass
            // chosen once per tile by a uniform branch. O is only touched in
            // straight-line code (the rescale and PV), so the branches merge no
            // accumulator state.
            const bool fast = !need_mask && !band && p.c2 > 0.f;
            const bool banded = BIAS && band;
            VisLim lim;
            if (!fast && !banded) vis_limits(lim, j0);
            float m_prev[T::NQB];
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) m_prev[qb] = m_run[qb];
            if (fast) max_fast(s);
            else if (banded) max_band(s, bb);
            else max_mask(s, lim);
            if (BF && !lo_check) {
                bool grew = false;
#pragma unroll
                for (int qb = 0; qb < T::NQB; qb++) grew = grew || m_run[qb] > m_prev[qb];
                if (__any(grew)) lo_resume(m_prev);
            }
            update_used_max();
            rescale_acc();
            if (fast) exp_fast(s);
            else if (banded) exp_band(s, bb);
            else exp_mask(s, lim);
            if (PRIO) __builtin_amdgcn_s_setprio(1);
            pv(vstage(st), s);
            if (PRIO) __builtin_amdgcn_s_setprio(0);
        }
        // tiles issued after kb+1: kb+2 .. min(kb+PREFETCH, kb_end-1)
        wait_tiles_after_next(min(kb + T::PREFETCH, kb_end - 1) - (kb + 1));
        __syncthreads();
    };
    // ---- software-pipelined run over the leading tiles that no wave of the work-group masks ----
    // Iteration r (K of tile r+1 and V of tile r in LDS): the MFMAs form S^T of tile r+1
    // while the VALU turns tile r's scores into exponentials (stage A), then the MFMAs add
    // tile r's P V to O while the VALU converts P, sums it into l and forms the row maxima
    // of tile r+1 (stage B). The per-row arithmetic is tile_step's, in the same order, so
    // a row's result does not depend on which tiles take this run. K runs one tile ahead
    // of V in the ring: with PF = PREFETCH, iteration r loads K of tile r+1+PF into the
    // slot tile r's K left and V of tile r+PF into the slot of tile r-1's V. The two S^T
    // tiles swap registers every iteration, so no accumulator is copied.
    // Only without the causal mask and the relative bias: there the run covers each row
    // tile's whole key range. With them every row tile ends its run within a few tiles of
    // the diagonal or the band, and the run's last step (which spills registers) plus the
    // hand-over to tile_step cost more than the run saves (varlen causal GQA, 8 sequences
    // of 512 .. 8192 tokens: +10% time).
    constexpr bool PIPE = (D == 64 || D == 128) && (T::NB == 2 || T::NB == 4) && !BIAS && !CAUSAL;
    constexpr int PF = T::PREFETCH;
    int nf = 0;  // tiles of the run (wave-uniform)
    if (PIPE && kb_begin < kb_end && p.c2 > 0.f) {
        const int wg_lo = row0 / gp;  // the work-group's first query: the most restrictive row
        int lim = k_len / T::BN;      // tiles inside the key range
        if (CAUSAL) {
            const int x = wg_lo + delta + 1;  // tile kb is below every diagonal iff (kb + 1) BN <= x
            lim = min(lim, x > 0 ? x / T::BN : 0);
        }
        if (BIAS) {
            const int x = wg_lo + delta - p.E + 1;  // and before every row's band
            lim = min(lim, x > 0 ? x / T::BN : 0);
        }
        nf = max(0, min(kb_end, lim) - kb_begin);
        // when tile_step takes over, let it start at ring stage 0 (it addresses the ring
        // with literal stages): the last nf % NB tiles of the run go to it instead
        if (nf < kb_end - kb_begin) nf -= nf % T::NB;
    }
    const int ntl = kb_end - kb_begin;  // tiles of this work-group's key range
    // the row maxima of an unmasked tile (raw scores; scaled when committed)
    float mx_next[T::NQB];
    auto raw_max = [&](const STile& s) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[qb][kb2][r]);
            mx_next[qb] = partner_max(mx) * p.c2;
        }
    };
    // Commit the maxima; only a row max that grew can call for a rescale (after one,
    // m_run <= m_used + kTau holds until m_run grows) or resume the remainder test.
    auto commit_max = [&]() __attribute__((always_inline)) {
        bool grew = false;
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) grew = grew || mx_next[qb] > m_run[qb];
        if (__any(grew)) {
            asm volatile("; row max grew" ::: "memory");
            float m_prev[T::NQB];
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) {
                m_prev[qb] = m_run[qb];
                m_run[qb] = fmaxf(m_run[qb], mx_next[qb]);
            }
            lo_resume(m_prev);
            update_used_max();
            rescale_acc();
        }
    };
    // The two stages are written in issue order, one K or V fragment at a time: its
    // MFMAs (one per row block), the LDS reads of a later fragment and a share of the
    // VALU work, each step fenced by a scheduling barrier, so the VALU work runs in the
    // shadow of the MFMAs before it and every fragment is read a few steps ahead of use.
    auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    // stage A: S^T of the next tile (K fragments from LDS); exponentials of the current one
    auto stage_a = [&](const char* kl, STile& sn, STile& sc, const char* vl, v8 (&vpre)[2]) __attribute__((always_inline)) {
        constexpr int NM = T::NKB * NCK;      // fragment steps
        constexpr int NE = 16 * T::NKB;       // exponentials per row block, shared out over the steps
        constexpr int AH = NCK < 4 ? NCK : 4; // fragments read ahead
        auto kread = [&](int g) __attribute__((always_inline)) {
            return *(const v8*)(kl + k_granule<D>((g / NCK) * 32 + l32, 2 * (g % NCK) + hf) * 16);
        };
        v8 ka[NM];
#pragma unroll
        for (int g = 0; g < AH; g++) ka[g] = kread(g);
        fence();
#pragma unroll
        for (int g = 0; g < NM; g++) {
            const int kb2 = g / NCK, c = g % NCK;
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++)
                sn[qb][kb2] = E::mma(ka[g], qf[qb][c], c == 0 ? f32x16{} : sn[qb][kb2]);
            if (g + AH < NM) ka[g + AH] = kread(g + AH);
            // stage B's first two V^T fragments go out in the last two steps, which read no K
            // fragment ahead, so PV finds them landed (c2 -0.3..-1% time, same results)
            if (g == NM - 2) vpre[0] = vfrag(vl, 0, dt0);
            if (g == NM - 1) vpre[1] = vfrag(vl, 1 / ODT, dt0 + 1 % ODT);
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
                for (int e = g * NE / NM; e < (g + 1) * NE / NM; e++)
                    sc[qb][e / 16][e % 16] =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][e / 16][e % 16], p.c2, -m_used[qb]));
            fence();
        }
    };
    // stage B: P V of the current tile (V^T fragments from LDS); P in the dtype, its sums
    // into l (tile_step's order) and the row maxima of the next tile
    auto stage_b = [&](const char* vl, const STile& sn, const STile& sc, bool with_max, const v8 (&vpre)[2], bool pre) __attribute__((always_inline)) {
        constexpr int NTS = T::BN / 16;         // 16-key steps
        constexpr int NM = NTS * ODT;           // fragment steps
        constexpr int AH = 2;                   // fragments read ahead
        constexpr int NX = 16 * T::NKB;         // maxima per row block, shared out over the steps
        v8 pt[T::NQB][NTS];
        auto cvt = [&](int qb, int t, int e) __attribute__((always_inline)) {
            pt[qb][t][e] = E::to_elem(sc[qb][t >> 1][8 * (t & 1) + e]);
        };
        float rs[T::NQB][T::NKB];  // row sums per 32-key block, as in pv
        float mx[T::NQB];
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            m_tile[qb] = mx_next[qb];  // this tile's max (mx_next moves on to the next tile below)
            mx[qb] = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++) rs[qb][kb2] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) cvt(qb, 0, e);
        }
        v8 va[NM];
        static_assert(AH == 2, "stage A reads the first two fragments ahead (vpre)");
        if (pre) {
            va[0] = vpre[0];
            va[1] = vpre[1];
        } else {
#pragma unroll
            for (int g = 0; g < AH; g++) va[g] = vfrag(vl, g / ODT, dt0 + g % ODT);
        }
        fence();
#pragma unroll
        for (int g = 0; g < NM; g++) {
            const int t = g / ODT, dt = g % ODT;
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) o[qb][dt] = E::mma(va[g], pt[qb][t], o[qb][dt]);
            if (g + AH < NM) va[g + AH] = vfrag(vl, (g + AH) / ODT, dt0 + (g + AH) % ODT);
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) {
                if (t + 1 < NTS)
#pragma unroll
                    for (int e = dt * 8 / ODT; e < (dt + 1) * 8 / ODT; e++) cvt(qb, t + 1, e);
                // the sums of step t (its 4 pairs over the step's fragments)
#pragma unroll
                for (int i = dt * 4 / ODT; i < (dt + 1) * 4 / ODT; i++)
                    rs[qb][t >> 1] = sum_pair(rs[qb][t >> 1], sc, pt[qb][t], qb, t, i);
                if (with_max)
#pragma unroll
                    for (int e = g * NX / NM; e < (g + 1) * NX / NM; e++) mx[qb] = fmaxf(mx[qb], sn[qb][e / 16][e % 16]);
            }
            fence();
        }
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            sums_into_l(rs[qb], qb);
            if (with_max) mx_next[qb] = partner_max(mx[qb]) * p.c2;
        }
    };
    // The work-group barrier of the run. Each wave has waited for exactly the loads the
    // next iteration reads (s_waitcnt vmcnt) and its LDS reads of the stages about to be
    // refilled have all returned (their MFMAs consumed them), so a plain s_barrier
    // suffices; __syncthreads would add a release fence, i.e. a wait for every load in
    // flight, including the tiles loaded further ahead. The empty asm statements keep
    // the compiler from moving LDS accesses across it.
    auto sync_run = []() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // s_waitcnt vmcnt(n * LOADS): at most n later K or V tile loads of this wave in flight
    auto wait_halves = [&](int n) __attribute__((always_inline)) {
        constexpr int L = T::LOADS;
        static_assert(2 * (PF - 1) * L < 64, "vmcnt field");
        if (n <= 0) wait_vm_loads<0>();
        else if (PF < 2 || n == 1) wait_vm_loads<L>();
        else if (n == 2) wait_vm_loads<2 * L>();
        else if (n == 3) wait_vm_loads<(PF > 2 ? 3 : 2) * L>();
        else wait_vm_loads<(PF > 2 ? 4 : 2) * L>();
    };
    static_assert(PF <= 3, "wait_halves covers up to four later loads");
    // K and V loads iteration i of the run issues (when the tile exists)
    auto iter_loads = [&](int i) __attribute__((always_inline)) {
        return (i + 1 + PF < ntl ? 1 : 0) + (i + PF < ntl ? 1 : 0);
    };
    // iteration r uses ring stage st = r % NB: a literal with two stages (the loop is
    // unrolled by two for the S^T tiles anyway), else a run-time value (uniform stage
    // bases that the per-lane LDS addresses add)
    auto pipe_iter = [&](int r, STile& sc, STile& sn, int st) __attribute__((always_inline)) {
        const int kb = kb_begin + r;
        // K of tile r+1+PF goes to K stage st, V of tile r+PF to V stage (st+PF) % NB
        if (r + 1 + PF < ntl) issue_tile(kbase, kb + 1 + PF, kstage(st), false);
        if (r + PF < ntl) issue_tile(vbase, kb + PF, vstage((st + PF) & (T::NB - 1)), true);
        float l0[T::NQB];
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) l0[qb] = l_part(qb);
        v8 vpre[2];
        stage_a(kstage((st + 1) & (T::NB - 1)), sn, sc, vstage(st), vpre);
        stage_b(vstage(st), sn, sc, true, vpre, true);
        lo_step(vstage(st), sc, l0);
        commit_max();
        // K of tile r+2 and V of tile r+1 must have landed: they were issued before the
        // loads of iterations max(0, r+2-PF) .. r
        int after = 0;
#pragma unroll
        for (int j = 0; j < PF - 1; j++)
            if (r - j >= 0) after += iter_loads(r - j);
        wait_halves(after);
        sync_run();
    };
    auto pipe_last = [&](int r, STile& sc, int st) __attribute__((always_inline)) {
        const int kb = kb_begin + r;
        if (r + PF < ntl) issue_tile(vbase, kb + PF, vstage((st + PF) & (T::NB - 1)), true);
        float l0[T::NQB];
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) l0[qb] = l_part(qb);
        exp_fast(sc);
        fence();
        v8 vpre[2];
        stage_b(vstage(st), sc, sc, false, vpre, false);
        lo_step(vstage(st), sc, l0);
        // the tile_step path keeps its own load order: start it with nothing in flight
        wait_vm_all();
        __syncthreads();
    };

    if (kb_begin < kb_end) {
        const int first_end = min(kb_begin + T::PREFETCH, kb_end);
        for (int j = kb_begin; j < first_end; j++) issue(j, j - kb_begin);
        wait_tiles_after_next(first_end - 1 - kb_begin);  // tile kb_begin has landed
        __syncthreads();
        int kb = kb_begin;
        if constexpr (PIPE) {
            if (nf > 0) {
                STile sa, sb;
                // prologue: K of tile PF goes out; S^T and maxima of tile 0; then K of tile 1
                // (issued before V of tile 1 .. PF-1 and K of tile 2 .. PF) must land
                if (PF < ntl) issue_tile(kbase, kb_begin + PF, kstage(PF % T::NB), false);
                qk(kstage(0), sa);
                raw_max(sa);
                commit_max();
                {
                    // issued after K of tile 1: V of tile 1, K and V of tiles 2 .. PF-1, K of tile PF
                    // (with PF = 1, K of tile 1 is the last load issued)
                    int after = (PF >= 2 && PF < ntl) ? 1 : 0;
#pragma unroll
                    for (int j = 1; j < PF; j++) after += (j >= 2 && j < ntl ? 1 : 0) + (j < ntl ? 1 : 0);
                    wait_halves(after);
                }
                sync_run();
                // unrolled by two: the S^T tiles alternate in step, so only one is live at the
                // loop's back edge
                // (r is even at each first call below)
                auto stage_of = [](int r, int lit) { return T::NB == 2 ? lit : r & (T::NB - 1); };
                int r = 0;
                for (; r + 2 < nf; r += 2) {
                    pipe_iter(r, sa, sb, stage_of(r, 0));
                    pipe_iter(r + 1, sb, sa, stage_of(r + 1, 1));
                }
                if (r + 1 < nf) {
                    pipe_iter(r, sa, sb, stage_of(r, 0));
                    pipe_last(r + 1, sb, stage_of(r + 1, 1));
                } else {
                    pipe_last(r, sa, stage_of(r, 0));
                }
                kb = kb_begin + nf;
            }
        }
        // unrolled over the ring stages (NB <= 5)
        for (; kb < kb_end; kb += T::NB) {
            tile_step(kb, 0);
            if (T::NB > 1 && kb + 1 < kb_end) tile_step(kb + 1, 1 % T::NB);
            if (T::NB > 2 && kb + 2 < kb_end) tile_step(kb + 2, 2 % T::NB);
            if (T::NB > 3 && kb + 3 < kb_end) tile_step(kb + 3, 3 % T::NB);
            if (T::NB > 4 && kb + 4 < kb_end) tile_step(kb + 4, 4 % T::NB);
        }
    }

    // ---- epilogue: O = O_acc / l, LSE = (m_used + log2 l) ln 2 ----
#pragma unroll
    for (int qb = 0; qb < T::NQB; qb++) {
        const float lt = row_l(qb);
        if (!qvalid[qb]) continue;
        const int i = qi[qb], h = qh[qb];
        const bool nonempty = lt > 0.f;
        const float inv = nonempty ? 1.0f / lt : 0.f;
        const float lse_v = nonempty ? (m_used[qb] + log2f(lt)) * kLn2 : -INFINITY;
        const long long orow = (q_off + i) * p.Hq + h;  // row of the [rows_q, Hq, Dv] output
        const long long lidx = VARLEN ? (long long)h * p.rows_q + q_off + i
                                      : ((long long)b * p.Hq + h) * p.Sq + i;
        if (!SPLIT) {
            uint16_t* orow_p = p.out + orow * p.Dv;
#pragma unroll
            for (int dt = 0; dt < ODT; dt++)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    const int dv = 32 * (dt0 + dt) + 8 * g4 + 4 * hf;
                    if (dv < p.Dv) {
                        const unsigned lo = (unsigned)E::narrow(o[qb][dt][4 * g4 + 0] * inv) |
                                            ((unsigned)E::narrow(o[qb][dt][4 * g4 + 1] * inv) << 16);
                        const unsigned hi = (unsigned)E::narrow(o[qb][dt][4 * g4 + 2] * inv) |
                                            ((unsigned)E::narrow(o[qb][dt][4 * g4 + 3] * inv) << 16);
                        *(u32x2*)(orow_p + dv) = u32x2{lo, hi};
                    }
                }
            if (p.lse && hf == 0 && (!DSPLIT || wave == 0)) p.lse[lidx] = lse_v;
        } else {
            float* op = p.o_part + ((long long)split * p.rows_q * p.Hq + orow) * p.Dv;
#pragma unroll
            for (int dt = 0; dt < ODT; dt++)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    const int dv = 32 * (dt0 + dt) + 8 * g4 + 4 * hf;
                    if (dv < p.Dv)
                        *(f32x4*)(op + dv) = f32x4{o[qb][dt][4 * g4 + 0] * inv, o[qb][dt][4 * g4 + 1] * inv,
                                                   o[qb][dt][4 * g4 + 2] * inv, o[qb][dt][4 * g4 + 3] * inv};
                }
            if (hf == 0 && (!DSPLIT || wave == 0)) p.lse_part[(long long)split * p.rows_q * p.Hq + lidx] = lse_v;
        }
    }
}

// ---- launch helpers ----
template <int D, int W, bool BF, bool CAUSAL, bool VARLEN, bool BIAS, bool SPLIT, bool DSPLIT>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
    const void* fn = (const void*)attn_fwd_kernel<D, BF, CAUSAL, VARLEN, BIAS, SPLIT, DSPLIT, W>;
    // bias instances may carry the fused producer's rows past the ring
    using T = Tile<D, CAUSAL>;
    constexpr unsigned lds_max = BIAS ? kLdsBytesPerCU / T::WG_PER_CU : T::LDS;
    // the LDS limit is raised once per device; a failure is returned and tried again on
    // the next call (only success is remembered)
    static std::atomic<uint64_t> attr_set{0};  // bit d: done on device d
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit == 0 || !(attr_set.load(std::memory_order_acquire) & bit)) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit, std::memory_order_acq_rel);
    }
    const unsigned lds = T::LDS + (BIAS ? (unsigned)p.lds_extra : 0u);
    if (lds > lds_max) return hipErrorInvalidValue;
    FwdParams pp = p;
    void* args[] = {(void*)&pp};
    return hipLaunchKernel(fn, dim3(p.nblocks), dim3(T::NT), args, lds, s);
}

typedef hipError_t (*FwdLauncher)(const FwdParams&, hipStream_t);

// instance index bits: bf16, causal, varlen, bias, split, dv split
template <int D, int W, int I>
hipError_t launch_idx(const FwdParams& p, hipStream_t s) {
    return launch_one<D, W, (I & 1) != 0, (I & 2) != 0, (I & 4) != 0, (I & 8) != 0, (I & 16) != 0,
                      (I & 32) != 0>(p, s);
}

template <int D, int W, size_t... I>
constexpr std::array<FwdLauncher, sizeof...(I)> make_fwd_table(std::index_sequence<I...>) {
    return {&launch_idx<D, W, (int)I>...};
}

// dsplit is honoured at class 256 only (the host asks for it only there); W narrows the
// arithmetic to the first W columns (see the kernel)
template <int D, int W = D>
hipError_t launch_fwd_any(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias, bool split,
                          bool dsplit, hipStream_t s) {
    constexpr bool HAS_DSPLIT = D == 256 && W == D;
    static constexpr auto table = make_fwd_table<D, W>(std::make_index_sequence<HAS_DSPLIT ? 64 : 32>{});
    if (dsplit && !HAS_DSPLIT) return hipErrorInvalidValue;
    const int idx = (bf16 ? 1 : 0) | (causal ? 2 : 0) | (varlen ? 4 : 0) | (bias ? 8 : 0) | (split ? 16 : 0) |
                    (dsplit ? 32 : 0);
    return table[idx](p, s);
}

}  // namespace mi355attn

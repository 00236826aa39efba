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
//     Lane l then holds 16 keys of query row l%32; lanes l and l^32 share a
//     row, so a row max is an in-lane max plus one permlane32_swap.
//   * O^T = V^T P^T on the same MFMA: B = P^T comes straight from the S^T
//     accumulators (same lane = same query), A = V^T is read from LDS with
//     ds_read_b64_tr_b16 out of a 4x4-blocked V layout, so each 16-lane group
//     reads 128 contiguous bytes. Every O^T register of a lane belongs to one
//     query, so the online-softmax rescale is a per-lane scalar multiply.
//   * K/V tiles of BN keys are double-buffered in LDS; global loads of tile
//     t+1 are in flight while tile t is computed; one barrier per tile.
//   * Only tiles that cross the key bound, the causal diagonal or the bias band
//     run the per-element mask / bias code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <utility>

#include "kernels.h"

namespace mi355attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4v __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4v lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLoThresh = 32.f;  // rows with a smaller softmax normaliser get the P remainder MFMA

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
};

template <int D>
struct Tile {
    static constexpr int NW = 4;                  // waves per work-group
    static constexpr int NT = NW * 64;            // threads
    static constexpr int NQB = tile_nqb(D);       // 32-row blocks per wave
    static constexpr int BM = tile_bm(D);         // rows per work-group
    static constexpr int BN = tile_bn(D);         // keys per tile
    static constexpr int NC = D / 16;             // 16-wide steps of the QK contraction
    static constexpr int NDT = (D + 31) / 32;     // 32-wide dv blocks of O^T
    static constexpr int NKB = BN / 32;           // 32-key blocks of S^T
    static constexpr int KSTRIDE = D * 2 + 16;    // bytes per K row in LDS (padded)
    static constexpr int K_BYTES = BN * KSTRIDE;
    static constexpr int V_BYTES = BN * D * 2;    // 4x4-blocked, unpadded
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int CHUNKS = BN * D / 8;     // 16-byte chunks per K (or V) tile
    static constexpr int NCH = (CHUNKS + NT - 1) / NT;
    static_assert(D == 16 || D == 64 || D == 128 || D == 256, "head dim");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Position of element r (0..15) of a 32x32 MFMA accumulator in lane half hf:
// row offset within the 32-row block (the "M" index).
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

template <int D, bool BF, bool CAUSAL, bool VARLEN, bool BIAS, bool SPLIT>
__global__ void __launch_bounds__(256, 1) attn_fwd_kernel(const FwdParams p) {
    using T = Tile<D>;
    using E = Elem<BF>;
    typedef typename E::v8 v8;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // ---- work-group -> (batch, head group, split, row tile), XCD-aware ----
    // Work-groups are handed to the 8 XCDs round-robin; give each XCD a
    // contiguous range of logical ids so tiles that read the same K/V share an L2.
    int lid;
    {
        const int nb = p.nblocks, bid = blockIdx.x;
        const int q8 = nb >> 3, r8 = nb & 7, x = bid & 7, slot = bid >> 3;
        lid = (x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8) + slot;
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
    const int i_lo = row0 / gp;
    const int i_hi = r_last / gp;

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
        const int row = row0 + (wave * T::NQB + qb) * 32 + l32;
        qvalid[qb] = row < n_rows;
        const int rr = qvalid[qb] ? row : r_last;
        qi[qb] = rr / gp;
        qh[qb] = h_base + rr % gp;
    }

    // ---- Q fragments (B operand of S^T = K Q^T): lane holds q[row][16c + 8hf .. +7] ----
    v8 qf[T::NQB][T::NC];
#pragma unroll
    for (int qb = 0; qb < T::NQB; qb++) {
        const uint16_t* qrow = p.q + ((q_off + qi[qb]) * p.Hq + qh[qb]) * (long long)D;
#pragma unroll
        for (int c = 0; c < T::NC; c++) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qvalid[qb]) x = *(const u32x4*)(qrow + 16 * c + 8 * hf);
            qf[qb][c] = __builtin_bit_cast(v8, x);
        }
    }

    f32x16 o[T::NQB][T::NDT];
    float m_run[T::NQB], l_run[T::NQB];
#pragma unroll
    for (int qb = 0; qb < T::NQB; qb++) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int dt = 0; dt < T::NDT; dt++)
#pragma unroll
            for (int r = 0; r < 16; r++) o[qb][dt][r] = 0.f;
    }

    const uint16_t* kbase = p.k + (k_off * p.Hkv + hk) * (long long)D;
    const uint16_t* vbase = p.v + (k_off * p.Hkv + hk) * (long long)D;
    const long long kv_row_stride = (long long)p.Hkv * D;  // elements between consecutive keys

    // ---- global -> register staging of one K/V tile ----
    u32x4 kst[T::NCH], vst[T::NCH];
    auto load_tile = [&](int kb) {
        const int j0 = kb * T::BN;
#pragma unroll
        for (int u = 0; u < T::NCH; u++) {
            const int c = tid + u * T::NT;
            kst[u] = u32x4{0u, 0u, 0u, 0u};
            vst[u] = u32x4{0u, 0u, 0u, 0u};
            if (c < T::CHUNKS) {
                // K: row-major chunks (8 consecutive elements of one key)
                const int kkey = c / (D / 8), kcol = c % (D / 8);
                if (j0 + kkey < k_len)
                    kst[u] = *(const u32x4*)(kbase + (long long)(j0 + kkey) * kv_row_stride + kcol * 8);
                // V: four consecutive keys per lane quad, for the blocked LDS layout
                const int vkr = c & 3, vcol = (c >> 2) % (D / 8), vkq = c / (4 * (D / 8));
                const int vkey = vkq * 4 + vkr;
                if (j0 + vkey < k_len)
                    vst[u] = *(const u32x4*)(vbase + (long long)(j0 + vkey) * kv_row_stride + vcol * 8);
            }
        }
    };
    auto store_tile = [&](int stage) {
        char* kl = smem + stage * T::STAGE;
        char* vl = kl + T::K_BYTES;
#pragma unroll
        for (int u = 0; u < T::NCH; u++) {
            const int c = tid + u * T::NT;
            if (c < T::CHUNKS) {
                const int kkey = c / (D / 8), kcol = c % (D / 8);
                *(u32x4*)(kl + kkey * T::KSTRIDE + kcol * 16) = kst[u];
                const int vkr = c & 3, vcol = (c >> 2) % (D / 8), vkq = c / (4 * (D / 8));
                // V[key][4*dq .. 4*dq+3] lives in block (key/4, dq) at row key%4
                char* vb = vl + (vkq * (D / 4) + 2 * vcol) * 32 + vkr * 8;
                *(u32x2*)(vb) = u32x2{vst[u][0], vst[u][1]};
                *(u32x2*)(vb + 32) = u32x2{vst[u][2], vst[u][3]};
            }
        }
    };

    // ---- per-tile compute ----
    auto compute_tile = [&](int kb, int stage) {
        const int j0 = kb * T::BN;
        const char* kl = smem + stage * T::STAGE;
        const char* vl = kl + T::K_BYTES;

        // S^T = K Q^T
        f32x16 s[T::NQB][T::NKB];
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) s[qb][kb2][r] = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < T::NKB; kb2++) {
            const char* krow = kl + (kb2 * 32 + l32) * T::KSTRIDE + 16 * hf;
#pragma unroll
            for (int c = 0; c < T::NC; c++) {
                const v8 a = *(const v8*)(krow + 32 * c);
#pragma unroll
                for (int qb = 0; qb < T::NQB; qb++) s[qb][kb2] = E::mma(a, qf[qb][c], s[qb][kb2]);
            }
        }

        // which per-element work this tile needs (uniform across the work-group)
        const bool need_kmask = (j0 + T::BN > k_len);
        const bool need_causal = CAUSAL && (j0 + T::BN - 1 > i_lo + delta);
        const bool need_mask = need_kmask || need_causal;
        const bool band = BIAS && (i_hi + delta - j0 >= 0) && (i_lo + delta - (j0 + T::BN - 1) < p.E);

        // online softmax, log2 domain: t = s * scale * log2(e) (+ bias * log2(e))
#pragma unroll
        for (int qb = 0; qb < T::NQB; qb++) {
            float mt = -INFINITY;
            const int i = qi[qb];
            if (need_mask || band) {
                const uint16_t* brow = nullptr;
                if (BIAS) brow = p.bias + ((q_off + i) * p.Hq + qh[qb]) * (long long)p.E;
#pragma unroll
                for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int j = j0 + kb2 * 32 + acc_row(r, hf);
                        float t = s[qb][kb2][r] * p.c2;
                        const bool vis = (j < k_len) && (!CAUSAL || j <= i + delta);
                        if (BIAS && band) {
                            const int d = i + delta - j;
                            if (vis && qvalid[qb] && d >= 0 && d < p.E) t += E::widen(brow[d]) * kLog2e;
                        }
                        t = vis ? t : -INFINITY;
                        s[qb][kb2][r] = t;
                        mt = fmaxf(mt, t);
                    }
            } else {
#pragma unroll
                for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const float t = s[qb][kb2][r] * p.c2;
                        s[qb][kb2][r] = t;
                        mt = fmaxf(mt, t);
                    }
            }
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
                mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float m_new = fmaxf(m_run[qb], mt);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
            m_run[qb] = m_new;
            float rs = 0.f;
#pragma unroll
            for (int kb2 = 0; kb2 < T::NKB; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const float pv = __builtin_amdgcn_exp2f(s[qb][kb2][r] - m_use);
                    s[qb][kb2][r] = pv;
                    rs += pv;
                }
            l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
            for (int dt = 0; dt < T::NDT; dt++)
#pragma unroll
                for (int r = 0; r < 16; r++) o[qb][dt][r] *= alpha;
        }

        // bf16 P carries a 2^-9 relative rounding error; for a row whose normaliser
        // is still small (few keys hold its weight) that error can reach the output
        // tolerance, so such rows also feed the remainder P - bf16(P) through a
        // second MFMA. A row with normaliser l has at least l effective keys, and
        // the error shrinks like 2^-9 / sqrt(3 l); rows at or above kLoThresh skip it.
        bool need_lo[T::NQB];
        bool any_lo = false;
        if (BF) {
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[qb]),
                                                                 __float_as_uint(l_run[qb]), false, false);
                need_lo[qb] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]) < kLoThresh;
                any_lo = any_lo || need_lo[qb];
            }
            any_lo = __any(any_lo);
        }

        // O^T += V^T P^T, 16 keys per MFMA step
#pragma unroll
        for (int t = 0; t < T::BN / 16; t++) {
            v8 pt[T::NQB], ptl[T::NQB];
#pragma unroll
            for (int qb = 0; qb < T::NQB; qb++)
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float pv = s[qb][t >> 1][8 * (t & 1) + e];
                    pt[qb][e] = E::to_elem(pv);
                    if (BF && any_lo) ptl[qb][e] = E::to_elem(need_lo[qb] ? pv - (float)pt[qb][e] : 0.f);
                }
            const int g = lane >> 4, jj = lane & 15;
#pragma unroll
            for (int dt = 0; dt < T::NDT; dt++) {
                // lanes of group g receive dv = 32dt + 16(g&1) + (lane&15); keys 16t + 4hf (+8)
                int dv0 = 32 * dt + 16 * (g & 1);
                const bool dv_ok = dv0 < D;
                if (!dv_ok) dv0 = 0;  // D = 16: the upper half of the dv block is padding
                const int key_a = 16 * t + 4 * hf;
                const char* pa = vl + ((key_a >> 2) * (D / 4) + (dv0 >> 2) + (jj & 3)) * 32 + (jj >> 2) * 8;
                const char* pb = pa + 2 * (D / 4) * 32;  // keys + 8 = two key-quads later
                const s16x4v ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
                const s16x4v rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pb);
                u32x4 w;
                w[0] = __builtin_bit_cast(u32x2, ra)[0];
                w[1] = __builtin_bit_cast(u32x2, ra)[1];
                w[2] = __builtin_bit_cast(u32x2, rb)[0];
                w[3] = __builtin_bit_cast(u32x2, rb)[1];
                if (!dv_ok) w = u32x4{0u, 0u, 0u, 0u};
                const v8 a = __builtin_bit_cast(v8, w);
#pragma unroll
                for (int qb = 0; qb < T::NQB; qb++) {
                    o[qb][dt] = E::mma(a, pt[qb], o[qb][dt]);
                    if (BF && any_lo) o[qb][dt] = E::mma(a, ptl[qb], o[qb][dt]);
                }
            }
        }
    };

    // ---- main loop: double-buffered K/V tiles ----
    if (kb_begin < kb_end) {
        load_tile(kb_begin);
        store_tile(0);
        __syncthreads();
        for (int kb = kb_begin; kb < kb_end; kb++) {
            const int stage = (kb - kb_begin) & 1;
            const bool more = kb + 1 < kb_end;
            if (more) load_tile(kb + 1);
            compute_tile(kb, stage);
            if (more) store_tile(stage ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2 ----
#pragma unroll
    for (int qb = 0; qb < T::NQB; qb++) {
        float lt = l_run[qb];
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
            lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        if (!qvalid[qb]) continue;
        const int i = qi[qb], h = qh[qb];
        const bool nonempty = lt > 0.f;
        const float inv = nonempty ? 1.0f / lt : 0.f;
        const float lse_v = nonempty ? (m_run[qb] + log2f(lt)) * kLn2 : -INFINITY;
        const long long orow = (q_off + i) * p.Hq + h;  // row of the [rows_q, Hq, Dv] output
        const long long lidx = VARLEN ? (long long)h * p.rows_q + q_off + i
                                      : ((long long)b * p.Hq + h) * p.Sq + i;
        if (!SPLIT) {
            uint16_t* orow_p = p.out + orow * D;
#pragma unroll
            for (int dt = 0; dt < T::NDT; dt++)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    const int dv = 32 * dt + 8 * g4 + 4 * hf;
                    if (dv < D) {
                        const unsigned lo = (unsigned)E::narrow(o[qb][dt][4 * g4 + 0] * inv) |
                                            ((unsigned)E::narrow(o[qb][dt][4 * g4 + 1] * inv) << 16);
                        const unsigned hi = (unsigned)E::narrow(o[qb][dt][4 * g4 + 2] * inv) |
                                            ((unsigned)E::narrow(o[qb][dt][4 * g4 + 3] * inv) << 16);
                        *(u32x2*)(orow_p + dv) = u32x2{lo, hi};
                    }
                }
            if (p.lse && hf == 0) p.lse[lidx] = lse_v;
        } else {
            float* op = p.o_part + ((long long)split * p.rows_q * p.Hq + orow) * D;
#pragma unroll
            for (int dt = 0; dt < T::NDT; dt++)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    const int dv = 32 * dt + 8 * g4 + 4 * hf;
                    if (dv < D)
                        *(f32x4*)(op + dv) = f32x4{o[qb][dt][4 * g4 + 0] * inv, o[qb][dt][4 * g4 + 1] * inv,
                                                   o[qb][dt][4 * g4 + 2] * inv, o[qb][dt][4 * g4 + 3] * inv};
                }
            if (hf == 0) p.lse_part[(long long)split * p.rows_q * p.Hq + lidx] = lse_v;
        }
    }
}

// ---- launch helpers ----
template <int D, bool BF, bool CAUSAL, bool VARLEN, bool BIAS, bool SPLIT>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
    const void* fn = (const void*)attn_fwd_kernel<D, BF, CAUSAL, VARLEN, BIAS, SPLIT>;
    constexpr unsigned lds = Tile<D>::LDS;
    static const hipError_t attr =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    FwdParams pp = p;
    void* args[] = {(void*)&pp};
    return hipLaunchKernel(fn, dim3(p.nblocks), dim3(Tile<D>::NT), args, lds, s);
}

typedef hipError_t (*FwdLauncher)(const FwdParams&, hipStream_t);

template <int D, int I>
hipError_t launch_idx(const FwdParams& p, hipStream_t s) {
    return launch_one<D, (I & 1) != 0, (I & 2) != 0, (I & 4) != 0, (I & 8) != 0, (I & 16) != 0>(p, s);
}

template <int D, size_t... I>
constexpr std::array<FwdLauncher, sizeof...(I)> make_fwd_table(std::index_sequence<I...>) {
    return {&launch_idx<D, (int)I>...};
}

template <int D>
hipError_t launch_fwd_any(const FwdParams& p, bool bf16, bool causal, bool varlen, bool bias, bool split,
                          hipStream_t s) {
    static constexpr auto table = make_fwd_table<D>(std::make_index_sequence<32>{});
    const int idx = (bf16 ? 1 : 0) | (causal ? 2 : 0) | (varlen ? 4 : 0) | (bias ? 8 : 0) | (split ? 16 : 0);
    return table[idx](p, s);
}

}  // namespace mi355attn

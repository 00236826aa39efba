// attn_api.cpp -- the C ABI: argument validation, planning and kernel dispatch.
//
// The host side stays short on purpose: one validation pass, a few integer
// divisions to size the grid, one launch (plus the combine launch when the key
// range is split). Per-call host overhead is what remains visible for short
// calls (TabPFN issue #1235, last comment), so nothing here allocates,
// synchronises or reads device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>

#include "../../include/attn.h"
#include "kernels.h"

using namespace mi355attn;

namespace {

constexpr int kFullChipCUs = 256;  // MI355X compute units (all XCDs of one GPU)

// Compute units of the current device, queried once per device (a partitioned MI355X
// shows fewer); the full chip's count when no device is visible, so the host-only
// entry points keep working without a GPU.
int num_cus() {
    static std::atomic<int> cached[64];
    static std::atomic<int> no_device{0};
    if (no_device.load(std::memory_order_relaxed)) return kFullChipCUs;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        no_device.store(1, std::memory_order_relaxed);
        return kFullChipCUs;
    }
    if (dev >= 64) return kFullChipCUs;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = kFullChipCUs;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool is_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// head dims of q/k and of v: multiples of 8 from 8 to 256 (any pair; the kernel
// runs the class of the larger one)
bool head_dim_ok(int d) { return d >= 8 && d <= 256 && d % 8 == 0; }

// product of non-negative ints, false if it reaches 2^62
bool mul_ok(long long& acc, long long x) {
    if (x < 0) return false;
    if (x == 0 || acc == 0) {
        acc = 0;
        return true;
    }
    if (acc > (1LL << 62) / x) return false;
    acc *= x;
    return true;
}

struct Plan {
    bool varlen, causal;
    int G, gp, n_hg, n_tiles, ns, nkb_max;
    int dclass;  // head-dim class the kernel is compiled for
    bool dsplit; // class 256 with at most 32 rows per tile: the waves share out the V columns
    long long rows_q;
    long long nblocks;
};

// Tile geometry shared with the kernels; returns false for sizes that cannot be planned.
bool make_plan(int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, int causal, int is_varlen, int max_seqlen_q,
               int max_seqlen_k, int pack_gqa, int num_splits, Plan& pl) {
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || !head_dim_ok(D) ||
        !head_dim_ok(Dv))
        return false;
    pl.dclass = head_dim_class(D > Dv ? D : Dv);
    const int dc = pl.dclass;
    pl.varlen = is_varlen != 0;
    pl.causal = causal != 0;
    pl.G = Hq / Hkv;
    const bool pack = pack_gqa == 1 || (pack_gqa == -1 && pl.G > 1);
    pl.gp = pack ? pl.G : 1;
    pl.n_hg = pack ? Hkv : Hq;
    const long long qmax = pl.varlen ? max_seqlen_q : Sq;
    const long long kmax = pl.varlen ? max_seqlen_k : Sk;
    const int bm = tile_bm(dc, pl.causal), bn = tile_bn(dc);
    const long long resident = (long long)num_cus() * tile_wg_per_cu(dc, pl.causal);
    const long long nt = (qmax * pl.gp + bm - 1) / bm;
    if (nt > INT32_MAX) return false;
    pl.n_tiles = (int)nt;
    pl.dsplit = dc == 256 && qmax * pl.gp <= 32;
    pl.nkb_max = (int)((kmax + bn - 1) / bn);
    pl.rows_q = pl.varlen ? (long long)Sq : (long long)B * Sq;
    const long long base = (long long)B * pl.n_hg * pl.n_tiles;
    int ns;
    if (pl.nkb_max <= 1) {
        ns = 1;
    } else if (num_splits >= 1) {
        ns = num_splits;
        if (ns > pl.nkb_max) ns = pl.nkb_max;
        if (ns > ATTN_MAX_SPLITS) ns = ATTN_MAX_SPLITS;
    } else if (base == 0 || base >= resident) {
        ns = 1;
    } else {
        // one wave of resident work-groups: CUs x work-groups per CU; then up to 8 such
        // waves while each split keeps at least 64 key blocks (the tail of the last
        // wave weighs less; measured c4c -12%, n1c -5% time against one wave)
        ns = (int)(resident / base);
        if (ns >= 1) {
            long long rounds = (long long)pl.nkb_max / ns / 64;
            if (rounds > 8) rounds = 8;
            if (rounds > 1) ns = (int)(ns * rounds);
        }
        const int cap = pl.nkb_max / 4 > 0 ? pl.nkb_max / 4 : 1;
        if (ns > cap) ns = cap;
        if (ns > ATTN_MAX_SPLITS) ns = ATTN_MAX_SPLITS;
        if (ns < 1) ns = 1;
    }
    pl.ns = ns;
    pl.nblocks = base * ns;
    return true;
}

size_t workspace_bytes_for(long long rows_q, int Hq, int Dv, int ns) {
    if (ns <= 1) return 0;
    return (size_t)ns * (size_t)rows_q * (size_t)Hq * ((size_t)Dv + 1) * sizeof(float);
}

attn_status_t validate(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale, int causal,
                       const int* cu_q, const int* cu_k, int max_seqlen_q, int max_seqlen_k,
                       const void* rel_bias, int rel_extent, int num_splits, int pack_gqa,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes, Plan& pl) {
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_BAD_DTYPE;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Dv <= 0) return ATTN_ERR_BAD_SHAPE;
    if (!head_dim_ok(D) || !head_dim_ok(Dv)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    if (Hq % Hkv) return ATTN_ERR_BAD_GQA;
    // The bytes of one K or V tile (tile_bn keys, consecutive keys Hkv * head dim * 2 bytes
    // apart) must not exceed 2^30: the kernels give the columns past D (Dv) a fixed load
    // offset of 2^30, which has to fall outside every tile's buffer range (and the range
    // is a 32-bit count). Hkv * max(D, Dv) <= 2^23, or 2^22 at head-dim class 16 (128-key
    // tiles).
    {
        const int dmax = D > Dv ? D : Dv;
        if ((long long)tile_bn(head_dim_class(dmax)) * Hkv * dmax * 2 > (1LL << 30)) return ATTN_ERR_BAD_SHAPE;
    }
    if (!isfinite(scale)) return ATTN_ERR_BAD_SCALE;
    if (pack_gqa < -1 || pack_gqa > 1) return ATTN_ERR_BAD_ARG;
    if ((cu_q == nullptr) != (cu_k == nullptr)) return ATTN_ERR_BAD_VARLEN;
    const bool varlen = cu_q != nullptr;
    if (varlen) {
        if (max_seqlen_q < 0 || max_seqlen_k < 0 || max_seqlen_q > Sq || max_seqlen_k > Sk)
            return ATTN_ERR_BAD_VARLEN;
        if (B > 0 && Sq > 0 && max_seqlen_q == 0) return ATTN_ERR_BAD_VARLEN;
        if (B > 0 && Sk > 0 && max_seqlen_k == 0) return ATTN_ERR_BAD_VARLEN;
    }
    // element counts below 2^62
    long long nq = 1, nk = 1;
    if (!mul_ok(nq, varlen ? 1 : B) || !mul_ok(nq, Sq) || !mul_ok(nq, Hq) || !mul_ok(nq, D))
        return ATTN_ERR_BAD_SHAPE;
    if (!mul_ok(nk, varlen ? 1 : B) || !mul_ok(nk, Sk) || !mul_ok(nk, Hkv) || !mul_ok(nk, D > Dv ? D : Dv))
        return ATTN_ERR_BAD_SHAPE;
    long long no = 1;
    if (!mul_ok(no, varlen ? 1 : B) || !mul_ok(no, Sq) || !mul_ok(no, Hq) || !mul_ok(no, Dv))
        return ATTN_ERR_BAD_SHAPE;
    if (rel_bias) {
        if (rel_extent <= 0 || rel_extent % 128) return ATTN_ERR_BAD_REL_EXTENT;
        long long nb = 1;
        if (!mul_ok(nb, varlen ? 1 : B) || !mul_ok(nb, Sq) || !mul_ok(nb, Hq) || !mul_ok(nb, rel_extent))
            return ATTN_ERR_BAD_SHAPE;
    } else if (rel_extent != 0) {
        return ATTN_ERR_BAD_REL_EXTENT;
    }
    if (!make_plan(B, Sq, Sk, Hq, Hkv, D, Dv, causal, varlen, max_seqlen_q, max_seqlen_k, pack_gqa, num_splits, pl))
        return ATTN_ERR_BAD_SHAPE;
    if (pl.nblocks > INT32_MAX) return ATTN_ERR_BAD_SHAPE;
    const bool has_rows = pl.rows_q > 0 && B > 0;
    if (has_rows && (!q || !out)) return ATTN_ERR_NULL_POINTER;
    if (has_rows && Sk > 0 && (!k || !v)) return ATTN_ERR_NULL_POINTER;
    if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(out, 16) ||
        !is_aligned(lse, 4) || !is_aligned(rel_bias, 2) || !is_aligned(workspace, 16))
        return ATTN_ERR_MISALIGNED;
    if (pl.ns > 1) {
        if (!workspace) return ATTN_ERR_WORKSPACE;
        if (workspace_bytes < workspace_bytes_for(pl.rows_q, Hq, Dv, pl.ns)) return ATTN_ERR_WORKSPACE;
    }
    return ATTN_OK;
}

bool log_enabled() {
    static const bool on = [] {
        const char* e = getenv("ATTN_LOG");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

}  // namespace

extern "C" {

attn_status_t attn_check_args(const void* q, const void* k, const void* v, void* out, float* lse,
                              int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale,
                              int causal, const int* cu_seqlens_q, const int* cu_seqlens_k,
                              int max_seqlen_q, int max_seqlen_k, const int* seqused_k,
                              const void* rel_bias, int rel_extent, int num_splits, int pack_gqa,
                              attn_dtype_t dtype, void* workspace, size_t workspace_bytes) {
    (void)seqused_k;
    Plan pl;
    return validate(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal, cu_seqlens_q, cu_seqlens_k,
                    max_seqlen_q, max_seqlen_k, rel_bias, rel_extent, num_splits, pack_gqa, dtype,
                    workspace, workspace_bytes, pl);
}

int attn_num_splits(int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, int causal, int is_varlen,
                    int max_seqlen_q, int max_seqlen_k, int pack_gqa, int num_splits) {
    Plan pl;
    if (!make_plan(B, Sq, Sk, Hq, Hkv, D, Dv, causal, is_varlen, max_seqlen_q, max_seqlen_k, pack_gqa, num_splits, pl))
        return 0;
    return pl.ns;
}

size_t attn_fwd_workspace_size(int B, int Sq, int Hq, int Dv, int is_varlen, int num_splits) {
    if (B < 0 || Sq < 0 || Hq <= 0 || Dv <= 0) return 0;
    const long long rows_q = is_varlen ? (long long)Sq : (long long)B * Sq;
    return workspace_bytes_for(rows_q, Hq, Dv, num_splits);
}

namespace {

// LDS the fused producer needs past the K/V ring: one key tile's bias values for each
// of the work-group's BM rows (BM x BN x 2 bytes, whatever rel_extent is)
long long rel_rows_lds_bytes(int dclass, bool causal) {
    return (long long)tile_bm(dclass, causal) * tile_bn(dclass) * 2;
}

// The fused-producer arguments on top of validate(): r and rel_proj given, d_rel a
// multiple of 8 in [8, 256], r 16-byte aligned.
attn_status_t validate_rel_proj(const void* rel_r, const void* rel_proj, int d_rel, const Plan& pl) {
    if (!rel_r || !rel_proj) return ATTN_ERR_NULL_POINTER;
    if (d_rel < 8 || d_rel > 256 || d_rel % 8) return ATTN_ERR_BAD_ARG;
    if (!is_aligned(rel_r, 16) || !is_aligned(rel_proj, 2)) return ATTN_ERR_MISALIGNED;
    if (tile_ring_bytes(pl.dclass) + rel_rows_lds_bytes(pl.dclass, pl.causal) >
        kLdsBytesPerCU / tile_wg_per_cu(pl.dclass, pl.causal))
        return ATTN_ERR_UNSUPPORTED_COMBO;  // (never: the ring and this region fit beside each other)
    return ATTN_OK;
}

attn_status_t run_fwd(const Plan& pl, const void* q, const void* k, const void* v, void* out, float* lse,
                      int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale, int causal,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, const int* seqused_k,
                      const void* rel_bias, const void* rel_r, const void* rel_proj, int d_rel,
                      int rel_extent, attn_dtype_t dtype, void* workspace, void* stream);

}  // namespace

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale, int causal,
                       const int* cu_seqlens_q, const int* cu_seqlens_k, int max_seqlen_q,
                       int max_seqlen_k, const int* seqused_k, const void* rel_bias, int rel_extent,
                       int num_splits, int pack_gqa, attn_dtype_t dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
    Plan pl;
    const attn_status_t st =
        validate(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal, cu_seqlens_q, cu_seqlens_k,
                 max_seqlen_q, max_seqlen_k, rel_bias, rel_extent, num_splits, pack_gqa, dtype,
                 workspace, workspace_bytes, pl);
    if (st != ATTN_OK) return st;
    if (pl.nblocks == 0) return ATTN_OK;  // no rows to compute
    return run_fwd(pl, q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal, cu_seqlens_q,
                   cu_seqlens_k, seqused_k, rel_bias, nullptr, nullptr, 0, rel_extent, dtype, workspace,
                   stream);
}

attn_status_t attn_fwd_rel_proj(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                                int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale, int causal,
                                const int* cu_seqlens_q, const int* cu_seqlens_k, int max_seqlen_q,
                                int max_seqlen_k, const int* seqused_k, const void* rel_r,
                                const void* rel_proj, int d_rel, int rel_extent, int num_splits,
                                int pack_gqa, attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                void* stream) {
    Plan pl;
    // validate as a call with a bias tensor (r stands in for its pointer: same row
    // order and dtype), then the producer's own arguments
    attn_status_t st =
        validate(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal, cu_seqlens_q, cu_seqlens_k,
                 max_seqlen_q, max_seqlen_k, rel_r ? rel_r : rel_proj, rel_extent, num_splits, pack_gqa,
                 dtype, workspace, workspace_bytes, pl);
    if (st != ATTN_OK) return st;
    st = validate_rel_proj(rel_r, rel_proj, d_rel, pl);
    if (st != ATTN_OK) return st;
    if (pl.nblocks == 0) return ATTN_OK;
    return run_fwd(pl, q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal, cu_seqlens_q,
                   cu_seqlens_k, seqused_k, nullptr, rel_r, rel_proj, d_rel, rel_extent, dtype, workspace,
                   stream);
}

namespace {

attn_status_t run_fwd(const Plan& pl, const void* q, const void* k, const void* v, void* out, float* lse,
                      int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale, int causal,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, const int* seqused_k,
                      const void* rel_bias, const void* rel_r, const void* rel_proj, int d_rel,
                      int rel_extent, attn_dtype_t dtype, void* workspace, void* stream) {
    const bool with_bias = rel_bias != nullptr || rel_r != nullptr;

    FwdParams p;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.out = (uint16_t*)out;
    p.lse = lse;
    p.bias = (const uint16_t*)rel_bias;
    p.rel_r = (const uint16_t*)rel_r;
    p.rel_proj = (const uint16_t*)rel_proj;
    p.d_rel = d_rel;
    p.lds_extra = rel_r ? (int)rel_rows_lds_bytes(pl.dclass, pl.causal) : 0;
    p.o_part = nullptr;
    p.lse_part = nullptr;
    if (pl.ns > 1) {
        p.o_part = (float*)workspace;
        p.lse_part = p.o_part + (size_t)pl.ns * (size_t)pl.rows_q * (size_t)Hq * (size_t)Dv;
    }
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.seqused_k = seqused_k;
    p.B = B;
    p.Sq = Sq;
    p.Sk = Sk;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.D = D;
    p.Dv = Dv;
    p.G = pl.G;
    p.gp = pl.gp;
    p.n_hg = pl.n_hg;
    p.n_tiles = pl.n_tiles;
    p.ns = pl.ns;
    p.E = with_bias ? rel_extent : 0;
    p.nblocks = (int)pl.nblocks;
    p.c2 = scale * 1.4426950408889634f;
    p.rows_q = pl.rows_q;

    const bool bf = dtype == ATTN_BF16;
    const bool split = pl.ns > 1;
    hipStream_t s = (hipStream_t)stream;
    if (log_enabled())
        fprintf(stderr, "[attn] D=%d Dv=%d class=%d dsplit=%d %s causal=%d varlen=%d bias=%d gp=%d n_hg=%d tiles=%d splits=%d grid=%lld\n",
                D, Dv, pl.dclass, pl.dsplit ? 1 : 0, bf ? "bf16" : "fp16", causal ? 1 : 0, pl.varlen ? 1 : 0, with_bias ? 1 : 0, pl.gp, pl.n_hg,
                pl.n_tiles, pl.ns, pl.nblocks);
    hipError_t e;
    switch (pl.dclass) {
        case 16: e = launch_fwd_d16(p, bf, causal != 0, pl.varlen, with_bias, split, pl.dsplit, s); break;
        case 64:
            // head dims up to 48: the same tiles with the QK contraction narrowed to 48 columns
            e = (D > Dv ? D : Dv) <= 48 ? launch_fwd_d64_n48(p, bf, causal != 0, pl.varlen, with_bias, split, pl.dsplit, s)
                                        : launch_fwd_d64(p, bf, causal != 0, pl.varlen, with_bias, split, pl.dsplit, s);
            break;
        case 128:
            // head dims up to 96: the same tiles with the arithmetic narrowed to 96 columns
            e = (D > Dv ? D : Dv) <= 96 ? launch_fwd_d128_n96(p, bf, causal != 0, pl.varlen, with_bias, split, pl.dsplit, s)
                                        : launch_fwd_d128(p, bf, causal != 0, pl.varlen, with_bias, split, pl.dsplit, s);
            break;
        case 256:
            // head dims up to 192 outside the decode form: the arithmetic narrowed to 192 columns
            e = (D > Dv ? D : Dv) <= 192 && !pl.dsplit
                    ? launch_fwd_d256_n192(p, bf, causal != 0, pl.varlen, with_bias, split, pl.dsplit, s)
                    : launch_fwd_d256(p, bf, causal != 0, pl.varlen, with_bias, split, pl.dsplit, s);
            break;
        default: return ATTN_ERR_UNSUPPORTED_COMBO;
    }
    if (e != hipSuccess) return ATTN_ERR_HIP;
    if (split) {
        CombineParams c;
        c.o_part = p.o_part;
        c.lse_part = p.lse_part;
        c.out = p.out;
        c.lse = lse;
        c.rows_q = pl.rows_q;
        c.Hq = Hq;
        c.Sq = Sq;
        c.ns = pl.ns;
        c.is_varlen = pl.varlen ? 1 : 0;
        c.Dv = Dv;
        if (launch_combine(c, Dv, bf, s) != hipSuccess) return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

}  // namespace

attn_status_t attn_combine(const float* o_partial, const float* lse_partial, int num_splits, void* out,
                           float* lse, int B, int Sq, int Hq, int Dv, int is_varlen, attn_dtype_t dtype,
                           void* stream) {
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_BAD_DTYPE;
    if (B < 0 || Sq < 0 || Hq <= 0) return ATTN_ERR_BAD_SHAPE;
    if (!head_dim_ok(Dv)) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
    if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_BAD_SPLITS;
    const long long rows_q = is_varlen ? (long long)Sq : (long long)B * Sq;
    long long n = rows_q;
    if (!mul_ok(n, Hq) || !mul_ok(n, Dv) || !mul_ok(n, num_splits)) return ATTN_ERR_BAD_SHAPE;
    if (rows_q == 0) return ATTN_OK;
    if (!o_partial || !lse_partial || !out) return ATTN_ERR_NULL_POINTER;
    if (!is_aligned(o_partial, 16) || !is_aligned(lse_partial, 4) || !is_aligned(out, 16) || !is_aligned(lse, 4))
        return ATTN_ERR_MISALIGNED;
    if (rows_q * Hq > INT32_MAX) return ATTN_ERR_BAD_SHAPE;  // one work-group per (row, head)
    CombineParams c;
    c.o_part = o_partial;
    c.lse_part = lse_partial;
    c.out = (uint16_t*)out;
    c.lse = lse;
    c.rows_q = rows_q;
    c.Hq = Hq;
    c.Sq = Sq;
    c.ns = num_splits;
    c.is_varlen = is_varlen ? 1 : 0;
    c.Dv = Dv;
    return launch_combine(c, Dv, dtype == ATTN_BF16, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char* attn_status_string(attn_status_t s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL_POINTER: return "a required pointer is NULL";
        case ATTN_ERR_BAD_SHAPE: return "invalid or overflowing sizes";
        case ATTN_ERR_BAD_DTYPE: return "dtype must be bf16 or fp16";
        case ATTN_ERR_UNSUPPORTED_HEAD_DIM: return "head dims D and Dv must be multiples of 8 in [8, 256]";
        case ATTN_ERR_BAD_GQA: return "Hq must be a multiple of Hkv";
        case ATTN_ERR_BAD_REL_EXTENT: return "rel_extent must be a positive multiple of 128 and needs rel_bias";
        case ATTN_ERR_BAD_VARLEN: return "cu_seqlens_q/k must be given together with valid max_seqlen";
        case ATTN_ERR_MISALIGNED: return "pointer misaligned (q/k/v/out/workspace 16 B, lse 4 B, rel_bias 2 B)";
        case ATTN_ERR_WORKSPACE: return "split-KV needs a workspace of attn_fwd_workspace_size bytes";
        case ATTN_ERR_UNSUPPORTED_COMBO: return "no kernel for this combination";
        case ATTN_ERR_HIP: return "HIP runtime error at launch";
        case ATTN_ERR_BAD_SPLITS: return "num_splits must be in [1, 256]";
        case ATTN_ERR_BAD_SCALE: return "scale must be finite";
        case ATTN_ERR_BAD_ARG: return "pack_gqa must be -1, 0 or 1";
        case ATTN_ERR_SCRATCH: return "the split partials exceed the library's 16 MiB array (attn_fwd_noalloc)";
    }
    return "unknown status";
}

const char* attn_version(void) { return "mi355-attn 0.2.0 gfx950"; }

}  // extern "C"

/*
 * attn.h -- C ABI of the exact attention forward for AMD Instinct MI355X (gfx950).
 *
 * One fused kernel computes, per (batch, query head, query row):
 *     S = scale * Q K^T  (+ relative bias on a band),  causal mask,
 *     online softmax,  O = softmax(S) V,  LSE = ln sum exp(S)   (fp32)
 * with GQA (several query heads share one K/V head), packed variable-length
 * batches, padded K/V (seqused_k) and a split-KV mode whose per-split partial
 * results are merged by an LSE-weighted combine kernel.
 *
 * Sources of the contract (the pages this library follows):
 *   - FlashAttention-4 forward returns (out, lse); the forward-only runtime card
 *     "flashrt/fa4-cute-runtime", section Functions (flash_attn_func,
 *     flash_attn_varlen_func, forward_static with a preallocated out,
 *     pack_gqa, seqused_k as a device int32 tensor).
 *   - "mgoin/tml-fa4", section Argument contract: varlen shapes, cu_seqlens,
 *     max_seqlen, rel_bias [total_q, n_q_heads, rel_extent] with rel_extent a
 *     multiple of 128, and the band rule d = i + (k_len - q_len) - j,
 *     score += rel_bias[cu_seqlens_q[b] + i, h, d] for 0 <= d < rel_extent.
 *   - "h3-blackwell-runtime" FLASH4.md, section API: native
 *     [batch, sequence, heads, head_dim] layout; an unmet requirement is an
 *     error, never a reason to use another kernel (no fallback).
 *   - TabPFN issue "FlashAttention-4 backend for Blackwell" (#1235), closing
 *     comment: the returned LSE lets split-KV be merged outside the kernel.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or keeps them. All tensors are dense and contiguous.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and runs asynchronously; the library never synchronises the host.
 *   - Device-resident metadata (cu_seqlens_*, seqused_k) is not read on the
 *     host; malformed contents are undefined behaviour.
 *   - Any violated requirement returns an error code, launches nothing and
 *     writes nothing. No other kernel is ever substituted.
 *   - The library keeps no state between calls beyond a lazily cached device
 *     property (the compute-unit count of each device) and, per kernel and device,
 *     whether its LDS limit has been raised; calls are reentrant.
 */
#ifndef MI355_ATTN_H
#define MI355_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL_POINTER = 1,      /* a required pointer is NULL */
    ATTN_ERR_BAD_SHAPE = 2,         /* negative / zero / overflowing sizes */
    ATTN_ERR_BAD_DTYPE = 3,         /* dtype is not ATTN_BF16 or ATTN_FP16 */
    ATTN_ERR_UNSUPPORTED_HEAD_DIM = 4, /* D or Dv not a multiple of 8 in [8, 256] */
    ATTN_ERR_BAD_GQA = 5,           /* Hq is not a multiple of Hkv */
    ATTN_ERR_BAD_REL_EXTENT = 6,    /* rel_extent <= 0, not a multiple of 128, or given without rel_bias */
    ATTN_ERR_BAD_VARLEN = 7,        /* only one of cu_seqlens_q/k given, or bad max_seqlen */
    ATTN_ERR_MISALIGNED = 8,        /* a pointer is not aligned as documented */
    ATTN_ERR_WORKSPACE = 9,         /* split-KV without a large enough workspace */
    ATTN_ERR_UNSUPPORTED_COMBO = 10, /* a valid combination this build has no kernel for */
    ATTN_ERR_HIP = 11,              /* the HIP runtime reported an error at launch */
    ATTN_ERR_BAD_SPLITS = 12,       /* attn_combine: num_splits outside [1, ATTN_MAX_SPLITS] */
    ATTN_ERR_BAD_SCALE = 13,        /* scale is NaN or infinite */
    ATTN_ERR_BAD_ARG = 14,          /* pack_gqa not in {-1, 0, 1} */
    ATTN_ERR_SCRATCH = 15           /* attn_fwd_noalloc: the split partials exceed ATTN_SCRATCH_BYTES */
} attn_status_t;

typedef enum { ATTN_BF16 = 0, ATTN_FP16 = 1 } attn_dtype_t;

#define ATTN_MAX_SPLITS 256

/* Bytes of split partials attn_fwd_noalloc can hold (its device-resident array). */
#define ATTN_SCRATCH_BYTES (16u << 20)

/*
 * attn_fwd -- the fused attention forward (dense or varlen, optional split-KV).
 *
 * Layout (16-bit elements of `dtype`, all contiguous):
 *   dense  (cu_seqlens_q == cu_seqlens_k == NULL):
 *     q [B, Sq, Hq, D], k [B, Sk, Hkv, D], v [B, Sk, Hkv, Dv], out [B, Sq, Hq, Dv]
 *     lse [B, Hq, Sq] (fp32)
 *   varlen (both cu_seqlens given, int32 [B+1], non-decreasing, first 0, last = total):
 *     Sq = total_q, Sk = total_k;  q [total_q, Hq, D], k [total_k, Hkv, D],
 *     v [total_k, Hkv, Dv], out [total_q, Hq, Dv], lse [Hq, total_q] (fp32)
 *     max_seqlen_q / max_seqlen_k >= every per-sequence length and <= total_q / total_k
 *     (used to size the grid; 0 only when that total is 0), else ATTN_ERR_BAD_VARLEN.
 *   Sequence b has q_len = Sq (dense) or cu_seqlens_q[b+1] - cu_seqlens_q[b],
 *   and k_len = seqused_k[b] if seqused_k != NULL (device int32 [B], keys
 *   past it are never read into the result, whatever they hold), else Sk or
 *   cu_seqlens_k[b+1] - cu_seqlens_k[b].
 *
 * Semantics, for every query row i < q_len and query head h:
 *   hk = h / (Hq / Hkv);  delta = k_len - q_len
 *   key j is visible iff j < k_len and (!causal || j <= i + delta)   (bottom-right aligned)
 *   s_j = scale * <q[i,h,:], k[j,hk,:]> + (rel_bias && 0 <= d < rel_extent ? rel_bias[row(i), h, d] : 0)
 *         with d = i + delta - j and row(i) the row of query i in q's flattened order
 *   lse = ln sum_visible exp(s_j);  out[i,h,:] = sum_visible exp(s_j - lse) v[j,hk,:]
 *   A row with no visible key gets out = 0 and lse = -inf.
 *   out is rounded to nearest even from fp32. lse may be NULL (not written).
 *
 * rel_bias: NULL, or [rows_q, Hq, rel_extent] of `dtype` flattened like q
 *   (rows_q = total_q in varlen mode, B*Sq in dense mode); rel_extent must be a
 *   positive multiple of 128 (tml-fa4 argument contract).
 * scale: any finite float (the usual value is 1/sqrt(D)); it is used as this float32.
 * pack_gqa: -1 automatic, 0 off, 1 on. Packing the G = Hq/Hkv query heads of a
 *   K/V head into one tile is a scheduling choice; results do not depend on it.
 * num_splits: <= 0 chooses with attn_num_splits; 1 = no split; n > 1 = n
 *   splits of the key range (clamped to the number of key blocks and to
 *   ATTN_MAX_SPLITS). With more than one split the partials live in `workspace`
 *   (device memory, 16-byte aligned, at least attn_fwd_workspace_size bytes) and
 *   the combine kernel runs on the same stream before the call returns.
 *   workspace may be NULL when no split is used.
 * Alignment: q, k, v, out and workspace 16 bytes; lse 4 bytes; rel_bias 2 bytes.
 * Head dims: D (q, k) and Dv (v, out) are each any multiple of 8 from 8 to 256
 *   (head_dim and head_dim_v of the tml-fa4 "Argument contract"; 8..256 in steps
 *   of 8 is the range the TabPFN issue thread gives for FA4 on sm_90);
 *   D = Dv = 64, 128 and 256 run at full efficiency, other pairs on the kernel
 *   of the next size up (16, 64, 128 or 256) with the extra columns zero.
 * Limits: one K or V tile must span at most 2^30 bytes, i.e. Hkv * max(D, Dv) <= 2^23
 *   (2^22 when max(D, Dv) <= 16, where a tile holds 128 keys instead of 64); sizes must
 *   keep every element count below 2^62.
 */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                       int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale,
                       int causal, const int* cu_seqlens_q, const int* cu_seqlens_k,
                       int max_seqlen_q, int max_seqlen_k, const int* seqused_k,
                       const void* rel_bias, int rel_extent, int num_splits, int pack_gqa,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * attn_fwd_rel_proj -- attn_fwd with the relative bias produced inside the kernel.
 *
 * The tml-fa4 page builds rel_bias as the product of r [total_q, n_q_heads, d_rel]
 * (flattened like q) with rel_proj [d_rel, rel_extent] (an einsum over d_rel) before
 * the call. Here the values each key tile of the band needs are formed on the MFMA
 * inside the kernel and kept in LDS, so the [rows_q, Hq, rel_extent] tensor is never
 * written to or read from HBM:
 *   rel_bias[t, h, d] = round_to_dtype( sum_e r[t, h, e] * rel_proj[e, d] )
 * with the sum in fp32 and the rounding to `dtype` (nearest even) that a rel_bias
 * materialised in q's dtype has; everything else is attn_fwd with that rel_bias.
 * r: [rows_q, Hq, d_rel] of `dtype`, device, 16-byte aligned; rel_proj: [d_rel,
 * rel_extent] of `dtype`, device. d_rel: a multiple of 8 in [8, 256]. rel_extent as
 * for attn_fwd (a positive multiple of 128), with no further limit. Other arguments,
 * errors and ownership as attn_fwd
 * (r stands in for rel_bias in the NULL / alignment checks; a missing rel_proj is
 * ATTN_ERR_NULL_POINTER, a bad d_rel ATTN_ERR_BAD_ARG).
 */
attn_status_t attn_fwd_rel_proj(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale,
                                int causal, const int* cu_seqlens_q, const int* cu_seqlens_k,
                                int max_seqlen_q, int max_seqlen_k, const int* seqused_k,
                                const void* rel_r, const void* rel_proj, int d_rel, int rel_extent,
                                int num_splits, int pack_gqa, attn_dtype_t dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * attn_fwd_noalloc -- attn_fwd for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments minus the workspace. When the key range is split, the partials go to an
 * array of ATTN_SCRATCH_BYTES (16 MiB) that the library holds in device memory on
 * every GPU it runs on, until the process ends; the call itself allocates and frees
 * nothing. Needs ns * rows_q * Hq * (Dv + 1) * 4 <= ATTN_SCRATCH_BYTES bytes for the
 * split count ns that attn_num_splits gives (rows_q = B * Sq dense, total_q varlen),
 * else returns ATTN_ERR_SCRATCH and launches nothing (pass a smaller num_splits, or use
 * attn_fwd with a workspace). Calls on one GPU share that array: calls that overlap in
 * time on the same GPU (other streams, other threads) must not be made. Results,
 * errors and ownership otherwise as attn_fwd (it is attn_fwd with that array as the
 * workspace).
 */
attn_status_t attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                               int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale,
                               int causal, const int* cu_seqlens_q, const int* cu_seqlens_k,
                               int max_seqlen_q, int max_seqlen_k, const int* seqused_k,
                               const void* rel_bias, int rel_extent, int num_splits, int pack_gqa,
                               attn_dtype_t dtype, void* stream);

/*
 * attn_check_args -- attn_fwd's validation alone, on the host, with no GPU work
 * (not from the pages: a check a caller can make before enqueueing).
 * Same arguments as attn_fwd minus the stream; returns the code attn_fwd would
 * return before launching anything. Pointers are only checked for NULL and
 * alignment, never dereferenced.
 */
attn_status_t attn_check_args(const void* q, const void* k, const void* v, void* out,
                              float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv,
                              float scale, int causal, const int* cu_seqlens_q,
                              const int* cu_seqlens_k, int max_seqlen_q, int max_seqlen_k,
                              const int* seqused_k, const void* rel_bias, int rel_extent,
                              int num_splits, int pack_gqa, attn_dtype_t dtype, void* workspace,
                              size_t workspace_bytes);

/*
 * attn_num_splits -- the number of key-range splits attn_fwd uses for these
 * sizes and this request (num_splits <= 0: the heuristic; otherwise the
 * request clamped). causal and is_varlen as in attn_fwd (causal changes the
 * work-group shape at head-dim class 128, hence the grid the heuristic sees).
 * Host function, no GPU work (it reads the current device's compute-unit count
 * once). Returns >= 1, or 0 for invalid sizes. Not from the pages: the split
 * count is this library's scheduling choice; every count gives the same result
 * up to rounding.
 * Heuristic: split only when the unsplit grid has fewer work-groups than fit
 * on the device at once (compute units of the current device -- 256 on a full
 * MI355X, also used when no device is visible -- times the work-groups resident
 * per CU: 2 up to head-dim class 64 and for causal class 128, 1 for non-causal
 * class 128 (eight-wave work-groups) and for class 256); then use
 * n = floor(that / work-groups) splits (one wave of work-groups fills the device),
 * times r = min(8, floor(key blocks / n / 64)) when r > 1 (several waves while
 * each split keeps at least 64 key blocks), never fewer than 4 key blocks per
 * split (64 keys per block; 128 for D <= 16) and never more than
 * ATTN_MAX_SPLITS splits. Rows per work-group: 256 for non-causal class 128,
 * 128 otherwise.
 */
int attn_num_splits(int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, int causal, int is_varlen,
                    int max_seqlen_q, int max_seqlen_k, int pack_gqa, int num_splits);

/*
 * attn_fwd_workspace_size -- (not from the pages: the partials' storage of this
 * library's split-KV path) bytes of workspace attn_fwd needs for `num_splits`
 * splits (0 when num_splits <= 1). Layout: fp32 O partials
 * [num_splits, rows_q, Hq, Dv] followed by fp32 LSE partials
 * [num_splits, <lse layout>] (rows_q = B*Sq dense, Sq = total_q varlen).
 */
size_t attn_fwd_workspace_size(int B, int Sq, int Hq, int Dv, int is_varlen, int num_splits);

/*
 * attn_combine -- LSE-weighted merge of split partials (the split-KV combine that
 * the returned LSE makes possible outside the kernel: TabPFN issue #1235, closing
 * comment; "split-KV combine" in the tml-fa4 page's introduction).
 *   o_partial [num_splits, rows_q, Hq, Dv] fp32, lse_partial [num_splits, <lse layout>] fp32,
 *   each split's O normalised within the split, an empty split marked by lse = -inf.
 *   M = max_s lse_s;  lse = M + ln sum_s exp(lse_s - M);  out = sum_s exp(lse_s - lse) o_s
 *   (rounded to `dtype`); all splits empty -> out = 0, lse = -inf.
 * Layouts of out / lse as in attn_fwd (is_varlen picks dense or varlen LSE order;
 * dense needs Sq = per-batch length, varlen Sq = total_q). lse may be NULL.
 * 1 <= num_splits <= ATTN_MAX_SPLITS; Dv a multiple of 8 in [8, 256].
 * Alignment: partials and out 16 bytes, lse 4 bytes.
 */
attn_status_t attn_combine(const float* o_partial, const float* lse_partial, int num_splits,
                           void* out, float* lse, int B, int Sq, int Hq, int Dv, int is_varlen,
                           attn_dtype_t dtype, void* stream);

/* Human-readable name of a status code (static storage; never NULL). Not from the pages. */
const char* attn_status_string(attn_status_t status);

/* Library version string, e.g. "mi355-attn 0.2.0 gfx950". Not from the pages. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ATTN_H */

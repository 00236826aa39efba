/*
 * attn_oracle.c -- plain, slow fp64 CPU reference of the exact attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg call this code; the product path never does.
 * It shares no code, header or table with the GPU library.
 *
 * What it computes (the plain definition; the tiled online-softmax method
 * reaches the same value up to rounding, since the "online softmax" figure of
 * the ATFlash-Kernel-FA4 page states that tiling, running max, normaliser and
 * PV are left as in the plain computation):
 *
 *   For batch b, query head h, query row i in [0, q_len):
 *     G = Hq / Hkv, hk = floor(h / G)                      (consecutive Q heads
 *                                                          share a KV head)
 *     q_off = cu_seqlens_q[b] (varlen) or b*Sq (dense)
 *     k_off = cu_seqlens_k[b] (varlen) or b*Sk (dense)
 *     q_len = cu_seqlens_q[b+1]-cu_seqlens_q[b] or Sq
 *     k_len = seqused_k[b] if given, else cu_seqlens_k[b+1]-cu_seqlens_k[b] or Sk
 *             (the "valid K/V length" of the fa4-cute-runtime card, Functions)
 *     delta = k_len - q_len
 *     key j is visible iff 0 <= j < k_len and (not causal or j <= i + delta)
 *             (bottom-right alignment: tml-fa4 page, "Argument contract",
 *              where d = i + (k_len - q_len) - j and d == 0 is the query's own
 *              key position)
 *     s_j = scale * sum_d q[q_off+i,h,d] * k[k_off+j,hk,d]
 *           + rel_bias[q_off+i, h, d_j]   when 0 <= d_j < E, d_j = i + delta - j
 *             (tml-fa4 page, "Argument contract": the bias is added to the
 *              score, i.e. after scaling, and only inside the band)
 *     LSE = ln sum_{visible j} exp(s_j)           (-inf if nothing is visible)
 *     O   = sum_{visible j} exp(s_j - LSE) v[k_off+j,hk,:]   (0 if nothing)
 *           (forward returns (out, lse): fa4-cute-runtime card, Functions;
 *            tml-fa4 page usage)
 *
 * Inputs are the 16-bit bit patterns (bfloat16 or IEEE half); they are widened
 * exactly to double. The scale arrives as the float32 the GPU path also uses.
 * Everything after widening is double precision, computed with plain loops.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_FP16 1

static double widen_bf16(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double widen_fp16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int mant = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);               /* zero / subnormal */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant + 1024), expo - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double widen(uint16_t x, int dtype) {
    return dtype == ORACLE_BF16 ? widen_bf16(x) : widen_fp16(x);
}

typedef struct {
    const uint16_t *q, *k, *v, *bias;
    int dtype;
    int B, Sq, Sk, Hq, Hkv, D, Dv, E;
    double scale;
    int causal;
    const int32_t *cu_q, *cu_k, *seqused_k;
    long long key_lo, key_hi; /* extra restriction of the key range (for split checks) */
} ctx_t;

/* Offsets and lengths of batch b. */
static void batch_geometry(const ctx_t* c, int b, long long* q_off, long long* k_off,
                           long long* q_len, long long* k_len) {
    if (c->cu_q) {
        *q_off = c->cu_q[b];
        *k_off = c->cu_k[b];
        *q_len = (long long)c->cu_q[b + 1] - c->cu_q[b];
        *k_len = (long long)c->cu_k[b + 1] - c->cu_k[b];
    } else {
        *q_off = (long long)b * c->Sq;
        *k_off = (long long)b * c->Sk;
        *q_len = c->Sq;
        *k_len = c->Sk;
    }
    if (c->seqused_k) *k_len = c->seqused_k[b];
}

/* One output row: o[0..Dv), *lse. s is scratch of at least k_len doubles. */
static void one_row(const ctx_t* c, int b, int h, long long i, double* s, double* o, double* lse) {
    long long q_off, k_off, q_len, k_len;
    batch_geometry(c, b, &q_off, &k_off, &q_len, &k_len);
    const int G = c->Hq / c->Hkv;
    const int hk = h / G;
    const long long delta = k_len - q_len;
    const uint16_t* qrow = c->q + ((q_off + i) * c->Hq + h) * (long long)c->D;

    double m = -INFINITY;
    long long nvis = 0;
    for (long long j = 0; j < k_len; j++) {
        int visible = 1;
        if (c->causal && j > i + delta) visible = 0;
        if (j < c->key_lo || j >= c->key_hi) visible = 0;
        if (!visible) {
            s[j] = -INFINITY;
            continue;
        }
        const uint16_t* krow = c->k + ((k_off + j) * c->Hkv + hk) * (long long)c->D;
        double dot = 0.0;
        for (int d = 0; d < c->D; d++) dot += widen(qrow[d], c->dtype) * widen(krow[d], c->dtype);
        double sj = c->scale * dot;
        if (c->bias) {
            long long dd = i + delta - j;
            if (dd >= 0 && dd < c->E)
                sj += widen(c->bias[((q_off + i) * c->Hq + h) * (long long)c->E + dd], c->dtype);
        }
        s[j] = sj;
        if (sj > m) m = sj;
        nvis++;
    }
    for (int d = 0; d < c->Dv; d++) o[d] = 0.0;
    if (nvis == 0) {
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (long long j = 0; j < k_len; j++) {
        if (s[j] == -INFINITY) continue;
        double p = exp(s[j] - m);
        l += p;
        const uint16_t* vrow = c->v + ((k_off + j) * c->Hkv + hk) * (long long)c->Dv;
        for (int d = 0; d < c->Dv; d++) o[d] += p * widen(vrow[d], c->dtype);
    }
    for (int d = 0; d < c->Dv; d++) o[d] /= l;
    *lse = m + log(l);
}

/*
 * Compute n_rows output rows. rows holds n_rows triples (b, h, i).
 * out_o: n_rows x Dv doubles; out_lse: n_rows doubles.
 * cu_q/cu_k: both NULL (dense) or both set (varlen, int32[B+1]).
 * seqused_k: NULL or int32[B]. bias: NULL or [rows_q, Hq, E] 16-bit.
 * key_lo/key_hi: keys outside [key_lo, key_hi) are treated as invisible
 * (pass 0 and a huge value for the plain definition).
 * Returns 0, or a negative code for malformed arguments.
 */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                     int B, int Sq, int Sk, int Hq, int Hkv, int D, int Dv, float scale,
                     int causal, const int32_t* cu_q, const int32_t* cu_k,
                     const int32_t* seqused_k, const uint16_t* bias, int E,
                     long long key_lo, long long key_hi, long long n_rows, const int32_t* rows,
                     double* out_o, double* out_lse, int nthreads) {
    if (!q || !k || !v || !rows || !out_o || !out_lse) return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return -2;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Dv <= 0 || Hq % Hkv) return -3;
    if ((cu_q == NULL) != (cu_k == NULL)) return -4;
    if (bias && E <= 0) return -5;
    ctx_t c;
    c.q = q; c.k = k; c.v = v; c.bias = bias; c.dtype = dtype;
    c.B = B; c.Sq = Sq; c.Sk = Sk; c.Hq = Hq; c.Hkv = Hkv; c.D = D; c.Dv = Dv; c.E = E;
    c.scale = (double)scale; c.causal = causal;
    c.cu_q = cu_q; c.cu_k = cu_k; c.seqused_k = seqused_k;
    c.key_lo = key_lo; c.key_hi = key_hi;

    long long kmax = 0;
    for (int b = 0; b < B; b++) {
        long long qo, ko, ql, kl;
        batch_geometry(&c, b, &qo, &ko, &ql, &kl);
        if (kl > kmax) kmax = kl;
    }
    if (nthreads <= 0) nthreads = 1;
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(kmax > 0 ? kmax : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long long r = 0; r < n_rows; r++) {
            if (!s) continue;
            int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            one_row(&c, b, h, i, s, out_o + r * (long long)Dv, out_lse + r);
        }
        free(s);
    }
    return bad ? -6 : 0;
}

/*
 * Merge per-split results with log-sum-exp weights (the split-KV combine:
 * the TabPFN issue's closing comment notes that the returned LSE lets a caller
 * split K/V outside the kernel and merge the pieces).
 *   M = max_s lse_s; LSE = M + ln sum_s exp(lse_s - M); O = sum_s exp(lse_s - LSE) o_s
 * All splits empty (every lse_s = -inf): O = 0, LSE = -inf.
 * o_parts: ns x n_rows x Dv, lse_parts: ns x n_rows.
 */
int oracle_combine(const double* o_parts, const double* lse_parts, int ns, long long n_rows,
                   int Dv, double* out_o, double* out_lse) {
    if (!o_parts || !lse_parts || !out_o || !out_lse || ns <= 0 || Dv <= 0) return -1;
    for (long long r = 0; r < n_rows; r++) {
        double M = -INFINITY;
        for (int s = 0; s < ns; s++) {
            double x = lse_parts[(long long)s * n_rows + r];
            if (x > M) M = x;
        }
        double* o = out_o + r * Dv;
        for (int d = 0; d < Dv; d++) o[d] = 0.0;
        if (M == -INFINITY) {
            out_lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int s = 0; s < ns; s++) sum += exp(lse_parts[(long long)s * n_rows + r] - M);
        double L = M + log(sum);
        for (int s = 0; s < ns; s++) {
            double w = exp(lse_parts[(long long)s * n_rows + r] - L);
            const double* os = o_parts + ((long long)s * n_rows + r) * Dv;
            for (int d = 0; d < Dv; d++) o[d] += w * os[d];
        }
        out_lse[r] = L;
    }
    return 0;
}

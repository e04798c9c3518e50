/*
 * fa_oracle.c -- the fp64 CPU oracle for exact attention, its split-KV
 * (partial output + log-sum-exp) combine, and its gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the package smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP kernels.
 *
 * What it computes (sources, by page and section):
 *
 *  - "FlashAttention-3 vs Triton Kernels: Warp-Specialization on GPUs"
 *    (dailyaiworld.com), introduction: FlashAttention computes ordinary
 *    softmax attention; its tiling only avoids storing the N x N score
 *    matrix in HBM.  The plain definition is therefore the oracle:
 *        s_ij = scale * <q_i, k_j>
 *        O_i  = sum_j softmax_j(s_i.) v_j
 *        lse_i = log sum_j exp(s_ij)
 *    over the keys j visible to query i.
 *  - Same page, "Benchmarking Triton vs FlashAttention-3 Kernels": tensors
 *    are laid out (batch, heads, seq_len, head_dim) and the benchmarked call
 *    is the non-causal default, whose scale is 1/sqrt(head_dim).
 *  - Same page, introduction and the pipeline figure: the FP8 variant of the
 *    forward.  Its oracle is the same definition on the dequantized inputs
 *    dq*q8, dk*k8, dv*v8 (per-tensor factors), with E4M3 bytes widened
 *    exactly (oracle_attention_rows_dq, dtype ORACLE_FP8).
 *  - post.smzdm.com digest on Triton warp specialisation, section 5
 *    (attention cannot be split like a GEMM): partial attention outputs over
 *    disjoint key shards cannot be added, because each shard has its own
 *    softmax denominator; each shard must carry its log-sum-exp, and the
 *    combine re-normalises the partial outputs with it.  oracle_combine()
 *    is that re-normalisation written out.
 *
 *  - "Warp Specialization in Triton: Design and Roadmap" (PyTorch blog),
 *    roadmap section: the attention backward is the next kernel.  Its oracle
 *    (oracle_attention_bwd) is the chain rule applied to the definition
 *    above, written out term by term.
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes): causal means key j is visible to query i iff j <= i; the
 * grouped-query map sends query head hq to key/value head hq / (Hq/Hkv);
 * lse is the natural log; a query with no visible key gets O = 0 and
 * lse = -inf.
 *
 * Precision: inputs are the exact values the GPU consumes (bf16, fp16 or
 * E4M3 bit patterns), widened exactly to double; everything after that is
 * plain fp64 in a two-pass (max, then exp-sum) softmax.
 *
 * ORACLE_MUTANT (compile-time, default 0) plants one deliberate mistake per
 * value.  Only the test that proves the pins can catch a wrong oracle builds
 * those variants; the normal build never defines it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#define ORACLE_BF16 0
#define ORACLE_FP16 1
#define ORACLE_FP8 2    /* OCP E4M3 ("e4m3fn"), one byte per element */

/* Exact widening of one 16-bit storage value to double. */
double oracle_widen(uint16_t bits, int dtype)
{
    if (dtype == ORACLE_FP8) {
        /* E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent 15
         * with fraction 7 is NaN; there are no infinities. */
        int sign8 = (bits >> 7) & 1, e8 = (bits >> 3) & 15, f8 = bits & 7;
#if ORACLE_MUTANT == 13
        const int bias8 = 8;
#else
        const int bias8 = 7;
#endif
        double mag8;
        if (e8 == 15 && f8 == 7)
            mag8 = NAN;
        else if (e8 == 0)
            mag8 = ldexp((double)f8, 1 - bias8 - 3);         /* subnormal */
        else
            mag8 = ldexp((double)(8 + f8), e8 - bias8 - 3);
        return sign8 ? -mag8 : mag8;
    }
    if (dtype == ORACLE_BF16) {
        /* bfloat16 is the top half of an IEEE binary32. */
#if ORACLE_MUTANT == 11
        uint32_t w = (uint32_t)bits << 15;
#else
        uint32_t w = (uint32_t)bits << 16;
#endif
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
#if ORACLE_MUTANT == 8
    const int bias = 14;
#else
    const int bias = 15;
#endif
    double mag;
    if (e == 0)
        mag = ldexp((double)frac, 1 - bias - 10);          /* subnormal */
    else if (e == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), e - bias - 10);
    return sign ? -mag : mag;
}

static int kv_head_of(long hq, long Hq, long Hkv)
{
#if ORACLE_MUTANT == 5
    (void)Hq;
    return (int)(hq % Hkv);
#else
    long group = Hq / Hkv;          /* query heads per key/value head */
    return (int)(hq / group);
#endif
}

static int key_visible(long j, long i, int causal)
{
    if (!causal)
        return 1;
#if ORACLE_MUTANT == 2
    return j < i;
#else
    return j <= i;
#endif
}

/*
 * Attention for an explicit list of query rows, restricted to keys in
 * [klo, khi) (the full key set is [0, Nk)), on the dequantized inputs
 * dq*q, dk*k, dv*v (dq = dk = dv = 1 for 16-bit inputs).
 *
 *   q     [B, Hq,  Nq, d]  bit patterns, d fastest (FP8 bytes zero-extended
 *                          to 16 bits)
 *   k, v  [B, Hkv, Nk, d]  bit patterns
 *   rows  nrows triples (b, hq, i)
 *   out_o [nrows, d] double, out_lse [nrows] double
 *
 * Returns 0, or -1 on a bad argument (nothing written).
 */
int oracle_attention_rows_dq(const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, int dtype, double dq, double dk,
                             double dv, long B, long Hq, long Hkv, long Nq,
                             long Nk, long d, int causal, double scale, long klo,
                             long khi, const long *rows, long nrows,
                             double *out_o, double *out_lse)
{
    if (!q || !k || !v || !rows || !out_o || !out_lse)
        return -1;
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 0 || Nk < 0 || d < 1)
        return -1;
    if (klo < 0) klo = 0;
    if (khi > Nk) khi = Nk;
    for (long r = 0; r < nrows; ++r) {
        long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Nq)
            return -1;
    }

    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < nrows; ++r) {
            if (!s || !qd)
                continue;
            long b = rows[3 * r], hq = rows[3 * r + 1], i = rows[3 * r + 2];
            long g = kv_head_of(hq, Hq, Hkv);
            const uint16_t *qi = q + ((b * Hq + hq) * Nq + i) * d;
            const uint16_t *kb = k + (b * Hkv + g) * Nk * d;
            const uint16_t *vb = v + (b * Hkv + g) * Nk * d;
#if ORACLE_MUTANT == 4
            kb = v + (b * Hkv + g) * Nk * d;
#endif
            double *o = out_o + r * d;
            for (long c = 0; c < d; ++c)
                qd[c] = dq * oracle_widen(qi[c], dtype);

            /* pass 1: scores of the visible keys and their maximum */
            double m = -INFINITY;
            long nvis = 0;
            for (long j = klo; j < khi; ++j) {
                if (!key_visible(j, i, causal))
                    continue;
                const uint16_t *kj = kb + j * d;
                double dot = 0.0;
#if ORACLE_MUTANT == 10
                for (long c = 0; c + 1 < d; ++c)
#else
                for (long c = 0; c < d; ++c)
#endif
                    dot += qd[c] * (dk * oracle_widen(kj[c], dtype));
#if ORACLE_MUTANT == 1
                s[j] = -scale * dot;
#else
                s[j] = scale * dot;
#endif
                if (s[j] > m)
                    m = s[j];
                ++nvis;
            }
            for (long c = 0; c < d; ++c)
                o[c] = 0.0;
            if (nvis == 0) {
                out_lse[r] = -INFINITY;
                continue;
            }

            /* pass 2: l = sum exp(s - m), O = sum exp(s - m) v / l */
            double l = 0.0;
            for (long j = klo; j < khi; ++j) {
                if (!key_visible(j, i, causal))
                    continue;
                double p = exp(s[j] - m);
                l += p;
#if ORACLE_MUTANT == 9
                const uint16_t *vj = vb + ((j + 1) % Nk) * d;
#else
                const uint16_t *vj = vb + j * d;
#endif
#if ORACLE_MUTANT == 14
                for (long c = 0; c < d; ++c)
                    o[c] += p * oracle_widen(vj[c], dtype);
#else
                for (long c = 0; c < d; ++c)
                    o[c] += p * (dv * oracle_widen(vj[c], dtype));
#endif
            }
#if ORACLE_MUTANT != 6
            for (long c = 0; c < d; ++c)
                o[c] /= l;
#endif
#if ORACLE_MUTANT == 3
            out_lse[r] = log(l);
#else
            out_lse[r] = m + log(l);
#endif
        }
        free(s);
        free(qd);
    }
    return bad ? -1 : 0;
}

/* The same for undequantized (16-bit) inputs. */
int oracle_attention_rows(const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, int dtype, long B, long Hq,
                          long Hkv, long Nq, long Nk, long d, int causal,
                          double scale, long klo, long khi, const long *rows,
                          long nrows, double *out_o, double *out_lse)
{
    return oracle_attention_rows_dq(q, k, v, dtype, 1.0, 1.0, 1.0, B, Hq, Hkv,
                                    Nq, Nk, d, causal, scale, klo, khi, rows,
                                    nrows, out_o, out_lse);
}

/*
 * Combine nsplit partial results of one query row, each the attention over a
 * disjoint key shard, into the attention over the union of the shards
 * (smzdm digest, section 5: every shard carries its log-sum-exp and the
 * combine re-normalises with it):
 *     lse = log sum_s exp(lse_s)          (computed as M + log sum exp(lse_s - M))
 *     O   = sum_s exp(lse_s - lse) O_s
 * A shard with lse_s = -inf (no visible key) has weight zero.
 *
 *   part_o [nsplit, d], part_lse [nsplit]  ->  o [d], *lse
 */
void oracle_combine(const double *part_o, const double *part_lse, long nsplit,
                    long d, double *o, double *lse)
{
    double M = -INFINITY;
    for (long s = 0; s < nsplit; ++s)
        if (part_lse[s] > M)
            M = part_lse[s];
    for (long c = 0; c < d; ++c)
        o[c] = 0.0;
    if (M == -INFINITY) {
        *lse = -INFINITY;
        return;
    }
    double wsum = 0.0;
    for (long s = 0; s < nsplit; ++s)
        wsum += exp(part_lse[s] - M);
#if ORACLE_MUTANT == 12
    double L = M;
#else
    double L = M + log(wsum);
#endif
    for (long s = 0; s < nsplit; ++s) {
#if ORACLE_MUTANT == 7
        double w = 1.0;
#else
        double w = exp(part_lse[s] - L);
#endif
        for (long c = 0; c < d; ++c)
            o[c] += w * part_o[s * d + c];
    }
    *lse = L;
}

/*
 * Single-token decode against a key/value cache, the unsplit definition:
 *   q [B, Hq, d], kcache, vcache [B, Hkv, L, d]  ->  o [B, Hq, d], lse [B, Hq]
 * All L cached keys are visible; scale is 1/sqrt(d) (the benchmarked
 * default on the dailyaiworld page).
 */
int oracle_decode(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                  int dtype, long B, long Hq, long Hkv, long L, long d,
                  double *out_o, double *out_lse)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || L < 0 || d < 1)
        return -1;
    long n = B * Hq;
    long *rows = (long *)malloc(sizeof(long) * 3 * (size_t)(n > 0 ? n : 1));
    if (!rows)
        return -1;
    for (long b = 0; b < B; ++b)
        for (long h = 0; h < Hq; ++h) {
            long r = b * Hq + h;
            rows[3 * r] = b;
            rows[3 * r + 1] = h;
            rows[3 * r + 2] = 0;
        }
    int rc = oracle_attention_rows(q, kc, vc, dtype, B, Hq, Hkv, 1, L, d, 0,
                                   1.0 / sqrt((double)d), 0, L, rows, n,
                                   out_o, out_lse);
    free(rows);
    return rc;
}

/*
 * ---------------------------------------------------------------------------
 * Gradients of attention (the backward pass).
 *
 * "Warp Specialization in Triton: Design and Roadmap" (PyTorch blog), section
 * on what is still missing by the authors' own roadmap: the attention
 * backward is the next kernel after the forward.  The pages give no formula
 * for it, so the oracle is the chain rule applied to the definition above,
 * for self-attention (Nq = Nk = N, one key/value head per query head).  With
 * P_ij = exp(s_ij - lse_i) on the keys visible to query i (0 elsewhere),
 * O_i = sum_j P_ij v_j and an upstream gradient dO:
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = <dO_i, v_j>
 *     dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)        (softmax Jacobian)
 *     dQ_i  = scale * sum_j dS_ij k_j
 *     dK_j  = scale * sum_i dS_ij q_i
 * A query with no visible key has no weights and contributes nothing.
 *
 * Inputs are bit patterns of dtype (bf16, fp16), or, with ORACLE_F64, plain
 * doubles: the finite-difference pin perturbs inputs continuously.
 * ---------------------------------------------------------------------------
 */
#define ORACLE_F64 3

static double elem_at(const void *p, long idx, int dtype)
{
    if (dtype == ORACLE_F64)
        return ((const double *)p)[idx];
    return oracle_widen(((const uint16_t *)p)[idx], dtype);
}

/* Per-row statistics of one head: lse_i and Dl_i = sum_k P_ik dP_ik, plus
 * O_i when o is not NULL, for the rows with want[i] != 0 (every row when
 * want is NULL).  Rows run in parallel. */
static int head_row_stats(const double *q, const double *k, const double *v,
                          const double *dout, long N, long d, int causal,
                          double scale, const char *want, double *lse,
                          double *dl, double *o)
{
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *oi = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !oi) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long i = 0; i < N; ++i) {
            if (!s || !oi || (want && !want[i]))
                continue;
            double m = -INFINITY;
            for (long j = 0; j < N; ++j) {
                if (!key_visible(j, i, causal))
                    continue;
                double dot = 0.0;
                for (long c = 0; c < d; ++c)
                    dot += q[i * d + c] * k[j * d + c];
                s[j] = scale * dot;
                if (s[j] > m)
                    m = s[j];
            }
            for (long c = 0; c < d; ++c)
                oi[c] = 0.0;
            if (m == -INFINITY) {
                lse[i] = -INFINITY;
                dl[i] = 0.0;
                if (o)
                    for (long c = 0; c < d; ++c)
                        o[i * d + c] = 0.0;
                continue;
            }
            double l = 0.0;
            for (long j = 0; j < N; ++j)
                if (key_visible(j, i, causal))
                    l += exp(s[j] - m);
            const double L = m + log(l);
            /* sum_k P_ik dP_ik, and O_i */
            double acc = 0.0;
            for (long j = 0; j < N; ++j) {
                if (!key_visible(j, i, causal))
                    continue;
                double p = exp(s[j] - L);
                double dp = 0.0;
                for (long c = 0; c < d; ++c) {
                    dp += dout[i * d + c] * v[j * d + c];
                    oi[c] += p * v[j * d + c];
                }
                acc += p * dp;
            }
            lse[i] = L;
            dl[i] = acc;
            if (o)
                for (long c = 0; c < d; ++c)
                    o[i * d + c] = oi[c];
        }
        free(s);
        free(oi);
    }
    return bad ? -1 : 0;
}

/*
 * Selected gradients of a [B, H, N, d] problem.
 *   q, k, v, dout  [B, H, N, d] of dtype (bits, or doubles with ORACLE_F64)
 *   qrows          nq triples (b, h, i): rows of dQ (and of O, lse) wanted
 *   kcols          nk triples (b, h, j): rows of dK and dV wanted
 *   out_dq [nq, d], out_o [nq, d] (may be NULL), out_lse [nq] (may be NULL),
 *   out_dk, out_dv [nk, d]
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attention_bwd(const void *q, const void *k, const void *v,
                         const void *dout, int dtype, long B, long H, long N,
                         long d, int causal, double scale, const long *qrows,
                         long nq, const long *kcols, long nk, double *out_dq,
                         double *out_o, double *out_lse, double *out_dk,
                         double *out_dv)
{
    if (!q || !k || !v || !dout || (nq && (!qrows || !out_dq)) ||
        (nk && (!kcols || !out_dk || !out_dv)))
        return -1;
    if (B < 0 || H < 1 || N < 0 || d < 1 || nq < 0 || nk < 0)
        return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16 && dtype != ORACLE_F64)
        return -1;
    for (long r = 0; r < nq + nk; ++r) {
        const long *t = r < nq ? qrows + 3 * r : kcols + 3 * (r - nq);
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= N)
            return -1;
    }
    const size_t nd = (size_t)N * (size_t)d;
    double *hq = (double *)malloc(sizeof(double) * (nd ? nd : 1));
    double *hk = (double *)malloc(sizeof(double) * (nd ? nd : 1));
    double *hv = (double *)malloc(sizeof(double) * (nd ? nd : 1));
    double *hdo = (double *)malloc(sizeof(double) * (nd ? nd : 1));
    double *lse = (double *)malloc(sizeof(double) * (size_t)(N ? N : 1));
    double *dl = (double *)malloc(sizeof(double) * (size_t)(N ? N : 1));
    double *ho = out_o ? (double *)malloc(sizeof(double) * (nd ? nd : 1)) : NULL;
    int rc = 0;
    if (!hq || !hk || !hv || !hdo || !lse || !dl || (out_o && !ho))
        rc = -1;

    /* One head at a time: every head named by either list. */
    for (long bh = 0; rc == 0 && bh < B * H; ++bh) {
        long b = bh / H, h = bh % H;
        int needed = 0;
        for (long r = 0; r < nq + nk && !needed; ++r) {
            const long *t = r < nq ? qrows + 3 * r : kcols + 3 * (r - nq);
            needed = t[0] == b && t[1] == h;
        }
        if (!needed)
            continue;
        const long base = bh * (long)nd;
        for (size_t e = 0; e < nd; ++e) {
            hq[e] = elem_at(q, base + (long)e, dtype);
            hk[e] = elem_at(k, base + (long)e, dtype);
            hv[e] = elem_at(v, base + (long)e, dtype);
            hdo[e] = elem_at(dout, base + (long)e, dtype);
        }
        /* dK and dV need every row's statistics; dQ rows only their own. */
        int all_rows = 0;
        for (long r = 0; r < nk && !all_rows; ++r)
            all_rows = kcols[3 * r] == b && kcols[3 * r + 1] == h;
        char *want = NULL;
        if (!all_rows) {
            want = (char *)calloc((size_t)(N ? N : 1), 1);
            if (!want) {
                rc = -1;
                break;
            }
            for (long r = 0; r < nq; ++r)
                if (qrows[3 * r] == b && qrows[3 * r + 1] == h)
                    want[qrows[3 * r + 2]] = 1;
        }
        int st = head_row_stats(hq, hk, hv, hdo, N, d, causal, scale, want, lse, dl, ho);
        free(want);
        if (st) {
            rc = -1;
            break;
        }

        /* dQ_i = scale * sum_j P_ij (dP_ij - Dl_i) k_j */
#pragma omp parallel for schedule(dynamic, 1)
        for (long r = 0; r < nq; ++r) {
            const long *t = qrows + 3 * r;
            if (t[0] != b || t[1] != h)
                continue;
            const long i = t[2];
            double *g = out_dq + r * d;
            for (long c = 0; c < d; ++c)
                g[c] = 0.0;
            if (out_o)
                for (long c = 0; c < d; ++c)
                    out_o[r * d + c] = ho[i * d + c];
            if (out_lse)
                out_lse[r] = lse[i];
            if (lse[i] == -INFINITY)
                continue;
            for (long j = 0; j < N; ++j) {
                if (!key_visible(j, i, causal))
                    continue;
                double dot = 0.0, dp = 0.0;
                for (long c = 0; c < d; ++c) {
                    dot += hq[i * d + c] * hk[j * d + c];
                    dp += hdo[i * d + c] * hv[j * d + c];
                }
                const double p = exp(scale * dot - lse[i]);
#if ORACLE_MUTANT == 15
                const double ds = p * dp;
#else
                const double ds = p * (dp - dl[i]);
#endif
                for (long c = 0; c < d; ++c)
                    g[c] += ds * hk[j * d + c];
            }
#if ORACLE_MUTANT != 16
            for (long c = 0; c < d; ++c)
                g[c] *= scale;
#endif
        }

        /* dV_j = sum_i P_ij dO_i;  dK_j = scale * sum_i dS_ij q_i */
#pragma omp parallel for schedule(dynamic, 1)
        for (long r = 0; r < nk; ++r) {
            const long *t = kcols + 3 * r;
            if (t[0] != b || t[1] != h)
                continue;
            const long j = t[2];
            double *gk = out_dk + r * d, *gv = out_dv + r * d;
            for (long c = 0; c < d; ++c)
                gk[c] = gv[c] = 0.0;
            for (long i = 0; i < N; ++i) {
#if ORACLE_MUTANT == 19
                if (lse[i] == -INFINITY)
#else
                if (!key_visible(j, i, causal) || lse[i] == -INFINITY)
#endif
                    continue;
                double dot = 0.0, dp = 0.0;
                for (long c = 0; c < d; ++c) {
                    dot += hq[i * d + c] * hk[j * d + c];
                    dp += hdo[i * d + c] * hv[j * d + c];
                }
#if ORACLE_MUTANT == 17
                const double p = exp(scale * dot);
#else
                const double p = exp(scale * dot - lse[i]);
#endif
                const double ds = p * (dp - dl[i]);
                for (long c = 0; c < d; ++c) {
                    gv[c] += p * hdo[i * d + c];
#if ORACLE_MUTANT == 18
                    gk[c] += ds * hdo[i * d + c];
#else
                    gk[c] += ds * hq[i * d + c];
#endif
                }
            }
            for (long c = 0; c < d; ++c)
                gk[c] *= scale;
        }
    }
    free(hq);
    free(hk);
    free(hv);
    free(hdo);
    free(lse);
    free(dl);
    free(ho);
    return rc;
}

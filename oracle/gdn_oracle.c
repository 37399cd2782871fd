/*
 * gdn_oracle.c -- fp64 CPU oracle of the Gated DeltaNet (GDN) token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library: it is a plain, slow, literal
 * token-by-token evaluation of the recurrence, kept obviously correct so that
 * the GPU kernels can be checked against it.
 *
 * What is computed (the gated delta rule).  The pages describe the GDN layer
 * only in words: a linear-attention block driven by a gated delta rule that
 * keeps a fixed-size recurrent state instead of a KV cache (kwkr.cn digest of
 * HyLo-Llama-8MLA8GDN-8K-SFT, section on the 8 MLA + 8 Gated DeltaNet
 * architecture), and which can erase or rewrite the value stored under one
 * key instead of decaying everything uniformly (we0.ai article on Priming,
 * comparison of Mamba-2, Gated DeltaNet and Gated KalmaNet).  The update used
 * here is the standard form of that rule:
 *
 *     S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     o_t = S_t q_t / sqrt(d_k)
 *     a_t = exp(g_t)              (g is the log-gate)
 *
 * with S in R^{d_v x d_k}.  Readout uses the updated state S_t.
 *
 * Second rule (ORC_RULE_GATED_DECAY): the same gated recurrence without the
 * erase term,
 *
 *     S_t = a_t * S_{t-1} + b_t v_t k_t^T
 *
 * i.e. the uniform decay the Priming article attributes to Mamba-2 (we0.ai
 * article, comparison of Mamba-2, Gated DeltaNet and Gated KalmaNet: the
 * state decays as a whole while new information is added), with b_t as the
 * write strength.  Readout and layouts are as above.
 *
 * Because (I - b k k^T) acts on the key side only, row i of S (value dim i)
 * evolves on its own:
 *     S_t[i,:] = a_t * (S_{t-1}[i,:] - b_t * (S_{t-1}[i,:] . k_t) * k_t)
 *                + b_t * v_t[i] * k_t
 *     o_t[i]   = (S_t[i,:] . q_t) / sqrt(d_k)
 * which is the same arithmetic as the matrix form written out one row at a
 * time; the oracle walks rows independently so it can also evaluate a subset
 * of value rows for very long inputs.
 *
 * Layouts (row-major, dense):
 *   q, k       [B, T, H, d_k]
 *   v          [B, T, H, d_v]
 *   g, beta    [B, T, H]
 *   s0, s_out  [B, H, d_k, d_v]   key-major: element (j, i) holds S[i][j]
 *   o          [B, T, H, d_v]
 * Inputs may be stored as fp64, fp32 or bf16 bits; every stored value is
 * widened exactly to fp64 before use.  All arithmetic is fp64.
 *
 * gdn_oracle_backward_rule gives the gradients of both rules by the adjoint of
 * the same recurrence, token by token (see its comment).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };
enum { ORC_RULE_GATED_DELTA = 0, ORC_RULE_GATED_DECAY = 1 };

static double orc_load(const void *p, int dtype, long idx)
{
    if (dtype == ORC_F64)
        return ((const double *)p)[idx];
    if (dtype == ORC_F32)
        return (double)((const float *)p)[idx];
    /* bf16: the upper 16 bits of an IEEE binary32 */
    uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Token-by-token prefill.
 *   rule:      ORC_RULE_GATED_DELTA or ORC_RULE_GATED_DECAY
 *   qkv_dtype: storage type of q, k, v (ORC_F64 / ORC_F32 / ORC_BF16)
 *   gb_dtype:  storage type of g and beta
 *   s0_dtype:  storage type of s0 (ignored when s0 == NULL, which means zeros)
 *   rows/nrows: value rows to evaluate (NULL = all d_v rows).  Only those
 *               entries of o and s_out are written.
 * Returns 0, or -1 on a bad argument.
 */
int gdn_oracle_prefill_rule(int rule, const void *q, const void *k, const void *v, int qkv_dtype,
                            const void *g, const void *beta, int gb_dtype,
                            const void *s0, int s0_dtype,
                            double *o, double *s_out,
                            long B, long T, long H, long dk, long dv,
                            const int *rows, long nrows)
{
    if (rule != ORC_RULE_GATED_DELTA && rule != ORC_RULE_GATED_DECAY)
        return -1;
    if (!q || !k || !v || !g || !beta || !o || !s_out)
        return -1;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (rows == NULL)
        nrows = dv;
    if (nrows <= 0 || nrows > dv)
        return -1;
    for (long r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= dv)
            return -1;

    const double scale = 1.0 / sqrt((double)dk);
    const long ntask = B * H * nrows;

#pragma omp parallel
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)dk);
#pragma omp for schedule(dynamic, 1)
        for (long task = 0; task < ntask; ++task) {
            const long r = task % nrows;
            const long h = (task / nrows) % H;
            const long b = task / (nrows * H);
            const long i = rows ? rows[r] : r;

            /* S[i][:] <- initial state row (or zeros) */
            for (long j = 0; j < dk; ++j)
                srow[j] = s0 ? orc_load(s0, s0_dtype, ((b * H + h) * dk + j) * dv + i) : 0.0;

            for (long t = 0; t < T; ++t) {
                const long bth = (b * T + t) * H + h;
                const double a = exp(orc_load(g, gb_dtype, bth));
                const double bt = orc_load(beta, gb_dtype, bth);
                const double vi = orc_load(v, qkv_dtype, bth * dv + i);

                if (rule == ORC_RULE_GATED_DECAY) {
                    /* S_t[i,:] = a S_{t-1}[i,:] + b v_i k_t */
                    for (long j = 0; j < dk; ++j)
                        srow[j] = a * srow[j] + bt * vi * orc_load(k, qkv_dtype, bth * dk + j);
                } else {
                    /* w = S_{t-1}[i,:] . k_t */
                    double w = 0.0;
                    for (long j = 0; j < dk; ++j)
                        w += srow[j] * orc_load(k, qkv_dtype, bth * dk + j);

                    /* S_t[i,:] = a (S_{t-1}[i,:] - b w k_t) + b v_i k_t */
                    for (long j = 0; j < dk; ++j) {
                        const double kj = orc_load(k, qkv_dtype, bth * dk + j);
                        srow[j] = a * (srow[j] - bt * w * kj) + bt * vi * kj;
                    }
                }

                /* o_t[i] = S_t[i,:] . q_t / sqrt(d_k) */
                double acc = 0.0;
                for (long j = 0; j < dk; ++j)
                    acc += srow[j] * orc_load(q, qkv_dtype, bth * dk + j);
                o[bth * dv + i] = acc * scale;
            }

            for (long j = 0; j < dk; ++j)
                s_out[((b * H + h) * dk + j) * dv + i] = srow[j];
        }
        free(srow);
    }
    return 0;
}

/* The gated delta rule (the library's default). */
int gdn_oracle_prefill(const void *q, const void *k, const void *v, int qkv_dtype,
                       const void *g, const void *beta, int gb_dtype,
                       const void *s0, int s0_dtype,
                       double *o, double *s_out,
                       long B, long T, long H, long dk, long dv,
                       const int *rows, long nrows)
{
    return gdn_oracle_prefill_rule(ORC_RULE_GATED_DELTA, q, k, v, qkv_dtype, g, beta, gb_dtype,
                                   s0, s0_dtype, o, s_out, B, T, H, dk, dv, rows, nrows);
}

/*
 * One decode step for N independent sequences: the prefill recurrence with
 * T = 1.  q, k, v: [N, H, d]; g, beta: [N, H]; state: [N, H, d_k, d_v]
 * (key-major, fp64, updated in place); o: [N, H, d_v].
 */
int gdn_oracle_decode_step_rule(int rule, const void *q, const void *k, const void *v, int qkv_dtype,
                                const void *g, const void *beta, int gb_dtype,
                                double *state, double *o, long N, long H, long dk, long dv)
{
    return gdn_oracle_prefill_rule(rule, q, k, v, qkv_dtype, g, beta, gb_dtype, state, ORC_F64,
                                   o, state, N, 1, H, dk, dv, NULL, 0);
}

int gdn_oracle_decode_step(const void *q, const void *k, const void *v, int qkv_dtype,
                           const void *g, const void *beta, int gb_dtype,
                           double *state, double *o, long N, long H, long dk, long dv)
{
    return gdn_oracle_decode_step_rule(ORC_RULE_GATED_DELTA, q, k, v, qkv_dtype, g, beta, gb_dtype,
                                       state, o, N, H, dk, dv);
}

/*
 * Gradients of the prefill (reverse-mode, token by token).
 *
 * The loss is taken to be L = sum_t <do_t, o_t> + <dS_T, S_T>: do holds the
 * gradient with respect to every output and ds_final the gradient with respect
 * to the final state (NULL = zero).  The adjoint of the recurrence, written out
 * from the forward definitions above, with D the gradient with respect to S_t
 * (d_v x d_k) accumulated from the end:
 *
 *   D     += scale do_t q_t^T                     (readout o_t = scale S_t q_t)
 *   dq_t   = scale S_t^T do_t
 *   dv_t   = b_t D k_t                            (write term b_t v_t k_t^T)
 *   db_t   = v_t^T D k_t  (+ erase part)
 *   dk_t   = b_t D^T v_t  (+ erase part)
 *   with M_t = a_t (I - b_t k_t k_t^T) (gated delta) or a_t I (gated decay) and
 *   dM = S_{t-1}^T D:
 *     da_t   = tr(dM) - b_t k_t^T dM k_t          (decay rule: tr(dM))
 *     erase: db_t -= a_t k_t^T dM k_t,  dk_t -= a_t b_t (dM + dM^T) k_t
 *     dg_t   = a_t da_t                           (a_t = exp(g_t))
 *   D      = D M_t^T                              (gradient passed to S_{t-1})
 * and finally ds0 = D.  dM is never formed: tr(dM) = <S_{t-1}, D>,
 * dM k = S_{t-1}^T (D k), dM^T k = D^T (S_{t-1} k), k^T dM k = (S_{t-1} k) . (D k).
 *
 * The forward states are recomputed from checkpoints (every ORC_CKPT tokens),
 * so memory stays O(T/ORC_CKPT * d_v * d_k) per (batch, head); the recomputed
 * states are bit for bit the ones of a single forward sweep.
 *
 * Layouts as the prefill; do [B, T, H, d_v] and ds_final [B, H, d_k, d_v]
 * (key-major) in do_dtype; outputs fp64: dq, dk [B, T, H, d_k], dv
 * [B, T, H, d_v], dg, dbeta [B, T, H], ds0 [B, H, d_k, d_v] (key-major).
 * Returns 0, or -1 on a bad argument.
 */
#define ORC_CKPT 64

int gdn_oracle_backward_rule(int rule, const void *q, const void *k, const void *v, int qkv_dtype,
                             const void *g, const void *beta, int gb_dtype,
                             const void *s0, int s0_dtype,
                             const void *d_o, const void *ds_final, int do_dtype,
                             double *dq, double *dk_out, double *dv_out, double *dg, double *dbeta,
                             double *ds0, long B, long T, long H, long dk, long dv)
{
    if (rule != ORC_RULE_GATED_DELTA && rule != ORC_RULE_GATED_DECAY)
        return -1;
    if (!ds0 || (T > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk_out || !dv_out ||
                           !dg || !dbeta)))
        return -1;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    const int delta = rule == ORC_RULE_GATED_DELTA;
    const double scale = 1.0 / sqrt((double)dk);
    const long ncp = (T + ORC_CKPT - 1) / ORC_CKPT;
    const long SZ = dv * dk; /* one state, row-major [i][j] = S[i][j] */

#pragma omp parallel
    {
        double *ckpt = (double *)malloc(sizeof(double) * (size_t)((ncp > 0 ? ncp : 1) * SZ));
        double *seg = (double *)malloc(sizeof(double) * (size_t)((ORC_CKPT + 1) * SZ));
        double *D = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *kt = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qt = (double *)malloc(sizeof(double) * (size_t)dk);
        double *vt = (double *)malloc(sizeof(double) * (size_t)dv);
        double *dot = (double *)malloc(sizeof(double) * (size_t)dv);
        double *Dk = (double *)malloc(sizeof(double) * (size_t)dv);
        double *Sk = (double *)malloc(sizeof(double) * (size_t)dv);
        double *dMk = (double *)malloc(sizeof(double) * (size_t)dk);
        double *dMtk = (double *)malloc(sizeof(double) * (size_t)dk);
#pragma omp for schedule(dynamic, 1)
        for (long task = 0; task < B * H; ++task) {
            const long h = task % H;
            const long b = task / H;

            /* forward sweep: the state at the start of every checkpoint segment */
            double *S = seg; /* scratch: the running state */
            for (long i = 0; i < dv; ++i)
                for (long j = 0; j < dk; ++j)
                    S[i * dk + j] = s0 ? orc_load(s0, s0_dtype, ((b * H + h) * dk + j) * dv + i) : 0.0;
            for (long t = 0; t < T; ++t) {
                if (t % ORC_CKPT == 0)
                    memcpy(ckpt + (t / ORC_CKPT) * SZ, S, sizeof(double) * (size_t)SZ);
                const long bth = (b * T + t) * H + h;
                const double a = exp(orc_load(g, gb_dtype, bth));
                const double bt = orc_load(beta, gb_dtype, bth);
                for (long j = 0; j < dk; ++j)
                    kt[j] = orc_load(k, qkv_dtype, bth * dk + j);
                for (long i = 0; i < dv; ++i) {
                    double *row = S + i * dk;
                    const double vi = orc_load(v, qkv_dtype, bth * dv + i);
                    double w = 0.0;
                    if (delta)
                        for (long j = 0; j < dk; ++j)
                            w += row[j] * kt[j];
                    for (long j = 0; j < dk; ++j)
                        row[j] = a * (row[j] - bt * w * kt[j]) + bt * vi * kt[j];
                }
            }

            /* reverse sweep */
            for (long i = 0; i < dv; ++i)
                for (long j = 0; j < dk; ++j)
                    D[i * dk + j] =
                        ds_final ? orc_load(ds_final, do_dtype, ((b * H + h) * dk + j) * dv + i) : 0.0;
            for (long c = ncp - 1; c >= 0; --c) {
                const long t0 = c * ORC_CKPT;
                const long t1 = (t0 + ORC_CKPT < T) ? t0 + ORC_CKPT : T;
                /* seg[u] = S_{t0 + u - 1}: the state before token t0 + u */
                memcpy(seg, ckpt + c * SZ, sizeof(double) * (size_t)SZ);
                for (long t = t0; t < t1; ++t) {
                    const double *Sp = seg + (t - t0) * SZ;
                    double *Sn = seg + (t - t0 + 1) * SZ;
                    const long bth = (b * T + t) * H + h;
                    const double a = exp(orc_load(g, gb_dtype, bth));
                    const double bt = orc_load(beta, gb_dtype, bth);
                    for (long j = 0; j < dk; ++j)
                        kt[j] = orc_load(k, qkv_dtype, bth * dk + j);
                    for (long i = 0; i < dv; ++i) {
                        const double vi = orc_load(v, qkv_dtype, bth * dv + i);
                        double w = 0.0;
                        if (delta)
                            for (long j = 0; j < dk; ++j)
                                w += Sp[i * dk + j] * kt[j];
                        for (long j = 0; j < dk; ++j)
                            Sn[i * dk + j] = a * (Sp[i * dk + j] - bt * w * kt[j]) + bt * vi * kt[j];
                    }
                }
                for (long t = t1 - 1; t >= t0; --t) {
                    const double *Sp = seg + (t - t0) * SZ;     /* S_{t-1} */
                    const double *St = seg + (t - t0 + 1) * SZ; /* S_t */
                    const long bth = (b * T + t) * H + h;
                    const double a = exp(orc_load(g, gb_dtype, bth));
                    const double bt = orc_load(beta, gb_dtype, bth);
                    for (long j = 0; j < dk; ++j) {
                        kt[j] = orc_load(k, qkv_dtype, bth * dk + j);
                        qt[j] = orc_load(q, qkv_dtype, bth * dk + j);
                    }
                    for (long i = 0; i < dv; ++i) {
                        vt[i] = orc_load(v, qkv_dtype, bth * dv + i);
                        dot[i] = orc_load(d_o, do_dtype, bth * dv + i);
                    }
                    /* readout: D += scale do q^T; dq = scale S_t^T do */
                    for (long i = 0; i < dv; ++i)
                        for (long j = 0; j < dk; ++j)
                            D[i * dk + j] += scale * dot[i] * qt[j];
                    for (long j = 0; j < dk; ++j) {
                        double acc = 0.0;
                        for (long i = 0; i < dv; ++i)
                            acc += St[i * dk + j] * dot[i];
                        dq[bth * dk + j] = scale * acc;
                    }
                    /* D k, S_{t-1} k, <S_{t-1}, D> */
                    double tr = 0.0, kdk = 0.0, vdk = 0.0;
                    for (long i = 0; i < dv; ++i) {
                        double x = 0.0, y = 0.0;
                        for (long j = 0; j < dk; ++j) {
                            x += D[i * dk + j] * kt[j];
                            y += Sp[i * dk + j] * kt[j];
                            tr += Sp[i * dk + j] * D[i * dk + j];
                        }
                        Dk[i] = x;
                        Sk[i] = y;
                        kdk += y * x;
                        vdk += vt[i] * x;
                    }
                    /* write term */
                    for (long i = 0; i < dv; ++i)
                        dv_out[bth * dv + i] = bt * Dk[i];
                    double db = vdk;
                    for (long j = 0; j < dk; ++j) {
                        double acc = 0.0;
                        for (long i = 0; i < dv; ++i)
                            acc += D[i * dk + j] * vt[i];
                        dk_out[bth * dk + j] = bt * acc;
                    }
                    /* decay / erase term */
                    double da = tr;
                    if (delta) {
                        da -= bt * kdk;
                        db -= a * kdk;
                        for (long j = 0; j < dk; ++j) {
                            double x = 0.0, y = 0.0;
                            for (long i = 0; i < dv; ++i) {
                                x += Sp[i * dk + j] * Dk[i];
                                y += D[i * dk + j] * Sk[i];
                            }
                            dMk[j] = x;
                            dMtk[j] = y;
                        }
                        for (long j = 0; j < dk; ++j)
                            dk_out[bth * dk + j] -= a * bt * (dMk[j] + dMtk[j]);
                    }
                    dbeta[bth] = db;
                    dg[bth] = a * da;
                    /* D <- D M_t^T */
                    for (long i = 0; i < dv; ++i)
                        for (long j = 0; j < dk; ++j)
                            D[i * dk + j] = a * (D[i * dk + j] - (delta ? bt * Dk[i] * kt[j] : 0.0));
                }
            }
            for (long i = 0; i < dv; ++i)
                for (long j = 0; j < dk; ++j)
                    ds0[((b * H + h) * dk + j) * dv + i] = D[i * dk + j];
        }
        free(ckpt);
        free(seg);
        free(D);
        free(kt);
        free(qt);
        free(vt);
        free(dot);
        free(Dk);
        free(Sk);
        free(dMk);
        free(dMtk);
    }
    return 0;
}

/* Threads an OpenMP parallel region of this library uses (for reporting). */
int gdn_oracle_num_threads(void)
{
    return omp_get_max_threads();
}

/* Threads the next calls use (n >= 1), for timing the oracle on fewer cores. */
void gdn_oracle_set_num_threads(int n)
{
    if (n >= 1) omp_set_num_threads(n);
}

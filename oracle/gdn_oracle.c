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

/* Threads an OpenMP parallel region of this library uses (for reporting). */
int gdn_oracle_num_threads(void)
{
    return omp_get_max_threads();
}

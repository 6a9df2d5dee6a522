/*
 * kda_oracle.c -- fp64 CPU oracle of the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow reference that the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the GPU library never does, and the
 * two share no code.
 *
 * What it computes (per sequence s and head h, tokens in order):
 *
 *   S <- initial state (zeros when absent), widened to fp64
 *   for each token t of the sequence:
 *     a   = exp(g_t)                    per-channel decay over the key rows
 *     S   = Diag(a) S                   forget first ...
 *     u   = beta_t (v_t - S^T k_t)      ... then one delta-rule step: the
 *     S   = S + k_t u^T                 value-retrieval error of key k_t
 *     o_t = S^T q_t                     readout from the updated state
 *
 * i.e. S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 * o_t = S_t^T q_t.  Sources: the delta rule as a step that minimises the L2
 * norm of the value-retrieval error and removes mismatched associations
 * (Kimi K3 report, English and Chinese editions, "Methodology notes" /
 * "DeltaNet and Delta Rule"; SemiAnalysis digest, section 1 on KDA), and the
 * forgetting factor widened to a diagonal matrix for per-channel decay
 * (same pages, "Kimi Delta Attention" bullet). The pages state these in prose;
 * the explicit matrix form above is the reading taken here.
 *
 * Readings where the pages are silent: no attention scale; q and k are used
 * exactly as given (the caller L2-normalises them; oracle/frontend.py holds
 * the parameter-free input transforms, applied in fp64 before this file's
 * recurrence when the inputs are raw); g = log(alpha) is the input; a checkpoint is a copy of S after every ckpt_interval tokens of a
 * sequence; a zero-length sequence returns its initial state.
 *
 * Columns of S (value channels) never interact, so a work unit is
 * (sequence, head, block of columns); running units in any order or on any
 * number of threads performs exactly the same floating-point operations.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* every input (q, k, v, g, beta) is fp64 */

static double in_val(const void *p, int dtype, int64_t i)
{
    if (dtype == ORC_F64)
        return ((const double *)p)[i];
    if (dtype == ORC_F32)
        return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* g and beta: fp64 with ORC_F64 inputs, fp32 otherwise. */
static double gb_val(const void *p, int dtype, int64_t i)
{
    return dtype == ORC_F64 ? ((const double *)p)[i] : (double)((const float *)p)[i];
}

/* One token on columns [j0, j0 + nc) of S (row-major Dk x nc, fp64). */
static void token_step(double *S, int Dk, int nc, int j0,
                       const void *q, const void *k, const void *v, int dtype,
                       int64_t qk_off, int64_t v_off, const void *g, double beta,
                       double *kv, double *qv, double *u, double *o_out /* nc or NULL */)
{
    for (int i = 0; i < Dk; ++i) {
        double a = exp(gb_val(g, dtype, qk_off + i));
        kv[i] = in_val(k, dtype, qk_off + i);
        qv[i] = in_val(q, dtype, qk_off + i);
        double *row = S + (int64_t)i * nc;
        for (int j = 0; j < nc; ++j)
            row[j] *= a;
    }
    for (int j = 0; j < nc; ++j) {
        double r = 0.0;
        for (int i = 0; i < Dk; ++i)
            r += S[(int64_t)i * nc + j] * kv[i];
        u[j] = beta * (in_val(v, dtype, v_off + j0 + j) - r);
    }
    for (int i = 0; i < Dk; ++i) {
        double *row = S + (int64_t)i * nc;
        for (int j = 0; j < nc; ++j)
            row[j] += kv[i] * u[j];
    }
    if (o_out) {
        for (int j = 0; j < nc; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i)
                acc += S[(int64_t)i * nc + j] * qv[i];
            o_out[j] = acc;
        }
    }
}

static int set_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
    return omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}

/*
 * Prefill over packed sequences.
 *   q, k [N, H, Dk], v [N, H, Dv]  fp32 or bf16 bits (dtype), or fp64
 *   g [N, H, Dk], beta [N, H]  fp32 (fp64 when dtype is ORC_F64)
 *   cu_seqlens [num_seqs + 1] (int64), packed token offsets
 *   initial_state [num_seqs, H, Dk, Dv] fp32 or NULL (zeros)
 *   final_state   [num_seqs, H, Dk, Dv] fp64 or NULL
 *   ckpt_interval 0 = none; ckpt [sum_s floor(L_s / interval), H, Dk, Dv] fp64
 *   o [N, H, Dv] fp64
 *   units: n_units triples (seq, head, column block) or NULL for all;
 *   only the outputs of the listed units are written.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int kda_oracle_prefill(const void *q, const void *k, const void *v, int dtype,
                       const void *g, const void *beta,
                       const int64_t *cu_seqlens, int num_seqs, int H, int Dk, int Dv,
                       const float *initial_state, double *final_state,
                       int64_t ckpt_interval, double *ckpt, double *o,
                       const int32_t *units, int64_t n_units, int col_block,
                       int n_threads)
{
    if (num_seqs < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || col_block <= 0)
        return -1;
    if (ckpt_interval < 0 || (ckpt_interval > 0 && !ckpt))
        return -1;
    int n_cb = (Dv + col_block - 1) / col_block;
    int64_t total_units = (int64_t)num_seqs * H * n_cb;
    int64_t nu = units ? n_units : total_units;

    int64_t *ckbase = (int64_t *)calloc((size_t)num_seqs + 1, sizeof(int64_t));
    if (!ckbase)
        return -1;
    for (int s = 0; s < num_seqs; ++s) {
        int64_t L = cu_seqlens[s + 1] - cu_seqlens[s];
        ckbase[s + 1] = ckbase[s] + (ckpt_interval > 0 ? L / ckpt_interval : 0);
    }

    set_threads(n_threads);
    int failed = 0;
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * col_block);
        double *kv = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *qv = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *u = (double *)malloc(sizeof(double) * (size_t)col_block);
        double *ob = (double *)malloc(sizeof(double) * (size_t)col_block);
        if (!S || !kv || !qv || !u || !ob) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t w = 0; w < nu; ++w) {
                int s, h, cb;
                if (units) {
                    s = units[3 * w];
                    h = units[3 * w + 1];
                    cb = units[3 * w + 2];
                } else {
                    s = (int)(w / ((int64_t)H * n_cb));
                    h = (int)((w / n_cb) % H);
                    cb = (int)(w % n_cb);
                }
                if (s < 0 || s >= num_seqs || h < 0 || h >= H || cb < 0 || cb >= n_cb) {
#pragma omp atomic write
                    failed = 1;
                    continue;
                }
                int j0 = cb * col_block;
                int nc = (Dv - j0 < col_block) ? Dv - j0 : col_block;
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < nc; ++j)
                        S[(int64_t)i * nc + j] = initial_state
                            ? (double)initial_state[(((int64_t)s * H + h) * Dk + i) * Dv + j0 + j]
                            : 0.0;
                int64_t t0 = cu_seqlens[s], t1 = cu_seqlens[s + 1];
                for (int64_t t = t0; t < t1; ++t) {
                    int64_t qk_off = (t * H + h) * (int64_t)Dk;
                    int64_t v_off = (t * H + h) * (int64_t)Dv;
                    token_step(S, Dk, nc, j0, q, k, v, dtype, qk_off, v_off, g,
                               gb_val(beta, dtype, t * H + h), kv, qv, u, ob);
                    for (int j = 0; j < nc; ++j)
                        o[v_off + j0 + j] = ob[j];
                    int64_t done = t + 1 - t0;
                    if (ckpt_interval > 0 && done % ckpt_interval == 0) {
                        int64_t c = ckbase[s] + done / ckpt_interval - 1;
                        for (int i = 0; i < Dk; ++i)
                            for (int j = 0; j < nc; ++j)
                                ckpt[((c * H + h) * Dk + i) * (int64_t)Dv + j0 + j] =
                                    S[(int64_t)i * nc + j];
                    }
                }
                if (final_state)
                    for (int i = 0; i < Dk; ++i)
                        for (int j = 0; j < nc; ++j)
                            final_state[(((int64_t)s * H + h) * Dk + i) * Dv + j0 + j] =
                                S[(int64_t)i * nc + j];
            }
        }
        free(S);
        free(kv);
        free(qv);
        free(u);
        free(ob);
    }
    free(ckbase);
    return failed ? -1 : 0;
}

/*
 * One decode step for B independent sequences: the same token body on an
 * fp64 state [B, H, Dk, Dv] that is read and updated in place.
 *   q, k [B, H, Dk], v [B, H, Dv] (dtype), g [B, H, Dk], beta [B, H] (fp32, or
 *   fp64 when dtype is ORC_F64), o [B, H, Dv] fp64.
 *   units: (batch, head, column block) triples or NULL for all.
 */
int kda_oracle_decode(const void *q, const void *k, const void *v, int dtype,
                      const void *g, const void *beta, int B, int H, int Dk, int Dv,
                      double *state, double *o, const int32_t *units, int64_t n_units,
                      int col_block, int n_threads)
{
    if (B < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || col_block <= 0 || !state)
        return -1;
    int n_cb = (Dv + col_block - 1) / col_block;
    int64_t nu = units ? n_units : (int64_t)B * H * n_cb;
    set_threads(n_threads);
    int failed = 0;
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * col_block);
        double *kv = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *qv = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *u = (double *)malloc(sizeof(double) * (size_t)col_block);
        double *ob = (double *)malloc(sizeof(double) * (size_t)col_block);
        if (!S || !kv || !qv || !u || !ob) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t w = 0; w < nu; ++w) {
                int b, h, cb;
                if (units) {
                    b = units[3 * w];
                    h = units[3 * w + 1];
                    cb = units[3 * w + 2];
                } else {
                    b = (int)(w / ((int64_t)H * n_cb));
                    h = (int)((w / n_cb) % H);
                    cb = (int)(w % n_cb);
                }
                if (b < 0 || b >= B || h < 0 || h >= H || cb < 0 || cb >= n_cb) {
#pragma omp atomic write
                    failed = 1;
                    continue;
                }
                int j0 = cb * col_block;
                int nc = (Dv - j0 < col_block) ? Dv - j0 : col_block;
                double *St = state + ((int64_t)b * H + h) * (int64_t)Dk * Dv;
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < nc; ++j)
                        S[(int64_t)i * nc + j] = St[(int64_t)i * Dv + j0 + j];
                int64_t qk_off = ((int64_t)b * H + h) * Dk;
                int64_t v_off = ((int64_t)b * H + h) * Dv;
                token_step(S, Dk, nc, j0, q, k, v, dtype, qk_off, v_off, g,
                           gb_val(beta, dtype, (int64_t)b * H + h), kv, qv, u, ob);
                for (int j = 0; j < nc; ++j)
                    o[v_off + j0 + j] = ob[j];
                for (int i = 0; i < Dk; ++i)
                    for (int j = 0; j < nc; ++j)
                        St[(int64_t)i * Dv + j0 + j] = S[(int64_t)i * nc + j];
            }
        }
        free(S);
        free(kv);
        free(qv);
        free(u);
        free(ob);
    }
    return failed ? -1 : 0;
}

int kda_oracle_num_threads(int n_threads) { return set_threads(n_threads); }

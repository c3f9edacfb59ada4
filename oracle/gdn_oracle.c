/*
 * gdn_oracle.c -- fp64 CPU oracle for the gated delta rule (TEST INFRASTRUCTURE ONLY).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load this
 * library.  It shares no code, header or table with the HIP implementation.
 *
 * What it computes (jianyuh.github.io reading notes, "Qwen3.8-Next-GDN-QSA-Gated-Residual",
 * section 2.1 "Gated DeltaNet", the four-line gated delta recurrence): for every sequence n
 * and head h, starting from S = S0[n,h] (zeros when no initial state is given), and for every
 * token t of the sequence in order,
 *
 *     S~  = alpha_t * S                      (decay the whole state)
 *     e   = v_t - S~^T k_t                   (what the key already retrieves, subtracted)
 *     S   = S~ + beta_t * k_t e^T            (write the residual along k_t)
 *     y_t = S^T q_t                          (read the updated state with the query)
 *
 * with S a d_k x d_v matrix (the page's "transposed convention": rows follow the key
 * dimension).  Every quantity is held in double precision; bf16 and fp32 inputs widen to
 * double exactly.  The loops are the definition written out, one token at a time, with no
 * blocking, chunking or reordering.  OpenMP only distributes independent (sequence, head)
 * pairs over threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to double. */
static double load_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_F64) return ((const double *)base)[idx];
    if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
    /* bf16: the upper half of an IEEE binary32 word. */
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Run the recurrence for every (sequence, head) pair.
 *
 * Row addressing: token s (0-based) of sequence n sits at row  seq_row0[n] + s * row_step
 * of the activation tensors, which are laid out [rows, H, d] (q, k: d = d_k; v: d = d_v)
 * and [rows, H] (alpha, beta).  A packed prefill batch uses row_step = 1 and seq_row0 =
 * cu_seqlens; a stack of decode steps laid out [steps, B, H, d] uses seq_row0[b] = b and
 * row_step = B.
 *
 * Heads head_lo <= h < head_hi are computed.  Outputs hold only those heads:
 *   y        [rows, head_hi - head_lo, d_v]           (rows not visited are left untouched)
 *   s_final  [nseq, head_hi - head_lo, d_k, d_v]
 * s0 is [nseq, H, d_k, d_v] (all heads) or NULL for zeros.  Either output may be NULL.
 * Returns 0 on success, -1 on a bad argument, -2 when scratch memory cannot be allocated.
 */
int gdn_oracle_run(const void *q, const void *k, const void *v, int dtype,
                   const double *alpha, const double *beta, const double *s0,
                   const int64_t *seq_row0, const int64_t *seq_len, int64_t row_step,
                   int nseq, int H, int dk, int dv, int head_lo, int head_hi,
                   double *y, double *s_final, int nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !seq_row0 || !seq_len) return -1;
    if (nseq < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (head_lo < 0 || head_hi > H || head_lo >= head_hi) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    const int nh = head_hi - head_lo;
    const int64_t units = (int64_t)nseq * nh;
    int failed = 0;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *kv = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qv = (double *)malloc(sizeof(double) * (size_t)dk);
        double *vv = (double *)malloc(sizeof(double) * (size_t)dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !kv || !qv || !vv || !e) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < units; ++u) {
                const int n = (int)(u / nh);
                const int h = head_lo + (int)(u % nh);
                const int hy = h - head_lo;

                /* initial state */
                if (s0) {
                    const double *src = s0 + ((int64_t)n * H + h) * dk * dv;
                    memcpy(S, src, sizeof(double) * (size_t)dk * dv);
                } else {
                    memset(S, 0, sizeof(double) * (size_t)dk * dv);
                }

                for (int64_t s = 0; s < seq_len[n]; ++s) {
                    const int64_t row = seq_row0[n] + s * row_step;
                    const double a = alpha[row * H + h];
                    const double b = beta[row * H + h];
                    const int64_t qk_base = (row * H + h) * (int64_t)dk;
                    const int64_t v_base = (row * H + h) * (int64_t)dv;
                    for (int i = 0; i < dk; ++i) {
                        kv[i] = load_elem(k, qk_base + i, dtype);
                        qv[i] = load_elem(q, qk_base + i, dtype);
                    }
                    for (int j = 0; j < dv; ++j) vv[j] = load_elem(v, v_base + j, dtype);

                    /* S~ = alpha_t S */
                    for (int64_t x = 0; x < (int64_t)dk * dv; ++x) S[x] *= a;

                    /* e = v_t - S~^T k_t */
                    for (int j = 0; j < dv; ++j) {
                        double r = 0.0;
                        for (int i = 0; i < dk; ++i) r += S[(int64_t)i * dv + j] * kv[i];
                        e[j] = vv[j] - r;
                    }

                    /* S = S~ + beta_t k_t e^T */
                    for (int i = 0; i < dk; ++i) {
                        const double bk = b * kv[i];
                        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += bk * e[j];
                    }

                    /* y_t = S^T q_t  (read from the updated state) */
                    if (y) {
                        double *yo = y + (row * nh + hy) * (int64_t)dv;
                        for (int j = 0; j < dv; ++j) {
                            double acc = 0.0;
                            for (int i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * qv[i];
                            yo[j] = acc;
                        }
                    }
                }

                if (s_final) {
                    double *dst = s_final + ((int64_t)n * nh + hy) * dk * dv;
                    memcpy(dst, S, sizeof(double) * (size_t)dk * dv);
                }
            }
        }
        free(S);
        free(kv);
        free(qv);
        free(vv);
        free(e);
    }
    return failed ? -2 : 0;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

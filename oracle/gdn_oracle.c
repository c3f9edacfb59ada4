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

/*
 * Reverse-mode derivative of gdn_oracle_run (TEST INFRASTRUCTURE ONLY).
 *
 * For the scalar  L = sum_t <dy_t, y_t> + <ds_final, S_T>  it returns dL/dq, dL/dk, dL/dv,
 * dL/dalpha, dL/dbeta and dL/dS0, taking the four lines of the recurrence backwards, one
 * token at a time from the last to the first, with the adjoint D of the state carried
 * between tokens (D starts as ds_final, or zero):
 *
 *     y_t  = S_t^T q_t           ->  D += q_t dy_t^T,         dq_t = S_t dy_t
 *     S_t  = S~ + beta_t k_t e^T ->  de = beta_t D^T k_t,     dbeta_t = k_t^T D e,
 *                                    dk_t = beta_t D e,       dS~ = D
 *     e    = v_t - S~^T k_t      ->  dv_t = de,  dS~ -= k_t de^T,  dk_t -= S~ de
 *     S~   = alpha_t S_{t-1}     ->  dalpha_t = <dS~, S_{t-1}>,  D = alpha_t dS~
 *
 * The states S_{t-1} that the backward pass needs are regenerated from the forward
 * recurrence: a first pass keeps the state at every BLOCK-th token, and each block is then
 * re-run from its kept state before it is walked backwards.  The re-run repeats the forward
 * arithmetic exactly, so the states are the same doubles as in gdn_oracle_run.
 *
 * Addressing follows gdn_oracle_run.  dy is [rows, H, d_v] (all heads); ds_final is
 * [nseq, H, d_k, d_v] or NULL (zero).  Outputs hold heads head_lo .. head_hi-1:
 * dq, dk [rows, nh, d_k]; dv [rows, nh, d_v]; dalpha, dbeta [rows, nh];
 * ds0 [nseq, nh, d_k, d_v].  Any output may be NULL.  Returns 0, -1 (bad argument) or
 * -2 (no memory).
 */
#define ORACLE_BWD_BLOCK 64

int gdn_oracle_backward(const void *q, const void *k, const void *v, int dtype,
                        const double *alpha, const double *beta, const double *s0,
                        const int64_t *seq_row0, const int64_t *seq_len, int64_t row_step,
                        int nseq, int H, int dk, int dv, int head_lo, int head_hi,
                        const double *dy, const double *ds_final,
                        double *dq, double *dk_out, double *dv_out, double *dalpha,
                        double *dbeta, double *ds0, int nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !seq_row0 || !seq_len || !dy) return -1;
    if (nseq < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (head_lo < 0 || head_hi > H || head_lo >= head_hi) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    const int nh = head_hi - head_lo;
    const int64_t units = (int64_t)nseq * nh;
    const size_t ss = (size_t)dk * dv;
    int failed = 0;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double *keep = NULL;                                              /* kept states */
        double *blk = (double *)malloc(sizeof(double) * ss * (ORACLE_BWD_BLOCK + 1));
        double *D = (double *)malloc(sizeof(double) * ss);
        double *St = (double *)malloc(sizeof(double) * ss);               /* S~ */
        double *kv = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qv = (double *)malloc(sizeof(double) * (size_t)dk);
        double *vv = (double *)malloc(sizeof(double) * (size_t)dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        double *de = (double *)malloc(sizeof(double) * (size_t)dv);
        double *dyv = (double *)malloc(sizeof(double) * (size_t)dv);
        int64_t keep_cap = 0;
        if (!blk || !D || !St || !kv || !qv || !vv || !e || !de || !dyv) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < units; ++u) {
                const int n = (int)(u / nh);
                const int h = head_lo + (int)(u % nh);
                const int hy = h - head_lo;
                const int64_t T = seq_len[n];
                const int64_t nblk = (T + ORACLE_BWD_BLOCK - 1) / ORACLE_BWD_BLOCK;

                if (nblk + 1 > keep_cap) {
                    free(keep);
                    keep_cap = nblk + 1;
                    keep = (double *)malloc(sizeof(double) * ss * (size_t)keep_cap);
                    if (!keep) {
                        keep_cap = 0;
#pragma omp atomic write
                        failed = 1;
                        continue;
                    }
                }

                /* token loaders (exact widening) */
#define LOAD_TOKEN(s_)                                                                     \
    do {                                                                                   \
        const int64_t row_ = seq_row0[n] + (s_) * row_step;                                \
        const int64_t qk_ = (row_ * H + h) * (int64_t)dk;                                  \
        const int64_t vb_ = (row_ * H + h) * (int64_t)dv;                                  \
        for (int i_ = 0; i_ < dk; ++i_) {                                                  \
            kv[i_] = load_elem(k, qk_ + i_, dtype);                                        \
            qv[i_] = load_elem(q, qk_ + i_, dtype);                                        \
        }                                                                                  \
        for (int j_ = 0; j_ < dv; ++j_) vv[j_] = load_elem(v, vb_ + j_, dtype);            \
    } while (0)

                /* one forward step S_out = step(S_in) for token s, as in gdn_oracle_run */
#define FORWARD_STEP(S_in, S_out, s_)                                                      \
    do {                                                                                   \
        const int64_t row_ = seq_row0[n] + (s_) * row_step;                                \
        const double a_ = alpha[row_ * H + h], b_ = beta[row_ * H + h];                    \
        LOAD_TOKEN(s_);                                                                    \
        for (size_t x_ = 0; x_ < ss; ++x_) (S_out)[x_] = a_ * (S_in)[x_];                  \
        for (int j_ = 0; j_ < dv; ++j_) {                                                  \
            double r_ = 0.0;                                                               \
            for (int i_ = 0; i_ < dk; ++i_) r_ += (S_out)[(int64_t)i_ * dv + j_] * kv[i_]; \
            e[j_] = vv[j_] - r_;                                                           \
        }                                                                                  \
        for (int i_ = 0; i_ < dk; ++i_) {                                                  \
            const double bk_ = b_ * kv[i_];                                                \
            for (int j_ = 0; j_ < dv; ++j_) (S_out)[(int64_t)i_ * dv + j_] += bk_ * e[j_]; \
        }                                                                                  \
    } while (0)

                /* forward pass: keep the state before every block */
                if (s0) memcpy(keep, s0 + ((int64_t)n * H + h) * ss, sizeof(double) * ss);
                else memset(keep, 0, sizeof(double) * ss);
                for (int64_t bi = 0; bi + 1 < nblk; ++bi) {
                    memcpy(blk, keep + bi * ss, sizeof(double) * ss);
                    for (int64_t s = bi * ORACLE_BWD_BLOCK; s < (bi + 1) * ORACLE_BWD_BLOCK; ++s) {
                        FORWARD_STEP(blk, St, s);
                        memcpy(blk, St, sizeof(double) * ss);
                    }
                    memcpy(keep + (bi + 1) * ss, blk, sizeof(double) * ss);
                }

                /* backward pass */
                if (ds_final) memcpy(D, ds_final + ((int64_t)n * H + h) * ss, sizeof(double) * ss);
                else memset(D, 0, sizeof(double) * ss);
                for (int64_t bi = nblk - 1; bi >= 0; --bi) {
                    const int64_t s_lo = bi * ORACLE_BWD_BLOCK;
                    const int64_t s_hi = s_lo + ORACLE_BWD_BLOCK < T ? s_lo + ORACLE_BWD_BLOCK : T;
                    /* blk[i] = state after token s_lo + i - 1 (blk[0] = the kept state) */
                    memcpy(blk, keep + bi * ss, sizeof(double) * ss);
                    for (int64_t s = s_lo; s < s_hi; ++s)
                        FORWARD_STEP(blk + (s - s_lo) * ss, blk + (s - s_lo + 1) * ss, s);
                    for (int64_t s = s_hi - 1; s >= s_lo; --s) {
                        const int64_t row = seq_row0[n] + s * row_step;
                        const double a = alpha[row * H + h], b = beta[row * H + h];
                        const double *Sp = blk + (s - s_lo) * ss;      /* S_{t-1} */
                        const double *Sn = blk + (s - s_lo + 1) * ss;  /* S_t */
                        LOAD_TOKEN(s);
                        for (int j = 0; j < dv; ++j) dyv[j] = dy[(row * H + h) * (int64_t)dv + j];

                        /* y_t = S_t^T q_t */
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dv; ++j) D[(int64_t)i * dv + j] += qv[i] * dyv[j];
                        if (dq) {
                            double *o = dq + (row * nh + hy) * (int64_t)dk;
                            for (int i = 0; i < dk; ++i) {
                                double acc = 0.0;
                                for (int j = 0; j < dv; ++j) acc += Sn[(int64_t)i * dv + j] * dyv[j];
                                o[i] = acc;
                            }
                        }
                        /* S~ = alpha_t S_{t-1};  e = v_t - S~^T k_t */
                        for (size_t x = 0; x < ss; ++x) St[x] = a * Sp[x];
                        for (int j = 0; j < dv; ++j) {
                            double r = 0.0;
                            for (int i = 0; i < dk; ++i) r += St[(int64_t)i * dv + j] * kv[i];
                            e[j] = vv[j] - r;
                        }
                        /* S_t = S~ + beta_t k_t e^T */
                        double db = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            double acc = 0.0;
                            for (int i = 0; i < dk; ++i) acc += D[(int64_t)i * dv + j] * kv[i];
                            de[j] = b * acc;
                            db += acc * e[j];
                        }
                        if (dbeta) dbeta[row * nh + hy] = db;
                        if (dv_out) {
                            double *o = dv_out + (row * nh + hy) * (int64_t)dv;
                            for (int j = 0; j < dv; ++j) o[j] = de[j];
                        }
                        if (dk_out) {
                            double *o = dk_out + (row * nh + hy) * (int64_t)dk;
                            for (int i = 0; i < dk; ++i) {
                                double acc = 0.0;
                                for (int j = 0; j < dv; ++j)
                                    acc += b * D[(int64_t)i * dv + j] * e[j] - St[(int64_t)i * dv + j] * de[j];
                                o[i] = acc;
                            }
                        }
                        /* dS~ = D - k_t de^T;  dalpha_t = <dS~, S_{t-1}>;  D = alpha_t dS~ */
                        double da = 0.0;
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dv; ++j) {
                                const int64_t x = (int64_t)i * dv + j;
                                const double g = D[x] - kv[i] * de[j];
                                da += g * Sp[x];
                                D[x] = a * g;
                            }
                        if (dalpha) dalpha[row * nh + hy] = da;
                    }
                }
                if (ds0) memcpy(ds0 + ((int64_t)n * nh + hy) * ss, D, sizeof(double) * ss);
#undef FORWARD_STEP
#undef LOAD_TOKEN
            }
        }
        free(keep);
        free(blk);
        free(D);
        free(St);
        free(kv);
        free(qv);
        free(vv);
        free(e);
        free(de);
        free(dyv);
    }
    return failed ? -2 : 0;
}

/*
 * Channel-wise gated variants of the rule (TEST INFRASTRUCTURE ONLY).
 *
 * The pages say of Kimi Delta Attention only that every feature channel gets its own gate,
 * and of Gated DeltaNet-2 only that erase and write get separate channel-wise gates.  The
 * reading taken (one form covering both, and the rule itself as a special case): per token,
 *
 *     S~  = Diag(a_t) S                          a_t in (0, 1]^{d_k}: decay per key channel
 *     r   = S~^T k_t                             what the key retrieves
 *     e   = (w_t .* v_t) - (b_t .* r)            b_t, w_t in [0, 1]^{d_v}: erase and write
 *     S   = S~ + k_t e^T                         gates per value channel
 *     y_t = S^T q_t
 *
 * a_t = alpha_t 1, b_t = w_t = beta_t 1 is the gated delta rule (gdn_oracle_run);
 * b_t = w_t = beta_t 1 with a free a_t is the channel-decay variant.  Addressing as in
 * gdn_oracle_run; a is [rows, H, d_k], b and w are [rows, H, d_v] (all heads).
 */
int gdn_oracle_channel_run(const void *q, const void *k, const void *v, int dtype,
                           const double *a, const double *b, const double *w,
                           const double *s0, const int64_t *seq_row0, const int64_t *seq_len,
                           int64_t row_step, int nseq, int H, int dk, int dv, int head_lo,
                           int head_hi, double *y, double *s_final, int nthreads)
{
    if (!q || !k || !v || !a || !b || !w || !seq_row0 || !seq_len) return -1;
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
                if (s0) memcpy(S, s0 + ((int64_t)n * H + h) * dk * dv, sizeof(double) * (size_t)dk * dv);
                else memset(S, 0, sizeof(double) * (size_t)dk * dv);
                for (int64_t s = 0; s < seq_len[n]; ++s) {
                    const int64_t row = seq_row0[n] + s * row_step;
                    const int64_t qk_base = (row * H + h) * (int64_t)dk;
                    const int64_t v_base = (row * H + h) * (int64_t)dv;
                    for (int i = 0; i < dk; ++i) {
                        kv[i] = load_elem(k, qk_base + i, dtype);
                        qv[i] = load_elem(q, qk_base + i, dtype);
                    }
                    for (int j = 0; j < dv; ++j) vv[j] = load_elem(v, v_base + j, dtype);
                    /* S~ = Diag(a_t) S */
                    for (int i = 0; i < dk; ++i) {
                        const double ai = a[qk_base + i];
                        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= ai;
                    }
                    /* e = w .* v - b .* (S~^T k) */
                    for (int j = 0; j < dv; ++j) {
                        double r = 0.0;
                        for (int i = 0; i < dk; ++i) r += S[(int64_t)i * dv + j] * kv[i];
                        e[j] = w[v_base + j] * vv[j] - b[v_base + j] * r;
                    }
                    /* S = S~ + k e^T */
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += kv[i] * e[j];
                    /* y_t = S^T q_t */
                    if (y) {
                        double *yo = y + (row * nh + hy) * (int64_t)dv;
                        for (int j = 0; j < dv; ++j) {
                            double acc = 0.0;
                            for (int i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * qv[i];
                            yo[j] = acc;
                        }
                    }
                }
                if (s_final)
                    memcpy(s_final + ((int64_t)n * nh + hy) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
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

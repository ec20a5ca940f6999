/*
 * rtopk_oracle.c -- CPU oracle for one beam-search decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. The product path
 * never calls it and shares no code, header or constant with it.
 *
 * What it computes is the plain definition the LightSeq inference article
 * (hierarchical-decoding passage) starts from: to pick the top-k tokens of a
 * decode step, take the softmax of every beam's row of the
 * [batch_size, beam_size, vocab_size] logit matrix and sort, once per batch
 * element. The article's hierarchical rewrite claims to return exactly this
 * result, so the oracle is that definition written out, slowly, in float64:
 *
 *   score(b, j, t) = alive[b][j] + (x[b][j][t] - lse[b][j]),
 *   lse[b][j]      = m + log(sum_t exp(x[b][j][t] - m)),  m = max_t x[b][j][t],
 *
 * i.e. the running score plus the token's log-softmax. For each batch element
 * every (j, t) pair of every alive beam enters one list; a finished beam
 * (mask != 0) enters only (j, eos_id) with its running score unchanged and
 * its row is never read. The list is sorted by score (descending), ties by
 * the flat index j*V + t (ascending), and the first k are returned, padded
 * with (-1, -1, -inf) when the list is shorter than k.
 *
 * The second routine group is pass 1 of the article's rough-select kernel,
 * used only to pin the GPU path's intermediate threshold: the logits are
 * split into k groups, the maximum of each group is taken, and the minimum of
 * those maxima (the "R-top-k") is a lower bound of the true k-th largest
 * logit. Elements are grouped by (position + offset) mod ngroups; with more
 * groups than k the k-th largest group maximum is returned, which is the
 * minimum when ngroups == k.
 *
 * Logits arrive in their storage type (float32, IEEE binary16 or bfloat16 bit
 * patterns) and are decoded to float64 exactly by the functions below, which
 * follow the IEEE 754 binary16 definition and bfloat16's definition as the
 * upper half of a binary32. Build: cc -O2 -shared -fPIC rtopk_oracle.c -lm -lpthread
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_F64 = 3 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double rtopk_oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);             /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE 754 binary32. */
double rtopk_oracle_decode_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_logit(const void *x, int dtype, int64_t i)
{
    if (dtype == ORACLE_F64)
        return ((const double *)x)[i];
    if (dtype == ORACLE_F32)
        return (double)((const float *)x)[i];
    if (dtype == ORACLE_F16)
        return rtopk_oracle_decode_f16(((const uint16_t *)x)[i]);
    return rtopk_oracle_decode_bf16(((const uint16_t *)x)[i]);
}

/* log-sum-exp of one row, max-shifted, summed in order t = 0..n-1. */
static double row_lse(const void *x, int dtype, int64_t base, int64_t n)
{
    double m = -INFINITY, s = 0.0;
    for (int64_t t = 0; t < n; t++) {
        double v = load_logit(x, dtype, base + t);
        if (v > m)
            m = v;
    }
    for (int64_t t = 0; t < n; t++)
        s += exp(load_logit(x, dtype, base + t) - m);
    return m + log(s);
}

void rtopk_oracle_lse(const void *logits, int dtype, int64_t nrows, int64_t V, double *lse_out)
{
    for (int64_t r = 0; r < nrows; r++)
        lse_out[r] = row_lse(logits, dtype, r * V, V);
}

typedef struct {
    double score;
    int64_t flat;
} entry_t;

/* Order: higher score first; equal scores by lower flat index. */
static int entry_cmp(const void *pa, const void *pb)
{
    const entry_t *a = (const entry_t *)pa, *b = (const entry_t *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->flat > b->flat) - (a->flat < b->flat);
}

typedef struct {
    const void *logits;
    int dtype;
    const float *alive;
    const uint8_t *finished;
    int B, beam, V, k, eos_id;
    int32_t *out_beam, *out_token;
    float *out_score;
    double *out_score64, *out_lse;
    int b_begin, b_end, status;
} job_t;

static void step_one_batch(job_t *J, int b, entry_t *ent)
{
    int64_t n = 0;
    for (int j = 0; j < J->beam; j++) {
        int64_t r = (int64_t)b * J->beam + j;
        double a = (double)J->alive[r];
        if (J->finished && J->finished[r]) {
            ent[n].score = a;
            ent[n].flat = (int64_t)j * J->V + J->eos_id;
            n++;
            if (J->out_lse)
                J->out_lse[r] = NAN;
            continue;
        }
        double lse = row_lse(J->logits, J->dtype, r * J->V, J->V);
        if (J->out_lse)
            J->out_lse[r] = lse;
        for (int t = 0; t < J->V; t++) {
            ent[n].score = a + (load_logit(J->logits, J->dtype, r * J->V + t) - lse);
            ent[n].flat = (int64_t)j * J->V + t;
            n++;
        }
    }
    qsort(ent, (size_t)n, sizeof(entry_t), entry_cmp);
    for (int p = 0; p < J->k; p++) {
        int64_t o = (int64_t)b * J->k + p;
        if (p < n) {
            J->out_beam[o] = (int32_t)(ent[p].flat / J->V);
            J->out_token[o] = (int32_t)(ent[p].flat % J->V);
            J->out_score[o] = (float)ent[p].score;
            if (J->out_score64)
                J->out_score64[o] = ent[p].score;
        } else {
            J->out_beam[o] = -1;
            J->out_token[o] = -1;
            J->out_score[o] = -INFINITY;
            if (J->out_score64)
                J->out_score64[o] = -INFINITY;
        }
    }
}

static void *step_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    entry_t *ent = (entry_t *)malloc(sizeof(entry_t) * (size_t)J->beam * (size_t)J->V);
    if (!ent) {
        J->status = -3;
        return NULL;
    }
    for (int b = J->b_begin; b < J->b_end; b++)
        step_one_batch(J, b, ent);
    free(ent);
    return NULL;
}

/*
 * Full decode-step selection. Host pointers; logits [B][beam][V] in dtype,
 * alive [B][beam], finished [B][beam] (NULL = none finished), outputs [B][k].
 * out_score64 / out_lse ([B][beam], NaN for finished beams) may be NULL.
 * Batch elements are independent and are spread over nthreads threads; the
 * arithmetic per element does not depend on nthreads.
 * Returns 0, -1 on bad arguments, -3 when memory runs out.
 */
int rtopk_oracle_step(const void *logits, int dtype, const float *alive, const uint8_t *finished,
                      int B, int beam, int V, int k, int eos_id,
                      int32_t *out_beam, int32_t *out_token, float *out_score,
                      double *out_score64, double *out_lse, int nthreads)
{
    if (!logits || !alive || !out_beam || !out_token || !out_score)
        return -1;
    if (B < 1 || beam < 1 || V < 1 || k < 1 || eos_id < 0 || eos_id >= V)
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > B)
        nthreads = B;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -3;
    }
    for (int i = 0; i < nthreads; i++) {
        job_t *J = &jobs[i];
        J->logits = logits;
        J->dtype = dtype;
        J->alive = alive;
        J->finished = finished;
        J->B = B;
        J->beam = beam;
        J->V = V;
        J->k = k;
        J->eos_id = eos_id;
        J->out_beam = out_beam;
        J->out_token = out_token;
        J->out_score = out_score;
        J->out_score64 = out_score64;
        J->out_lse = out_lse;
        J->b_begin = (int)((int64_t)B * i / nthreads);
        J->b_end = (int)((int64_t)B * (i + 1) / nthreads);
    }
    int status = 0;
    if (nthreads == 1) {
        step_worker(&jobs[0]);
    } else {
        for (int i = 0; i < nthreads; i++)
            if (pthread_create(&th[i], NULL, step_worker, &jobs[i]) != 0)
                status = -3, jobs[i].status = -99;
        for (int i = 0; i < nthreads; i++)
            if (jobs[i].status != -99)
                pthread_join(th[i], NULL);
    }
    for (int i = 0; i < nthreads; i++)
        if (jobs[i].status == -3)
            status = -3;
    free(jobs);
    free(th);
    return status;
}

/*
 * The oracle's score of one (b, j, t) pair, given lse[b][j] from
 * rtopk_oracle_lse/step: the running score plus the log-softmax for an alive
 * beam; for a finished beam the running score at t == eos_id and -inf for
 * every other token (those pairs are not candidates). j or t out of range
 * (the padding pair) gives -inf.
 */
double rtopk_oracle_score_of(const void *logits, int dtype, const float *alive,
                             const uint8_t *finished, const double *lse,
                             int B, int beam, int V, int eos_id, int b, int j, int t)
{
    if (b < 0 || b >= B || j < 0 || j >= beam || t < 0 || t >= V)
        return -INFINITY;
    int64_t r = (int64_t)b * beam + j;
    if (finished && finished[r])
        return t == eos_id ? (double)alive[r] : -INFINITY;
    return (double)alive[r] + (load_logit(logits, dtype, r * V + t) - lse[r]);
}

static int double_desc_cmp(const void *pa, const void *pb)
{
    double a = *(const double *)pa, b = *(const double *)pb;
    return (a < b) - (a > b);
}

/*
 * Pass 1 of the rough-select kernel on n consecutive logits starting at
 * element `base`: element i belongs to group (i + offset) mod ngroups; each
 * group's maximum is taken; the k-th largest of the ngroups maxima is
 * returned (the minimum when ngroups == k). Empty groups have maximum -inf.
 */
double rtopk_oracle_threshold(const void *logits, int dtype, int64_t base, int64_t n,
                              int ngroups, int k, int64_t offset)
{
    if (ngroups < 1 || k < 1 || k > ngroups)
        return NAN;
    double *gmax = (double *)malloc(sizeof(double) * (size_t)ngroups);
    if (!gmax)
        return NAN;
    for (int g = 0; g < ngroups; g++)
        gmax[g] = -INFINITY;
    for (int64_t i = 0; i < n; i++) {
        int g = (int)(((i + offset) % ngroups + ngroups) % ngroups);
        double v = load_logit(logits, dtype, base + i);
        if (v > gmax[g])
            gmax[g] = v;
    }
    /* k-th largest of the group maxima: sort them descending, take position k-1 */
    qsort(gmax, (size_t)ngroups, sizeof(double), double_desc_cmp);
    double result = gmax[k - 1];
    free(gmax);
    return result;
}

/* Number of the n logits from `base` that are >= T (the survivors of pass 2). */
int64_t rtopk_oracle_count_ge(const void *logits, int dtype, int64_t base, int64_t n, double T)
{
    int64_t c = 0;
    for (int64_t i = 0; i < n; i++)
        if (load_logit(logits, dtype, base + i) >= T)
            c++;
    return c;
}

/*
 * The LM head in front of the step: logits[m][v] = sum_h x[m][h] * w[v][h],
 * x the [M][H] hidden states and w the [V][H] output projection (one row of
 * H weights per vocabulary entry), both bfloat16 bit patterns. Every product
 * of two bfloat16 values is exact in float64 and the sum runs in float64 in
 * h order, so the result is the exact dot product up to float64 rounding of
 * the sum. The LightSeq inference article computes the logits with a GEMM
 * ahead of the decoding step and names fusing the operations around GEMMs as
 * its kernel-fusion principle; this is that GEMM written out, for composing
 * with rtopk_oracle_step (float64 logits, dtype 3).
 */
void rtopk_oracle_lmhead_logits(const uint16_t *x, const uint16_t *w, int64_t M, int64_t V, int64_t H,
                                double *logits)
{
    for (int64_t m = 0; m < M; m++)
        for (int64_t v = 0; v < V; v++) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; h++)
                acc += rtopk_oracle_decode_bf16(x[m * H + h]) * rtopk_oracle_decode_bf16(w[v * H + h]);
            logits[m * V + v] = acc;
        }
}

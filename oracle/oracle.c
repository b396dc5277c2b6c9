/*
 * CPU oracle for the frequency-ranked drafter LM head.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow definition that the
 * GPU library is checked against. Only the tests, the package's smoke check
 * and the benchmark's CPU-baseline leg may load it; the product path never
 * does. It shares no code, header, table or constant with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [VT]  "VocabTrim: Memory-Efficient Vocabulary Pruning for Speculative
 *         Decoding" skill page (English and Japanese renderings):
 *         Implementation, Steps 1-4.
 *   [FR]  "FR-Spec: Accelerating Large-Vocabulary Language Models via
 *         Frequency-Ranked Speculative Sampling" paper notes:
 *         Method / key design "frequency-ranked vocabulary compression".
 *
 * Precision: every floating-point step is done in double (fp64); bfloat16
 * inputs are widened exactly. Results do not depend on the OpenMP thread
 * count: each output element is produced by one thread in a fixed order.
 *
 * Readings of points the pages leave open (each is also listed with the
 * design notes of this repository):
 *   - ids outside [0, V) are not counted; they are tallied in n_invalid.
 *   - ranking is by count descending, ties by lower id; every id in [0, V)
 *     is eligible, including ids never seen (count 0).
 *   - the draft row's pick is a deterministic top-k (ties: lower full id),
 *     not the page's multinomial draw; probabilities are the softmax over
 *     the kept subset, not renormalised over the top k; temperature 1.
 *
 * Parity pins: every function here is pinned by the CPU tests against
 * library routines, closed forms, brute force or hand-worked examples.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_BAD -1

/* bfloat16 bit pattern -> exact real value. A bfloat16 is the upper half of
 * an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int or_version(void) { return 1; }

/* Threads the OpenMP loops use (1 when built without OpenMP). */
int or_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Step 1 of [VT] (count every sampled token id) and [FR]'s corpus frequency
 * statistics: counts[v] = number of i with ids[i] == v.
 * With accumulate != 0 the counts and n_invalid are added to, as when the
 * calibration stream arrives in batches. */
int or_count(const int32_t *ids, uint64_t n, int32_t V, uint32_t *counts,
             int accumulate, uint64_t *n_invalid)
{
    if (V <= 0 || !counts || !n_invalid || (n && !ids))
        return OR_BAD;
    if (!accumulate) {
        for (int32_t v = 0; v < V; ++v)
            counts[v] = 0;
        *n_invalid = 0;
    }
    for (uint64_t i = 0; i < n; ++i) {
        int32_t id = ids[i];
        if (id >= 0 && id < V)
            counts[id] += 1;
        else
            *n_invalid += 1;
    }
    return OR_OK;
}

typedef struct {
    uint32_t count;
    int32_t id;
} or_rank_t;

/* Order of Step 2 of [VT] (sort by frequency, most frequent first), with the
 * lower id first among equal counts. It is a total order on distinct ids. */
static int rank_cmp(const void *pa, const void *pb)
{
    const or_rank_t *a = (const or_rank_t *)pa, *b = (const or_rank_t *)pb;
    if (a->count != b->count)
        return a->count > b->count ? -1 : 1;
    return (a->id > b->id) - (a->id < b->id);
}

/* Step 2 of [VT] ("select vocabulary and create remapping") and [FR]'s
 * top-|V_high| frequency subset:
 *   t2f[i]       = id of the i-th entry of all V ids in rank order, i < V_high
 *   f2t[t2f[i]]  = i, and -1 for every id not kept (f2t may be NULL)
 *   sel          = sum of counts of the kept ids
 *   tot          = sum of all counts
 * Coverage is sel / tot, taken by the caller. */
int or_select(const uint32_t *counts, int32_t V, int32_t V_high, int32_t *t2f,
              int32_t *f2t, uint64_t *sel, uint64_t *tot)
{
    if (!counts || !t2f || !sel || !tot || V <= 0 || V_high <= 0 || V_high > V)
        return OR_BAD;
    or_rank_t *all = (or_rank_t *)malloc(sizeof(or_rank_t) * (size_t)V);
    if (!all)
        return OR_BAD;
    for (int32_t v = 0; v < V; ++v) {
        all[v].count = counts[v];
        all[v].id = v;
    }
    qsort(all, (size_t)V, sizeof(or_rank_t), rank_cmp);
    uint64_t s = 0, t = 0;
    for (int32_t i = 0; i < V_high; ++i) {
        t2f[i] = all[i].id;
        s += all[i].count;
    }
    for (int32_t v = 0; v < V; ++v)
        t += counts[v];
    if (f2t) {
        for (int32_t v = 0; v < V; ++v)
            f2t[v] = -1;
        for (int32_t i = 0; i < V_high; ++i)
            f2t[t2f[i]] = i;
    }
    *sel = s;
    *tot = t;
    free(all);
    return OR_OK;
}

/* Step 3 of [VT] (keep only the head rows of the kept ids) and [FR]'s
 * d x 128k -> d x 32k head: W_trim[i, :] = W[t2f[i], :], rows of d bf16. */
int or_gather(const uint16_t *W, int32_t V, int32_t d, const int32_t *t2f,
              int32_t V_high, uint16_t *W_trim)
{
    if (!W || !t2f || !W_trim || V <= 0 || d <= 0 || V_high <= 0)
        return OR_BAD;
    for (int32_t i = 0; i < V_high; ++i)
        if (t2f[i] < 0 || t2f[i] >= V)
            return OR_BAD;
    for (int32_t i = 0; i < V_high; ++i)
        memcpy(W_trim + (size_t)i * d, W + (size_t)t2f[i] * d,
               sizeof(uint16_t) * (size_t)d);
    return OR_OK;
}

/* The trimmed head's forward pass ([VT] Step 4: drafter logits over the
 * trimmed vocabulary; [FR]: the head projects onto the subset only):
 *   z[m, j] = sum_{t < d} h[m, t] * W[j, t]   for m < M, j < rows,
 * summed in ascending t in double. Every bf16 x bf16 product is exact in
 * double; the only rounding is in the running sum. */
int or_logits(const uint16_t *h, int32_t M, int32_t d, const uint16_t *W,
              int32_t rows, double *z)
{
    if (!h || !W || !z || M <= 0 || d <= 0 || rows <= 0)
        return OR_BAD;
    for (int32_t m = 0; m < M; ++m) {
        const uint16_t *hm = h + (size_t)m * d;
        double *zm = z + (size_t)m * rows;
#pragma omp parallel for schedule(static)
        for (int32_t j = 0; j < rows; ++j) {
            const uint16_t *wj = W + (size_t)j * d;
            double acc = 0.0;
            for (int32_t t = 0; t < d; ++t)
                acc += bf16_value(hm[t]) * bf16_value(wj[t]);
            zm[j] = acc;
        }
    }
    return OR_OK;
}

/* Softmax over the kept subset only ([FR]: the softmax is also computed on
 * the subset; [VT] Step 4 takes the softmax of the trimmed logits):
 *   mu[m] = max_j z[m, j],  S[m] = sum_j exp(z[m, j] - mu[m]) (ascending j),
 *   p[m, j] = exp(z[m, j] - mu[m]) / S[m].   p may be NULL. */
int or_softmax(const double *z, int32_t M, int32_t n, double *p, double *mu,
               double *S)
{
    if (!z || !mu || !S || M <= 0 || n <= 0)
        return OR_BAD;
    for (int32_t m = 0; m < M; ++m) {
        const double *zm = z + (size_t)m * n;
        double mx = zm[0];
        for (int32_t j = 1; j < n; ++j)
            if (zm[j] > mx)
                mx = zm[j];
        double s = 0.0;
        for (int32_t j = 0; j < n; ++j)
            s += exp(zm[j] - mx);
        mu[m] = mx;
        S[m] = s;
        if (p)
            for (int32_t j = 0; j < n; ++j)
                p[(size_t)m * n + j] = exp(zm[j] - mx) / s;
    }
    return OR_OK;
}

typedef struct {
    double z;
    int32_t full_id;
    int32_t j;
} or_cand_t;

/* Larger logit first; among equal logits the lower full id first. */
static int cand_cmp(const void *pa, const void *pb)
{
    const or_cand_t *a = (const or_cand_t *)pa, *b = (const or_cand_t *)pb;
    if (a->z != b->z)
        return a->z > b->z ? -1 : 1;
    return (a->full_id > b->full_id) - (a->full_id < b->full_id);
}

/* Per-row top-k and remap: the k largest trimmed logits of row m, in rank
 * order, each mapped to its full id through t2f ([VT] Step 4: map the
 * trimmed index back with trimmed_to_full, done here as a table lookup as
 * the page's pitfalls advise). Outputs: full_ids[m, r] and the trimmed index
 * trim_idx[m, r] (may be NULL). */
int or_topk(const double *z, const int32_t *t2f, int32_t M, int32_t V_high,
            int32_t k, int32_t *full_ids, int32_t *trim_idx)
{
    if (!z || !t2f || !full_ids || M <= 0 || V_high <= 0 || k <= 0 ||
        k > V_high)
        return OR_BAD;
    or_cand_t *c = (or_cand_t *)malloc(sizeof(or_cand_t) * (size_t)V_high);
    if (!c)
        return OR_BAD;
    for (int32_t m = 0; m < M; ++m) {
        for (int32_t j = 0; j < V_high; ++j) {
            c[j].z = z[(size_t)m * V_high + j];
            c[j].full_id = t2f[j];
            c[j].j = j;
        }
        qsort(c, (size_t)V_high, sizeof(or_cand_t), cand_cmp);
        for (int32_t r = 0; r < k; ++r) {
            full_ids[(size_t)m * k + r] = c[r].full_id;
            if (trim_idx)
                trim_idx[(size_t)m * k + r] = c[r].j;
        }
    }
    free(c);
    return OR_OK;
}

/* One draft-head call, composed from the steps above:
 * logits over the trimmed head, softmax over the subset, top-k, remap.
 *   full_ids[m, r] = t2f of the r-th largest logit of row m
 *   probs[m, r]    = its subset-softmax probability, rounded to float
 * z_out (may be NULL) receives the fp64 logits [M, V_high]; mu_out and
 * S_out (may be NULL) the per-row max and sum. */
int or_draft_head(const uint16_t *h, int32_t M, int32_t d,
                  const uint16_t *W_trim, int32_t V_high, const int32_t *t2f,
                  int32_t k, int32_t *full_ids, float *probs, double *z_out,
                  double *mu_out, double *S_out)
{
    if (!h || !W_trim || !t2f || !full_ids || !probs || M <= 0 || d <= 0 ||
        V_high <= 0 || k <= 0 || k > V_high)
        return OR_BAD;
    double *z = z_out ? z_out
                      : (double *)malloc(sizeof(double) * (size_t)M * V_high);
    double *mu = (double *)malloc(sizeof(double) * (size_t)M);
    double *S = (double *)malloc(sizeof(double) * (size_t)M);
    int32_t *ti = (int32_t *)malloc(sizeof(int32_t) * (size_t)M * k);
    int rc = OR_BAD;
    if (!z || !mu || !S || !ti)
        goto done;
    if ((rc = or_logits(h, M, d, W_trim, V_high, z)) != OR_OK)
        goto done;
    if ((rc = or_softmax(z, M, V_high, NULL, mu, S)) != OR_OK)
        goto done;
    if ((rc = or_topk(z, t2f, M, V_high, k, full_ids, ti)) != OR_OK)
        goto done;
    for (int32_t m = 0; m < M; ++m) {
        for (int32_t r = 0; r < k; ++r) {
            double zj = z[(size_t)m * V_high + ti[(size_t)m * k + r]];
            probs[(size_t)m * k + r] = (float)(exp(zj - mu[m]) / S[m]);
        }
        if (mu_out)
            mu_out[m] = mu[m];
        if (S_out)
            S_out[m] = S[m];
    }
done:
    if (!z_out)
        free(z);
    free(mu);
    free(S);
    free(ti);
    return rc;
}

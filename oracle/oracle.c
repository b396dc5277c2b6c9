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
 *   [VT] Step 4's draft loop samples one token from the subset softmax
 *         (a multinomial draw) and maps it back to its full id.
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
 *   - the draft row's pick is a deterministic top-k (ties: lower full id);
 *     probabilities are the softmax over the kept subset, not renormalised
 *     over the top k; temperature 1.
 *   - the page's multinomial draw (or_draft_sample) is a Gumbel-max draw
 *     whose uniforms come from the counter-based generator Philox4x32-10
 *     (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
 *     1, 2, 3", SC 2011); one generator call per (block of four rows,
 *     trimmed index) gives the four rows' uniforms, one output word each.
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

/* Sets the number of threads of later OpenMP loops (results do not depend
 * on it); returns the number now in effect. */
int or_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
    return or_threads();
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

/* The bias term of a head that carries one ([VT] Step 3 keeps the bias of
 * the kept ids; the trimmed head is a linear layer with that bias):
 *   z[m, j] += bias[j]   for m < M, j < rows (bias as bf16 payloads). */
static void add_bias(double *z, int32_t M, int32_t rows, const uint16_t *bias)
{
    for (int32_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < rows; ++j)
            z[(size_t)m * rows + j] += bf16_value(bias[j]);
}

/* One draft-head call, composed from the steps above:
 * logits over the trimmed head (plus its bias when bias is not NULL),
 * softmax over the subset, top-k, remap.
 *   full_ids[m, r] = t2f of the r-th largest logit of row m
 *   probs[m, r]    = its subset-softmax probability, rounded to float
 * z_out (may be NULL) receives the fp64 logits [M, V_high]; mu_out and
 * S_out (may be NULL) the per-row max and sum. */
int or_draft_head(const uint16_t *h, int32_t M, int32_t d,
                  const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                  const int32_t *t2f, int32_t k, int32_t *full_ids, float *probs,
                  double *z_out, double *mu_out, double *S_out)
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
    if (bias)
        add_bias(z, M, V_high, bias);
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

/* Philox4x32-10 (Salmon et al., SC 2011): a 4 x 32-bit counter and a
 * 2 x 32-bit key; each of the 10 rounds multiplies words 0 and 2 by two
 * fixed odd constants (full 64-bit products), swaps the halves and mixes in
 * the other words and the key; the key is advanced by two Weyl constants
 * between rounds. */
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                      uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The Gumbel variate of draft row m and trimmed index j for a draw keyed by
 * (seed, offset): Philox4x32-10 with counter (j, m div 4, offset low, offset
 * high) and key (seed low, seed high) yields four words, one for each of the
 * draft rows 4 (m div 4) .. 4 (m div 4) + 3; row m takes word m mod 4. The
 * top 24 bits x of that word give the uniform u = (x + 1/2) / 2^24 in (0, 1),
 * exactly representable; the variate is -log(-log u). */
double or_gumbel(uint64_t seed, uint64_t offset, int32_t m, int32_t j)
{
    const uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(m / 4), (uint32_t)offset,
                             (uint32_t)(offset >> 32)};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t o[4];
    or_philox4x32_10(ctr, key, o);
    const double u = ((double)(o[m % 4] >> 8) + 0.5) / 16777216.0;
    return -log(-log(u));
}

/* The variates G[m, j] of or_gumbel for all m < M, j < n, row-major. */
int or_gumbel_block(uint64_t seed, uint64_t offset, int32_t M, int32_t n, double *g)
{
    if (!g || M <= 0 || n <= 0)
        return OR_BAD;
    for (int32_t m = 0; m < M; ++m)
#pragma omp parallel for schedule(static)
        for (int32_t j = 0; j < n; ++j)
            g[(size_t)m * n + j] = or_gumbel(seed, offset, m, j);
    return OR_OK;
}

/* One sampled draft token per row, the page's multinomial draw from the
 * subset softmax ([VT] Step 4's draft loop), by the Gumbel-max rule: the
 * draw is argmax_j (z[m, j] + G[m, j]) (z with the bias when bias is not
 * NULL) with independent standard Gumbel
 * variates G, which picks j with probability exp(z_j) / sum_i exp(z_i).
 * Equal perturbed logits: the lower full id. Outputs:
 *   full_ids[m] = t2f[j*],  probs[m] = p[m, j*] (subset softmax, float)
 *   trim_idx[m] = j* (may be NULL); z_out [M, V_high] (may be NULL). */
int or_draft_sample(const uint16_t *h, int32_t M, int32_t d,
                    const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                    const int32_t *t2f, uint64_t seed, uint64_t offset,
                    int32_t *full_ids, float *probs, int32_t *trim_idx, double *z_out)
{
    if (!h || !W_trim || !t2f || !full_ids || !probs || M <= 0 || d <= 0 ||
        V_high <= 0)
        return OR_BAD;
    double *z = z_out ? z_out
                      : (double *)malloc(sizeof(double) * (size_t)M * V_high);
    double *mu = (double *)malloc(sizeof(double) * (size_t)M);
    double *S = (double *)malloc(sizeof(double) * (size_t)M);
    int rc = OR_BAD;
    if (!z || !mu || !S)
        goto done;
    if ((rc = or_logits(h, M, d, W_trim, V_high, z)) != OR_OK)
        goto done;
    if (bias)
        add_bias(z, M, V_high, bias);
    if ((rc = or_softmax(z, M, V_high, NULL, mu, S)) != OR_OK)
        goto done;
    for (int32_t m = 0; m < M; ++m) {
        const double *zm = z + (size_t)m * V_high;
        int32_t best = 0;
        double bv = zm[0] + or_gumbel(seed, offset, m, 0);
        for (int32_t j = 1; j < V_high; ++j) {
            const double v = zm[j] + or_gumbel(seed, offset, m, j);
            if (v > bv || (v == bv && t2f[j] < t2f[best])) {
                bv = v;
                best = j;
            }
        }
        full_ids[m] = t2f[best];
        probs[m] = (float)(exp(zm[best] - mu[m]) / S[m]);
        if (trim_idx)
            trim_idx[m] = best;
    }
done:
    if (!z_out)
        free(z);
    free(mu);
    free(S);
    return rc;
}

/* Coverage of every prefix of a ranking ([VT] Step 2's coverage, the
 * fraction of counted tokens the kept ids cover, for every V_high at once;
 * the guidance table's coverage threshold then picks V_high; with counts of
 * an evaluation stream it is Step 5's share of tokens inside the trimmed
 * vocabulary, one minus the miss rate):
 *   cum[i]  = sum_{r <= i} counts[order[r]]   for i < L (ids outside [0, V)
 *             count as 0)
 *   tot     = sum_{v < V} counts[v]
 *   v_high  = smallest n in [1, L] with (double)cum[n-1] >= min_coverage *
 *             (double)tot, or -1 if there is none (v_high may be NULL).
 * Coverage at n is cum[n-1] / tot. */
int or_coverage_curve(const uint32_t *counts, int32_t V, const int32_t *order,
                      int32_t L, double min_coverage, uint64_t *cum,
                      uint64_t *tot, int32_t *v_high)
{
    if (!counts || !order || !cum || !tot || V <= 0 || L <= 0 || L > V)
        return OR_BAD;
    uint64_t t = 0;
    for (int32_t v = 0; v < V; ++v)
        t += counts[v];
    *tot = t;
    const double x = min_coverage * (double)t;
    uint64_t c = 0;
    int32_t n = -1;
    for (int32_t i = 0; i < L; ++i) {
        const int32_t id = order[i];
        if (id >= 0 && id < V)
            c += counts[id];
        cum[i] = c;
        if (n < 0 && (double)c >= x)
            n = i + 1;
    }
    if (v_high)
        *v_high = n;
    return OR_OK;
}

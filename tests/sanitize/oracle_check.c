/* Runs every function of the CPU oracle on small inputs and on its edge
 * cases (empty streams, ids out of range, V_high = V, k = V_high, exact ties,
 * optional outputs left NULL, invalid arguments) in a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer. Values are checked only
 * for invariants that hold at any size; the oracle's values are pinned by the
 * Python tests. Exits 0 and prints "oracle_check ok" when every call behaved. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int or_version(void);
int or_threads(void);
int or_set_threads(int n);
int or_count(const int32_t *ids, uint64_t n, int32_t V, uint32_t *counts, int accumulate,
             uint64_t *n_invalid);
int or_select(const uint32_t *counts, int32_t V, int32_t V_high, int32_t *t2f, int32_t *f2t,
              uint64_t *sel, uint64_t *tot);
int or_gather(const uint16_t *W, int32_t V, int32_t d, const int32_t *t2f, int32_t V_high,
              uint16_t *W_trim);
int or_logits(const uint16_t *h, int32_t M, int32_t d, const uint16_t *W, int32_t rows,
              double *z);
int or_softmax(const double *z, int32_t M, int32_t n, double *p, double *mu, double *S);
int or_topk(const double *z, const int32_t *t2f, int32_t M, int32_t V_high, int32_t k,
            int32_t *full_ids, int32_t *trim_idx);
int or_draft_head(const uint16_t *h, int32_t M, int32_t d, const uint16_t *W_trim,
                  const uint16_t *bias, int32_t V_high, const int32_t *t2f, int32_t k,
                  int32_t *full_ids, float *probs, double *z_out, double *mu_out,
                  double *S_out);
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
double or_gumbel(uint64_t seed, uint64_t offset, int32_t m, int32_t j);
int or_gumbel_block(uint64_t seed, uint64_t offset, int32_t M, int32_t n, double *g);
int or_draft_sample(const uint16_t *h, int32_t M, int32_t d, const uint16_t *W_trim,
                    const uint16_t *bias, int32_t V_high, const int32_t *t2f, uint64_t seed,
                    uint64_t offset, int32_t *full_ids, float *probs, int32_t *trim_idx,
                    double *z_out);
int or_coverage_curve(const uint32_t *counts, int32_t V, const int32_t *order, int32_t L,
                      double min_coverage, uint64_t *cum, uint64_t *tot, int32_t *v_high);

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

/* xorshift64*: the driver's own inputs, nothing of the method */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* a bf16 payload of a value in about [-scale, scale] */
static uint16_t bf16_rand(float scale)
{
    float f = ((float)(rnd() & 0xFFFF) / 32768.0f - 1.0f) * scale;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void check_prep(int32_t V, int32_t V_high, uint64_t n)
{
    int32_t *ids = xmalloc(sizeof(int32_t) * (n + 2));
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t r = rnd();
        /* mostly small ids (a skewed stream), some out of range */
        ids[i] = (r % 17 == 0) ? (int32_t)(r % 3) - 2 - (int32_t)(r % 2) * V
                               : (int32_t)((r >> 8) % (uint32_t)(1 + (r & 7) * V / 8));
    }
    uint32_t *counts = xmalloc(sizeof(uint32_t) * V);
    uint64_t bad = 0, bad2 = 0;
    CHECK(or_count(ids, n, V, counts, 0, &bad) == 0);
    uint64_t s = 0;
    for (int32_t v = 0; v < V; ++v)
        s += counts[v];
    CHECK(s + bad == n);
    CHECK(or_count(ids, n, V, counts, 1, &bad2) == 0); /* accumulate: doubles */
    (void)bad2;
    CHECK(or_count(NULL, 0, V, counts, 0, &bad) == 0 && bad == 0);
    CHECK(or_count(NULL, 3, V, counts, 0, &bad) != 0);
    CHECK(or_count(ids, n, 0, counts, 0, &bad) != 0);

    for (uint64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= V)
            ids[i] = 0;
    CHECK(or_count(ids, n, V, counts, 0, &bad) == 0 && bad == 0);
    int32_t *t2f = xmalloc(sizeof(int32_t) * V_high), *f2t = xmalloc(sizeof(int32_t) * V);
    uint64_t sel = 0, tot = 0;
    CHECK(or_select(counts, V, V_high, t2f, f2t, &sel, &tot) == 0);
    CHECK(tot == n && sel <= tot);
    for (int32_t i = 0; i < V_high; ++i) {
        CHECK(t2f[i] >= 0 && t2f[i] < V);
        CHECK(f2t[t2f[i]] == i);
        if (i)
            CHECK(counts[t2f[i - 1]] > counts[t2f[i]] ||
                  (counts[t2f[i - 1]] == counts[t2f[i]] && t2f[i - 1] < t2f[i]));
    }
    CHECK(or_select(counts, V, V_high, t2f, NULL, &sel, &tot) == 0);
    CHECK(or_select(counts, V, V + 1, t2f, NULL, &sel, &tot) != 0);

    uint64_t *cum = xmalloc(sizeof(uint64_t) * V_high);
    int32_t vh = 0;
    CHECK(or_coverage_curve(counts, V, t2f, V_high, 0.5, cum, &tot, &vh) == 0);
    CHECK(cum[V_high - 1] == sel);
    CHECK(or_coverage_curve(counts, V, t2f, V_high, 2.0, cum, &tot, &vh) == 0);
    CHECK(vh == (tot ? -1 : 1)); /* nothing counted: every prefix reaches 0 */
    CHECK(or_coverage_curve(counts, V, t2f, V_high, 0.5, cum, &tot, NULL) == 0);
    CHECK(or_coverage_curve(counts, V, t2f, V + 1, 0.5, cum, &tot, &vh) != 0);
    free(cum);
    free(ids);
    free(counts);
    free(t2f);
    free(f2t);
}

static void check_head(int32_t M, int32_t d, int32_t V, int32_t V_high, int32_t k, int ties)
{
    uint16_t *h = xmalloc(sizeof(uint16_t) * (size_t)M * d);
    uint16_t *W = xmalloc(sizeof(uint16_t) * (size_t)V * d);
    uint16_t *Wt = xmalloc(sizeof(uint16_t) * (size_t)V_high * d);
    uint16_t *bias = xmalloc(sizeof(uint16_t) * (size_t)V_high);
    for (size_t i = 0; i < (size_t)M * d; ++i)
        h[i] = bf16_rand(2.0f);
    for (size_t i = 0; i < (size_t)V * d; ++i)
        W[i] = ties ? (uint16_t)(0x3F80 * (rnd() & 1)) : bf16_rand(0.1f);
    for (int32_t j = 0; j < V_high; ++j)
        bias[j] = bf16_rand(1.0f);
    int32_t *t2f = xmalloc(sizeof(int32_t) * V_high);
    for (int32_t i = 0; i < V_high; ++i)
        t2f[i] = (int32_t)(((int64_t)i * 7919) % V); /* distinct when gcd(7919, V) = 1 */
    CHECK(or_gather(W, V, d, t2f, V_high, Wt) == 0);
    t2f[0] = V; /* out of range: refused */
    CHECK(or_gather(W, V, d, t2f, V_high, Wt) != 0);
    t2f[0] = 0;

    double *z = xmalloc(sizeof(double) * (size_t)M * V_high);
    double *p = xmalloc(sizeof(double) * (size_t)M * V_high);
    double *mu = xmalloc(sizeof(double) * M), *S = xmalloc(sizeof(double) * M);
    CHECK(or_logits(h, M, d, Wt, V_high, z) == 0);
    CHECK(or_softmax(z, M, V_high, p, mu, S) == 0);
    for (int32_t m = 0; m < M; ++m) {
        double sum = 0.0;
        for (int32_t j = 0; j < V_high; ++j)
            sum += p[(size_t)m * V_high + j];
        CHECK(fabs(sum - 1.0) < 1e-12 && S[m] >= 1.0);
    }
    CHECK(or_softmax(z, M, V_high, NULL, mu, S) == 0);
    int32_t *ids = xmalloc(sizeof(int32_t) * (size_t)M * k);
    int32_t *tix = xmalloc(sizeof(int32_t) * (size_t)M * k);
    CHECK(or_topk(z, t2f, M, V_high, k, ids, tix) == 0);
    for (int32_t m = 0; m < M; ++m)
        for (int32_t r = 1; r < k; ++r)
            CHECK(z[(size_t)m * V_high + tix[m * k + r - 1]] >= z[(size_t)m * V_high + tix[m * k + r]]);
    CHECK(or_topk(z, t2f, M, V_high, k, ids, NULL) == 0);
    CHECK(or_topk(z, t2f, M, V_high, V_high + 1, ids, NULL) != 0);

    float *probs = xmalloc(sizeof(float) * (size_t)M * k);
    CHECK(or_draft_head(h, M, d, Wt, NULL, V_high, t2f, k, ids, probs, NULL, NULL, NULL) == 0);
    CHECK(or_draft_head(h, M, d, Wt, bias, V_high, t2f, k, ids, probs, z, mu, S) == 0);
    for (size_t i = 0; i < (size_t)M * k; ++i)
        CHECK(probs[i] >= 0.0f && probs[i] <= 1.0f);
    CHECK(or_draft_head(h, M, d, Wt, NULL, V_high, t2f, 0, ids, probs, NULL, NULL, NULL) != 0);

    float *pr1 = xmalloc(sizeof(float) * M);
    CHECK(or_draft_sample(h, M, d, Wt, NULL, V_high, t2f, 7, 11, ids, pr1, NULL, NULL) == 0);
    CHECK(or_draft_sample(h, M, d, Wt, bias, V_high, t2f, 7, 11, ids, pr1, tix, z) == 0);
    for (int32_t m = 0; m < M; ++m)
        CHECK(tix[m] >= 0 && tix[m] < V_high && ids[m] == t2f[tix[m]]);
    double *g = xmalloc(sizeof(double) * (size_t)M * V_high);
    CHECK(or_gumbel_block(7, 11, M, V_high, g) == 0);
    CHECK(g[0] == or_gumbel(7, 11, 0, 0));
    CHECK(or_gumbel_block(7, 11, 0, V_high, g) != 0);

    free(h); free(W); free(Wt); free(bias); free(t2f); free(z); free(p); free(mu); free(S);
    free(ids); free(tix); free(probs); free(pr1); free(g);
}

int main(void)
{
    CHECK(or_version() >= 1);
    CHECK(or_set_threads(2) >= 1);
    const uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0};
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    check_prep(1, 1, 0);
    check_prep(5, 5, 40);
    check_prep(257, 64, 5000);
    check_prep(3000, 1000, 20000);
    check_head(1, 8, 1, 1, 1, 0);
    check_head(3, 64, 101, 101, 101, 0);  /* k = V_high = V */
    check_head(5, 136, 331, 70, 10, 1);   /* exact ties */
    check_head(9, 256, 1009, 300, 64, 0);
    or_set_threads(0);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle_check ok\n");
    return 0;
}

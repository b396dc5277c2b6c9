/*
 * vocabtrim.h - C ABI of the frequency-ranked drafter LM head for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (two pages describe it):
 *   [VT] "VocabTrim: Memory-Efficient Vocabulary Pruning for Speculative
 *        Decoding" (skill page; Implementation, Steps 1-4; Practical
 *        Guidance; pitfalls).
 *   [FR] "FR-Spec: Accelerating Large-Vocabulary Language Models via
 *        Frequency-Ranked Speculative Sampling" (paper notes; Method,
 *        overall framework and key design).
 * A drafter's LM head W[V, d] is cut down to the V_high most frequent token
 * ids. Preparation counts ids, ranks them and gathers the kept rows into
 * W_trim[V_high, d]; every draft step then computes the logits of the kept
 * rows only, a softmax over the kept subset, the k best tokens per draft row,
 * and maps them back to full-vocabulary ids.
 *
 * Conventions shared by every call:
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device (e.g. torch tensors); they are owned by the caller,
 *     contiguous and row-major. bfloat16 values are passed as uint16_t bit
 *     patterns. Device pointers to 16-byte vectors must be 16-byte aligned
 *     where stated.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream) and never blocks the host. The library
 *     allocates no memory: scratch space is passed in as a workspace whose
 *     size the matching *_workspace_size call returns.
 *   - Arguments are validated on the host before any HIP call. A call that
 *     returns an error status has launched nothing and written nothing.
 *     VT_ERR_HIP means a launch failed; hipGetLastError() was cleared.
 *   - Calls are not synchronised with each other except by stream order.
 *     Two calls that share a workspace must run in stream order (not
 *     concurrently on different streams).
 */
#ifndef VOCABTRIM_H
#define VOCABTRIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VT_ABI_VERSION 1

/* Limits of the library. */
#define VT_K_MAX 64           /* top-k per draft row                        */
#define VT_M_MAX 512          /* draft rows per vt_draft_head call           */
#define VT_D_MAX 8192         /* hidden size; d must also be a multiple of 8 */
#define VT_VHIGH_MAX 262144   /* kept vocabulary per vt_draft_head call     */
#define VT_V_MAX (1 << 26)    /* full vocabulary of the count, select,
                                 coverage and gather calls               */

typedef enum {
    VT_OK = 0,
    VT_ERR_INVALID_ARG = -1,  /* null/misaligned pointer or size out of range */
    VT_ERR_UNSUPPORTED = -2,  /* valid request beyond the library's limits   */
    VT_ERR_WORKSPACE = -3,    /* workspace missing, misaligned or too small   */
    VT_ERR_HIP = -4,          /* a HIP launch or query failed                 */
    VT_ERR_TIMEOUT = -5,      /* a bounded wait inside a kernel gave up       */
    VT_ERR_SCRATCH_LIMIT = -6 /* vt_draft_head_noalloc: request exceeds the
                                 library's fixed scratch                      */
} vt_status;

/* Static text for a status code (never NULL). */
const char *vt_status_string(int status);

/* VT_ABI_VERSION of the loaded library. */
int vt_version(void);

/* ------------------------------------------------------------------ count
 * Token-id histogram: [VT] Step 1 counts every id the drafter samples on
 * calibration data; [FR] key design counts token frequencies over a corpus.
 *
 *   counts[v] (+)= number of i < n with ids[i] == v, for 0 <= v < V
 *   n_invalid (+)= number of i < n with ids[i] < 0 or ids[i] >= V
 *
 * ids       device, int32[n], 16-byte aligned (may be NULL when n == 0)
 * n         number of ids, n <= UINT32_MAX
 * V         full vocabulary, 1 <= V <= VT_V_MAX (larger: VT_ERR_UNSUPPORTED)
 * counts    device, uint32[V]; overwritten, or added to when accumulate != 0
 * n_invalid device, uint64[1]; overwritten, or added to when accumulate != 0
 * ws        device workspace of at least vt_count_freq_workspace_size(n, V)
 *           bytes, 256-byte aligned; no initial contents required.
 * Counts are exact. With accumulate the caller keeps each count below 2^32
 * (it wraps modulo 2^32 otherwise). Ids out of range are never counted and
 * cause no out-of-bounds access. */
size_t vt_count_freq_workspace_size(uint64_t n, int32_t V);
int vt_count_freq(const int32_t *ids, uint64_t n, int32_t V, uint32_t *counts,
                  int accumulate, uint64_t *n_invalid, void *ws,
                  size_t ws_bytes, void *stream);

/* ----------------------------------------------------------------- select
 * Top-V_high vocabulary and both maps: [VT] Step 2 sorts ids by count, keeps
 * the first target_vocab_size, builds trimmed_to_full / full_to_trimmed and
 * the coverage; [FR] key design keeps the |V_high| most frequent tokens.
 *
 * All V ids are ranked by (count descending, id ascending); ids never seen
 * (count 0) rank last by id. Then
 *   t2f[i]       = id at rank i, for i < V_high (trimmed_to_full)
 *   f2t[t2f[i]]  = i, and -1 for every id that is not kept (full_to_trimmed)
 *   sel_sum      = sum of counts[t2f[i]],  tot_sum = sum of counts[v]
 * Coverage is sel_sum / tot_sum (the caller divides; tot_sum == 0 means no
 * id was counted).
 *
 * counts  device, uint32[V], 16-byte aligned
 * V, V_high  1 <= V_high <= V <= VT_V_MAX (larger V: VT_ERR_UNSUPPORTED)
 * t2f     device, int32[V_high]
 * f2t     device, int32[V], or NULL to skip it
 * sel_sum, tot_sum  device, uint64[1] each
 * ws      device workspace of vt_select_vocab_workspace_size(V, V_high)
 *         bytes, 256-byte aligned; no initial contents required.
 * The result is unique (the order is total), so it is bit-exact. */
size_t vt_select_vocab_workspace_size(int32_t V, int32_t V_high);
int vt_select_vocab(const uint32_t *counts, int32_t V, int32_t V_high,
                    int32_t *t2f, int32_t *f2t, uint64_t *sel_sum,
                    uint64_t *tot_sum, void *ws, size_t ws_bytes,
                    void *stream);

/* --------------------------------------------------------- coverage curve
 * Coverage of every prefix of a ranking: [VT] Step 2's coverage (the share
 * of counted tokens the kept ids cover) for every V_high at once, and the
 * smallest V_high that reaches a coverage threshold (the guidance table
 * recommends 85-95 %). Given an evaluation stream's counts and the
 * calibration ranking, 1 - coverage is [VT] Step 5's share of tokens that
 * fall outside the trimmed vocabulary.
 *
 *   cum[i]  = sum_{r <= i} counts[order[r]]   (i < L; ids outside [0, V) add 0)
 *   tot_sum = sum_{v < V} counts[v]
 *   v_high  = smallest n in [1, L] with (double)cum[n - 1] >= min_coverage *
 *             (double)tot_sum, or -1 if none (e.g. min_coverage > 1)
 * Coverage at n is cum[n - 1] / tot_sum (tot_sum == 0: no token counted).
 *
 * counts  device, uint32[V], V <= VT_V_MAX (larger: VT_ERR_UNSUPPORTED)
 * order   device, int32[L], 1 <= L <= V, e.g. the t2f of vt_select_vocab
 *         with V_high = L
 * cum     device, uint64[L];  tot_sum  device, uint64[1]
 * v_high  device, int32[1], or NULL to skip it
 * ws      device workspace of vt_coverage_curve_workspace_size(V, L) bytes,
 *         256-byte aligned; no initial contents required.
 * The sums are exact integers; the threshold test is taken in double. */
size_t vt_coverage_curve_workspace_size(int32_t V, int32_t L);
int vt_coverage_curve(const uint32_t *counts, int32_t V, const int32_t *order,
                      int32_t L, double min_coverage, uint64_t *cum,
                      uint64_t *tot_sum, int32_t *v_high, void *ws,
                      size_t ws_bytes, void *stream);

/* ----------------------------------------------------------------- gather
 * Trimmed head: [VT] Step 3 keeps the head rows of the kept ids; [FR] key
 * design shrinks the head from d x 128k to d x 32k.
 *
 *   W_trim[i, :] = W[t2f[i], :]   for i < V_high  (bit copy)
 *
 * W       device, bf16[V, d], 16-byte aligned;  d % 8 == 0, 8 <= d <= VT_D_MAX
 * V, V_high  at most VT_V_MAX each (larger: VT_ERR_UNSUPPORTED)
 * t2f     device, int32[V_high] (from vt_select_vocab or the caller)
 * W_trim  device, bf16[V_high, d], 16-byte aligned; must not overlap W
 * n_bad   device uint32[1] or NULL. A t2f entry outside [0, V) is not read
 *         through: its output row is filled with zeros and, when n_bad is
 *         given, counted into *n_bad (which the call first sets to 0). */
int vt_gather_head(const uint16_t *W, int32_t V, int32_t d,
                   const int32_t *t2f, int32_t V_high, uint16_t *W_trim,
                   uint32_t *n_bad, void *stream);

/* Bias of a trimmed head that has one: [VT] Step 3 copies the bias entries
 * of the kept ids next to their rows when the original head carries a bias.
 *
 *   b_trim[i] = b[t2f[i]]   for i < V_high  (bit copy)
 *
 * b       device, bf16[V];  t2f as for vt_gather_head
 * b_trim  device, bf16[V_high]; must not overlap b
 * n_bad   as for vt_gather_head: entries outside [0, V) give 0 and are
 *         counted when n_bad is not NULL. */
int vt_gather_bias(const uint16_t *b, int32_t V, const int32_t *t2f, int32_t V_high,
                   uint16_t *b_trim, uint32_t *n_bad, void *stream);

/* ------------------------------------------------------------- draft head
 * One draft step of the trimmed head: [VT] Step 4 (logits of the trimmed
 * head, softmax over the trimmed vocabulary, pick, remap trimmed -> full id
 * with a table lookup as the page's pitfalls advise) and [FR] key design
 * (the head and its softmax cover the subset only).
 *
 * For every draft row m < M:
 *   z[m, j]   = sum_t h[m, t] * W_trim[j, t]   (bf16 inputs, fp32 sums)
 *   mu, S     = max_j z[m, j],  sum_j exp(z[m, j] - mu)   over j < V_high
 *   the k largest z[m, j] in rank order (equal logits: lower full id first)
 *   full_ids[m, r] = t2f[j_r],   probs[m, r] = exp(z[m, j_r] - mu) / S
 * The pick is a deterministic top-k; probs are subset-softmax values (not
 * renormalised over the k picks); temperature is 1. Partial results of
 * tiles of 64 kept rows are merged in a fixed order, so repeated calls give
 * identical bits.
 *
 * What runs, by number of draft rows (W_trim is read from memory once in
 * every case):
 *   M = 1, and M = 2 when V_high <= 32640
 *               one kernel: a GEMV over W_trim whose workgroups rank each
 *               tile's logits on chip and publish per tile only the softmax
 *               partial and the tile's top-k keys; the last workgroups to
 *               finish merge them. No logit is written to memory.
 *   otherwise   a GEMM-tiled MFMA kernel (one workgroup per 128 kept rows,
 *               or per 64 up to 64 draft rows when V_high <= 32640 and up
 *               to 128 when V_high <= 16384, over every draft row, both
 *               operands copied into an LDS ring), then one merge workgroup
 *               per draft row. The fp32 logits of every tile of 64 kept rows
 *               go to the workspace and the merge reads back those of the
 *               few tiles that can hold a pick. With 3 <= M <= 32 and
 *               V_high <= 16320 an MFMA skinny GEMM with one workgroup per
 *               tile takes the GEMM-tiled kernel's place.
 *
 * h         device, bf16[M, d], 16-byte aligned; 1 <= M <= VT_M_MAX
 * d         d % 8 == 0, 8 <= d <= VT_D_MAX
 * W_trim    device, bf16[V_high, d], 16-byte aligned; 1 <= V_high <= VT_VHIGH_MAX
 * t2f       device, int32[V_high]; only copied to the output and used to
 *           break ties, never used as an address. Its entries must be
 *           distinct (vt_select_vocab makes them so); with a repeated id
 *           and equal logits some output slots are left unwritten.
 * k         1 <= k <= min(V_high, VT_K_MAX)
 * full_ids  device, int32[M, k];  probs  device, float[M, k]
 * ws        device workspace of vt_draft_head_workspace_size(M, V_high, d, k)
 *           bytes, 256-byte aligned. It must be zero-filled once before its
 *           first use; every call leaves its counters at zero again. Its
 *           first 256 bytes hold the library's counters and status words
 *           (see vt_draft_head_status).
 * A merging workgroup waits, boundedly, for the other workgroups to arrive
 * (only on the GEMV path with two draft rows). If that wait gives up
 * (another process kept workgroups from running for tens of milliseconds),
 * the affected rows get full_ids = -1 and NaN probabilities, and the
 * workspace's error word is raised; vt_draft_head_status reports and clears
 * it. */
size_t vt_draft_head_workspace_size(int32_t M, int32_t V_high, int32_t d,
                                    int32_t k);
int vt_draft_head(const uint16_t *h, int32_t M, int32_t d,
                  const uint16_t *W_trim, int32_t V_high, const int32_t *t2f,
                  int32_t k, int32_t *full_ids, float *probs, void *ws,
                  size_t ws_bytes, void *stream);

/* vt_draft_head for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: its scratch is a fixed array of
 * VT_NOALLOC_WS_BYTES inside the library, one per GPU, held until the
 * process ends. The call allocates nothing (the first call on a device
 * takes the array's address and clears its counters with a kernel on
 * `stream`; do not make that first call under graph capture). Every call on
 * a GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, threads or processes without stream order) race and give wrong
 * results. Requests whose vt_draft_head_workspace_size exceeds
 * VT_NOALLOC_WS_BYTES return VT_ERR_SCRATCH_LIMIT and launch nothing.
 * Results are those of vt_draft_head. vt_draft_head_status(NULL, stream)
 * reports on this scratch. Other arguments as for vt_draft_head. */
#define VT_NOALLOC_WS_BYTES (16u << 20)
int vt_draft_head_noalloc(const uint16_t *h, int32_t M, int32_t d,
                          const uint16_t *W_trim, int32_t V_high, const int32_t *t2f,
                          int32_t k, int32_t *full_ids, float *probs, void *stream);

/* vt_draft_head for a trimmed head with a bias ([VT] Step 3 keeps the bias
 * of the kept ids; the trimmed head is a linear layer with that bias):
 *   z[m, j] = sum_t h[m, t] * W_trim[j, t] + bias[j]   (fp32)
 * and everything else as for vt_draft_head.
 * bias  device, bf16[V_high] (e.g. from vt_gather_bias); not NULL. */
int vt_draft_head_bias(const uint16_t *h, int32_t M, int32_t d,
                       const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                       const int32_t *t2f, int32_t k, int32_t *full_ids, float *probs,
                       void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------ draft sample
 * One draft token per row drawn from the subset softmax: the multinomial
 * draw of [VT] Step 4's draft loop (softmax over the trimmed logits, one
 * sample, then the trimmed index mapped back through trimmed_to_full).
 * The draw is taken by the Gumbel-max rule, which selects index j with
 * probability exp(z_j) / sum_i exp(z_i):
 *   j*[m]       = argmax_j ( z[m, j] + G[m, j] )   (equal values: lower full id)
 *   G[m, j]     = -log(-log u),  u = (x + 1/2) / 2^24, x = the top 24 bits of
 *                 word (m mod 4) of Philox4x32-10 (Salmon et al., SC 2011)
 *                 with counter (j, m div 4, offset low, offset high) and key
 *                 (seed low, seed high): one generator call serves four rows
 *   full_ids[m] = t2f[j*[m]],   probs[m] = exp(z[m, j*] - mu) / S  (as above)
 * z, mu and S are as for vt_draft_head (fp32 sums); G is computed in fp32.
 * The draw is a function of (seed, offset, m, logits) only: repeated calls
 * give identical results, and a caller advances `offset` once per draft
 * step to get independent draws.
 *
 * h, d, W_trim, V_high, t2f, ws, ws_bytes, stream: as for vt_draft_head,
 *           with ws of at least vt_draft_head_workspace_size(M, V_high, d, 1)
 *           bytes (zero-filled once; every call leaves its counters at zero).
 * full_ids  device, int32[M];  probs  device, float[M], or NULL to skip it */
int vt_draft_sample(const uint16_t *h, int32_t M, int32_t d,
                    const uint16_t *W_trim, int32_t V_high, const int32_t *t2f,
                    uint64_t seed, uint64_t offset, int32_t *full_ids,
                    float *probs, void *ws, size_t ws_bytes, void *stream);

/* vt_draft_sample for a trimmed head with a bias: z as for
 * vt_draft_head_bias, the draw as for vt_draft_sample.
 * bias  device, bf16[V_high]; not NULL. */
int vt_draft_sample_bias(const uint16_t *h, int32_t M, int32_t d,
                         const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                         const int32_t *t2f, uint64_t seed, uint64_t offset,
                         int32_t *full_ids, float *probs, void *ws, size_t ws_bytes,
                         void *stream);

/* Status of the kernels that last used a draft-head workspace. Waits on the
 * stream (host-blocking: not for use under graph capture), then returns
 * VT_ERR_TIMEOUT if a bounded wait inside a kernel gave up since the last
 * query (the affected outputs hold -1 / NaN) and clears the word, else
 * VT_OK. ws: a draft-head workspace, or NULL for the library's own scratch
 * on the current device (vt_draft_head_noalloc; VT_OK if never used).
 *
 * Workspace words (byte offsets; all zero in normal use):
 *   VT_WS_ERROR_OFFSET       uint32, set to 1 when a bounded wait gives up.
 *   VT_WS_HOLD_OFFSET        uint32, for tests of the timeout path: the
 *                            merging workgroups wait for this many extra
 *                            arrivals that never come, so their wait gives
 *                            up while every kernel still ends normally.
 *   VT_WS_SPIN_LIMIT_OFFSET  uint32, when nonzero it replaces the wait's
 *                            bound (in sleeps of about 128 clocks), so that
 *                            such a test ends quickly. */
#define VT_WS_ERROR_OFFSET 128
#define VT_WS_HOLD_OFFSET 132
#define VT_WS_SPIN_LIMIT_OFFSET 136
int vt_draft_head_status(const void *ws, void *stream);

/* ------------------------------------------------------- logits (checks)
 * The trimmed logits alone, z[m, j] as defined for vt_draft_head, written to
 * logits (device, float[M, V_high]), and the subset softmax statistics of
 * each row from those fp32 logits: row_max[m] = max_j z[m, j] and
 * row_sum[m] = sum_j exp(z[m, j] - row_max[m]) (device, float[M] each, or
 * NULL to skip). For parity diagnostics: it writes the M x V_high logits to
 * memory, which the draft head avoids.
 * Same argument rules as vt_draft_head. */
int vt_head_logits(const uint16_t *h, int32_t M, int32_t d,
                   const uint16_t *W_trim, int32_t V_high, float *logits,
                   float *row_max, float *row_sum, void *stream);

/* ------------------------------------------------------- remap cost (checks)
 * vt_draft_head without the remap: the picks are returned as trimmed
 * indices j (so equal logits rank by lower j) and t2f is not read. The
 * VocabTrim page's guidance table puts the cost of mapping trimmed ids back
 * to full ids below 1 %; comparing this call with vt_draft_head measures it.
 * Arguments as for vt_draft_head, with t2f absent and trimmed_ids in place of
 * full_ids (device, int32[M, k]). */
int vt_draft_head_trimmed(const uint16_t *h, int32_t M, int32_t d,
                          const uint16_t *W_trim, int32_t V_high, int32_t k,
                          int32_t *trimmed_ids, float *probs, void *ws,
                          size_t ws_bytes, void *stream);

/* ----------------------------------------------------- streaming ceiling
 * A plain read of `bytes` bytes of device memory with the draft head's load
 * width and cache policy (16-byte non-temporal loads, one pass), folding
 * the data into one word written to *sink (device uint64). It does no other
 * work, so its time is the practical ceiling of the draft head, which reads
 * W_trim once. p and bytes must be 16-byte aligned / a multiple of 16. */
int vt_stream_read(const void *p, size_t bytes, uint64_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VOCABTRIM_H */

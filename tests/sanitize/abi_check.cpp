// Host-side check of the C ABI's argument validation and workspace sizing,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the CPU (the
// library's sources compiled for the host only: no kernel is ever launched).
// Every call below is refused before any HIP call, so no GPU is needed. The
// sizing functions are swept over the whole range of their arguments, where
// an overflow in the size arithmetic would be undefined behaviour.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "vocabtrim.h"

static int failures = 0;

#define EXPECT_EQ(got, want)                                                        \
  do {                                                                              \
    const long long g_ = (long long)(got), w_ = (long long)(want);                  \
    if (g_ != w_) {                                                                 \
      fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #got, \
              g_, w_);                                                              \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

#define EXPECT(cond)                                                           \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond);       \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

// Stand-in addresses: validation only looks at nullness, alignment and
// overlap, never at the memory, so these are never dereferenced.
alignas(4096) static unsigned char arena[1 << 16];

template <typename T>
static T *at(size_t off) {
  return reinterpret_cast<T *>(arena + off);
}

static void check_status_strings() {
  const int codes[] = {VT_OK, VT_ERR_INVALID_ARG, VT_ERR_UNSUPPORTED, VT_ERR_WORKSPACE,
                       VT_ERR_HIP, VT_ERR_TIMEOUT, VT_ERR_SCRATCH_LIMIT, 12345, -999};
  for (int c : codes) {
    const char *s = vt_status_string(c);
    EXPECT(s != nullptr && s[0] != '\0');
  }
  EXPECT_EQ(vt_version(), VT_ABI_VERSION);
}

static void check_sizes() {
  // count: every n up to the limit, small and huge vocabularies.
  const uint64_t ns[] = {0, 1, 15, 16, 1u << 20, 100000000ull, UINT32_MAX, UINT32_MAX + 1ull,
                         UINT64_MAX};
  const int32_t Vs[] = {1, 2, 257, 65536, 128256, 152064, 1 << 24, INT32_MAX};
  for (uint64_t n : ns)
    for (int32_t V : Vs) {
      const size_t b = vt_count_freq_workspace_size(n, V);
      if (V > VT_V_MAX)
        EXPECT_EQ(b, 0);
      else
        EXPECT(b > 0 && b < ((size_t)1 << 48));
    }
  EXPECT_EQ(vt_count_freq_workspace_size(10, 0), 0);
  EXPECT_EQ(vt_count_freq_workspace_size(10, -5), 0);
  // select and coverage: every kept size against the vocabulary.
  for (int32_t V : Vs) {
    const int32_t highs[] = {1, V / 7 + 1, V / 2 + 1, V - 1 > 0 ? V - 1 : 1, V};
    for (int32_t vh : highs) {
      EXPECT((vt_select_vocab_workspace_size(V, vh) > 0) == (V <= VT_V_MAX));
      EXPECT((vt_coverage_curve_workspace_size(V, vh) > 0) == (V <= VT_V_MAX));
    }
    EXPECT_EQ(vt_select_vocab_workspace_size(V, 0), 0);
    EXPECT_EQ(vt_coverage_curve_workspace_size(V, -1), 0);
  }
  EXPECT_EQ(vt_select_vocab_workspace_size(10, 11), 0);
  EXPECT_EQ(vt_coverage_curve_workspace_size(10, 11), 0);
  // draft head: every M, a spread of vocabularies and k.
  const int32_t vhs[] = {1, 63, 64, 65, 1000, 8192, 32768, 128256, VT_VHIGH_MAX};
  const int32_t ks[] = {1, 10, VT_K_MAX};
  for (int32_t M = 1; M <= VT_M_MAX; ++M)
    for (int32_t vh : vhs)
      for (int32_t k : ks) {
        const size_t b = vt_draft_head_workspace_size(M, vh, 4096, k);
        EXPECT(b >= (size_t)VT_WS_SPIN_LIMIT_OFFSET + 4);
        EXPECT(b % 256 == 0);
      }
  EXPECT_EQ(vt_draft_head_workspace_size(0, 100, 64, 1), 0);
  EXPECT_EQ(vt_draft_head_workspace_size(VT_M_MAX + 1, 100, 64, 1), 0);
  EXPECT_EQ(vt_draft_head_workspace_size(1, VT_VHIGH_MAX + 1, 64, 1), 0);
  EXPECT_EQ(vt_draft_head_workspace_size(1, 100, 64, VT_K_MAX + 1), 0);
  EXPECT_EQ(vt_draft_head_workspace_size(1, 100, 64, 0), 0);
}

static void check_refusals() {
  uint16_t *h = at<uint16_t>(0), *W = at<uint16_t>(4096);
  int32_t *t2f = at<int32_t>(8192), *ids = at<int32_t>(12288);
  float *probs = at<float>(16384);
  uint32_t *counts = at<uint32_t>(20480);
  uint64_t *u64 = at<uint64_t>(24576);
  void *ws = at<void>(32768);
  const size_t big = (size_t)1 << 40;  // claimed workspace size; never touched
  const int E = VT_ERR_INVALID_ARG, U = VT_ERR_UNSUPPORTED, WS = VT_ERR_WORKSPACE;

  // count
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), 10, 0, counts, 0, u64, ws, big, nullptr), E);
  EXPECT_EQ(vt_count_freq(at<int32_t>(4), 10, 100, counts, 0, u64, ws, big, nullptr), E);
  EXPECT_EQ(vt_count_freq(nullptr, 10, 100, counts, 0, u64, ws, big, nullptr), E);
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), UINT32_MAX + 1ull, 100, counts, 0, u64, ws, big,
                          nullptr), E);
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), 10, 100, nullptr, 0, u64, ws, big, nullptr), E);
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), 10, 100, counts, 0, nullptr, ws, big, nullptr), E);
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), 10, 100, counts, 0, u64, nullptr, big, nullptr), WS);
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), 10, 100, counts, 0, u64, at<void>(32768 + 16), big,
                          nullptr), WS);
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), 1000000, 128256, counts, 0, u64, ws, 0, nullptr), WS);
  EXPECT_EQ(vt_count_freq(at<int32_t>(0), 10, VT_V_MAX + 1, counts, 0, u64, ws, big, nullptr), U);

  // select
  EXPECT_EQ(vt_select_vocab(nullptr, 100, 10, t2f, nullptr, u64, u64, ws, big, nullptr), E);
  EXPECT_EQ(vt_select_vocab(at<uint32_t>(4), 100, 10, t2f, nullptr, u64, u64, ws, big, nullptr),
            E);
  EXPECT_EQ(vt_select_vocab(counts, 100, 101, t2f, nullptr, u64, u64, ws, big, nullptr), E);
  EXPECT_EQ(vt_select_vocab(counts, 100, 0, t2f, nullptr, u64, u64, ws, big, nullptr), E);
  EXPECT_EQ(vt_select_vocab(counts, INT32_MAX, INT32_MAX, t2f, nullptr, u64, u64, ws, big,
                            nullptr), U);
  EXPECT_EQ(vt_select_vocab(counts, VT_V_MAX, VT_V_MAX, t2f, nullptr, u64, u64, ws, 64,
                            nullptr), WS);
  EXPECT_EQ(vt_select_vocab(counts, 128256, 32768, t2f, nullptr, u64, u64, nullptr, big,
                            nullptr), WS);

  // coverage curve
  EXPECT_EQ(vt_coverage_curve(counts, 100, t2f, 101, 0.9, u64, u64, nullptr, ws, big, nullptr),
            E);
  EXPECT_EQ(vt_coverage_curve(counts, 100, nullptr, 10, 0.9, u64, u64, nullptr, ws, big,
                              nullptr), E);
  EXPECT_EQ(vt_coverage_curve(counts, 128256, t2f, 128256, 0.9, u64, u64, nullptr, ws, 0,
                              nullptr), WS);
  EXPECT_EQ(vt_coverage_curve(counts, INT32_MAX, t2f, 10, 0.9, u64, u64, nullptr, ws, big,
                              nullptr), U);

  // gather: bad d, misalignment, overlap of source and destination
  EXPECT_EQ(vt_gather_head(W, 100, 12, t2f, 10, at<uint16_t>(40960), nullptr, nullptr), E);
  EXPECT_EQ(vt_gather_head(W, 100, VT_D_MAX + 8, t2f, 10, at<uint16_t>(40960), nullptr, nullptr),
            E);
  EXPECT_EQ(vt_gather_head(at<uint16_t>(4098), 100, 64, t2f, 10, at<uint16_t>(40960), nullptr,
                           nullptr), E);
  EXPECT_EQ(vt_gather_head(W, 100, 64, t2f, 10, W + 64, nullptr, nullptr), E);
  EXPECT_EQ(vt_gather_head(W, INT32_MAX, VT_D_MAX, t2f, INT32_MAX, at<uint16_t>(40960), nullptr,
                           nullptr), U);
  EXPECT_EQ(vt_gather_bias(W, 100, t2f, 10, W + 50, nullptr, nullptr), E);
  EXPECT_EQ(vt_gather_bias(W, 0, t2f, 10, at<uint16_t>(40960), nullptr, nullptr), E);
  EXPECT_EQ(vt_gather_bias(W, VT_V_MAX + 1, t2f, 10, at<uint16_t>(40960), nullptr, nullptr), U);

  // draft head and its variants
  const int32_t d = 64, vh = 1000, k = 10, M = 4;
  const size_t need = vt_draft_head_workspace_size(M, vh, d, k);
  EXPECT(need > 0);
  EXPECT_EQ(vt_draft_head(nullptr, M, d, W, vh, t2f, k, ids, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_head(h, 0, d, W, vh, t2f, k, ids, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_head(h, M, 60, W, vh, t2f, k, ids, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_head(h + 1, M, d, W, vh, t2f, k, ids, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_head(h, VT_M_MAX + 1, d, W, vh, t2f, k, ids, probs, ws, big, nullptr), U);
  EXPECT_EQ(vt_draft_head(h, M, d, W, VT_VHIGH_MAX + 1, t2f, k, ids, probs, ws, big, nullptr),
            U);
  EXPECT_EQ(vt_draft_head(h, M, d, W, vh, t2f, vh + 1, ids, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_head(h, M, d, W, vh, t2f, VT_K_MAX + 1, ids, probs, ws, big, nullptr), U);
  EXPECT_EQ(vt_draft_head(h, M, d, W, vh, nullptr, k, ids, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_head(h, M, d, W, vh, t2f, k, ids, probs, ws, need - 1, nullptr), WS);
  EXPECT_EQ(vt_draft_head(h, M, d, W, vh, t2f, k, ids, probs, at<void>(32768 + 128), big,
                          nullptr), WS);
  EXPECT_EQ(vt_draft_head_bias(h, M, d, W, nullptr, vh, t2f, k, ids, probs, ws, big, nullptr),
            E);
  EXPECT_EQ(vt_draft_head_bias(h, M, d, W, W, vh, t2f, k, ids, probs, ws, need - 1, nullptr),
            WS);
  EXPECT_EQ(vt_draft_sample(h, M, d, W, vh, nullptr, 1, 2, ids, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_sample(h, M, d, W, vh, t2f, 1, 2, ids, probs, nullptr, big, nullptr), WS);
  EXPECT_EQ(vt_draft_sample_bias(h, M, d, W, nullptr, vh, t2f, 1, 2, ids, probs, ws, big,
                                 nullptr), E);
  EXPECT_EQ(vt_draft_head_trimmed(h, M, d, W, vh, k, nullptr, probs, ws, big, nullptr), E);
  EXPECT_EQ(vt_draft_head_trimmed(h, M, d, W, vh, k, ids, probs, ws, need - 1, nullptr), WS);
  EXPECT_EQ(vt_head_logits(h, M, d, W, vh, nullptr, nullptr, nullptr, nullptr), E);
  EXPECT_EQ(vt_head_logits(h, M, d, W, VT_VHIGH_MAX + 1, probs, nullptr, nullptr, nullptr), U);
  // the allocation-free variant refuses what does not fit its fixed scratch
  // before touching any device
  EXPECT_EQ(vt_draft_head_noalloc(h, VT_M_MAX, VT_D_MAX, W, VT_VHIGH_MAX, t2f, VT_K_MAX, ids,
                                  probs, nullptr), VT_ERR_SCRATCH_LIMIT);
  EXPECT_EQ(vt_draft_head_noalloc(h, M, d, W, vh, t2f, 0, ids, probs, nullptr), E);
  EXPECT_EQ(vt_draft_head_noalloc(nullptr, M, d, W, vh, t2f, k, ids, probs, nullptr), E);
  // streaming read
  EXPECT_EQ(vt_stream_read(W, 1000, u64, nullptr), E);
  EXPECT_EQ(vt_stream_read(W, 0, u64, nullptr), E);
  EXPECT_EQ(vt_stream_read(at<void>(8), 1024, u64, nullptr), E);
  EXPECT_EQ(vt_stream_read(W, 1024, nullptr, nullptr), E);
}

int main() {
  check_status_strings();
  check_sizes();
  check_refusals();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi_check ok\n");
  return 0;
}

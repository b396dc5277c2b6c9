// Internal interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vocabtrim.h"
#include "vt_device.hpp"

namespace vt {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// gfx950 has 160 KB of LDS per CU; one counting workgroup uses up to
// kRangeBinsMax 32-bit bins of it.
constexpr int kRangeBinsMax = 38912;  // 152 KB
constexpr int kRange16Max = 76800;    // 16-bit bins: 150 KB
constexpr int kSpillCap = 1024;       // overflow records per 16-bit workgroup
constexpr int kMaxChunks = 256;       // counting workgroups (chunks x ranges), about one per CU

struct CountPlan {
  int32_t n_ranges, range_bins, n_chunks;
  uint64_t chunk_len;
  bool bins16;              // 16-bit LDS bins (vocabularies past kRangeBinsMax ids)
  int32_t row_pitch;        // partial-table row length in bins
  size_t partial_bytes, inv_bytes, spill_bytes;
};
CountPlan count_plan(uint64_t n, int32_t V);
hipError_t launch_count(const int32_t *ids, uint64_t n, int32_t V,
                        uint32_t *counts, int accumulate, uint64_t *n_invalid,
                        void *ws, hipStream_t stream);

size_t select_ws_bytes(int32_t V, int32_t V_high);
hipError_t launch_select(const uint32_t *counts, int32_t V, int32_t V_high,
                         int32_t *t2f, int32_t *f2t, uint64_t *sel,
                         uint64_t *tot, void *ws, hipStream_t stream);

hipError_t launch_gather(const uint16_t *W, int32_t V, int32_t d,
                         const int32_t *t2f, int32_t V_high, uint16_t *W_trim,
                         uint32_t *n_bad, hipStream_t stream);

// Draft head: tiles of kTileRows rows of W_trim; the last tile to finish
// merges every tile's partial result.
constexpr int kTileRows = 64;
// Fixed words at the start of a draft-head workspace (byte offsets). The
// status words are described with vt_draft_head_status in vocabtrim.h.
constexpr size_t kWsTicket = 0;     // uint32 ticket counter, zero between calls
constexpr size_t kWsMerged = 64;    // uint32 finished row mergers, zero between calls
constexpr size_t kWsError = VT_WS_ERROR_OFFSET;        // uint32 sticky error word
constexpr size_t kWsHold = VT_WS_HOLD_OFFSET;          // uint32, see vocabtrim.h
constexpr size_t kWsSpinLimit = VT_WS_SPIN_LIMIT_OFFSET;  // uint32, see vocabtrim.h
struct HeadPlan {
  int32_t tiles;
  size_t off_group, zero_bytes, off_tile_keys, off_tile_ms, off_tile_z, off_zbuf;
  size_t bytes;
};
HeadPlan head_plan(int32_t M, int32_t V_high, int32_t k);
// Bytes at the start of every draft-head workspace that must be zero before
// the first call (every call leaves them so).
size_t head_zero_bytes();
// Zero-fills n bytes (n a multiple of 16) on the stream with a kernel.
hipError_t launch_zero(void *p, size_t n, hipStream_t stream);
// bias: bf16[V_high] added to the logits, or nullptr for a head without one.
// remap: full ids through t2f (the method); false: trimmed indices j.
hipError_t launch_draft_head(const uint16_t *h, int32_t M, int32_t d,
                             const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                             const int32_t *t2f, int32_t k, int32_t *full_ids,
                             float *probs, void *ws, hipStream_t stream, bool remap = true);
hipError_t launch_draft_sample(const uint16_t *h, int32_t M, int32_t d,
                               const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                               const int32_t *t2f, uint64_t seed, uint64_t offset,
                               int32_t *full_ids, float *probs, void *ws, hipStream_t stream);
hipError_t launch_gather_bias(const uint16_t *b, int32_t V, const int32_t *t2f,
                              int32_t V_high, uint16_t *b_trim, uint32_t *n_bad,
                              hipStream_t stream);
// Coverage curve of a ranking.
size_t coverage_ws_bytes(int32_t V, int32_t L);
hipError_t launch_coverage(const uint32_t *counts, int32_t V, const int32_t *order, int32_t L,
                           double min_coverage, uint64_t *cum, uint64_t *tot_sum,
                           int32_t *v_high, void *ws, hipStream_t stream);

hipError_t launch_head_logits(const uint16_t *h, int32_t M, int32_t d,
                              const uint16_t *W_trim, int32_t V_high,
                              float *logits, float *row_max, float *row_sum,
                              hipStream_t stream);

// Streaming read of a buffer (the draft head's practical ceiling).
hipError_t launch_stream_read(const void *p, size_t bytes, uint64_t *sink, hipStream_t stream);

}  // namespace vt

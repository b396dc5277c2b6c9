// C ABI of the frequency-ranked drafter head (declared in vocabtrim.h):
// argument validation before any HIP call, workspace sizing, and dispatch
// to the kernels on the caller's stream.
#include "vocabtrim.h"

#include <stdint.h>

#include <mutex>

#include "vt_internal.hpp"

namespace {

bool aligned(const void *p, uintptr_t a) {
  return ((uintptr_t)p & (a - 1)) == 0;
}

bool valid_d(int32_t d) { return d >= 8 && d <= VT_D_MAX && d % 8 == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return VT_OK;
  (void)hipGetLastError();
  return VT_ERR_HIP;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Scratch of vt_draft_head_noalloc: a fixed array in device memory, one
// copy per GPU (each device that loads the library holds it until the
// process ends). Host code never passes the array's name to a kernel: its
// device address is taken once per device with hipGetSymbolAddress and kept
// in g_scratch.
static __device__ __align__(256) unsigned char scratch[VT_NOALLOC_WS_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, once set up

// The current device's scratch address. On the first call on a device it
// takes the address and clears the counters at its start (a fill kernel on
// `stream`, ahead of the caller's kernels). Returns a vt_status.
int device_scratch(bool set_up, hipStream_t stream, void **out) {
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hip_status(hipErrorInvalidDevice);
  if (dev < 0 || dev >= kMaxDevices) return VT_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev] && set_up) {
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e == hipSuccess ? hipErrorInvalidSymbol : e);
    e = vt::launch_zero(p, vt::head_zero_bytes(), stream);
    if (e != hipSuccess) return hip_status(e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return VT_OK;
}

}  // namespace

extern "C" {

const char *vt_status_string(int status) {
  switch (status) {
    case VT_OK: return "ok";
    case VT_ERR_INVALID_ARG: return "invalid argument";
    case VT_ERR_UNSUPPORTED: return "size beyond the library's limits";
    case VT_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case VT_ERR_HIP: return "HIP launch failed";
    case VT_ERR_TIMEOUT: return "a bounded wait inside a kernel gave up (outputs hold -1 / NaN)";
    case VT_ERR_SCRATCH_LIMIT:
      return "request needs more scratch than the library's fixed scratch (VT_NOALLOC_WS_BYTES)";
    default: return "unknown status";
  }
}

int vt_version(void) { return VT_ABI_VERSION; }

// ------------------------------------------------------------------ count
size_t vt_count_freq_workspace_size(uint64_t n, int32_t V) {
  if (V <= 0 || V > VT_V_MAX) return 0;
  const vt::CountPlan p = vt::count_plan(n, V);
  return p.partial_bytes + p.inv_bytes + p.spill_bytes;
}

int vt_count_freq(const int32_t *ids, uint64_t n, int32_t V, uint32_t *counts,
                  int accumulate, uint64_t *n_invalid, void *ws,
                  size_t ws_bytes, void *stream) {
  if (V <= 0 || n > UINT32_MAX || !counts || !n_invalid) return VT_ERR_INVALID_ARG;
  if (n > 0 && (!ids || !aligned(ids, 16))) return VT_ERR_INVALID_ARG;
  if (V > VT_V_MAX) return VT_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256) || ws_bytes < vt_count_freq_workspace_size(n, V))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_count(ids, n, V, counts, accumulate ? 1 : 0,
                                     n_invalid, ws, as_stream(stream)));
}

// ----------------------------------------------------------------- select
size_t vt_select_vocab_workspace_size(int32_t V, int32_t V_high) {
  if (V <= 0 || V_high <= 0 || V_high > V || V > VT_V_MAX) return 0;
  return vt::select_ws_bytes(V, V_high);
}

int vt_select_vocab(const uint32_t *counts, int32_t V, int32_t V_high,
                    int32_t *t2f, int32_t *f2t, uint64_t *sel_sum,
                    uint64_t *tot_sum, void *ws, size_t ws_bytes,
                    void *stream) {
  if (!counts || !t2f || !sel_sum || !tot_sum) return VT_ERR_INVALID_ARG;
  if (!aligned(counts, 16)) return VT_ERR_INVALID_ARG;
  if (V <= 0 || V_high <= 0 || V_high > V) return VT_ERR_INVALID_ARG;
  if (V > VT_V_MAX) return VT_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256) ||
      ws_bytes < vt_select_vocab_workspace_size(V, V_high))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_select(counts, V, V_high, t2f, f2t, sel_sum,
                                      tot_sum, ws, as_stream(stream)));
}

// --------------------------------------------------------- coverage curve
size_t vt_coverage_curve_workspace_size(int32_t V, int32_t L) {
  if (V <= 0 || L <= 0 || L > V || V > VT_V_MAX) return 0;
  return vt::coverage_ws_bytes(V, L);
}

int vt_coverage_curve(const uint32_t *counts, int32_t V, const int32_t *order,
                      int32_t L, double min_coverage, uint64_t *cum,
                      uint64_t *tot_sum, int32_t *v_high, void *ws,
                      size_t ws_bytes, void *stream) {
  if (!counts || !order || !cum || !tot_sum) return VT_ERR_INVALID_ARG;
  if (V <= 0 || L <= 0 || L > V) return VT_ERR_INVALID_ARG;
  if (V > VT_V_MAX) return VT_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256) || ws_bytes < vt_coverage_curve_workspace_size(V, L))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_coverage(counts, V, order, L, min_coverage, cum,
                                        tot_sum, v_high, ws, as_stream(stream)));
}

// ----------------------------------------------------------------- gather
int vt_gather_head(const uint16_t *W, int32_t V, int32_t d,
                   const int32_t *t2f, int32_t V_high, uint16_t *W_trim,
                   uint32_t *n_bad, void *stream) {
  if (!W || !t2f || !W_trim) return VT_ERR_INVALID_ARG;
  if (V <= 0 || V_high <= 0 || !valid_d(d)) return VT_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(W_trim, 16)) return VT_ERR_INVALID_ARG;
  if (V > VT_V_MAX || V_high > VT_V_MAX) return VT_ERR_UNSUPPORTED;
  if (overlaps(W, (size_t)V * d * 2, W_trim, (size_t)V_high * d * 2))
    return VT_ERR_INVALID_ARG;
  return hip_status(vt::launch_gather(W, V, d, t2f, V_high, W_trim, n_bad,
                                      as_stream(stream)));
}

int vt_gather_bias(const uint16_t *b, int32_t V, const int32_t *t2f, int32_t V_high,
                   uint16_t *b_trim, uint32_t *n_bad, void *stream) {
  if (!b || !t2f || !b_trim) return VT_ERR_INVALID_ARG;
  if (V <= 0 || V_high <= 0) return VT_ERR_INVALID_ARG;
  if (V > VT_V_MAX || V_high > VT_V_MAX) return VT_ERR_UNSUPPORTED;
  if (overlaps(b, (size_t)V * 2, b_trim, (size_t)V_high * 2)) return VT_ERR_INVALID_ARG;
  return hip_status(vt::launch_gather_bias(b, V, t2f, V_high, b_trim, n_bad,
                                           as_stream(stream)));
}

// ------------------------------------------------------------- draft head
static int check_head(const uint16_t *h, int32_t M, int32_t d,
                      const uint16_t *W_trim, int32_t V_high) {
  if (!h || !W_trim) return VT_ERR_INVALID_ARG;
  if (M <= 0 || V_high <= 0 || !valid_d(d)) return VT_ERR_INVALID_ARG;
  if (!aligned(h, 16) || !aligned(W_trim, 16)) return VT_ERR_INVALID_ARG;
  if (M > VT_M_MAX || V_high > VT_VHIGH_MAX) return VT_ERR_UNSUPPORTED;
  return VT_OK;
}

size_t vt_draft_head_workspace_size(int32_t M, int32_t V_high, int32_t d,
                                    int32_t k) {
  (void)d;
  if (M <= 0 || M > VT_M_MAX || V_high <= 0 || V_high > VT_VHIGH_MAX ||
      k <= 0 || k > VT_K_MAX)
    return 0;
  return vt::head_plan(M, V_high, k).bytes;
}

int vt_draft_head(const uint16_t *h, int32_t M, int32_t d,
                  const uint16_t *W_trim, int32_t V_high, const int32_t *t2f,
                  int32_t k, int32_t *full_ids, float *probs, void *ws,
                  size_t ws_bytes, void *stream) {
  int st = check_head(h, M, d, W_trim, V_high);
  if (st != VT_OK) return st;
  if (!t2f || !full_ids || !probs) return VT_ERR_INVALID_ARG;
  if (k <= 0 || k > V_high) return VT_ERR_INVALID_ARG;
  if (k > VT_K_MAX) return VT_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256) ||
      ws_bytes < vt_draft_head_workspace_size(M, V_high, d, k))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_draft_head(h, M, d, W_trim, nullptr, V_high, t2f, k,
                                          full_ids, probs, ws, as_stream(stream)));
}

int vt_draft_head_bias(const uint16_t *h, int32_t M, int32_t d,
                       const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                       const int32_t *t2f, int32_t k, int32_t *full_ids, float *probs,
                       void *ws, size_t ws_bytes, void *stream) {
  int st = check_head(h, M, d, W_trim, V_high);
  if (st != VT_OK) return st;
  if (!bias || !t2f || !full_ids || !probs) return VT_ERR_INVALID_ARG;
  if (k <= 0 || k > V_high) return VT_ERR_INVALID_ARG;
  if (k > VT_K_MAX) return VT_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256) ||
      ws_bytes < vt_draft_head_workspace_size(M, V_high, d, k))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_draft_head(h, M, d, W_trim, bias, V_high, t2f, k, full_ids,
                                          probs, ws, as_stream(stream)));
}

int vt_draft_sample(const uint16_t *h, int32_t M, int32_t d,
                    const uint16_t *W_trim, int32_t V_high, const int32_t *t2f,
                    uint64_t seed, uint64_t offset, int32_t *full_ids,
                    float *probs, void *ws, size_t ws_bytes, void *stream) {
  int st = check_head(h, M, d, W_trim, V_high);
  if (st != VT_OK) return st;
  if (!t2f || !full_ids) return VT_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256) ||
      ws_bytes < vt_draft_head_workspace_size(M, V_high, d, 1))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_draft_sample(h, M, d, W_trim, nullptr, V_high, t2f, seed,
                                            offset, full_ids, probs, ws, as_stream(stream)));
}

int vt_draft_sample_bias(const uint16_t *h, int32_t M, int32_t d,
                         const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                         const int32_t *t2f, uint64_t seed, uint64_t offset,
                         int32_t *full_ids, float *probs, void *ws, size_t ws_bytes,
                         void *stream) {
  int st = check_head(h, M, d, W_trim, V_high);
  if (st != VT_OK) return st;
  if (!bias || !t2f || !full_ids) return VT_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256) ||
      ws_bytes < vt_draft_head_workspace_size(M, V_high, d, 1))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_draft_sample(h, M, d, W_trim, bias, V_high, t2f, seed, offset,
                                            full_ids, probs, ws, as_stream(stream)));
}

int vt_draft_head_noalloc(const uint16_t *h, int32_t M, int32_t d,
                          const uint16_t *W_trim, int32_t V_high, const int32_t *t2f,
                          int32_t k, int32_t *full_ids, float *probs, void *stream) {
  int st = check_head(h, M, d, W_trim, V_high);
  if (st != VT_OK) return st;
  if (!t2f || !full_ids || !probs) return VT_ERR_INVALID_ARG;
  if (k <= 0 || k > V_high) return VT_ERR_INVALID_ARG;
  if (k > VT_K_MAX) return VT_ERR_UNSUPPORTED;
  if (vt_draft_head_workspace_size(M, V_high, d, k) > (size_t)VT_NOALLOC_WS_BYTES)
    return VT_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  st = device_scratch(true, as_stream(stream), &ws);
  if (st != VT_OK) return st;
  return hip_status(vt::launch_draft_head(h, M, d, W_trim, nullptr, V_high, t2f, k, full_ids,
                                          probs, ws, as_stream(stream)));
}

int vt_draft_head_trimmed(const uint16_t *h, int32_t M, int32_t d,
                          const uint16_t *W_trim, int32_t V_high, int32_t k,
                          int32_t *trimmed_ids, float *probs, void *ws,
                          size_t ws_bytes, void *stream) {
  int st = check_head(h, M, d, W_trim, V_high);
  if (st != VT_OK) return st;
  if (!trimmed_ids || !probs) return VT_ERR_INVALID_ARG;
  if (k <= 0 || k > V_high) return VT_ERR_INVALID_ARG;
  if (k > VT_K_MAX) return VT_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256) ||
      ws_bytes < vt_draft_head_workspace_size(M, V_high, d, k))
    return VT_ERR_WORKSPACE;
  return hip_status(vt::launch_draft_head(h, M, d, W_trim, nullptr, V_high, nullptr, k,
                                          trimmed_ids, probs, ws, as_stream(stream),
                                          /*remap=*/false));
}

int vt_draft_head_status(const void *ws, void *stream) {
  const hipStream_t s = as_stream(stream);
  if (!ws) {  // the library's own scratch on the current device
    void *p = nullptr;
    const int st = device_scratch(false, s, &p);
    if (st != VT_OK) return st;
    if (!p) return VT_OK;  // never used on this device
    ws = p;
  }
  char *word = static_cast<char *>(const_cast<void *>(ws)) + VT_WS_ERROR_OFFSET;
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return hip_status(hipErrorUnknown);
  if (v == 0) return VT_OK;
  const uint32_t zero = 0;
  if (hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return hip_status(hipErrorUnknown);
  return VT_ERR_TIMEOUT;
}

int vt_head_logits(const uint16_t *h, int32_t M, int32_t d,
                   const uint16_t *W_trim, int32_t V_high, float *logits,
                   float *row_max, float *row_sum, void *stream) {
  int st = check_head(h, M, d, W_trim, V_high);
  if (st != VT_OK) return st;
  if (!logits) return VT_ERR_INVALID_ARG;
  return hip_status(vt::launch_head_logits(h, M, d, W_trim, V_high, logits, row_max, row_sum,
                                           as_stream(stream)));
}

int vt_stream_read(const void *p, size_t bytes, uint64_t *sink, void *stream) {
  if (!p || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(p, 16)) return VT_ERR_INVALID_ARG;
  return hip_status(vt::launch_stream_read(p, bytes, sink, as_stream(stream)));
}

}  // extern "C"

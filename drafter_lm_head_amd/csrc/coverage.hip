// Coverage curve of a ranking (VocabTrim page, Step 2: the coverage of the
// kept ids, here for every prefix of the ranking at once; the guidance
// table's coverage threshold picks V_high; with an evaluation stream's counts
// it is Step 5's share of tokens inside the trimmed vocabulary).
//
//   cum[i] = sum_{r <= i} counts[order[r]] (exact uint64; ids outside [0, V)
//   count 0), tot = sum_v counts[v], v_high = smallest n with
//   (double)cum[n - 1] >= min_coverage * (double)tot, or -1.
//
// Three launches on the caller's stream: per-block sums (4096 entries per
// workgroup, coalesced 16-byte loads of order and counts), one workgroup that
// scans the block sums, then per block a local scan plus its offset, with
// the threshold crossing found where cum steps over it (cum never
// decreases, so exactly one entry crosses).
#include "vt_internal.hpp"
#include "vocabtrim.h"

namespace vt {

namespace {

constexpr int kCovThreads = 1024;
constexpr int kCovPer = 4;
constexpr int kCovBlock = kCovThreads * kCovPer;
constexpr int kCovWaves = kCovThreads / kWave;

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    const uint64_t y = __shfl_up(x, s);
    if (lane >= s) x += y;
  }
  return x;
}

// Exclusive prefix of x over the workgroup (in thread order) and the total.
__device__ uint64_t block_excl_scan_u64(uint64_t x, uint64_t *s_w, uint64_t &total) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const uint64_t incl = wave_incl_scan_u64(x);
  if (lane == kWave - 1) s_w[wave] = incl;
  __syncthreads();
  uint64_t before = 0;
  total = 0;
  for (int w = 0; w < kCovWaves; ++w) {
    const uint64_t t = s_w[w];
    before += w < wave ? t : 0ull;
    total += t;
  }
  __syncthreads();  // s_w may be reused by the caller
  return before + incl - x;
}

__device__ __forceinline__ uint32_t gathered(const uint32_t *counts, int32_t V, int32_t id) {
  return (id >= 0 && id < V) ? counts[id] : 0u;
}

__global__ __launch_bounds__(kCovThreads) void cov_block_sums_kernel(
    const uint32_t *__restrict__ counts, int32_t V, const int32_t *__restrict__ order, int32_t L,
    uint64_t *__restrict__ sumL, uint64_t *__restrict__ sumV) {
  __shared__ uint64_t s_w[kCovWaves];
  const int64_t i0 = (int64_t)blockIdx.x * kCovBlock + (int64_t)threadIdx.x * kCovPer;
  uint64_t l = 0, v = 0;
#pragma unroll
  for (int q = 0; q < kCovPer; ++q) {
    const int64_t i = i0 + q;
    if (i < L) l += gathered(counts, V, order[i]);
    if (i < V) v += counts[i];
  }
  uint64_t tl, tv;
  block_excl_scan_u64(l, s_w, tl);
  block_excl_scan_u64(v, s_w, tv);
  if (threadIdx.x == 0) {
    sumL[blockIdx.x] = tl;
    sumV[blockIdx.x] = tv;
  }
}

// One workgroup: offL = exclusive scan of sumL, the total of sumV, v_high = -1.
__global__ __launch_bounds__(kCovThreads) void cov_scan_kernel(
    const uint64_t *__restrict__ sumL, const uint64_t *__restrict__ sumV, int32_t nb,
    uint64_t *__restrict__ offL, uint64_t *__restrict__ tot_sum, int32_t *v_high) {
  __shared__ uint64_t s_w[kCovWaves];
  uint64_t carry = 0, tot = 0;
  for (int base = 0; base < nb; base += kCovThreads) {
    const int b = base + threadIdx.x;
    const uint64_t x = b < nb ? sumL[b] : 0ull;
    const uint64_t y = b < nb ? sumV[b] : 0ull;
    uint64_t tx, ty;
    const uint64_t ex = block_excl_scan_u64(x, s_w, tx);
    block_excl_scan_u64(y, s_w, ty);
    if (b < nb) offL[b] = carry + ex;
    carry += tx;
    tot += ty;
  }
  if (threadIdx.x == 0) {
    *tot_sum = tot;
    if (v_high) *v_high = -1;
  }
}

__global__ __launch_bounds__(kCovThreads) void cov_write_kernel(
    const uint32_t *__restrict__ counts, int32_t V, const int32_t *__restrict__ order, int32_t L,
    const uint64_t *__restrict__ offL, const uint64_t *__restrict__ tot_sum, double min_coverage,
    uint64_t *__restrict__ cum, int32_t *v_high) {
  __shared__ uint64_t s_w[kCovWaves];
  const int64_t i0 = (int64_t)blockIdx.x * kCovBlock + (int64_t)threadIdx.x * kCovPer;
  uint32_t c[kCovPer];
  uint64_t run = 0;
#pragma unroll
  for (int q = 0; q < kCovPer; ++q) {
    const int64_t i = i0 + q;
    c[q] = i < L ? gathered(counts, V, order[i]) : 0u;
    run += c[q];
  }
  uint64_t total;
  uint64_t prev = offL[blockIdx.x] + block_excl_scan_u64(run, s_w, total);  // cum[i0 - 1]
  const double x = min_coverage * (double)*tot_sum;
#pragma unroll
  for (int q = 0; q < kCovPer; ++q) {
    const int64_t i = i0 + q;
    if (i < L) {
      const uint64_t cur = prev + c[q];
      cum[i] = cur;
      if (v_high && (double)cur >= x && (i == 0 || (double)prev < x)) *v_high = (int32_t)(i + 1);
      prev = cur;
    }
  }
}

}  // namespace

size_t coverage_ws_bytes(int32_t V, int32_t L) {
  (void)L;
  const size_t nb = ((size_t)V + kCovBlock - 1) / kCovBlock;
  return align_up(3 * nb * sizeof(uint64_t), 256);
}

hipError_t launch_coverage(const uint32_t *counts, int32_t V, const int32_t *order, int32_t L,
                           double min_coverage, uint64_t *cum, uint64_t *tot_sum,
                           int32_t *v_high, void *ws, hipStream_t stream) {
  const int nb = (int)(((int64_t)V + kCovBlock - 1) / kCovBlock);
  const int nbL = (int)(((int64_t)L + kCovBlock - 1) / kCovBlock);
  uint64_t *sumL = static_cast<uint64_t *>(ws);
  uint64_t *sumV = sumL + nb;
  uint64_t *offL = sumV + nb;
  hipLaunchKernelGGL(cov_block_sums_kernel, dim3(nb), dim3(kCovThreads), 0, stream, counts, V,
                     order, L, sumL, sumV);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cov_scan_kernel, dim3(1), dim3(kCovThreads), 0, stream, sumL, sumV, nb,
                     offL, tot_sum, v_high);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cov_write_kernel, dim3(nbL), dim3(kCovThreads), 0, stream, counts, V, order,
                     L, offL, tot_sum, min_coverage, cum, v_high);
  return hipGetLastError();
}

}  // namespace vt

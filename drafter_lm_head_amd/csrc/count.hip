// Token-id histogram (VocabTrim page, Implementation, Step 1; FR-Spec notes,
// key design: token frequencies over a corpus), for gfx950.
//
// The bins of a large vocabulary (128k-152k ids) do not fit one CU's LDS, so
// the id range is cut into R ranges of at most kRangeBins bins and every
// (range, chunk-of-ids) pair is one workgroup that counts into LDS with LDS
// atomics. The R workgroups of one chunk read the same ids; they are placed
// on the same XCD and dispatched back to back, so the repeated reads are
// served by that XCD's L2 and the Infinity Cache rather than HBM. Each
// workgroup then stores its range of counts to its own row of a partial
// table (no global atomics), and a second kernel sums the rows, which keeps
// the result independent of scheduling.
#include <algorithm>
#include <atomic>

#include "vt_internal.hpp"

namespace vt {

namespace {

constexpr int kCountThreads = 1024;

__device__ __forceinline__ void count_one(int32_t id, uint32_t lo, uint32_t nb,
                                          uint32_t *s_bins) {
  const uint32_t b = (uint32_t)id - lo;  // wraps for ids below the range
  if (b < nb) atomicAdd(&s_bins[b], 1u);
}

__global__ __launch_bounds__(kCountThreads) void count_partial_kernel(
    const int32_t *__restrict__ ids, uint64_t n, int32_t V, int32_t range_bins,
    int32_t n_ranges, int32_t n_chunks, uint64_t chunk_len, int32_t pitch,
    uint32_t *__restrict__ partial, unsigned long long *__restrict__ inv_part) {
  extern __shared__ uint32_t s_bins[];
  __shared__ unsigned long long s_inv;

  // blockIdx -> (range, chunk): workgroups are dispatched to XCDs round
  // robin, so XCD = blockIdx % 8. The ranges of one chunk get consecutive
  // slots on one XCD.
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int r = slot % n_ranges;
  const int c = (slot / n_ranges) * 8 + xcd;
  if (c >= n_chunks) return;  // grid is rounded up to whole XCD rows

  const uint32_t lo = (uint32_t)r * (uint32_t)range_bins;
  const uint32_t nb = (uint32_t)min((int64_t)range_bins, (int64_t)V - lo);
  for (uint32_t i = threadIdx.x; i < nb; i += kCountThreads) s_bins[i] = 0;
  if (threadIdx.x == 0) s_inv = 0;
  __syncthreads();

  const uint64_t beg = (uint64_t)c * chunk_len;
  const uint64_t end = beg + chunk_len < n ? beg + chunk_len : n;
  unsigned long long inv = 0;
  const bool tally = (r == 0);
  if (beg < end) {
    // chunk_len is a multiple of 4 and ids is 16-byte aligned.
    const u32x4 *v4 = reinterpret_cast<const u32x4 *>(ids + beg);
    const uint64_t n4 = (end - beg) >> 2;
    constexpr int kUnroll = 4;
    uint64_t i = threadIdx.x;
    for (; i + (kUnroll - 1) * kCountThreads < n4; i += kUnroll * kCountThreads) {
      u32x4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = load_stream16(v4 + i + u * kCountThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t a[4] = {(int32_t)q[u].x, (int32_t)q[u].y, (int32_t)q[u].z,
                              (int32_t)q[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          count_one(a[e], lo, nb, s_bins);
          if (tally) inv += (uint32_t)a[e] >= (uint32_t)V;
        }
      }
    }
    for (; i < n4; i += kCountThreads) {
      const u32x4 q = load_stream16(v4 + i);
      const int32_t a[4] = {(int32_t)q.x, (int32_t)q.y, (int32_t)q.z, (int32_t)q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        count_one(a[e], lo, nb, s_bins);
        if (tally) inv += (uint32_t)a[e] >= (uint32_t)V;
      }
    }
    for (uint64_t j = beg + (n4 << 2) + threadIdx.x; j < end; j += kCountThreads) {
      const int32_t a = ids[j];
      count_one(a, lo, nb, s_bins);
      if (tally) inv += (uint32_t)a >= (uint32_t)V;
    }
  }
  if (tally && inv) atomicAdd(&s_inv, inv);
  __syncthreads();

  uint32_t *row = partial + (size_t)c * (size_t)pitch + lo;
  for (uint32_t i = threadIdx.x; i < nb; i += kCountThreads) row[i] = s_bins[i];
  if (tally && threadIdx.x == 0) inv_part[c] = s_inv;
}

// 16-bit bins, for vocabularies past kRangeBinsMax ids: two bins share an
// LDS word, so a range holds up to kRange16Max ids and each chunk of ids is
// read by half as many range workgroups. A 16-bit count is kept below 2^15
// plus the increments in flight: the increment that takes it from 0x7FFF to
// 0x8000 (exactly one thread sees 0x7FFF in the atomic's return value)
// subtracts 0x8000 again and records an overflow of 32768 for that id, so a
// count never wraps and never carries into its neighbour. The records are
// added to the totals after the reduction.
__device__ __forceinline__ void count_one16(int32_t id, uint32_t lo, uint32_t nb,
                                            uint32_t *s_words, uint32_t *s_spill,
                                            uint32_t *s_nspill) {
  const uint32_t b = (uint32_t)id - lo;  // wraps for ids below the range
  if (b < nb) {
    const uint32_t sh = (b & 1u) << 4;
    const uint32_t old = atomicAdd(&s_words[b >> 1], 1u << sh);
    if (((old >> sh) & 0xFFFFu) == 0x7FFFu) {
      atomicSub(&s_words[b >> 1], 0x8000u << sh);
      const uint32_t pos = atomicAdd(s_nspill, 1u);
      if (pos < (uint32_t)kSpillCap) s_spill[pos] = lo + b;
    }
  }
}

// The same for N ids at once: every atomic of the batch is issued before
// any returned value is looked at, so that a wave waits for the LDS once per
// batch rather than once per id.
template <int N>
__device__ __forceinline__ void count_batch16(const int32_t (&id)[N], uint32_t lo, uint32_t nb,
                                              uint32_t *s_words, uint32_t *s_spill,
                                              uint32_t *s_nspill) {
  uint32_t old[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint32_t b = (uint32_t)id[e] - lo;
    old[e] = b < nb ? atomicAdd(&s_words[b >> 1], 1u << ((b & 1u) << 4)) : 0u;
  }
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint32_t b = (uint32_t)id[e] - lo, sh = (b & 1u) << 4;
    if (b < nb && ((old[e] >> sh) & 0xFFFFu) == 0x7FFFu) {
      atomicSub(&s_words[b >> 1], 0x8000u << sh);
      const uint32_t pos = atomicAdd(s_nspill, 1u);
      if (pos < (uint32_t)kSpillCap) s_spill[pos] = lo + b;
    }
  }
}

// kShared: the chunk is read by several range workgroups. Its ids are then
// loaded with plain loads, which stay in L2 for the other readers (with
// non-temporal loads the second reader went to HBM: 159 against 139 us at
// 1e8 ids over 128256); a chunk read once streams past the caches.
template <bool kShared>
__device__ __forceinline__ u32x4 load_ids16(const u32x4 *p) {
  return kShared ? *p : load_stream16(p);
}

template <bool kShared>
__global__ __launch_bounds__(kCountThreads) void count_partial16_kernel(
    const int32_t *__restrict__ ids, uint64_t n, int32_t V, int32_t range_bins,
    int32_t n_ranges, int32_t n_chunks, uint64_t chunk_len, int32_t pitch,
    uint16_t *__restrict__ partial, unsigned long long *__restrict__ inv_part,
    uint32_t *__restrict__ spill) {
  extern __shared__ uint32_t s_words[];
  __shared__ uint32_t s_spill[kSpillCap];
  __shared__ uint32_t s_nspill;
  __shared__ unsigned long long s_inv;

  // blockIdx -> (range, chunk) as for the 32-bit kernel.
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int r = slot % n_ranges;
  const int c = (slot / n_ranges) * 8 + xcd;
  if (c >= n_chunks) return;

  const uint32_t lo = (uint32_t)r * (uint32_t)range_bins;
  const uint32_t nb = (uint32_t)min((int64_t)range_bins, (int64_t)V - lo);
  const uint32_t nw = (nb + 1) / 2;
  for (uint32_t i = threadIdx.x; i < nw; i += kCountThreads) s_words[i] = 0;
  if (threadIdx.x == 0) {
    s_inv = 0;
    s_nspill = 0;
  }
  __syncthreads();

  const uint64_t beg = (uint64_t)c * chunk_len;
  const uint64_t end = beg + chunk_len < n ? beg + chunk_len : n;
  unsigned long long inv = 0;
  const bool tally = (r == 0);
  if (beg < end) {
    const u32x4 *v4 = reinterpret_cast<const u32x4 *>(ids + beg);
    const uint64_t n4 = (end - beg) >> 2;
    constexpr int kUnroll = 4;
    uint64_t i = threadIdx.x;
    for (; i + (kUnroll - 1) * kCountThreads < n4; i += kUnroll * kCountThreads) {
      u32x4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = load_ids16<kShared>(v4 + i + u * kCountThreads);
      int32_t a[4 * kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        a[4 * u] = (int32_t)q[u].x;
        a[4 * u + 1] = (int32_t)q[u].y;
        a[4 * u + 2] = (int32_t)q[u].z;
        a[4 * u + 3] = (int32_t)q[u].w;
      }
      count_batch16(a, lo, nb, s_words, s_spill, &s_nspill);
      if (tally) {
#pragma unroll
        for (int e = 0; e < 4 * kUnroll; ++e) inv += (uint32_t)a[e] >= (uint32_t)V;
      }
    }
    for (; i < n4; i += kCountThreads) {
      const u32x4 q = load_ids16<kShared>(v4 + i);
      const int32_t a[4] = {(int32_t)q.x, (int32_t)q.y, (int32_t)q.z, (int32_t)q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        count_one16(a[e], lo, nb, s_words, s_spill, &s_nspill);
        if (tally) inv += (uint32_t)a[e] >= (uint32_t)V;
      }
    }
    for (uint64_t j = beg + (n4 << 2) + threadIdx.x; j < end; j += kCountThreads) {
      const int32_t a = ids[j];
      count_one16(a, lo, nb, s_words, s_spill, &s_nspill);
      if (tally) inv += (uint32_t)a >= (uint32_t)V;
    }
  }
  if (tally && inv) atomicAdd(&s_inv, inv);
  __syncthreads();

  // The row's bins as words (range_bins and the pitch are even, so the row
  // segment is 4-byte aligned; an odd last range pads with a zero bin).
  uint32_t *row = reinterpret_cast<uint32_t *>(partial + (size_t)c * (size_t)pitch + lo);
  for (uint32_t w = threadIdx.x; w < nw; w += kCountThreads) row[w] = s_words[w];
  if (tally && threadIdx.x == 0) inv_part[c] = s_inv;
  uint32_t *sp = spill + (size_t)(c * n_ranges + r) * (kSpillCap + 1);
  const uint32_t ns = min(s_nspill, (uint32_t)kSpillCap);
  if (threadIdx.x == 0) sp[0] = ns;
  for (uint32_t i = threadIdx.x; i < ns; i += kCountThreads) sp[1 + i] = s_spill[i];
}

__device__ __forceinline__ void reduce_invalid(const unsigned long long *__restrict__ inv_part,
                                               int32_t n_chunks, int accumulate,
                                               uint64_t *__restrict__ n_invalid) {
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    unsigned long long t = 0;
    for (int c = threadIdx.x; c < n_chunks; c += 64) t += inv_part[c];
    for (int s = 32; s > 0; s >>= 1) t += __shfl_xor(t, s);
    if (threadIdx.x == 0) *n_invalid = (accumulate ? *n_invalid : 0) + t;
  }
}

// Sums of the 16-bit partial rows. A workgroup takes 512 ids, 8 per lane
// (one 16-byte load per row; the row pitch is a multiple of 8 ids, so a
// load never leaves its row); its 8 waves split the rows, and the 8
// partial sums are added in LDS in a fixed order.
constexpr int kRedWaves = 8;
constexpr int kRedIds = 8 * kWave;  // ids per workgroup

__global__ __launch_bounds__(kRedWaves *kWave) void count_reduce16_kernel(
    const uint16_t *__restrict__ partial, const unsigned long long *__restrict__ inv_part,
    int32_t V, int32_t pitch, int32_t n_chunks, int accumulate, uint32_t *__restrict__ counts,
    uint64_t *__restrict__ n_invalid) {
  __shared__ u32x4 s_sum[kRedWaves][2 * kWave];
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int32_t v0 = blockIdx.x * kRedIds + 8 * lane;
  uint32_t s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (v0 < V) {
#pragma unroll 8
    for (int c = wave; c < n_chunks; c += kRedWaves) {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(partial + (size_t)c * (size_t)pitch + v0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += w[j] & 0xFFFFu;
        s[2 * j + 1] += w[j] >> 16;
      }
    }
  }
  s_sum[wave][2 * lane] = u32x4{s[0], s[1], s[2], s[3]};
  s_sum[wave][2 * lane + 1] = u32x4{s[4], s[5], s[6], s[7]};
  __syncthreads();
  const int32_t v = blockIdx.x * kRedIds + threadIdx.x;
  if (v < V) {
    uint32_t tot = accumulate ? counts[v] : 0u;
#pragma unroll
    for (int w = 0; w < kRedWaves; ++w)
      tot += reinterpret_cast<const uint32_t *>(s_sum[w])[threadIdx.x];
    counts[v] = tot;
  }
  reduce_invalid(inv_part, n_chunks, accumulate, n_invalid);
}

// Adds the 32768-count overflow records of one counting workgroup.
__global__ __launch_bounds__(256) void count_spill_kernel(const uint32_t *__restrict__ spill,
                                                          uint32_t *__restrict__ counts) {
  const uint32_t *sp = spill + (size_t)blockIdx.x * (kSpillCap + 1);
  const uint32_t ns = sp[0];
  for (uint32_t i = threadIdx.x; i < ns; i += 256) atomicAdd(&counts[sp[1 + i]], 32768u);
}

// Sums of the 32-bit partial rows, laid out as the 16-bit reduction: 4 ids
// per lane (the row pitch is a multiple of 4 ids), rows split over the
// waves, partial sums added in LDS in a fixed order.
__global__ __launch_bounds__(kRedWaves *kWave) void count_reduce_kernel(
    const uint32_t *__restrict__ partial, const unsigned long long *__restrict__ inv_part,
    int32_t V, int32_t pitch, int32_t n_chunks, int accumulate, uint32_t *__restrict__ counts,
    uint64_t *__restrict__ n_invalid) {
  __shared__ u32x4 s_sum[kRedWaves][kWave];
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int32_t v0 = blockIdx.x * (4 * kWave) + 4 * lane;
  u32x4 s = {0, 0, 0, 0};
  if (v0 < V) {
#pragma unroll 8
    for (int c = wave; c < n_chunks; c += kRedWaves)
      s += *reinterpret_cast<const u32x4 *>(partial + (size_t)c * (size_t)pitch + v0);
  }
  s_sum[wave][lane] = s;
  __syncthreads();
  if (threadIdx.x < 4 * kWave) {
    const int32_t v = blockIdx.x * (4 * kWave) + threadIdx.x;
    if (v < V) {
      uint32_t tot = accumulate ? counts[v] : 0u;
#pragma unroll
      for (int w = 0; w < kRedWaves; ++w)
        tot += reinterpret_cast<const uint32_t *>(s_sum[w])[threadIdx.x];
      counts[v] = tot;
    }
  }
  reduce_invalid(inv_part, n_chunks, accumulate, n_invalid);
}

}  // namespace

CountPlan count_plan(uint64_t n, int32_t V) {
  CountPlan p;
  p.bins16 = V > kRangeBinsMax;
  const int32_t range_max = p.bins16 ? kRange16Max : kRangeBinsMax;
  p.n_ranges = (V + range_max - 1) / range_max;
  p.range_bins = (V + p.n_ranges - 1) / p.n_ranges;
  if (p.bins16) p.range_bins = (p.range_bins + 1) / 2 * 2;  // word-aligned ranges
  // Chunks of ids: a multiple of 8 (whole chunks per XCD), at least 64k ids
  // each, and about 256 workgroups over the ranges (one per CU). 16-bit
  // bins: also enough chunks that no workgroup sees more than
  // kSpillCap * 32768 ids (the bound on its overflow records).
  int64_t c = (int64_t)((n + 65535) / 65536);
  const int64_t cap = (kMaxChunks / p.n_ranges + 7) / 8 * 8;
  if (c > cap) c = cap;
  if (p.bins16) {
    const uint64_t per = (uint64_t)kSpillCap << 15;
    c = std::max<int64_t>(c, (int64_t)((n + per - 1) / per));
  }
  if (c < 1) c = 1;
  c = (c + 7) / 8 * 8;
  p.n_chunks = (int32_t)c;
  uint64_t len = (n + c - 1) / c;
  p.chunk_len = (len + 3) / 4 * 4;
  if (p.chunk_len == 0) p.chunk_len = 4;
  p.row_pitch = p.bins16 ? (V + 7) / 8 * 8 : (V + 3) / 4 * 4;
  p.partial_bytes =
      align_up((size_t)p.n_chunks * (size_t)p.row_pitch * (p.bins16 ? 2 : 4), 256);
  p.inv_bytes = align_up((size_t)p.n_chunks * 8, 256);
  p.spill_bytes =
      p.bins16 ? align_up((size_t)p.n_chunks * p.n_ranges * (kSpillCap + 1) * 4, 256) : 0;
  return p;
}

hipError_t launch_count(const int32_t *ids, uint64_t n, int32_t V,
                        uint32_t *counts, int accumulate, uint64_t *n_invalid,
                        void *ws, hipStream_t stream) {
  const CountPlan p = count_plan(n, V);
  unsigned long long *inv = reinterpret_cast<unsigned long long *>(
      static_cast<char *>(ws) + p.partial_bytes);
  const int slots = p.n_ranges * (p.n_chunks / 8);
  // The counting kernels need more than 64 KB of LDS: opt in once per device
  // (a bit per device; setting the attribute twice is harmless).
  static std::atomic<uint64_t> lds_opt_in{0};
  int dev = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(lds_opt_in.load(std::memory_order_acquire) & bit)) {
    hipError_t a = hipFuncSetAttribute((const void *)count_partial_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(kRangeBinsMax * 4));
    if (a != hipSuccess) return a;
    for (const void *f : {(const void *)count_partial16_kernel<false>,
                          (const void *)count_partial16_kernel<true>}) {
      a = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kRange16Max * 2));
      if (a != hipSuccess) return a;
    }
    lds_opt_in.fetch_or(bit, std::memory_order_release);
  }
  if (p.bins16) {
    uint16_t *partial = static_cast<uint16_t *>(ws);
    uint32_t *spill = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + p.partial_bytes +
                                                   p.inv_bytes);
    const size_t lds = (size_t)(p.range_bins + 1) / 2 * 4;
    if (p.n_ranges > 1)
      hipLaunchKernelGGL(count_partial16_kernel<true>, dim3(slots * 8), dim3(kCountThreads),
                         lds, stream, ids, n, V, p.range_bins, p.n_ranges, p.n_chunks,
                         p.chunk_len, p.row_pitch, partial, inv, spill);
    else
      hipLaunchKernelGGL(count_partial16_kernel<false>, dim3(slots * 8), dim3(kCountThreads),
                         lds, stream, ids, n, V, p.range_bins, p.n_ranges, p.n_chunks,
                         p.chunk_len, p.row_pitch, partial, inv, spill);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(count_reduce16_kernel, dim3((V + kRedIds - 1) / kRedIds),
                       dim3(kRedWaves * kWave), 0, stream,
                       partial, inv, V, p.row_pitch, p.n_chunks, accumulate, counts, n_invalid);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(count_spill_kernel, dim3(p.n_chunks * p.n_ranges), dim3(256), 0, stream,
                       spill, counts);
    return hipGetLastError();
  }
  uint32_t *partial = static_cast<uint32_t *>(ws);
  const size_t lds = (size_t)p.range_bins * 4;
  hipLaunchKernelGGL(count_partial_kernel, dim3(slots * 8), dim3(kCountThreads),
                     lds, stream, ids, n, V, p.range_bins, p.n_ranges,
                     p.n_chunks, p.chunk_len, p.row_pitch, partial, inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(count_reduce_kernel, dim3((V + 4 * kWave - 1) / (4 * kWave)),
                     dim3(kRedWaves * kWave), 0, stream, partial, inv, V, p.row_pitch,
                     p.n_chunks, accumulate, counts, n_invalid);
  return hipGetLastError();
}

}  // namespace vt

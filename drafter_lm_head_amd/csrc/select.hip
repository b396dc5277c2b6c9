// Top-V_high vocabulary selection (VocabTrim page, Implementation, Step 2;
// FR-Spec notes, key design: keep the |V_high| most frequent tokens), for
// gfx950.
//
// The order is (count descending, id ascending) over all V ids. The counts
// (at most 608 KB) stay in L2, so one workgroup of 1024 threads does the
// whole selection in one launch:
//   1. radix select (11/11/10-bit digits) of the V_high-th largest count c*,
//      and `need`, the number of ids with count c* that are kept; the first
//      pass also sums all counts and finds the largest;
//   2. stable compaction, in id order, of the ids with count > c* and the
//      first `need` ids with count == c*;
//   3. stable LSD radix sort (8-bit digits) of the kept (count, id) pairs by
//      descending count, over only the bits the largest count uses; since the
//      pairs start in id order, equal counts stay in ascending id order;
//   4. t2f, f2t and the two sums.
// Counts of a frequency histogram are very skewed (most ids share a few
// small values), so digit histograms combine each wave's most common digit
// into one LDS atomic; loads are 16 bytes wide with several in flight.
// From kMtMinV ids on, the selection runs over many workgroups instead (see
// below).
#include <algorithm>

#include "vt_internal.hpp"

namespace vt {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

struct SelShared {
  uint32_t hist[2048];
  uint32_t wsum[kSelWaves];
  uint32_t total;
  uint32_t digit, need;
  unsigned long long r64[kSelWaves];
  uint32_t r32[kSelWaves];
  uint32_t dbase[256];
  uint32_t drun[256];
  uint32_t wcnt[kSelWaves][256];
};

// Exclusive prefix sum over the 1024 threads; *total receives the sum.
__device__ uint32_t block_excl_scan(uint32_t x, SelShared &s, uint32_t *total) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(x);
  if (lane == kWave - 1) s.wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const uint32_t y = lane < kSelWaves ? s.wsum[lane] : 0u;
    const uint32_t yi = wave_incl_scan(y);
    if (lane < kSelWaves) s.wsum[lane] = yi - y;
    if (lane == kSelWaves - 1) s.total = yi;
  }
  __syncthreads();
  const uint32_t r = s.wsum[wave] + incl - x;
  *total = s.total;
  __syncthreads();
  return r;
}

__device__ unsigned long long block_sum_u64(unsigned long long x, SelShared &s) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if (lane == 0) s.r64[wave] = x;
  __syncthreads();
  unsigned long long t = 0;
  for (int w = 0; w < kSelWaves; ++w) t += s.r64[w];
  __syncthreads();
  return t;
}

__device__ uint32_t block_max_u32(uint32_t x, SelShared &s) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor(x, o));
  if (lane == 0) s.r32[wave] = x;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < kSelWaves; ++w) t = max(t, s.r32[w]);
  __syncthreads();
  return t;
}

// counts[4 i .. 4 i + 3] with entries past V read as 0 and never loaded
// (counts is 16-byte aligned; only the last, partial vector uses scalars).
__device__ __forceinline__ u32x4 load_counts4(const uint32_t *counts, int32_t V, int32_t i) {
  if (4 * i + 3 < V) return reinterpret_cast<const u32x4 *>(counts)[i];
  u32x4 q = {0, 0, 0, 0};
  if (4 * i + 0 < V) q.x = counts[4 * i + 0];
  if (4 * i + 1 < V) q.y = counts[4 * i + 1];
  if (4 * i + 2 < V) q.z = counts[4 * i + 2];
  return q;
}

// hist[d] += 1 for every active lane. The lanes that share the first active
// lane's digit add with one atomic; the others add one by one. Every lane of
// the wave must call it.
__device__ __forceinline__ void hist_add(uint32_t *hist, uint32_t d, bool active) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int leader = (int)__builtin_ctzll(act);
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
  const uint64_t same = __ballot(active && d == d0);
  if (__lane_id() == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
  if (active && d != d0) atomicAdd(&hist[d], 1u);
}

// Calls f(v, c) for every id v < V (coalesced 16-byte loads, kUnroll in
// flight); the loop trip count is uniform so f may use wave-wide ops, and
// ids past V are passed with valid = false.
template <typename F>
__device__ __forceinline__ void for_counts(const uint32_t *counts, int32_t V, F f) {
  const int32_t n4 = (V + 3) / 4;
  for (int32_t base = 0; base < n4; base += kUnroll * kSelThreads) {
    u32x4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t i = base + u * kSelThreads + (int)threadIdx.x;
      q[u] = i < n4 ? load_counts4(counts, V, i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t v = 4 * (base + u * kSelThreads + (int)threadIdx.x);
      f(v + 0, q[u].x, v + 0 < V);
      f(v + 1, q[u].y, v + 1 < V);
      f(v + 2, q[u].z, v + 2 < V);
      f(v + 3, q[u].w, v + 3 < V);
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const uint32_t *__restrict__ counts, int32_t V, int32_t V_high,
    int32_t *__restrict__ t2f, int32_t *__restrict__ f2t,
    uint64_t *__restrict__ sel_out, uint64_t *__restrict__ tot_out,
    uint64_t *__restrict__ bufA, uint64_t *__restrict__ bufB) {
  __shared__ SelShared s;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;

  // ---- 1. radix select of c*, the V_high-th largest count (the first pass
  // also totals the counts and finds the largest)
  unsigned long long tot = 0;
  uint32_t cmax = 0;
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)V_high;
  const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
  for (int p = 0; p < 3; ++p) {
    const int sh = shifts[p];
    const uint32_t nd = 1u << widths[p], dm = nd - 1;
    for (uint32_t i = tid; i < nd; i += kSelThreads) s.hist[i] = 0;
    __syncthreads();
    for_counts(counts, V, [&](int32_t, uint32_t c, bool valid) {
      if (p == 0 && valid) {
        tot += c;
        cmax = max(cmax, c);
      }
      hist_add(s.hist, (c >> sh) & dm, valid && (c & pmask) == prefix);
    });
    __syncthreads();
    // Thread t owns digits d0 = nd-1-2t and d1 = d0-1 (largest first).
    const int d0 = (int)nd - 1 - 2 * tid, d1 = d0 - 1;
    const uint32_t h0 = d0 >= 0 ? s.hist[d0] : 0u, h1 = d1 >= 0 ? s.hist[d1] : 0u;
    uint32_t tot_unused;
    const uint32_t above = block_excl_scan(h0 + h1, s, &tot_unused);  // # with digit > d0
    if (d0 >= 0 && above < need && above + h0 >= need) {
      s.digit = (uint32_t)d0;
      s.need = need - above;
    } else if (d1 >= 0 && above + h0 < need && above + h0 + h1 >= need) {
      s.digit = (uint32_t)d1;
      s.need = need - above - h0;
    }
    __syncthreads();
    prefix |= s.digit << sh;
    pmask |= dm << sh;
    need = s.need;
    __syncthreads();
  }
  tot = block_sum_u64(tot, s);
  cmax = block_max_u32(cmax, s);
  const uint32_t cstar = prefix;  // ids with count > c* all kept; `need` ties kept

  // ---- 2. stable compaction in id order: thread t owns the ids of a
  // contiguous run of 16-byte vectors.
  const int32_t n4 = (V + 3) / 4;
  const int32_t run4 = (n4 + kSelThreads - 1) / kSelThreads;
  const int32_t i4b = min(n4, tid * run4), i4e = min(n4, i4b + run4);
  uint32_t n_gt = 0, n_eq = 0;
  for (int32_t i4 = i4b; i4 < i4e; i4 += kUnroll) {
    u32x4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = i4 + u < i4e ? load_counts4(counts, V, i4 + u) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t cc[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = i4 + u < i4e && 4 * (i4 + u) + e < V;
        n_gt += valid && cc[e] > cstar;
        n_eq += valid && cc[e] == cstar;
      }
    }
  }
  uint32_t scan_total;
  const uint32_t eq_before = block_excl_scan(n_eq, s, &scan_total);
  const uint32_t eq_take =
      eq_before >= need ? 0u : min(n_eq, need - eq_before);
  uint32_t pos = block_excl_scan(n_gt + eq_take, s, &scan_total);
  {
    uint32_t eq_rank = eq_before;
    for (int32_t i4 = i4b; i4 < i4e; i4 += kUnroll) {
      u32x4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = i4 + u < i4e ? load_counts4(counts, V, i4 + u) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t cc[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int32_t v = 4 * (i4 + u) + e;
          if (i4 + u >= i4e || v >= V) continue;
          const uint32_t c = cc[e];
          bool keep = c > cstar;
          if (c == cstar) keep = eq_rank++ < need;
          // pos < V_high always holds; the test keeps a logic error in bounds
          if (keep && pos < (uint32_t)V_high) bufA[pos++] = ((uint64_t)c << 32) | (uint32_t)v;
        }
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  // ---- 3. stable LSD radix sort by descending count
  const int nbits = cmax ? 32 - __clz(cmax) : 0;
  const uint32_t kmask = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
  const int passes = (nbits + 7) / 8;
  uint64_t *src = bufA, *dst = bufB;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int p = 0; p < passes; ++p) {
    const int sh = 8 * p;
    for (int i = tid; i < 256; i += kSelThreads) {
      s.hist[i] = 0;
      s.drun[i] = 0;
    }
    __syncthreads();
    for (int32_t base = 0; base < V_high; base += kUnroll * kSelThreads) {
      uint64_t e[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t i = base + u * kSelThreads + tid;
        e[u] = i < V_high ? src[i] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t i = base + u * kSelThreads + tid;
        const uint32_t key = (~(uint32_t)(e[u] >> 32)) & kmask;
        hist_add(s.hist, (key >> sh) & 255u, i < V_high);
      }
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the 256 digit counts
      uint32_t a[4], t = 0;
      for (int j = 0; j < 4; ++j) {
        a[j] = s.hist[lane * 4 + j];
        t += a[j];
      }
      const uint32_t before = wave_incl_scan(t) - t;
      uint32_t run_sum = before;
      for (int j = 0; j < 4; ++j) {
        s.dbase[lane * 4 + j] = run_sum;
        run_sum += a[j];
      }
    }
    __syncthreads();
    // Tiles of 1024 elements in order; the next tile's element is loaded
    // while this one is ranked.
    uint64_t e_next = tid < V_high ? src[tid] : 0ull;
    for (int32_t base = 0; base < V_high; base += kSelThreads) {
      const int32_t i = base + tid;
      const bool valid = i < V_high;
      const uint64_t e = e_next;
      e_next = i + kSelThreads < V_high ? src[i + kSelThreads] : 0ull;
      const uint32_t dg = valid ? (((~(uint32_t)(e >> 32)) & kmask) >> sh) & 255u : 0u;
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (dg >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
      }
      for (int j = lane; j < 256; j += kWave) s.wcnt[wave][j] = 0;
      const uint32_t rank = __popcll(peers & lt_mask);
      if (valid && rank == 0) s.wcnt[wave][dg] = __popcll(peers);
      __syncthreads();
      if (tid < 256) {  // prefix over waves, per digit
        uint32_t acc = s.drun[tid];
        for (int w = 0; w < kSelWaves; ++w) {
          const uint32_t t = s.wcnt[w][tid];
          s.wcnt[w][tid] = acc;
          acc += t;
        }
        s.drun[tid] = acc;
      }
      __syncthreads();
      const uint32_t at = s.dbase[dg] + s.wcnt[wave][dg] + rank;
      if (valid && at < (uint32_t)V_high) dst[at] = e;
      __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
    uint64_t *t = src;
    src = dst;
    dst = t;
  }

  // ---- 4. maps and sums
  if (f2t)
    for (int32_t v = tid; v < V; v += kSelThreads) f2t[v] = -1;
  __threadfence_block();
  __syncthreads();
  unsigned long long sel = 0;
  for (int32_t base = 0; base < V_high; base += kUnroll * kSelThreads) {
    uint64_t e[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t i = base + u * kSelThreads + tid;
      e[u] = i < V_high ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t i = base + u * kSelThreads + tid;
      if (i >= V_high) continue;
      const int32_t id = (int32_t)(uint32_t)e[u];
      t2f[i] = id;
      if (f2t && (uint32_t)id < (uint32_t)V) f2t[id] = i;
      sel += e[u] >> 32;
    }
  }
  sel = block_sum_u64(sel, s);
  if (tid == 0) {
    *sel_out = sel;
    *tot_out = tot;
  }
}

// ------------------------------------------------------- many workgroups
// A large vocabulary is selected by the whole chip. Id v gets the key
// (counts[v] << 32) | ~v: the keys are distinct and a larger key is exactly a
// higher rank (count descending, id ascending), so the kept set is
// {v : key(v) >= P} for P the V_high-th largest key, with no tie rule left to
// apply at the cut:
//   1. P by radix select over the 64 key bits, six digits (11 bits, the last
//      9): each pass histograms the keys that share the digits chosen so far
//      (per-workgroup LDS histograms folded into one with atomics) and the
//      last workgroup to finish picks the next digit;
//   2. the kept keys are compacted (in any order) and their counts summed;
//   3. blocks of kSortBlock keys are sorted in LDS (bitonic, descending); the
//      rank of a key is its position in its block plus the number of larger
//      keys in every other block (binary search), summed over groups of
//      blocks in a fixed order;
//   4. t2f[rank] = id and f2t[id] = rank.
constexpr int kSortBlock = 2048;  // keys per sorted block (two per thread)
constexpr int kRankGroup = 4;     // blocks searched per rank workgroup (at least)
constexpr int kRankGroupsMax = 32;  // partial ranks summed per key (at most)
constexpr int kPasses = 6;

struct MtState {
  unsigned long long pref, mask, tot, sel;
  uint32_t rank, ticket, ncomp, pad;
};

__device__ __forceinline__ uint64_t sel_key(uint32_t c, int32_t v) {
  return ((uint64_t)c << 32) | (uint32_t)(~(uint32_t)v);
}
__device__ __forceinline__ uint32_t fetch_u32(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void mt_init_kernel(MtState *st, uint32_t *ghist,
                                                      int32_t V_high, int32_t *f2t, int32_t V) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i == 0) {
    st->pref = 0;
    st->mask = 0;
    st->tot = 0;
    st->sel = 0;
    st->rank = (uint32_t)V_high;
    st->ticket = 0;
    st->ncomp = 0;
  }
  if (i < 2048) ghist[i] = 0;
  if (f2t && i < V) f2t[i] = -1;
}

// One radix-select pass over the ids of this workgroup (4 per thread).
__global__ __launch_bounds__(kSelThreads) void mt_hist_kernel(const uint32_t *counts,
                                                              int32_t V, MtState *st,
                                                              uint32_t *ghist, int pass) {
  __shared__ SelShared s;
  __shared__ uint32_t s_slot;
  const int tid = threadIdx.x;
  const int lo = pass < kPasses - 1 ? 53 - 11 * pass : 0;
  const uint32_t nbins = pass < kPasses - 1 ? 2048u : 512u;
  for (int i = tid; i < 2048; i += kSelThreads) s.hist[i] = 0;
  const uint64_t pref = st->pref, mask = st->mask;
  __syncthreads();
  const int32_t i4 = blockIdx.x * kSelThreads + tid;
  const u32x4 q = 4 * i4 < V ? load_counts4(counts, V, i4) : u32x4{0, 0, 0, 0};
  unsigned long long tsum = 0;
  const uint32_t qc[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int32_t v = 4 * i4 + c;
    const uint64_t key = sel_key(qc[c], v);
    const bool active = v < V && ((key ^ pref) & mask) == 0;
    hist_add(s.hist, (uint32_t)(key >> lo) & (nbins - 1), active);
    if (v < V) tsum += qc[c];
  }
  __syncthreads();
  for (uint32_t i = tid; i < nbins; i += kSelThreads)
    if (s.hist[i])
      __hip_atomic_fetch_add(&ghist[i], s.hist[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (pass == 0) {
    tsum = block_sum_u64(tsum, s);
    if (tid == 0 && tsum)
      __hip_atomic_fetch_add(&st->tot, tsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (arrive(&st->ticket, &s_slot) != gridDim.x - 1) return;

  // Last workgroup: the digit holding the rank-th largest key. Thread t
  // takes digits nbins - 1 - 2t and nbins - 2 - 2t (descending order).
  const int d0 = (int)nbins - 1 - 2 * tid, d1 = d0 - 1;
  const uint32_t h0 = d0 >= 0 ? fetch_u32(&ghist[d0]) : 0u;
  const uint32_t h1 = d1 >= 0 ? fetch_u32(&ghist[d1]) : 0u;
  uint32_t total;
  const uint32_t before = block_excl_scan(h0 + h1, s, &total);
  const uint32_t r = st->rank;
  const uint64_t dmask = (uint64_t)(nbins - 1) << lo;
  if (d0 >= 0 && before < r && r <= before + h0) {
    st->pref = pref | ((uint64_t)d0 << lo);
    st->mask = mask | dmask;
    st->rank = r - before;
  } else if (d1 >= 0 && before + h0 < r && r <= before + h0 + h1) {
    st->pref = pref | ((uint64_t)d1 << lo);
    st->mask = mask | dmask;
    st->rank = r - before - h0;
  }
  for (uint32_t i = tid; i < nbins; i += kSelThreads)
    __hip_atomic_store(&ghist[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) reset_counter(&st->ticket);
}

// The kept keys (key >= P) to comp[], in any order, and the sum of their counts.
__global__ __launch_bounds__(kSelThreads) void mt_compact_kernel(const uint32_t *counts,
                                                                 int32_t V, MtState *st,
                                                                 uint64_t *comp) {
  __shared__ SelShared s;
  __shared__ uint32_t s_base;
  const int tid = threadIdx.x;
  const uint64_t P = st->pref;
  const int32_t i4 = blockIdx.x * kSelThreads + tid;
  const u32x4 q = 4 * i4 < V ? load_counts4(counts, V, i4) : u32x4{0, 0, 0, 0};
  const uint32_t qc[4] = {q.x, q.y, q.z, q.w};
  bool keep[4];
  uint32_t nk = 0;
  unsigned long long csum = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int32_t v = 4 * i4 + c;
    keep[c] = v < V && sel_key(qc[c], v) >= P;
    nk += keep[c];
    if (keep[c]) csum += qc[c];
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan(nk, s, &total);
  csum = block_sum_u64(csum, s);
  if (tid == 0) {
    s_base = total ? __hip_atomic_fetch_add(&st->ncomp, total, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                   : 0u;
    if (csum)
      __hip_atomic_fetch_add(&st->sel, csum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  uint32_t o = s_base + excl;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (keep[c]) comp[o++] = sel_key(qc[c], 4 * i4 + c);
}

// Sorts block b of the n compacted keys descending in LDS (0 pads the block).
__global__ __launch_bounds__(kSelThreads) void mt_block_sort_kernel(const uint64_t *comp,
                                                                    int32_t n,
                                                                    uint64_t *sorted) {
  __shared__ uint64_t sk[kSortBlock];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kSortBlock;
  for (int i = tid; i < kSortBlock; i += kSelThreads)
    sk[i] = base + i < n ? comp[base + i] : 0ull;
  __syncthreads();
  // kSortBlock / 2 compare-exchanges per stage, one per thread. Up to a
  // stride of 64 both keys of every exchange of wave w lie in keys
  // 128 w .. 128 w + 127, and a wave's LDS accesses are performed in order,
  // so a workgroup barrier is needed only after a stage that crosses waves
  // (stride >= 128) or before one (the first stage of a size >= 256).
  for (uint32_t size = 2; size <= (uint32_t)kSortBlock; size <<= 1)
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t i = tid;
      const uint32_t lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
      const uint64_t x = sk[lo], y = sk[hi];
      if ((x < y) == ((lo & size) == 0)) {
        sk[lo] = y;
        sk[hi] = x;
      }
      if (stride > (uint32_t)kWave || (stride == 1 && size >= 2 * kWave)) {
        __syncthreads();
      } else {
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
  for (int i = tid; i < kSortBlock; i += kSelThreads) sorted[base + i] = sk[i];
}

// Number of keys in the descending block ob that are larger than x.
__device__ __forceinline__ uint32_t count_greater(const uint64_t *ob, uint64_t x) {
  uint32_t lo = 0, hi = kSortBlock;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (ob[mid] > x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Partial ranks of the keys of block b against the blocks of group g (blocks
// g * group .. g * group + group - 1): rank_part[g][j] for position
// j = b * kSortBlock + i.
__global__ __launch_bounds__(kSelThreads) void mt_rank_kernel(const uint64_t *sorted, int32_t nb,
                                                              int32_t ngroups, int32_t group,
                                                              uint32_t *rank_part) {
  __shared__ uint64_t ob[kSortBlock];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / ngroups, g = blockIdx.x % ngroups;
  const int64_t npos = (int64_t)nb * kSortBlock;
  const int64_t j0 = (int64_t)b * kSortBlock + tid, j1 = j0 + kSelThreads;
  const uint64_t x0 = sorted[j0], x1 = sorted[j1];
  uint32_t r0 = 0, r1 = 0;
  const int ob_end = min(nb, (g + 1) * group);
  for (int o = g * group; o < ob_end; ++o) {
    if (o == b) {  // within its own sorted block a key's rank is its position
      r0 += tid;
      r1 += tid + kSelThreads;
      continue;
    }
    __syncthreads();
    ob[tid] = sorted[(int64_t)o * kSortBlock + tid];
    ob[tid + kSelThreads] = sorted[(int64_t)o * kSortBlock + tid + kSelThreads];
    __syncthreads();
    r0 += count_greater(ob, x0);
    r1 += count_greater(ob, x1);
  }
  rank_part[(int64_t)g * npos + j0] = r0;
  rank_part[(int64_t)g * npos + j1] = r1;
}

__global__ __launch_bounds__(256) void mt_scatter_kernel(const uint64_t *sorted,
                                                         const uint32_t *rank_part,
                                                         int32_t ngroups, int32_t npos,
                                                         int32_t V, int32_t V_high,
                                                         int32_t *t2f, int32_t *f2t,
                                                         const MtState *st, uint64_t *sel_out,
                                                         uint64_t *tot_out) {
  const int32_t j = blockIdx.x * 256 + threadIdx.x;
  if (j < npos) {
    const uint64_t key = sorted[j];
    if (key != 0) {  // not a pad
      uint32_t r = 0;
      for (int g = 0; g < ngroups; ++g) r += rank_part[(int64_t)g * npos + j];
      const int32_t id = (int32_t)(~(uint32_t)key);
      if (r < (uint32_t)V_high) {
        t2f[r] = id;
        if (f2t && (uint32_t)id < (uint32_t)V) f2t[id] = (int32_t)r;
      }
    }
  }
  if (j == 0) {
    *sel_out = st->sel;
    *tot_out = st->tot;
  }
}

struct MtPlan {
  int32_t nb, group, ngroups;
  size_t off_hist, off_comp, off_sorted, off_rank, bytes;
};

MtPlan mt_plan(int32_t V_high) {
  MtPlan p;
  p.nb = (V_high + kSortBlock - 1) / kSortBlock;
  p.group = std::max(kRankGroup, (p.nb + kRankGroupsMax - 1) / kRankGroupsMax);
  p.ngroups = (p.nb + p.group - 1) / p.group;
  size_t off = align_up(sizeof(MtState), 256);
  p.off_hist = off;
  off += align_up(2048 * 4, 256);
  p.off_comp = off;
  off += align_up((size_t)V_high * 8, 256);
  p.off_sorted = off;
  off += align_up((size_t)p.nb * kSortBlock * 8, 256);
  p.off_rank = off;
  off += align_up((size_t)p.ngroups * p.nb * kSortBlock * 4, 256);
  p.bytes = off;
  return p;
}

// One workgroup does the whole selection up to this many ids; past it the
// many-workgroup path is faster.
constexpr int32_t kMtMinV = 16384;

}  // namespace

size_t select_ws_bytes(int32_t V, int32_t V_high) {
  if (V >= kMtMinV) return mt_plan(V_high).bytes;
  return 2 * align_up((size_t)V_high * 8, 256);
}

hipError_t launch_select(const uint32_t *counts, int32_t V, int32_t V_high,
                         int32_t *t2f, int32_t *f2t, uint64_t *sel,
                         uint64_t *tot, void *ws, hipStream_t stream) {
  if (V < kMtMinV) {
    uint64_t *a = static_cast<uint64_t *>(ws);
    uint64_t *b = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) +
                                               align_up((size_t)V_high * 8, 256));
    hipLaunchKernelGGL(select_kernel, dim3(1), dim3(kSelThreads), 0, stream,
                       counts, V, V_high, t2f, f2t, sel, tot, a, b);
    return hipGetLastError();
  }
  const MtPlan p = mt_plan(V_high);
  char *base = static_cast<char *>(ws);
  MtState *st = reinterpret_cast<MtState *>(base);
  uint32_t *ghist = reinterpret_cast<uint32_t *>(base + p.off_hist);
  uint64_t *comp = reinterpret_cast<uint64_t *>(base + p.off_comp);
  uint64_t *sorted = reinterpret_cast<uint64_t *>(base + p.off_sorted);
  uint32_t *rank_part = reinterpret_cast<uint32_t *>(base + p.off_rank);
  const int32_t init_n = std::max(std::max(V, V_high), 2048);
  hipLaunchKernelGGL(mt_init_kernel, dim3((init_n + 255) / 256), dim3(256), 0, stream, st, ghist,
                     V_high, f2t, V);
  const int32_t wgs = (int32_t)(((int64_t)V + 4 * kSelThreads - 1) / (4 * kSelThreads));
  for (int pass = 0; pass < kPasses; ++pass)
    hipLaunchKernelGGL(mt_hist_kernel, dim3(wgs), dim3(kSelThreads), 0, stream, counts, V, st,
                       ghist, pass);
  hipLaunchKernelGGL(mt_compact_kernel, dim3(wgs), dim3(kSelThreads), 0, stream, counts, V, st,
                     comp);
  hipLaunchKernelGGL(mt_block_sort_kernel, dim3(p.nb), dim3(kSelThreads), 0, stream, comp,
                     V_high, sorted);
  hipLaunchKernelGGL(mt_rank_kernel, dim3(p.nb * p.ngroups), dim3(kSelThreads), 0, stream,
                     sorted, p.nb, p.ngroups, p.group, rank_part);
  const int32_t npos = p.nb * kSortBlock;
  hipLaunchKernelGGL(mt_scatter_kernel, dim3((npos + 255) / 256), dim3(256), 0, stream, sorted,
                     rank_part, p.ngroups, npos, V, V_high, t2f, f2t, st, sel, tot);
  return hipGetLastError();
}

}  // namespace vt

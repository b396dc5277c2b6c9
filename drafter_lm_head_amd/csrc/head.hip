// Frequency-ranked drafter head, one draft step (VocabTrim page,
// Implementation, Step 4; FR-Spec notes, key design), for gfx950.
//
// One kernel streams W_trim[V_high, d] once and never writes the logits:
//   * a workgroup owns a tile of kTileRows = 64 rows; each wave computes
//     whole rows (16-byte coalesced loads over d, packed bf16 dot products
//     with fp32 accumulation against h held in registers, then a DPP
//     reduction across the wave);
//   * the tile's logits go to LDS; per draft row one wave sorts the 64
//     (logit, full id) keys, and writes the tile's top-k keys and its
//     softmax partial (max, sum of exp(z - max)) to the workspace;
//   * tiles are grouped; the last workgroup of a group to finish (atomic
//     ticket) merges the group's partials, and the last group merger merges
//     the groups and writes full_ids and probs. Every merge runs in a fixed
//     order, so results do not depend on scheduling.
// The kernel is bound by HBM bandwidth: it moves 2 * V_high * d bytes of
// W_trim and does 2 * M * V_high * d flops.
#include "vt_internal.hpp"

#ifndef VT_GEMV_WAVES
#define VT_GEMV_WAVES 4
#endif
#ifndef VT_GEMV_ROWS
#define VT_GEMV_ROWS 4
#endif

namespace vt {

namespace {

struct HeadArgs {
  const u32x4 *h;        // [M, c16]
  const u32x4 *W;        // [V_high, c16]
  const int32_t *t2f;    // [V_high]
  int32_t M, c16, V_high, k;
  int32_t tiles, group_size, groups;
  uint64_t *tile_keys;   // [M][tiles][k]
  float2 *tile_ms;       // [M][tiles]
  uint64_t *group_keys;  // [M][groups][k]
  float2 *group_ms;      // [M][groups]
  uint32_t *counters;    // [groups + 1], zero between calls
  int32_t *full_ids;     // [M][k]
  float *probs;          // [M][k]
  float *logits;         // [M][V_high], logits-only variant
};

// Merges P <= 64 parts. Part p has its k largest keys in descending order at
// lists[p * k ...] and its softmax partial ms[p] = (max, sum of exp(z - max)).
// Returns the overall rank-`lane` key for lanes < k; *mu and *S receive the
// merged max and sum. The k-th largest key overall is at least T, the
// largest of the parts' k-th keys, so only keys >= T can be picked; they are
// collected and sorted in one wave. If more than 64 keys tie above T, the
// parts' heads are merged one rank at a time instead.
__device__ uint64_t merge_parts(const uint64_t *lists, const float2 *ms, int P,
                                int k, uint64_t *s_buf, float *mu, float *S) {
  const int lane = __lane_id();
  const float2 p = lane < P ? ms[lane] : make_float2(-INFINITY, 0.f);
  const float m = wave_max(p.x);
  *S = wave_sum(lane < P ? p.y * __expf(p.x - m) : 0.f);
  *mu = m;

  const uint64_t T =
      wave_max_u64(lane < P ? lists[(size_t)lane * k + (k - 1)] : 0ull);
  const int n = P * k;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t found = 0;
  for (int j0 = 0; j0 < n; j0 += 4 * kWave) {
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = j0 + u * kWave + lane;
      v[u] = idx < n ? lists[idx] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool take = v[u] != 0ull && v[u] >= T;
      const uint64_t bal = __ballot(take);
      const uint32_t pos = found + (uint32_t)__popcll(bal & lt);
      if (take && pos < kWave) s_buf[pos] = v[u];
      found += (uint32_t)__popcll(bal);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  uint64_t key = 0;
  if (found <= (uint32_t)kWave) {
    key = lane < (int)found ? s_buf[lane] : 0ull;
    key = wave_sort_desc(key);
  } else {
    int pos = 0;
    uint64_t head = lane < P ? lists[(size_t)lane * k] : 0ull;
    for (int r = 0; r < k; ++r) {
      const uint64_t mx = wave_max_u64(head);
      if (lane == r) key = mx;
      const uint64_t win = __ballot(lane < P && head == mx);
      if (lane == __ffsll((unsigned long long)win) - 1) {
        ++pos;
        head = pos < k ? lists[(size_t)lane * k + pos] : 0ull;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  return key;
}

// Rows a wave loads per step: VT_GEMV_ROWS, halved while the step's loads
// plus h would need more than about 200 VGPRs ((U + MT) * CPL * 4).
template <int MT, int CPL>
constexpr int rows_per_step() {
  int u = VT_GEMV_ROWS;
  while (u > 1 && (u + MT) * CPL > 50) u >>= 1;
  return u;
}

template <int MT, int CPL, bool RAGGED, bool LOGITS>
__global__ __launch_bounds__(VT_GEMV_WAVES *kWave) void head_gemv_kernel(HeadArgs a) {
  constexpr int WAVES = VT_GEMV_WAVES, U = rows_per_step<MT, CPL>();
  static_assert(kTileRows % (WAVES * U) == 0, "tile must split evenly");
  static_assert(MT <= WAVES, "one wave per draft row in the epilogue");
  __shared__ float s_z[MT][kTileRows];
  __shared__ uint64_t s_buf[MT][kWave];
  __shared__ uint32_t s_slot;

  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int tile = blockIdx.x, row0 = tile * kTileRows;
  const int c16 = a.c16;

  int32_t fid = 0;
  if (!LOGITS && wave < MT && row0 + lane < a.V_high) fid = a.t2f[row0 + lane];

  u32x4 hr[MT][CPL];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int idx = c * kWave + lane;
      hr[m][c] = (!RAGGED || idx < c16) ? a.h[(size_t)m * c16 + idx]
                                        : u32x4{0, 0, 0, 0};
    }

  constexpr int kSteps = kTileRows / (WAVES * U);
#pragma unroll 1
  for (int s = 0; s < kSteps; ++s) {
    const int rl = (s * WAVES + wave) * U;  // first tile-local row of the wave
    u32x4 w[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // Rows past V_high re-read the last row (in bounds) and are dropped.
      const int row = min(row0 + rl + u, a.V_high - 1);
      const u32x4 *p = a.W + (size_t)row * c16;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int idx = c * kWave + lane;
        w[u][c] = (!RAGGED || idx < c16) ? load_stream16(p + idx)
                                         : u32x4{0, 0, 0, 0};
      }
    }
    // Issue every load of the step before any math, so that U * CPL 16-byte
    // loads per lane are in flight (the scheduler would otherwise interleave
    // them with the dot products to save registers).
    __builtin_amdgcn_sched_barrier(0);
    float z[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc = dot8_bf16(w[u][c], hr[m][c], acc);
        z[m][u] = acc;
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) z[m][u] = wave_sum(z[m][u]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (LOGITS) {
            const int row = row0 + rl + u;
            if (row < a.V_high) a.logits[(size_t)m * a.V_high + row] = z[m][u];
          } else {
            s_z[m][rl + u] = z[m][u];
          }
        }
    }
  }
  if (LOGITS) return;
  __syncthreads();

  // Tile partial: top-k keys and softmax partial of each draft row.
  const int k = a.k;
  if (wave < MT) {
    const int m = wave;
    const bool valid = row0 + lane < a.V_high;
    const float z = s_z[m][lane];
    uint64_t key = valid ? make_key(z, fid) : 0ull;
    key = wave_sort_desc(key);
    const float mu = key_logit(readlane_u64(key, 0));
    const float S = wave_sum(valid ? __expf(z - mu) : 0.f);
    uint64_t *dst = a.tile_keys + ((size_t)m * a.tiles + tile) * k;
    if (lane < k) dst[lane] = key;
    if (lane == 0) a.tile_ms[(size_t)m * a.tiles + tile] = make_float2(mu, S);
  }

  // Group merge by the group's last workgroup.
  const int g = tile / a.group_size;
  const int g_beg = g * a.group_size;
  const int g_n = min(a.group_size, a.tiles - g_beg);
  if (arrive(&a.counters[g], &s_slot) != (uint32_t)(g_n - 1)) return;
  if (wave < MT) {
    const int m = wave;
    float mu, S;
    const uint64_t key = merge_parts(
        a.tile_keys + ((size_t)m * a.tiles + g_beg) * k,
        a.tile_ms + (size_t)m * a.tiles + g_beg, g_n, k, s_buf[m], &mu, &S);
    if (lane < k) a.group_keys[((size_t)m * a.groups + g) * k + lane] = key;
    if (lane == 0) a.group_ms[(size_t)m * a.groups + g] = make_float2(mu, S);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[g], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);

  // Final merge by the last group merger: picks, probabilities, remap.
  if (arrive(&a.counters[a.groups], &s_slot) != (uint32_t)(a.groups - 1)) return;
  if (wave < MT) {
    const int m = wave;
    float mu, S;
    const uint64_t key = merge_parts(a.group_keys + (size_t)m * a.groups * k,
                                     a.group_ms + (size_t)m * a.groups,
                                     a.groups, k, s_buf[m], &mu, &S);
    if (lane < k) {
      a.full_ids[(size_t)m * k + lane] = key_id(key);
      a.probs[(size_t)m * k + lane] = __expf(key_logit(key) - mu) / S;
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[a.groups], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- dispatch
constexpr int kCplSet[] = {1, 2, 3, 4, 5, 6, 7, 8, 12, 16};

template <int MT, bool LOGITS, int CPL, bool RAGGED>
hipError_t launch_one(const HeadArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((head_gemv_kernel<MT, CPL, RAGGED, LOGITS>), dim3(a.tiles),
                     dim3(VT_GEMV_WAVES * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int MT, bool LOGITS, int I = 0>
hipError_t launch_cpl(const HeadArgs &a, hipStream_t stream) {
  constexpr int n_set = sizeof(kCplSet) / sizeof(kCplSet[0]);
  if constexpr (I >= n_set) {
    return hipErrorInvalidValue;
  } else {
    constexpr int CPL = kCplSet[I];
    if (a.c16 <= CPL * kWave) {
      if (a.c16 == CPL * kWave) return launch_one<MT, LOGITS, CPL, false>(a, stream);
      return launch_one<MT, LOGITS, CPL, true>(a, stream);
    }
    return launch_cpl<MT, LOGITS, I + 1>(a, stream);
  }
}

hipError_t launch_gemv(const HeadArgs &a, hipStream_t stream) {
  switch (a.M) {
    case 1: return launch_cpl<1, false>(a, stream);
    case 2: return launch_cpl<2, false>(a, stream);
    case 3: return launch_cpl<3, false>(a, stream);
    case 4: return launch_cpl<4, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

HeadPlan head_plan(int32_t M, int32_t V_high, int32_t k) {
  HeadPlan p;
  p.tiles = (V_high + kTileRows - 1) / kTileRows;
  int gs = 1;
  while (gs * gs < p.tiles) ++gs;
  if (gs > 64) gs = 64;
  if ((p.tiles + gs - 1) / gs > 64) gs = (p.tiles + 63) / 64;
  p.group_size = gs;
  p.groups = (p.tiles + gs - 1) / gs;
  size_t off = align_up((size_t)(p.groups + 1) * 4, 256);
  p.off_tile_keys = off;
  off += align_up((size_t)M * p.tiles * k * 8, 256);
  p.off_tile_ms = off;
  off += align_up((size_t)M * p.tiles * 8, 256);
  p.off_group_keys = off;
  off += align_up((size_t)M * p.groups * k * 8, 256);
  p.off_group_ms = off;
  off += align_up((size_t)M * p.groups * 8, 256);
  p.bytes = off;
  return p;
}

hipError_t launch_draft_head(const uint16_t *h, int32_t M, int32_t d,
                             const uint16_t *W_trim, int32_t V_high,
                             const int32_t *t2f, int32_t k, int32_t *full_ids,
                             float *probs, void *ws, hipStream_t stream) {
  const HeadPlan p = head_plan(M, V_high, k);
  char *base = static_cast<char *>(ws);
  HeadArgs a{};
  a.W = reinterpret_cast<const u32x4 *>(W_trim);
  a.t2f = t2f;
  a.c16 = d / 8;
  a.V_high = V_high;
  a.k = k;
  a.tiles = p.tiles;
  a.group_size = p.group_size;
  a.groups = p.groups;
  a.counters = reinterpret_cast<uint32_t *>(base);
  a.tile_keys = reinterpret_cast<uint64_t *>(base + p.off_tile_keys);
  a.tile_ms = reinterpret_cast<float2 *>(base + p.off_tile_ms);
  a.group_keys = reinterpret_cast<uint64_t *>(base + p.off_group_keys);
  a.group_ms = reinterpret_cast<float2 *>(base + p.off_group_ms);
  // Up to 4 draft rows per pass over W_trim.
  for (int32_t m0 = 0; m0 < M; m0 += 4) {
    HeadArgs c = a;
    c.M = min(4, M - m0);
    c.h = reinterpret_cast<const u32x4 *>(h + (size_t)m0 * d);
    c.full_ids = full_ids + (size_t)m0 * k;
    c.probs = probs + (size_t)m0 * k;
    hipError_t e = launch_gemv(c, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_head_logits(const uint16_t *h, int32_t M, int32_t d,
                              const uint16_t *W_trim, int32_t V_high,
                              float *logits, hipStream_t stream) {
  HeadArgs a{};
  a.W = reinterpret_cast<const u32x4 *>(W_trim);
  a.c16 = d / 8;
  a.V_high = V_high;
  a.M = 1;
  a.tiles = (V_high + kTileRows - 1) / kTileRows;
  for (int32_t m = 0; m < M; ++m) {
    HeadArgs c = a;
    c.h = reinterpret_cast<const u32x4 *>(h + (size_t)m * d);
    c.logits = logits + (size_t)m * V_high;
    hipError_t e = launch_cpl<1, true>(c, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace vt

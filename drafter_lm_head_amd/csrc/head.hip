// Frequency-ranked drafter head, one draft step (VocabTrim page,
// Implementation, Step 4; FR-Spec notes, key design), for gfx950. Every path
// reads W_trim[V_high, d] from memory once; they differ in what else they
// write, by number of draft rows M:
//   * M = 1 (and M = 2 on a head of fewer than 512 tiles), one kernel
//     (head_gemv_kernel), no logit written to memory:
//     each wave computes whole rows (16-byte coalesced loads over d, packed
//     bf16 dot products with fp32 accumulation against h held in
//     registers, a DPP reduction); a tile's 64 logits go to LDS, where per
//     draft row one wave ranks the (logit, full id) keys and publishes the
//     tile's top-k keys and softmax partial (max, sum of exp(z - max)); the
//     workgroup that finishes last (atomic ticket) reads every partial once
//     and merges them: the softmax partials in a fixed order, the keys by a
//     threshold filter and a rank, so results do not depend on scheduling.
//   * 2 <= M <= 512: a GEMM tiling on the matrix cores (head_gemm_kernel:
//     one workgroup per pair of W tiles, or per tile on heads of fewer than
//     512 tiles, over every draft row, both operands copied into an LDS
//     ring), which writes each tile's fp32 logits and softmax partials to
//     the workspace, then one merge workgroup per draft row
//     (tree_merge_kernel) that reads the partials and the logits of only the
//     tiles that can hold a pick. From 3 to 32 rows on a head of fewer than
//     256 tiles a skinny GEMM with one workgroup per tile whose waves stream
//     their own quarters of d (head_mfma_kernel) takes its place.
// Sampling (one draw per row) runs the same contraction kernels with a
// per-tile draw in place of the logits. Up to M of about 312 the head is
// bound by HBM bandwidth: it moves 2 * V_high * d bytes of W_trim for
// 2 * M * V_high * d flops.
#include <algorithm>

#include "vt_internal.hpp"
#include "vocabtrim.h"

namespace vt {

namespace {

constexpr int kGroups = 64;  // tile groups whose maxima bound the k-th key
// Up to this many draft rows the GEMV path can run. From three rows on the
// MFMA path is faster (measured: 49.8 us at 3 to 12 rows against 55.4 /
// 59.4 us for the GEMV at 3 / 4 rows on the 4096 x 32768 head), and at two
// rows the GEMM tiling is where its tile pairs fill the chip (46.7 against
// 47.0 us on that head, 41.0 against 42.0 us at d = 3584).
constexpr int kGemvMaxRows = 2;

struct HeadArgs {
  const u32x4 *h;        // [M, c16]
  const u32x4 *W;        // [V_high, c16]
  const int32_t *t2f;    // [V_high]
  int32_t M, c16, V_high, k;
  int32_t tiles;
  uint64_t *tile_keys;   // [M][tiles][k], published
  uint64_t *tile_ms;     // [M][tiles], (bits(S) << 32) | bits(max), published
  uint64_t *group_max;   // [M][kGroups]: largest tile head per tile group
  uint64_t *group_kth;   // [M][kGroups]: largest tile k-th key per group
  int32_t tiles_per_group;
  uint32_t *counter;     // tickets, zero between calls
  int32_t *full_ids;     // [M][k]
  float *probs;          // [M][k]
  float *logits;         // [M][V_high], logits-only variant
  uint32_t *merged;      // GEMV path, two draft rows: finished row mergers (zero between calls)
  int32_t zstream;       // MFMA path: logits to the workspace with streaming stores
  // Sampling mode (k = 1): the pick is the largest z + Gumbel(seed, offset).
  int32_t sample;
  uint32_t seed_lo, seed_hi, off_lo, off_hi;
  uint64_t *tile_z;      // [M][tiles]: bits of z of each tile's drawn row
  const uint16_t *bias;  // bf16[V_high] added to every logit, or nullptr
  int32_t remap;         // 1: keys carry t2f[j] (full ids); 0: the trimmed index j
  uint32_t *status;      // the workspace's fixed words (error, hold, spin limit)
  float *zbuf;           // MFMA path, top-k mode: logits [M][zpitch]
  int32_t zpitch;        // tiles * kTileRows floats
};

__device__ __forceinline__ uint64_t pack_ms(float mu, float S) {
  return ((uint64_t)__float_as_uint(S) << 32) | __float_as_uint(mu);
}
__device__ __forceinline__ float ms_max(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float ms_sum(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

// Id that a kept row j carries into the keys and the outputs: its full id
// t2f[j] (the remap), or j itself when the caller asks for trimmed indices.
__device__ __forceinline__ int32_t fid_at(const HeadArgs &a, int j) {
  return a.remap ? a.t2f[j] : j;
}

// Sampling-mode tile partial of one draft row, by one wave (lane = tile row,
// g = its Gumbel variate): the tile's largest sampling key, (z + g) in key
// order and then the lower full id, with that row's z, and the tile's
// softmax partial over the unperturbed z. The draw is the largest key over
// all tiles.
__device__ __forceinline__ void wave_publish_sample(const HeadArgs &a, int m, int tile,
                                                    float z, float g, int32_t fid,
                                                    bool valid) {
  const int lane = __lane_id();
  const uint64_t key = valid ? make_key(z + g, fid) : 0ull;
  const uint64_t best = wave_max_u64(key);
  const uint64_t hit = __ballot(valid && key == best);
  const float zb = __shfl(z, hit ? (int)__builtin_ctzll(hit) : 0);
  const float mu = wave_max(valid ? z : -INFINITY);
  const float S = wave_sum(valid ? __expf(z - mu) : 0.f);
  if (lane == 0) {
    publish_u64(a.tile_keys + (size_t)m * a.tiles + tile, best);
    publish_u64(a.tile_z + (size_t)m * a.tiles + tile, __float_as_uint(zb));
    publish_u64(a.tile_ms + (size_t)m * a.tiles + tile, pack_ms(mu, S));
  }
}


typedef float f32x4 __attribute__((ext_vector_type(4)));

// The same draw for the 16 draft rows m0 + r16 that a wave holds in the
// MFMA accumulator layout: lane (g, r16) has z[rb][i], the logit of draft
// row m0 + r16 at tile row trow0 + 16 rb + 4 g + i, and fid[rb][i], that
// row's full id. The four lanes r16 = 4 q .. 4 q + 3 of one g (a quad)
// share the Philox block (m0 + r16) / 4 and the same 16 tile rows: quad
// lane r makes the calls of the tile rows (rb, i = r), whose word s is the
// variate of the block's draft row s, and three exchanges within the quad
// (exchange k: send word r ^ k, receive from lane r ^ k) give every lane
// its own row's variates. Each lane reduces its draft row over its 16 tile
// rows and two cross-lane steps combine the four lanes of a row. m0 is a
// multiple of 16; every lane of the wave must call it.
__device__ __forceinline__ uint32_t pick4(u32x4 w, int i) {
  return i == 0 ? w[0] : i == 1 ? w[1] : i == 2 ? w[2] : w[3];
}

// The Gumbel variates of the quad-transposed draw: lane (g, r16) gets, for
// each 16-row block rb and exchange k, the variate of draft row m0 + r16 at
// tile row trow0 + 16 rb + 4 g + (r16 % 4 ^ k). Each quad lane draws the
// Philox block of four draft rows at one of the quad's four tile rows, and
// three exchanges within the quad (exchange k: send word r ^ k, receive from
// lane r ^ k) hand every lane its own row's variates. They depend on nothing
// but the seed, the offset and the indices, so a caller may draw them ahead.
__device__ __forceinline__ void gumbel_quad(const HeadArgs &a, int m0, int trow0,
                                            float (&gq)[4][4]) {
  const int lane = __lane_id(), g = lane >> 4, r16 = lane & 15, qr = r16 & 3;
  const int m = m0 + r16;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const u32x4 w = gumbel_words(a.seed_lo, a.seed_hi, a.off_lo, a.off_hi, (uint32_t)(m >> 2),
                                 trow0 + 16 * rb + 4 * g + qr);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = k == 0 ? pick4(w, qr) : (uint32_t)__shfl_xor((int)pick4(w, qr ^ k), k);
      gq[rb][k] = gumbel_from_word(x);
    }
  }
}

// kPre: the variates come in gq (from gumbel_quad), else they are drawn here.
template <bool kPre = false>
__device__ __forceinline__ void quad_draw_publish(const HeadArgs &a, int m0, int tile,
                                                  int trow0, const f32x4 (&z)[4],
                                                  const int32_t (&fid)[4][4],
                                                  const float (*gpre)[4] = nullptr) {
  const int lane = __lane_id(), g = lane >> 4, r16 = lane & 15, qr = r16 & 3;
  const int m = m0 + r16;
  auto pickf = [](f32x4 w, int i) -> float {
    return i == 0 ? w[0] : i == 1 ? w[1] : i == 2 ? w[2] : w[3];
  };
  float gq[4][4];
  if constexpr (kPre) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int k = 0; k < 4; ++k) gq[rb][k] = gpre[rb][k];
  } else {
    gumbel_quad(a, m0, trow0, gq);
  }
  uint64_t best = 0;
  float zb = 0.f, mu = -INFINITY;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = qr ^ k;  // tile row (rb, i) of this variate
      const int32_t f = i == 0 ? fid[rb][0] : i == 1 ? fid[rb][1] : i == 2 ? fid[rb][2]
                                                                          : fid[rb][3];
      const float zv = pickf(z[rb], i);
      if (trow0 + 16 * rb + 4 * g + i < a.V_high) {
        const uint64_t key = make_key(zv + gq[rb][k], f);
        if (key > best) {
          best = key;
          zb = zv;
        }
        mu = fmaxf(mu, zv);
      }
    }
  }
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
    const uint64_t ob = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), x) << 32) |
                        (uint32_t)__shfl_xor((int)(uint32_t)best, x);
    const float oz = __shfl_xor(zb, x);
    if (ob > best) {
      best = ob;
      zb = oz;
    }
    mu = fmaxf(mu, __shfl_xor(mu, x));
  }
  float S = 0.f;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (trow0 + 16 * rb + 4 * g + i < a.V_high) S += __expf(z[rb][i] - mu);
  S += __shfl_xor(S, 16);
  S += __shfl_xor(S, 32);
  if (g == 0 && m < a.M) {
    publish_u64(a.tile_keys + (size_t)m * a.tiles + tile, best);
    publish_u64(a.tile_z + (size_t)m * a.tiles + tile, __float_as_uint(zb));
    publish_u64(a.tile_ms + (size_t)m * a.tiles + tile, pack_ms(mu, S));
  }
}

constexpr int kMaxTiles = VT_VHIGH_MAX / kTileRows;

constexpr int kCandCap = 4096;   // survivors the final merge can hold (every logit of 64 tiles)

template <int WAVES>
struct alignas(16) MergeShared {
  alignas(16) uint64_t cand[kCandCap];       // survivors of the threshold
  alignas(16) uint64_t sc[2][kWave];         // rank inputs / outputs
  uint32_t prank[4][4][kWave];               // partial ranks
  uint32_t gm[WAVES][kWave];                 // per-wave maxima of the tile groups
  unsigned long long kmax;
  uint32_t cnt;
  float f[WAVES], f2[WAVES], zw[WAVES];
};

// Ranks (0 = largest) of NR rows of 64 keys in LDS, keys[r * 64 + lane],
// counted by up to 4 waves per row: wave w takes row w % NR and a quarter
// (half, whole) of the keys to compare against, so the latency of a rank
// is that of 16 to 64 compares. Keys must be distinct apart from 0. Every
// thread must call it (it has a barrier); the rank of keys[w * 64 + lane]
// is returned to wave w < NR.
template <int WAVES, int NR>
__device__ __forceinline__ uint32_t block_rank(const uint64_t *keys,
                                               uint32_t *prank) {
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  constexpr int P = (WAVES / NR) < 4 ? (WAVES / NR) : 4;
  constexpr int SPAN = kWave / P;
  static_assert(P >= 1 && SPAN % 2 == 0, "parts must split 64 keys evenly");
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  if (wave < NR * P) {
    const int r = wave % NR, part = wave / NR;
    const uint64_t v = keys[r * kWave + lane];
    const uint64_t *kr = keys + r * kWave + part * SPAN;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < SPAN; j += 2) {
      const u64x2 q = *reinterpret_cast<const u64x2 *>(kr + j);
      c += q.x > v;
      c += q.y > v;
    }
    prank[(part * NR + r) * kWave + lane] = c;
  }
  __syncthreads();
  uint32_t rank = 0;
  if (wave < NR)
#pragma unroll
    for (int p = 0; p < P; ++p) rank += prank[(p * NR + wave) * kWave + lane];
  return rank;
}

// Survivors collected with an LDS counter, one key at a time.
__device__ __forceinline__ void offer(uint64_t v, uint64_t T, uint64_t *cand,
                                      uint32_t *cnt) {
  if (v != 0ull && v >= T) {
    const uint32_t pos = atomicAdd(cnt, 1u);
    if (pos < (uint32_t)kCandCap) cand[pos] = v;
  }
}

// Sorts cand[0, n) descending in place (n <= kCandCap) with a bitonic
// network over the workgroup; only used when many keys tie above the bound.
template <int WAVES>
__device__ void block_sort_desc(uint64_t *cand, uint32_t n) {
  constexpr int NT = WAVES * kWave;
  uint32_t P = 2;
  while (P < n) P <<= 1;
  for (uint32_t i = n + threadIdx.x; i < P; i += NT) cand[i] = 0;
  __syncthreads();
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t i = threadIdx.x; i < P / 2; i += NT) {
        const uint32_t lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const uint64_t x = cand[lo], y = cand[hi];
        if ((x < y) == ((lo & size) == 0)) {
          cand[lo] = y;
          cand[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Final merge for draft row m, run by the whole last workgroup after one
// round of loads of the published tile partials:
//   * softmax: global max of the tile maxima, then the sum of the tile sums
//     rescaled to it, in a fixed order (no dependence on timing);
//   * picks: the k-th largest key overall is at least T, the larger of the
//     largest tile k-th key and the k-th largest of the 64 tile-group
//     maxima (both are k-th largest keys of sets of real candidates; the
//     tiles fold them in with atomic max). Keys >= T, typically a few
//     dozen, are collected in LDS and ranked. With more than 64 survivors
//     (exact ties, large k) a workgroup sort or, past kCandCap, k exact
//     max rounds take over.
// Sampling-mode merge of draft row m: the largest published key (the draw)
// with its row's z, and the softmax max and sum over the tile partials in a
// fixed order; full_ids[m] and probs[m] = exp(z - max) / sum.
template <int WAVES>
__device__ void sample_merge(const HeadArgs &a, int m, MergeShared<WAVES> &sh) {
  constexpr int NT = WAVES * kWave;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int tiles = a.tiles;
  const uint64_t *keys = a.tile_keys + (size_t)m * tiles;
  const uint64_t *zs = a.tile_z + (size_t)m * tiles;
  const uint64_t *ms = a.tile_ms + (size_t)m * tiles;
  // The thread's tiles t = tid + j NT in index order (uniform bound on j):
  // keys and their z, and the softmax partials, relative to the thread's
  // own max and then to the wave's.
  constexpr int kB = 4;
  const int tpt = (tiles + NT - 1) / NT;
  uint64_t best = 0;
  float zb = 0.f, mu_l = -INFINITY, s_l = 0.f;
  for (int base = 0; base < tpt; base += kB) {
    uint64_t kv[kB], zv[kB], mv[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      kv[j] = zv[j] = mv[j] = 0ull;
      const int t = tid + (base + j) * NT;
      if (base + j < tpt && t < tiles) {
        kv[j] = fetch_u64(keys + t);
        zv[j] = fetch_u64(zs + t);
        mv[j] = fetch_u64(ms + t);
      }
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (kv[j] > best) {
        best = kv[j];
        zb = __uint_as_float((uint32_t)zv[j]);
      }
      if (base + j < tpt && tid + (base + j) * NT < tiles) {
        const float mj = ms_max(mv[j]);
        if (mj > mu_l) {
          s_l = s_l * __expf(mu_l - mj) + ms_sum(mv[j]);
          mu_l = mj;
        } else {
          s_l += ms_sum(mv[j]) * __expf(mj - mu_l);
        }
      }
    }
  }
  const float mu_w = wave_max(mu_l);
  if (mu_l != -INFINITY) s_l *= __expf(mu_l - mu_w);
  const float s_w = wave_sum(s_l);
  const uint64_t bw = wave_max_u64(best);
  const uint64_t hit = __ballot(best == bw && bw != 0ull);
  const float zw = __shfl(zb, hit ? (int)__builtin_ctzll(hit) : 0);
  if (lane == 0) {
    sh.sc[0][wave] = bw;
    sh.f[wave] = mu_w;
    sh.f2[wave] = s_w;
    sh.zw[wave] = zw;
  }
  __syncthreads();
  if (tid == 0) {
    float mu = sh.f[0];
    for (int w = 1; w < WAVES; ++w) mu = fmaxf(mu, sh.f[w]);
    float S = 0.f;
    uint64_t kbest = 0;
    float z = 0.f;
    for (int w = 0; w < WAVES; ++w) {
      if (sh.f[w] != -INFINITY) S += sh.f2[w] * __expf(sh.f[w] - mu);
      if (sh.sc[0][w] > kbest) {
        kbest = sh.sc[0][w];
        z = sh.zw[w];
      }
    }
    a.full_ids[m] = key_id(kbest);
    if (a.probs) a.probs[m] = __expf(z - mu) / S;
  }
  __syncthreads();  // sh is reused by the next draft row's merge
}

// Final merge over the published tile partials of draft row m, by the
// first WAVES waves of the last workgroup (SW waves share its LDS):
//   * softmax: global max of the tile maxima, then the sum of the tile sums
//     rescaled to it, in a fixed order (no dependence on timing);
//   * picks: the k-th largest key overall is at least T, the larger of the
//     largest tile k-th key and the k-th largest of the 64 tile-group
//     maxima (both are k-th largest keys of sets of real candidates; the
//     tiles fold them in with atomic max). Keys >= T, typically a few
//     dozen, are collected in LDS and ranked. With more than 64 survivors
//     (exact ties, large k) a workgroup sort or, past kCandCap, k exact
//     max rounds take over.
template <int WAVES, int SW>
__device__ void final_merge(const HeadArgs &a, int m, MergeShared<SW> &sh) {
  constexpr int NT = WAVES * kWave;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int k = a.k, tiles = a.tiles;
  const uint64_t *keys = a.tile_keys + (size_t)m * tiles * k;
  const uint64_t *ms = a.tile_ms + (size_t)m * tiles;
  uint64_t *gmax = a.group_max + (size_t)m * kGroups;
  uint64_t *gkth = a.group_kth + (size_t)m * kGroups;
  const int n = tiles * k;

  // One round of loads: two batches of keys, the tile softmax partials and
  // the group maxima.
  constexpr int kBatch = 8;
  uint64_t kb[2][kBatch];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int f = tid + (b * kBatch + j) * NT;
      kb[b][j] = f < n ? fetch_u64(keys + f) : 0ull;
    }
  constexpr int kTpt = (kMaxTiles + NT - 1) / NT;  // tiles per thread
  uint64_t mst[kTpt];
#pragma unroll
  for (int j = 0; j < kTpt; ++j) {
    const int t = tid + j * NT;
    mst[j] = t < tiles ? fetch_u64(ms + t) : 0ull;
  }
  uint64_t g = 0, gk = 0;
  if (wave == 0) {
    g = fetch_u64(gmax + lane);
    gk = fetch_u64(gkth + lane);
  }
  float mu_l = -INFINITY;
#pragma unroll
  for (int j = 0; j < kTpt; ++j)
    if (tid + j * NT < tiles) mu_l = fmaxf(mu_l, ms_max(mst[j]));
  const float mu_w = wave_max(mu_l);
  if (wave == 0) {
    sh.sc[0][lane] = g;
    sh.kmax = wave_max_u64(gk);
  }
  if (lane == 0) sh.f[wave] = mu_w;
  if (tid == 0) sh.cnt = 0;
  __syncthreads();
  float mu = sh.f[0];
  for (int w = 1; w < WAVES; ++w) mu = fmaxf(mu, sh.f[w]);
  // Rank of each group maximum (distinct keys, 0 for an empty group): every
  // wave counts the larger keys among its 64 / WAVES of them; after the
  // barrier every wave sums the partial counts and forms T itself.
  constexpr int kSpan = kWave / WAVES;
  static_assert(kSpan * WAVES == kWave && WAVES <= 16, "group keys split evenly over the waves");
  const uint64_t gkey = sh.sc[0][lane];
  uint32_t gc = 0;
#pragma unroll
  for (int j = 0; j < kSpan; ++j) gc += sh.sc[0][wave * kSpan + j] > gkey;
  uint32_t *prank = &sh.prank[0][0][0];
  prank[wave * kWave + lane] = gc;
  __syncthreads();  // partial ranks ready; all reads of sh.f done
  uint64_t T;
  {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) r += prank[w * kWave + lane];
    const uint64_t hit = __ballot(r == (uint32_t)(k - 1) && gkey != 0ull);
    T = max_u64(hit ? readlane_u64(gkey, __builtin_ctzll(hit)) : 0ull, sh.kmax);
  }
  if (wave == 0) {  // g and gk are in registers: reset the maxima for the next call
    publish_u64(gmax + lane, 0ull);
    publish_u64(gkth + lane, 0ull);
  }
  float s_l = 0.f;
#pragma unroll
  for (int j = 0; j < kTpt; ++j)
    if (tid + j * NT < tiles) s_l += ms_sum(mst[j]) * __expf(ms_max(mst[j]) - mu);
  const float s_w = wave_sum(s_l);
  if (lane == 0) sh.f[wave] = s_w;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < kBatch; ++j) offer(kb[b][j], T, sh.cand, &sh.cnt);
  for (int base = 2 * kBatch * NT; base < n; base += kBatch * NT) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int f = base + tid + j * NT;
      kb[0][j] = f < n ? fetch_u64(keys + f) : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) offer(kb[0][j], T, sh.cand, &sh.cnt);
  }
  __syncthreads();
  const uint32_t found = sh.cnt;
  float S = sh.f[0];
  for (int w = 1; w < WAVES; ++w) S += sh.f[w];
  uint64_t key = 0;  // rank `tid` for tid < k
  if (found <= (uint32_t)kWave) {
    // Wave 0 ranks the few survivors against each other (a loop over the
    // survivors only) and writes each one to its output slot; at least k
    // keys survive because T is at most the k-th largest key.
    if (wave == 0) {
      const uint64_t v = lane < (int)found ? sh.cand[lane] : 0ull;
      uint32_t r = 0;
      for (uint32_t j = 0; j < found; ++j) r += sh.cand[j] > v;
      if (lane < (int)found && r < (uint32_t)k) {
        a.full_ids[(size_t)m * k + r] = key_id(v);
        a.probs[(size_t)m * k + r] = __expf(key_logit(v) - mu) / S;
      }
    }
    __syncthreads();  // sh is reused by the next draft row's merge
    return;
  } else if (found <= (uint32_t)kCandCap) {
    block_sort_desc<WAVES>(sh.cand, found);
    if (wave == 0) key = sh.cand[lane];
  } else {
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
      for (int f = tid; f < n; f += NT) {
        const uint64_t v = fetch_u64(keys + f);
        if (v < prev) best = max_u64(best, v);
      }
      best = wave_max_u64(best);
      __syncthreads();
      if (tid == 0) sh.kmax = 0;
      __syncthreads();
      if (lane == 0) atomicMax(&sh.kmax, (unsigned long long)best);
      __syncthreads();
      best = sh.kmax;
      if (tid == r) key = best;
      prev = best;
    }
  }
  if (tid < k) {
    a.full_ids[(size_t)m * k + tid] = key_id(key);
    a.probs[(size_t)m * k + tid] = __expf(key_logit(key) - mu) / S;
  }
  __syncthreads();
}

// GEMV workgroups. Within a CU the memory pipeline serves the oldest waves
// first, so of two workgroups sharing a CU one finishes long before the
// other, and for the rest of the call that CU has half as many rows in
// flight; the XCDs then no longer get equal shares of the bandwidth, and
// two or three of them finish several microseconds after the others. A CU
// therefore runs one workgroup of 16 waves over a block of two 64-row tiles,
// and its waves take the block's rows one at a time from an LDS counter, so
// that all 16 keep loading until the block's rows run out. Where 16 waves
// would not fit in the registers (long rows with two draft rows) the
// workgroups have 8 waves and one tile each. Each tile's partial (top-k keys,
// softmax partial) is published as before.
// Several draft rows, R = min(rows, workgroups) mergers: the workgroup with
// the q-th ticket from the end (q = 0: the last to arrive) merges rows q,
// q + R, ...; all but the last first wait until every workgroup has arrived
// (a bounded wait: the mergers are resident and no other workgroup waits,
// so it ends within microseconds). Every thread must call it (it has a
// barrier).
constexpr uint32_t kArriveWaitMax = 1u << 20;

// Waits until n workgroups have taken a ticket. Returns false if it gave up
// (after kArriveWaitMax sleeps, or the workspace's spin-limit word when that
// is nonzero); it then raises the workspace's error word, which
// vt_draft_head_status reports. The workspace's hold word, zero unless a
// test sets it, adds that many arrivals that never come. Every thread must
// call it (it has a barrier); the result is uniform.
__device__ __forceinline__ bool wait_arrivals(const HeadArgs &a, uint32_t n, uint32_t *s_ok) {
  if (threadIdx.x == 0) {
    const uint32_t hold = a.status[kWsHold / 4];
    const uint32_t lim = a.status[kWsSpinLimit / 4] ? a.status[kWsSpinLimit / 4] : kArriveWaitMax;
    const uint32_t want = n + hold;
    uint32_t spins = 0;
    bool ok;
    while (!(ok = __hip_atomic_load(a.counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                  want) &&
           ++spins < lim)
      __builtin_amdgcn_s_sleep(2);
    if (!ok)
      __hip_atomic_store(a.status + kWsError / 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_ok = ok ? 1u : 0u;
  }
  __syncthreads();
  return *s_ok != 0;
}

// Outputs of a draft row whose merge could not be trusted: id -1, NaN
// probabilities (k entries, or one when sampling).
__device__ __forceinline__ void write_sentinel(const HeadArgs &a, int m) {
  const int n = a.sample ? 1 : a.k;
  for (int r = threadIdx.x; r < n; r += blockDim.x) {
    a.full_ids[(size_t)m * n + r] = -1;
    if (a.probs) a.probs[(size_t)m * n + r] = __builtin_nanf("");
  }
}

// The last of R mergers to finish returns the ticket counter (and the count
// of finished mergers) to zero: only then has every merger seen the count
// of arrivals it waited for.
__device__ __forceinline__ void finish_merge(const HeadArgs &a, int R) {
  if (threadIdx.x != 0) return;
  if (R == 1 || __hip_atomic_fetch_add(a.merged, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)R - 1) {
    if (R > 1) reset_counter(a.merged);
    reset_counter(a.counter);
  }
}

template <int MT, int CPL>
constexpr int gemv_waves() {
  return (CPL <= 8 || (MT == 1 && CPL <= 12)) ? 16 : 8;
}

template <int WAVES, int MT, int CPL, bool RAGGED, bool LOGITS>
__global__ __launch_bounds__(WAVES *kWave) void head_gemv_kernel(HeadArgs a) {
  // Rows per wave and step: short rows (small d) take several per step so
  // that about 8 loads per lane are in flight; from 6 loads per row on, one
  // row per step measured best.
  constexpr int U = CPL >= 6 ? 1 : CPL >= 3 ? 2 : CPL == 2 ? 4 : 8;
  constexpr int kTiles = WAVES / 8;            // 64-row tiles per workgroup
  constexpr int kRows = kTiles * kTileRows;
  static_assert(kRows % U == 0, "units must split the block evenly");
  static_assert(kTiles * MT <= WAVES, "one wave per (tile, draft row) in the epilogue");
  __shared__ float s_z[MT][kRows];
  __shared__ MergeShared<WAVES> sh;
  __shared__ uint32_t s_slot, s_next, s_ok;

  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int tile0 = blockIdx.x * kTiles, row0 = tile0 * kTileRows;
  const int c16 = a.c16;
  // Units of U rows in this block (the last block may be short).
  const int units = (min(kRows, a.V_high - row0) + U - 1) / U;

  // Epilogue roles: wave e = sub * MT + m takes tile tile0 + sub, draft row m.
  const int e_sub = wave / MT, e_m = wave % MT;
  const bool e_on = wave < kTiles * MT && tile0 + e_sub < a.tiles;
  const int e_row = row0 + e_sub * kTileRows + lane;
  int32_t fid = 0;
  if (!LOGITS && e_on && e_row < a.V_high) fid = fid_at(a, e_row);

  if (threadIdx.x == 0) s_next = WAVES;  // unit w < WAVES is wave w's first
  __syncthreads();

  u32x4 hr[MT][CPL];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int idx = c * kWave + lane;
      hr[m][c] = (!RAGGED || idx < c16) ? a.h[(size_t)m * c16 + idx]
                                        : u32x4{0, 0, 0, 0};
    }

#pragma unroll 1
  for (int u0 = wave; u0 < units;) {
    const int rl = u0 * U;  // first block-local row of the unit
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
    uint32_t next = 0;
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
      next = atomicAdd(&s_next, 1u);
    }
    u0 = (int)__builtin_amdgcn_readfirstlane(next);
  }
  if (LOGITS) return;
  __syncthreads();

  const int tile = tile0 + e_sub;
  const bool valid = e_on && e_row < a.V_high;
  // Wave e works on draft row e_m of tile `tile`: its logit of tile row
  // `lane`, with the head's bias when it has one.
  float zl = 0.f;
  if (e_on) {
    zl = s_z[e_m][e_sub * kTileRows + lane];
    if (a.bias && valid) zl += bf16_to_f32(a.bias[e_row]);
  }
  if (a.sample) {  // one draw per draft row
    if (e_on)
      wave_publish_sample(a, e_m, tile, zl,
                          gumbel(a.seed_lo, a.seed_hi, a.off_lo, a.off_hi, e_m, e_row),
                          fid, valid);
    const uint32_t ticket = arrive(a.counter, &s_slot);
    if (MT == 1) {
      if (ticket != gridDim.x - 1) return;
      sample_merge<WAVES>(a, 0, sh);
      if (threadIdx.x == 0) reset_counter(a.counter);
      return;
    }
    const int R = min(MT, (int)gridDim.x), q = (int)gridDim.x - 1 - (int)ticket;
    if (q >= R) return;
    const bool ok = q == 0 || wait_arrivals(a, gridDim.x, &s_ok);
    for (int m = q; m < MT; m += R) {
      if (ok)
        sample_merge<WAVES>(a, m, sh);
      else
        write_sentinel(a, m);
    }
    finish_merge(a, R);
    return;
  }

  // Tile partials: top-k keys and softmax partial of each (tile, draft row).
  constexpr int NR = kTiles * MT;
  const int k = a.k;
  uint64_t *s_key = sh.cand;               // [NR][64] keys of the tiles
  uint64_t *s_top = sh.cand + NR * kWave;  // [NR][64] ranked keys
  if (wave < NR) {
    s_key[wave * kWave + lane] = valid ? make_key(zl, fid) : 0ull;
    s_top[wave * kWave + lane] = 0;
  }
  __syncthreads();
  const uint32_t rank = block_rank<WAVES, NR>(s_key, &sh.prank[0][0][0]);
  if (e_on) {
    const int m = e_m;
    if (rank < (uint32_t)k) s_top[wave * kWave + rank] = s_key[wave * kWave + lane];
    __builtin_amdgcn_wave_barrier();
    const uint64_t key = s_top[wave * kWave + lane];
    const float mu = key_logit(s_top[wave * kWave]);
    const float S = wave_sum(valid ? __expf(zl - mu) : 0.f);
    if (lane < k) publish_u64(a.tile_keys + ((size_t)m * a.tiles + tile) * k + lane, key);
    if (lane == 0) {
      publish_u64(a.tile_ms + (size_t)m * a.tiles + tile, pack_ms(mu, S));
      const int grp = tile / a.tiles_per_group;
      __hip_atomic_fetch_max(a.group_max + (size_t)m * kGroups + grp,
                             s_top[wave * kWave], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(a.group_kth + (size_t)m * kGroups + grp,
                             s_top[wave * kWave + k - 1], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // The last workgroup to finish merges every tile's partial; with two
  // draft rows the one before it takes the second row at the same time.
  // The merge is latency-bound: past 8 waves more waves only add work.
  const uint32_t ticket = arrive(a.counter, &s_slot);
  constexpr int MW = WAVES < 8 ? WAVES : 8;
  if (MT == 1) {
    if (ticket != gridDim.x - 1) return;
    if (threadIdx.x == 0) reset_counter(a.counter);
    if (wave >= MW) return;
    final_merge<MW, WAVES>(a, 0, sh);
    return;
  }
  const int R = min(MT, (int)gridDim.x), q = (int)gridDim.x - 1 - (int)ticket;
  if (q >= R || wave >= MW) return;
  const bool ok = q == 0 || wait_arrivals(a, gridDim.x, &s_ok);
  for (int m = q; m < MT; m += R) {
    if (ok)
      final_merge<MW, WAVES>(a, m, sh);
    else
      write_sentinel(a, m);
  }
  finish_merge(a, R);
}

// Top-k merge of the MFMA path, one workgroup per draft row m, from the
// tiles' softmax partials and the logits in the workspace:
//   * the softmax max and sum over the row come from the tile partials,
//     combined in a fixed order;
//   * each tile's max is a logit of that tile, so the k-th largest of the
//     maxima of 64 disjoint groups of tiles (with multiplicity) is at most
//     the row's k-th largest logit: only tiles whose max reaches it can hold
//     a pick, typically k to 2k of them;
//   * the logits of those tiles at or above the bound become keys in LDS
//     and are ranked as in the tile merge.
// The partials and logits were written by an earlier kernel.
template <int WAVES>
__device__ void row_merge(const HeadArgs &a, int m, MergeShared<WAVES> &sh, int32_t *s_tiles,
                          uint32_t &s_ntiles) {
  constexpr int NT = WAVES * kWave;
  constexpr int kTpt = (kMaxTiles + NT - 1) / NT;  // tiles per thread
  static_assert(NT % kGroups == 0, "a thread's tiles share its group");
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int k = a.k, V = a.V_high, tiles = a.tiles;
  const uint64_t *ms = a.tile_ms + (size_t)m * tiles;
  const float *zr = a.zbuf + (size_t)m * a.zpitch;

  // Slots past the tile count are skipped by uniform branches (a load
  // instruction costs issue time even with no lane active).
  const int tpt = (tiles + NT - 1) / NT;
  uint64_t mst[kTpt];
#pragma unroll
  for (int j = 0; j < kTpt; ++j) {
    const int t = tid + j * NT;
    mst[j] = 0ull;
    if (j < tpt && t < tiles) mst[j] = ms[t];
  }
  float mu_l = -INFINITY;
#pragma unroll
  for (int j = 0; j < kTpt; ++j)
    if (j < tpt && tid + j * NT < tiles) mu_l = fmaxf(mu_l, ms_max(mst[j]));
  // Tile t belongs to group t mod 64, the lane of the thread that holds it:
  // every group has a tile once there are 64, and up to 64 tiles each tile
  // is a group of its own, so whenever there are k tiles the k-th largest
  // group maximum is a logit that bounds the row's k-th largest from below.
  // (Groups of consecutive threads instead left most groups empty on small
  // heads or with large k, and the bound fell to zero.)
  sh.gm[wave][lane] = mu_l == -INFINITY ? 0u : ord_from_f32(mu_l);
  const float mw = wave_max(mu_l);
  if (lane == 0) sh.f[wave] = mw;
  if (tid == 0) {
    sh.cnt = 0;
    s_ntiles = 0;
  }
  __syncthreads();
  float mu = sh.f[0];
  for (int w = 1; w < WAVES; ++w) mu = fmaxf(mu, sh.f[w]);
  float s_l = 0.f;
#pragma unroll
  for (int j = 0; j < kTpt; ++j)
    if (j < tpt && tid + j * NT < tiles) s_l += ms_sum(mst[j]) * __expf(ms_max(mst[j]) - mu);
  const float sw = wave_sum(s_l);
  if (lane == 0) sh.f2[wave] = sw;
  // Group maxima as distinct keys (max, then 64 - group): the key of rank
  // k - 1 holds the k-th largest maximum counted with multiplicity. Every
  // wave forms all 64 keys (lane = group); each counts the larger keys among
  // 64 / WAVES of them; after the barrier every wave sums the partial
  // counts and takes the key of rank k - 1.
  uint32_t gmx = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) gmx = max(gmx, sh.gm[w][lane]);
  const uint64_t gkey = ((uint64_t)gmx << 32) | (uint32_t)(kWave - lane);
  constexpr int kSpan = kWave / WAVES;
  static_assert(kSpan * WAVES == kWave && WAVES <= 16, "group keys split evenly over the waves");
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kSpan; ++j) c += readlane_u64(gkey, wave * kSpan + j) > gkey;
  uint32_t *prank = &sh.prank[0][0][0];
  prank[wave * kWave + lane] = c;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) r += prank[w * kWave + lane];
  const uint64_t hit = __ballot(r == (uint32_t)(k - 1));
  const uint32_t T = hit ? (uint32_t)(readlane_u64(gkey, __builtin_ctzll(hit)) >> 32) : 0u;
  float S = sh.f2[0];
  for (int w = 1; w < WAVES; ++w) S += sh.f2[w];
#pragma unroll
  for (int j = 0; j < kTpt; ++j) {
    const int t = tid + j * NT;
    if (j < tpt && t < tiles && ord_from_f32(ms_max(mst[j])) >= T)
      s_tiles[atomicAdd(&s_ntiles, 1u)] = t;
  }
  __syncthreads();
  const int ne = (int)s_ntiles * kTileRows;  // candidate logits
  constexpr int kRound = 4;
  for (int base = 0; base < ne; base += kRound * NT) {
    float zv[kRound];
    int jv[kRound];
    int32_t fv[kRound];
    // The full ids are loaded beside the logits (one round trip to memory
    // instead of a second one for the survivors).
#pragma unroll
    for (int i = 0; i < kRound; ++i) {
      const int e = base + i * NT + tid;
      jv[i] = e < ne ? s_tiles[e / kTileRows] * kTileRows + e % kTileRows : V;
      zv[i] = jv[i] < V ? zr[jv[i]] : 0.f;
      fv[i] = jv[i] < V ? fid_at(a, jv[i]) : 0;
    }
#pragma unroll
    for (int i = 0; i < kRound; ++i)
      if (jv[i] < V && ord_from_f32(zv[i]) >= T) {
        const uint32_t pos = atomicAdd(&sh.cnt, 1u);
        if (pos < (uint32_t)kCandCap) sh.cand[pos] = make_key(zv[i], fv[i]);
      }
  }
  __syncthreads();
  const uint32_t found = sh.cnt;
  uint64_t key = 0;  // rank `tid` for tid < k
  if (found <= (uint32_t)kWave) {
    if (wave == 0) {
      const uint64_t x = lane < (int)found ? sh.cand[lane] : 0ull;
      uint32_t r = 0;
      for (uint32_t j = 0; j < found; ++j) r += sh.cand[j] > x;
      if (lane < (int)found && r < (uint32_t)k) {
        a.full_ids[(size_t)m * k + r] = key_id(x);
        a.probs[(size_t)m * k + r] = __expf(key_logit(x) - mu) / S;
      }
    }
    __syncthreads();  // sh is reused by the next row's merge
    return;
  } else if (found <= (uint32_t)kCandCap) {
    block_sort_desc<WAVES>(sh.cand, found);
    if (tid < k) key = sh.cand[tid];
  } else {
    // Massive exact ties: k rounds of "largest key below the previous one"
    // over the candidate logits.
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
      for (int e = tid; e < ne; e += NT) {
        const int j = s_tiles[e / kTileRows] * kTileRows + e % kTileRows;
        if (j < V) {
          const float z = zr[j];
          if (ord_from_f32(z) >= T) {
            const uint64_t kv = make_key(z, fid_at(a, j));
            if (kv < prev) best = max_u64(best, kv);
          }
        }
      }
      best = wave_max_u64(best);
      __syncthreads();
      if (tid == 0) sh.kmax = 0;
      __syncthreads();
      if (lane == 0) atomicMax(&sh.kmax, (unsigned long long)best);
      __syncthreads();
      best = sh.kmax;
      if (tid == r) key = best;
      prev = best;
    }
  }
  if (tid < k) {
    a.full_ids[(size_t)m * k + tid] = key_id(key);
    a.probs[(size_t)m * k + tid] = __expf(key_logit(key) - mu) / S;
  }
  __syncthreads();  // sh is reused by the next row's merge
}

// ---------------------------------------------------------------- MFMA path
// Draft trees and batches (M = 3..512 rows): the head is a skinny GEMM, z^T = W_trim h^T.
// v_mfma_f32_16x16x32_bf16 takes 16 W rows as the A operand and 16 draft rows
// as the B operand; lane l supplies 16 bytes (8 k-values) of row l % 16 at
// k-chunk 4 s + l / 16 of k-step s, the same chunk for A and B, and receives
// C[4 (l / 16) + r][l % 16] in accumulator register r. A workgroup owns a
// tile of 64 W rows; its 4 waves split d into contiguous k ranges, stream
// their slices of W once (16 KiB per wave in flight) and read h from L2. The
// partial products are summed over the waves in a fixed order in LDS. For
// top-k the tile's logits go to the workspace and each draft row's softmax
// partial over the tile is published; tree_merge_kernel then finds each
// row's picks among the few tiles whose maximum can reach them. Ranking
// inside every tile instead (as the GEMV path does for one or two rows)
// costs hundreds of VALU instructions per (draft row, tile) pair, all of it
// issued after the streaming ends. Sampling publishes each tile's draw.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kMfmaWaves = 4;
// A logit buffer of this size or more is written with streaming stores: left
// dirty in the L2s it would be written back at the kernel's end, after the
// last tile, while streaming stores send it to memory during the
// contraction. Smaller buffers stay in L2 for the merge kernel that reads
// them back.
constexpr size_t kZStreamBytes = 6u << 20;
constexpr int kCpolNt = 2;                     // cache policy: non-temporal (streaming)
constexpr int kBufferRsrcWord3 = 0x00020000;   // raw 32-bit data, no swizzle
constexpr int kGroupRows = 32;  // draft rows of the 64-row kernel (2 column blocks)

// W is staged through wave-private LDS: the operand layout (16 rows x 64
// bytes per load) is slow to fetch from HBM directly, so each load
// instruction instead reads 4 rows x 256 contiguous bytes; rows are padded
// by 32 bytes in LDS so that the operand reads (16 rows at one chunk) are
// free of bank conflicts (measured with the LDS counters: 4 cycles per read
// instruction, against 8 with 16 bytes of padding).
constexpr int kStageChunks = 16;                      // 16-byte chunks per row and stage
constexpr int kStagePitch = kStageChunks + 2;         // row pitch in chunks
constexpr int kStageSize = kTileRows * kStagePitch;   // chunks per wave
constexpr int kPartPitch = kTileRows + 4;             // floats per partial-sum row

// Up to 32 draft rows on small heads, one workgroup per tile; each W tile is
// read once and streams past the caches (non-temporal loads; plain ones cost
// 4.5 us at M = 60 when this kernel also served 60 rows).
template <int NT>
__global__ __launch_bounds__(kMfmaWaves *kWave) __attribute__((amdgpu_waves_per_eu(2)))
void head_mfma_kernel(HeadArgs a) {
  union alignas(16) Smem {
    u32x4 stage[kMfmaWaves][kStageSize];
    float part[kMfmaWaves][NT * 16][kPartPitch];
  };
  __shared__ Smem sm;
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int tile = blockIdx.x;
  const int row0 = tile * kTileRows;
  const int M = a.M;  // draft rows, at most kGroupRows
  const int c16 = a.c16;
  const int g = lane >> 4, r16 = lane & 15;
  // This wave's contiguous range of 16-byte chunks (a multiple of 4).
  const int cq = ((c16 + kMfmaWaves - 1) / kMfmaWaves + 3) / 4 * 4;
  const int c_lo = min(c16, wave * cq), c_hi = min(c16, c_lo + cq);

  // W loads through a buffer resource over the tile's rows that exist (rows
  // past V_high read as zero): one per-lane byte offset plus a uniform
  // offset per group of 4 rows.
  const int vrows = min(kTileRows, a.V_high - row0);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(a.W + (size_t)row0 * c16), 0, vrows * c16 * 16, kBufferRsrcWord3);
  const int row4_bytes = 4 * c16 * 16;
  u32x4 *st = sm.stage[wave];

  f32x4 acc[4][NT];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < NT; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage loads: instruction q covers tile rows 4q .. 4q + 3, 256 bytes each.
  // Every load is issued (chunks past the wave's range re-read its last one
  // and are zeroed when staged), so the number of loads in flight is fixed.
  auto load_stage = [&](u32x4 (&v)[kStageChunks], int base) {
    const int off = (g * c16 + min(base + r16, c_hi - 1)) * 16;
#pragma unroll
    for (int q = 0; q < kStageChunks; ++q)
      v[q] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, q * row4_bytes,
                                                       kCpolNt));
  };
  // One stage: its loads (v) go to LDS, then the B operands of the whole
  // stage are loaded (contiguous loads from L2), then v is refilled with the
  // next stage, and per k-step the A operands come from LDS for the MFMAs.
  // The B loads go first so that the MFMAs wait for them only and not for
  // the next stage, which stays in flight through the stage's MFMAs. The
  // scheduling barriers keep the compiler from hoisting every A read.
  auto do_stage = [&](u32x4 (&v)[kStageChunks], int base, auto prefetch) {
    const bool in = base + r16 < c_hi;
#pragma unroll
    for (int q = 0; q < kStageChunks; ++q)
      st[(4 * q + g) * kStagePitch + r16] = in ? v[q] : u32x4{0, 0, 0, 0};
    __builtin_amdgcn_wave_barrier();
    u32x4 bv[kStageChunks / 4][NT];
#pragma unroll
    for (int t = 0; t < kStageChunks / 4; ++t) {
      // The B operands straight from h (16 rows x 64 bytes per load).
      const bool ok = base + 4 * t + g < c_hi;
      const int ch = base + 4 * t + g;
#pragma unroll
      for (int cb = 0; cb < NT; ++cb) {
        const int row = cb * 16 + r16;
        bv[t][cb] = (ok && row < M) ? a.h[(size_t)row * c16 + ch] : u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (decltype(prefetch)::value) load_stage(v, base + kStageChunks);
#pragma unroll
    for (int t = 0; t < kStageChunks / 4; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      const int cl = 4 * t + g;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const u32x4 av = st[(rb * 16 + r16) * kStagePitch + cl];
#pragma unroll
        for (int cb = 0; cb < NT; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv[t][cb]), acc[rb][cb],
              0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  u32x4 v[kStageChunks];
  if (c_lo < c_hi) {
    load_stage(v, c_lo);
    int base = c_lo;
#pragma unroll 1
    for (; base + kStageChunks < c_hi; base += kStageChunks)
      do_stage(v, base, std::true_type{});
    do_stage(v, base, std::false_type{});
  }
  __syncthreads();  // every wave is done with its stage before part[] reuses it

  // Partial products to LDS as [draft row][tile row] (rows padded to break
  // bank conflicts; each accumulator is 4 consecutive tile rows), then a
  // fixed-order sum over the waves into wave 0's slot.
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < NT; ++cb)
      *reinterpret_cast<f32x4 *>(&sm.part[wave][cb * 16 + r16][rb * 16 + 4 * g]) = acc[rb][cb];
  __syncthreads();
  // Top-k mode: the sums go straight to the logit buffer, which the row
  // merge reads; sampling mode keeps them in LDS for the tile epilogue.
  // Streaming stores go through a buffer resource over the draft rows from
  // this tile on (uniform base, per-lane byte offsets, bounds-checked).
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      a.zbuf + row0, 0,
      (int)(((size_t)M * a.zpitch - row0) * 4), kBufferRsrcWord3);
  for (int i = threadIdx.x; i < NT * 16 * (kTileRows / 4); i += kMfmaWaves * kWave) {
    const int row = i / (kTileRows / 4), c4 = 4 * (i % (kTileRows / 4));
    f32x4 val = *reinterpret_cast<const f32x4 *>(&sm.part[0][row][c4]);
#pragma unroll
    for (int w = 1; w < kMfmaWaves; ++w)
      val += *reinterpret_cast<const f32x4 *>(&sm.part[w][row][c4]);
    if (a.bias) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (row0 + c4 + c < a.V_high) val[c] += bf16_to_f32(a.bias[row0 + c4 + c]);
    }
    *reinterpret_cast<f32x4 *>(&sm.part[0][row][c4]) = val;
    if (!a.sample && row < M) {
      if (a.zstream)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), zrs,
                                               (row * a.zpitch + c4) * 4, 0, kCpolNt);
      else
        *reinterpret_cast<f32x4 *>(a.zbuf + (size_t)row * a.zpitch + row0 + c4) = val;
    }
  }
  __syncthreads();
  if (!a.sample) {
    // Softmax partial of each draft row over the tile, one lane per draft row:
    // wave q takes tile rows 16 q .. 16 q + 15, then wave 0 combines the four
    // quarters in a fixed order and publishes (max, sum of exp(z - max)).
    const int m = lane, q = wave;
    float mq = -INFINITY, sq = 0.f;
    if (m < M) {
      float zq[16];
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<f32x4 *>(&zq[i]) =
            *reinterpret_cast<const f32x4 *>(&sm.part[0][m][16 * q + i]);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (row0 + 16 * q + i < a.V_high) mq = fmaxf(mq, zq[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (row0 + 16 * q + i < a.V_high) sq += __expf(zq[i] - mq);
    }
    __syncthreads();  // every quarter has read part[0] before it is reused
    float *qm = &sm.part[1][0][0], *qs = &sm.part[2][0][0];
    qm[q * kWave + lane] = mq;
    qs[q * kWave + lane] = sq;
    __syncthreads();
    if (wave == 0 && m < M) {
      float mu = qm[lane];
#pragma unroll
      for (int w = 1; w < kMfmaWaves; ++w) mu = fmaxf(mu, qm[w * kWave + lane]);
      float S = 0.f;
#pragma unroll
      for (int w = 0; w < kMfmaWaves; ++w) {
        const float mw = qm[w * kWave + lane];
        if (mw != -INFINITY) S += qs[w * kWave + lane] * __expf(mw - mu);
      }
      a.tile_ms[(size_t)m * a.tiles + tile] = pack_ms(mu, S);
    }
  } else if (NT == 1) {
    // Sampling, up to 16 draft rows: per tile row (lane), draft rows in
    // blocks of four over the four waves; one Philox call per lane and block
    // gives the variates of all four rows.
    const bool valid = row0 + lane < a.V_high;
    const int32_t fid = valid ? fid_at(a, row0 + lane) : 0;
    for (int b = wave; 4 * b < M; b += kMfmaWaves) {
      const u32x4 x = gumbel_words(a.seed_lo, a.seed_hi, a.off_lo, a.off_hi, b, row0 + lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * b + r;
        if (m < M)
          wave_publish_sample(a, m, tile, sm.part[0][m][lane], gumbel_from_word(x[r]),
                              fid, valid);
      }
    }
  } else if (16 * wave < M) {
    // Sampling, more rows: wave w draws for the column block of draft rows
    // 16 w .. 16 w + 15, reading the tile's logits (bias included) back from
    // LDS in the accumulator layout for the quad-transposed draw (with one
    // block the per-row draw above spreads the rows over all four waves).
    f32x4 z[4];
    int32_t fid[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      z[rb] = *reinterpret_cast<const f32x4 *>(&sm.part[0][16 * wave + r16][16 * rb + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + 16 * rb + 4 * g + i;
        fid[rb][i] = row < a.V_high ? fid_at(a, row) : 0;
      }
    }
    quad_draw_publish(a, 16 * wave, tile, row0, z, fid);
  }
}



// Sampling mode: one workgroup per draft row merges the published tile
// partials.
template <int WAVES>
__global__ __launch_bounds__(WAVES *kWave) void head_merge_kernel(HeadArgs a) {
  __shared__ MergeShared<WAVES> sh;
  sample_merge<WAVES>(a, blockIdx.x, sh);
}

constexpr int kTreeWaves = 8;

// Top-k mode of the MFMA path: the row merges, one workgroup per draft row.
template <int WAVES>
__global__ __launch_bounds__(WAVES *kWave) void tree_merge_kernel(HeadArgs a) {
  __shared__ MergeShared<WAVES> sh;
  __shared__ int32_t s_tiles[kMaxTiles];
  __shared__ uint32_t s_ntiles;
  row_merge<WAVES>(a, blockIdx.x, sh, s_tiles, s_ntiles);
}

// ------------------------------------------- MFMA path, many draft rows
// The contraction tiled as a GEMM: one workgroup of 8 waves per pair of W
// tiles (128 W rows) covers up to 64 CB draft rows, so that W_trim streams
// from memory once. Wave (wr, wc) owns the 64 x 16 CB block of tile 2 p + wr
// and draft rows 16 CB wc .. over the whole of d, so it ends with final
// sums: logits and the (draft row, tile) softmax partials (or the tile's
// draws) go out as on the 64-row path and the same row merges follow.
constexpr int kGemmKC = 8;                      // 16-byte chunks per row and K step

// Slot of 16-byte chunk c of staged row r (rows of 8 chunks). The chunk index
// is XOR-swizzled by the row's low three bits: the operand reads (16 rows at
// one chunk for each of four chunks per instruction) then hit distinct banks.
// Measured with the LDS counters: 4 cycles per read instruction against 8 for
// an unswizzled row pitch of 9 chunks.
static_assert(kGemmKC == 8, "the swizzle permutes the 8 chunks of a row");
__device__ __forceinline__ int gemm_slot(int r, int c) { return r * kGemmKC + (c ^ (r & 7)); }

// The quad-transposed draw for column blocks I .. CB - 1 of a wave's
// accumulators (blocks past M skipped), expanded at compile time so that
// every accumulator index is static.
template <int I, int CB, bool kPre>
__device__ __forceinline__ void draw_blocks(const HeadArgs &a, const f32x4 (&acc)[4][CB], int mw0,
                                            int tile, int trow0, const int32_t (&fid)[4][4],
                                            const float (*gq)[4][4]) {
  if constexpr (I < CB) {
    if (mw0 + 16 * I < a.M) {  // uniform: the block has rows
      const f32x4 z[4] = {acc[0][I], acc[1][I], acc[2][I], acc[3][I]};
      quad_draw_publish<kPre>(a, mw0 + 16 * I, tile, trow0, z, fid, kPre ? gq[I] : nullptr);
    }
    draw_blocks<I + 1, CB, kPre>(a, acc, mw0, tile, trow0, fid, gq);
  }
}

// Up to two 16-row blocks per wave the GEMM tiling draws its Gumbel
// variates and loads the tile rows' full ids before its K loop, while the
// ring fills (16 registers per block), instead of after it.
template <int CB>
constexpr bool kEarlyDraw = CB <= 2;
template <int CB>
struct EarlyDraw {
  float gq[kEarlyDraw<CB> ? CB : 1][4][4];
  int32_t fid[4][4];
};

// Epilogue of wave (wr, wc) of a GEMM-tiled workgroup over W tile pair p,
// whose first draft row is mw0: lane (g, r16) holds, per (rb, cb), the
// logits of tile rows 16 rb + 4 g .. + 3 for draft row mw0 + 16 cb + r16.
template <int CB>
__device__ __forceinline__ void gemm_epilogue(const HeadArgs &a, f32x4 (&acc)[4][CB], int tile,
                                              int mw0, int g, int r16,
                                              const EarlyDraw<CB> &early) {
  const int trow0 = tile * kTileRows;
  // Sampling: the quad-transposed draw per 16-row column block (not
  // compiled for 8 blocks per wave, whose registers it would overflow; the
  // host runs draws on narrower shapes).
  if constexpr (CB <= 6) if (a.sample) {
    if (tile >= a.tiles) return;
    int32_t fid[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = trow0 + 16 * rb + 4 * g + i;
        if constexpr (kEarlyDraw<CB>)
          fid[rb][i] = early.fid[rb][i];
        else
          fid[rb][i] = row < a.V_high ? fid_at(a, row) : 0;
        if (a.bias && row < a.V_high)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[rb][cb][i] += bf16_to_f32(a.bias[row]);
      }
    draw_blocks<0, CB, kEarlyDraw<CB>>(a, acc, mw0, tile, trow0, fid, early.gq);
    return;
  }
  if (tile >= a.tiles) return;
  // Over the wave's draft rows that exist, from this tile on (none: no
  // stores follow).
  const int zrows = min(16 * CB, a.M - mw0);
  const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc(
      a.zbuf + (size_t)max(0, min(mw0, a.M - 1)) * a.zpitch + trow0, 0,
      zrows > 0 ? (int)(((size_t)zrows * a.zpitch - trow0) * 4) : 0, kBufferRsrcWord3);
  auto store = [&](const f32x4 &v, int idx) {  // logits v at float index idx past zres
    if (a.zstream)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), zres, idx * 4, 0,
                                             kCpolNt);
    else
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), zres, idx * 4, 0, 0);
  };
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int m = mw0 + 16 * cb + r16;
    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = trow0 + 16 * rb + 4 * g + i;
        if (a.bias && row < a.V_high) acc[rb][cb][i] += bf16_to_f32(a.bias[row]);
        if (row < a.V_high) mx = fmaxf(mx, acc[rb][cb][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float S = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (trow0 + 16 * rb + 4 * g + i < a.V_high) S += __expf(acc[rb][cb][i] - mx);
    S += __shfl_xor(S, 16);
    S += __shfl_xor(S, 32);
    // Logits out in whole 128-byte lines: for each pair of 16-row blocks
    // (rb, rb + 1) lanes r16 and r16 ^ 8 swap one block (a DPP rotation by
    // 8 within each row of 16 lanes), so that one store writes tile rows
    // 32 pr .. 32 pr + 31 of draft rows 0..7 of the block (8 lanes per draft
    // row) and the next those of draft rows 8..15. Storing each lane's own
    // block instead (64 bytes per draft row and store) wrote 1.4 times the
    // bytes past L2 (M = 60: 11.9 against 8.4 MB; M = 512: 98 against 71 MB)
    // and took 4.7 us longer at M = 512.
    const bool lo = r16 < 8;
    const int rowA = lo ? r16 : r16 - 8, rowB = lo ? r16 + 8 : r16;
    const int col = (lo ? 0 : 16) + 4 * g;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const f32x4 a0 = acc[2 * pr][cb], a1 = acc[2 * pr + 1][cb];
      const f32x4 send = lo ? a1 : a0;
      // (__float_as_int, not __builtin_bit_cast: hipcc's bit_cast of a vector
      // element send[i] reads element 0 whatever i is.)
      f32x4 recv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        recv[i] = __int_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_int(send[i]), 0x128, 0xf, 0xf, false));
      const f32x4 vA = lo ? a0 : recv, vB = lo ? recv : a1;
      if (mw0 + 16 * cb + rowA < a.M) store(vA, (16 * cb + rowA) * a.zpitch + 32 * pr + col);
      if (mw0 + 16 * cb + rowB < a.M) store(vB, (16 * cb + rowB) * a.zpitch + 32 * pr + col);
    }
    if (m < a.M && g == 0) a.tile_ms[(size_t)m * a.tiles + tile] = pack_ms(mx, S);
  }
}

// A workgroup of the GEMM tiling covers a pair of W tiles once there are
// enough pairs to give each of the 256 CUs one (heads of 512 tiles or more),
// else a single tile (4 waves): up to 64 draft rows such workgroups also fit
// two to a CU, past 64 rows one, so past 64 rows the single-tile form is
// taken only up to 256 tiles. Up to 32 rows on heads of fewer than 256 tiles
// the 64-row kernel (one workgroup per tile, its four waves streaming their
// own quarters of d with no barrier per step) is faster still.
constexpr int kRingMinPairs = 256;

// Both operands are copied from memory straight into LDS (buffer loads with
// the LDS flag: each lane's 16 bytes land in slot lane of a 64-slot block, no
// registers involved), through a ring of S stages, so that up to S - 1 K
// steps are in flight per workgroup at no register cost. A stage holds the
// W rows, then the draft rows, 8 chunks each in the swizzled order of
// gemm_slot; lane l of a load fills row l / 8 of its 8-row block at position
// l % 8, so it reads chunk (l % 8) ^ (l / 8) of that row. Chunks past d and rows past
// V_high or M are addressed outside the buffer ranges, which the hardware
// turns into zeros in LDS.
template <int CB, int S, int TPW>
struct GemmRing {
  static constexpr int kRows = TPW * kTileRows;        // W rows per workgroup
  static constexpr int kWaves = 4 * TPW;
  static constexpr int kDraftRows = 4 * 16 * CB;
  static constexpr int kSlots = (kRows + kDraftRows) * kGemmKC;  // per stage
  static constexpr int kLoads = (kRows + kDraftRows) / 8 / kWaves;
  static constexpr int kWLoads = kRows / 8 / kWaves;
  static_assert(kLoads * 8 * kWaves == kRows + kDraftRows && kWLoads * 8 * kWaves == kRows,
                "every wave issues whole 8-row blocks of each operand");
  static_assert(S >= 2 && (S - 1) * kLoads <= 63, "the in-flight loads must fit vmcnt");
  static_assert(S * kSlots * 16 <= 160 * 1024, "the ring must fit the LDS");
};

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, the other counters at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// kShared: more than one group of draft rows, so each pair of W tiles is
// read by two workgroups of one XCD (plain loads keep it in L2 for the
// other); otherwise W is streamed once, non-temporally.
template <bool kShared, int CB, int S, int TPW>
__global__ __launch_bounds__(4 * TPW * kWave) void head_gemm_kernel(HeadArgs a) {
  using Ring = GemmRing<CB, S, TPW>;
  constexpr int kDR = Ring::kDraftRows, kWaves = Ring::kWaves, kRows = Ring::kRows;
  constexpr int kLoads = Ring::kLoads, kWLoads = Ring::kWLoads, kSlots = Ring::kSlots;
  __shared__ u32x4 ring[S * kSlots];
  // The wave index is uniform (the LDS address of a load must be).
  const int tid = threadIdx.x, lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tpairs = (a.tiles + TPW - 1) / TPW, gpairs = (a.M + kDR - 1) / kDR;
  // Workgroup -> (tile pair p, draft-row group q); past 384 draft rows (draws
  // only) the groups of one tile pair take consecutive slots of one XCD, so
  // that the later one finds the W rows in that XCD's L2.
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int q = slot % gpairs, p = xcd + 8 * (slot / gpairs);
  if (p >= tpairs) return;
  const int c16 = a.c16;
  const int wrow0 = p * kRows, mrow0 = q * kDR;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(a.W + (size_t)wrow0 * c16), 0,
      min(kRows, a.V_high - wrow0) * c16 * 16, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(a.h + (size_t)mrow0 * c16), 0,
      min(kDR, a.M - mrow0) * c16 * 16, kBufferRsrcWord3);
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ lrow;
  // Load j of this wave fills 8-row block wave + kWaves j of a stage: W
  // rows for j < kWLoads, draft rows after them.
  uint32_t voff[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int blk = wave + kWaves * j;
    const int row = 8 * (j < kWLoads ? blk : blk - kRows / 8) + lrow;
    voff[j] = (uint32_t)(row * c16 + lchunk) * 16u;
  }
  // Workgroups start their K loop at staggered steps and wrap around, so
  // that at any moment the rows in flight are spread over the width of d. In
  // step with one another they would all read the same 128-byte column of
  // 8 KiB-strided rows and crowd onto a few memory channels. The workgroups
  // of one XCD (tile pairs p, p + 8, ...) start one step apart (three up to
  // 32 draft rows), so that their columns cover all of that XCD's L2
  // channels; every XCD uses the same offsets, and the two row groups of a
  // tile pair (draws past 384 rows) the same one. Measured on the
  // 4096 x 32768 head against no stagger: M = 60 67.4 -> 46.2 us, M = 128
  // 68.7 -> 56.0 us; starting tile pair p at step p mod steps instead (8
  // distinct offsets per XCD) gave 49.6 and 56.6 us, and shifting alternate
  // XCDs by half of d 72.6 and 77.7 us. Three steps apart is 1 us faster up
  // to 32 rows and 0.5 to 4 us slower from 60 rows on.
  const int steps = (c16 + kGemmKC - 1) / kGemmKC;
  const int rot = ((a.M <= 32 ? 3 : 1) * (p / 8)) % steps;
  // K step s (the workgroup's s-th, step se of d) into ring stage s % S:
  // its W loads (part 1), its draft-row loads (part 2) or both; every step
  // is issued, steps past the last (and chunks past d) as out-of-range zero
  // loads.
  auto issue = [&](int s, int part) {
    const int se = s < steps ? (s + rot < steps ? s + rot : s + rot - steps) : s;
    // All ones past d, else zero (arithmetic, so that no lane branches).
    const uint32_t past = ~(uint32_t)((se * kGemmKC + lchunk - c16) >> 31);
    u32x4 *stage = ring + (s % S) * kSlots;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint32_t off = (voff[j] + (uint32_t)se * (kGemmKC * 16)) | (past & 0x7fffff00u);
      auto *dst = (__attribute__((address_space(3))) void *)(stage + 64 * (wave + kWaves * j));
      if (j < kWLoads) {
        if (part & 1)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, dst, 16, off, 0, 0, kShared ? 0 : kCpolNt);
      } else if (part & 2) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(hres, dst, 16, off, 0, 0, 0);
      }
    }
  };
  const int wr = TPW == 2 ? wave & 1 : 0, wc = TPW == 2 ? wave >> 1 : wave;
  const int g = lane >> 4, r16 = lane & 15;
  f32x4 acc[4][CB];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s, 3);
  EarlyDraw<CB> early;
  if constexpr (kEarlyDraw<CB>) {
    if (a.sample) {
      const int trow0 = (TPW * p + wr) * kTileRows;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        gumbel_quad(a, mrow0 + 16 * CB * wc + 16 * cb, trow0, early.gq[cb]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = trow0 + 16 * rb + 4 * g + i;
          early.fid[rb][i] = row < a.V_high ? fid_at(a, row) : 0;
        }
    }
  }
#pragma unroll 1
  for (int s = 0; s < steps; ++s) {
    // This wave's loads of step s have landed (the S - 2 later steps may
    // still be in flight) and its reads of the previous stage have
    // returned; after the barrier every wave's loads of step s have, and no
    // wave reads the stage that the next issue overwrites.
    wait_vmcnt<(S - 2) * kLoads>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // With three stages or more the next step's loads go out after this
    // step's MFMAs, behind its LDS reads, which they would otherwise hold up
    // (4096 x 32768 head, M = 160 / 192 / 256: 77.3 / 79.0 / 83.9 -> 72.6 /
    // 75.3 / 79.1 us; with four stages, up to 128 rows, no change). With two
    // they must land within this step: the W loads, from HBM, go out at
    // once, and the draft-row loads, which hit in L2 and are most of the
    // bytes, halfway through the step (M = 320 / 384 on 6 blocks per wave
    // and 512 on 8: 110.0 / 113.7 / 143.6 us all at once, 98.9 / 104.6 /
    // 128.5 so; a quarter of the way 103.6 / 109.2 / 136.1, after the MFMAs
    // 110.3 / 114.1 / 141.9).
    if constexpr (S == 2) issue(s + 1, 1);
    const u32x4 *st = ring + (s % S) * kSlots;
#pragma unroll
    for (int t = 0; t < kGemmKC / 4; ++t) {
      const int cl = 4 * t + g;
      u32x4 av[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) av[rb] = st[gemm_slot(64 * wr + 16 * rb + r16, cl)];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const u32x4 bv = st[kRows * kGemmKC + gemm_slot(16 * CB * wc + 16 * cb + r16, cl)];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av[rb]), __builtin_bit_cast(bf16x8, bv), acc[rb][cb],
              0, 0, 0);
      }
      if constexpr (S == 2) if (t == 0) issue(s + 1, 2);
    }
    if constexpr (S > 2) issue(s + S - 1, 3);
  }
  // No load into this workgroup's LDS may outlive it.
  wait_vmcnt<0>();
  gemm_epilogue<CB>(a, acc, TPW * p + wr, mrow0 + 16 * CB * wc, g, r16, early);
}

template <int CB, int S, int TPW = 2>
hipError_t launch_gemm_shape(const HeadArgs &a, hipStream_t stream) {
  using Ring = GemmRing<CB, S, TPW>;
  const int units = (a.tiles + TPW - 1) / TPW;
  const int gpairs = (a.M + Ring::kDraftRows - 1) / Ring::kDraftRows;
  const dim3 grid(8 * ((units + 7) / 8) * gpairs), block(Ring::kWaves * kWave);
  if (gpairs > 1)
    hipLaunchKernelGGL((head_gemm_kernel<true, CB, S, TPW>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((head_gemm_kernel<false, CB, S, TPW>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// The block of each wave grows with M in steps of 16 x 4 = 64 draft rows per
// workgroup: 64 x 16 up to 64 draft rows, then 64 x 32, 64 x 48, ... up to
// 64 x 128 (512 rows; 64 x 112 up to 448), with as many ring stages as fit
// the LDS (4, 4, 4, 3, 2, 2, 2, 2). Against shapes that cover twice the
// range (64, 128, 256, 384, 512 rows), the intermediate ones are 5 to 11 %
// faster (4096 x 32768 head, M = 160 / 300 / 420: 68.5 / 96.6 / 120.3 ->
// 61.3 / 91.6 / 112.7 us). Draws past 384 rows run two groups of 256 rows
// on the 64 x 64 shape (the draw does not fit the registers next to 8
// column blocks).
hipError_t launch_gemm(const HeadArgs &a, hipStream_t stream) {
  hipError_t e;
  const bool pairs = (a.tiles + 1) / 2 >= kRingMinPairs;
  if (a.M <= 64)
    e = pairs ? launch_gemm_shape<1, 4, 2>(a, stream) : launch_gemm_shape<1, 4, 1>(a, stream);
  else if (a.M <= 128)
    e = a.tiles > kRingMinPairs ? launch_gemm_shape<2, 4, 2>(a, stream)
                                : launch_gemm_shape<2, 4, 1>(a, stream);
  else if (a.M <= 192)
    e = launch_gemm_shape<3, 4>(a, stream);
  else if (a.M <= 256 || (a.sample && a.M > 384))
    e = launch_gemm_shape<4, 3>(a, stream);
  else if (a.M <= 320)
    e = launch_gemm_shape<5, 2>(a, stream);
  else if (a.M <= 384)
    e = launch_gemm_shape<6, 2>(a, stream);
  else if (a.M <= 448)
    e = launch_gemm_shape<7, 2>(a, stream);
  else
    e = launch_gemm_shape<8, 2>(a, stream);
  if (e != hipSuccess) return e;
  if (a.sample)
    hipLaunchKernelGGL((head_merge_kernel<8>), dim3(a.M), dim3(8 * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((tree_merge_kernel<kTreeWaves>), dim3(a.M), dim3(kTreeWaves * kWave), 0,
                       stream, a);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_mfma(const HeadArgs &a, hipStream_t stream) {
  static_assert(NT == 1 || NT == 2, "up to 32 draft rows");
  hipLaunchKernelGGL((head_mfma_kernel<NT>), dim3(a.tiles), dim3(kMfmaWaves * kWave), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.sample)
    hipLaunchKernelGGL((head_merge_kernel<8>), dim3(a.M), dim3(8 * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((tree_merge_kernel<kTreeWaves>), dim3(a.M), dim3(kTreeWaves * kWave), 0,
                       stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch
constexpr int kCplSet[] = {1, 2, 3, 4, 5, 6, 7, 8, 12, 16};

// Workgroups of two tiles need 512 tiles to give every CU one; below that
// one-tile workgroups (two per CU) spread the rows over more CUs.
constexpr int kWideMinTiles = 512;

template <int WAVES, int MT, bool LOGITS, int CPL, bool RAGGED>
hipError_t launch_waves(const HeadArgs &a, hipStream_t stream) {
  constexpr int kTiles = WAVES / 8;
  hipLaunchKernelGGL((head_gemv_kernel<WAVES, MT, CPL, RAGGED, LOGITS>),
                     dim3((a.tiles + kTiles - 1) / kTiles), dim3(WAVES * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int MT, bool LOGITS, int CPL, bool RAGGED>
hipError_t launch_one(const HeadArgs &a, hipStream_t stream) {
  constexpr int WIDE = gemv_waves<MT, CPL>();
  if (WIDE == 16 && a.tiles >= kWideMinTiles)
    return launch_waves<WIDE, MT, LOGITS, CPL, RAGGED>(a, stream);
  return launch_waves<8, MT, LOGITS, CPL, RAGGED>(a, stream);
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Counters and status words (256 bytes), then the GEMV path's group maxima.
constexpr size_t head_zero_prefix = 256;
static_assert(kWsSpinLimit + 4 <= head_zero_prefix, "status words inside the prefix");

size_t head_zero_bytes() {
  return head_zero_prefix + (size_t)kGemvMaxRows * 2 * kGroups * 8;
}

// One draft row always takes the GEMV path; two rows take it on a head of
// fewer than 256 tile pairs (on larger heads the GEMM tiling is faster).
static bool gemv_path(int32_t M, int32_t tiles) {
  return M == 1 || (M <= kGemvMaxRows && (tiles + 1) / 2 < kRingMinPairs);
}

HeadPlan head_plan(int32_t M, int32_t V_high, int32_t k) {
  // Fixed-offset prefix that every call leaves at zero: the ticket counter
  // (byte 0), the count of finished row mergers (byte 64), then the group
  // maxima of the GEMV path's draft rows. Per-call data after.
  HeadPlan p;
  p.tiles = (V_high + kTileRows - 1) / kTileRows;
  size_t off = head_zero_prefix;
  p.off_group = off;
  off += (size_t)kGemvMaxRows * 2 * kGroups * 8;
  p.zero_bytes = off;
  // Tile keys: k per tile on the GEMV path; the MFMA path publishes one key
  // per tile, and only when sampling.
  const bool mfma = !gemv_path(M, p.tiles);
  p.off_tile_keys = off;
  off += align_up((size_t)M * p.tiles * (mfma ? 1 : k) * 8, 256);
  p.off_tile_ms = off;
  off += align_up((size_t)M * p.tiles * 8, 256);
  p.off_tile_z = off;  // sampling mode: z of each tile's drawn row
  off += align_up((size_t)M * p.tiles * 8, 256);
  p.off_zbuf = off;  // MFMA path, top-k mode: logits [M][tiles * kTileRows] fp32
  off += mfma ? align_up((size_t)M * p.tiles * kTileRows * 4, 256) : 0;
  p.bytes = off;
  return p;
}

namespace {
hipError_t launch_head_call(const uint16_t *h, int32_t M, int32_t d, const uint16_t *W_trim,
                            const uint16_t *bias, int32_t V_high, const int32_t *t2f,
                            int32_t k, int32_t *full_ids,
                            float *probs, void *ws, bool sample, uint64_t seed,
                            uint64_t offset, bool remap, hipStream_t stream) {
  const HeadPlan p = head_plan(M, V_high, k);
  char *base = static_cast<char *>(ws);
  HeadArgs a{};
  a.W = reinterpret_cast<const u32x4 *>(W_trim);
  a.bias = bias;
  a.t2f = t2f;
  a.c16 = d / 8;
  a.V_high = V_high;
  a.k = k;
  a.tiles = p.tiles;
  a.counter = reinterpret_cast<uint32_t *>(base + kWsTicket);
  a.merged = reinterpret_cast<uint32_t *>(base + kWsMerged);
  a.status = reinterpret_cast<uint32_t *>(base);
  a.remap = remap ? 1 : 0;
  a.tile_keys = reinterpret_cast<uint64_t *>(base + p.off_tile_keys);
  a.tile_ms = reinterpret_cast<uint64_t *>(base + p.off_tile_ms);
  a.group_max = reinterpret_cast<uint64_t *>(base + p.off_group);
  a.group_kth = a.group_max + (size_t)kGemvMaxRows * kGroups;
  a.tiles_per_group = (p.tiles + kGroups - 1) / kGroups;
  a.M = M;
  a.h = reinterpret_cast<const u32x4 *>(h);
  a.full_ids = full_ids;
  a.probs = probs;
  a.sample = sample ? 1 : 0;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.off_lo = (uint32_t)offset;
  a.off_hi = (uint32_t)(offset >> 32);
  a.tile_z = reinterpret_cast<uint64_t *>(base + p.off_tile_z);
  a.zbuf = reinterpret_cast<float *>(base + p.off_zbuf);
  a.zpitch = p.tiles * kTileRows;
  a.zstream = (size_t)M * p.tiles * kTileRows * 4 >= kZStreamBytes ? 1 : 0;
  // One draft row (two on a head of fewer than 256 tile pairs): one GEMV
  // pass with the merge in the same kernel. Up to 32 rows on a head of
  // fewer than 256 tiles: the 64-row MFMA kernel, one workgroup per tile.
  // Otherwise the GEMM tiling. Then one merge workgroup per draft row.
  if (gemv_path(M, p.tiles)) return launch_gemv(a, stream);
  if (M > kGroupRows || p.tiles >= kRingMinPairs) return launch_gemm(a, stream);
  return M <= 16 ? launch_mfma<1>(a, stream) : launch_mfma<2>(a, stream);
}
}  // namespace

hipError_t launch_draft_head(const uint16_t *h, int32_t M, int32_t d,
                             const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                             const int32_t *t2f, int32_t k, int32_t *full_ids,
                             float *probs, void *ws, hipStream_t stream, bool remap) {
  return launch_head_call(h, M, d, W_trim, bias, V_high, t2f, k, full_ids, probs, ws, false, 0,
                          0, remap, stream);
}

hipError_t launch_draft_sample(const uint16_t *h, int32_t M, int32_t d,
                               const uint16_t *W_trim, const uint16_t *bias, int32_t V_high,
                               const int32_t *t2f, uint64_t seed, uint64_t offset,
                               int32_t *full_ids, float *probs, void *ws, hipStream_t stream) {
  return launch_head_call(h, M, d, W_trim, bias, V_high, t2f, 1, full_ids, probs, ws, true,
                          seed, offset, true, stream);
}

namespace {
// Per-row softmax statistics of logits already in memory (the logits-only
// check call): mu = max_j z[m, j], S = sum_j exp(z[m, j] - mu), one
// workgroup per row. Each thread takes the indices tid, tid + 256, ... in
// order; the waves and then the workgroup combine in a fixed order.
constexpr int kStatWaves = 4;
__global__ __launch_bounds__(kStatWaves *kWave) void row_stats_kernel(const float *__restrict__ z,
                                                                      int n, float *row_max,
                                                                      float *row_sum) {
  __shared__ float s_m[kStatWaves], s_s[kStatWaves];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const float *zr = z + (size_t)blockIdx.x * n;
  float mu = -INFINITY;
  for (int j = tid; j < n; j += kStatWaves * kWave) mu = fmaxf(mu, zr[j]);
  mu = wave_max(mu);
  if (lane == 0) s_m[wave] = mu;
  __syncthreads();
  mu = s_m[0];
  for (int w = 1; w < kStatWaves; ++w) mu = fmaxf(mu, s_m[w]);
  float S = 0.f;
  for (int j = tid; j < n; j += kStatWaves * kWave) S += __expf(zr[j] - mu);
  S = wave_sum(S);
  if (lane == 0) s_s[wave] = S;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < kStatWaves; ++w) t += s_s[w];
    if (row_max) row_max[blockIdx.x] = mu;
    if (row_sum) row_sum[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(u32x4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0, 0, 0, 0};
}
}  // namespace

hipError_t launch_zero(void *p, size_t n, hipStream_t stream) {
  const size_t n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n16 + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<u32x4 *>(p),
                     n16);
  return hipGetLastError();
}

hipError_t launch_head_logits(const uint16_t *h, int32_t M, int32_t d,
                              const uint16_t *W_trim, int32_t V_high,
                              float *logits, float *row_max, float *row_sum,
                              hipStream_t stream) {
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
  if (row_max || row_sum) {
    hipLaunchKernelGGL(row_stats_kernel, dim3(M), dim3(kStatWaves * kWave), 0, stream, logits,
                       V_high, row_max, row_sum);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace vt

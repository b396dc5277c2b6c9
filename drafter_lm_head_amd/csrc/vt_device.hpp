// Device helpers shared by the gfx950 kernels: wave64 reductions on DPP,
// order-preserving 64-bit top-k keys, the counter-based generator of the
// multinomial draw, and the hand-off of partial results between workgroups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vt {

constexpr int kWave = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- loads
// Streaming 16-byte load that should not displace reused lines.
__device__ __forceinline__ u32x4 load_stream16(const u32x4 *p) {
  return __builtin_nontemporal_load(p);
}

// fp32 += a.lo*b.lo + a.hi*b.hi on two packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// bf16 payload -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float c) {
  c = dot2_bf16(a.x, b.x, c);
  c = dot2_bf16(a.y, b.y, c);
  c = dot2_bf16(a.z, b.z, c);
  c = dot2_bf16(a.w, b.w, c);
  return c;
}

// ---------------------------------------------------------- DPP shuffles
// GFX9 DPP controls used below.
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF,
                                               false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(x)));
}

__device__ __forceinline__ float readlane_f32(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int lane) {
  uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
  uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Sum over the 64 lanes in a fixed order; every lane must be active. The
// result is wave-uniform.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  x += dpp_f32<kDppRowMirror>(x);
  return (readlane_f32(x, 0) + readlane_f32(x, 16)) +
         (readlane_f32(x, 32) + readlane_f32(x, 48));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return fmaxf(fmaxf(readlane_f32(x, 0), readlane_f32(x, 16)),
               fmaxf(readlane_f32(x, 32), readlane_f32(x, 48)));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  uint32_t lo = dpp_u32<CTRL>((uint32_t)x);
  uint32_t hi = dpp_u32<CTRL>((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) {
  return a > b ? a : b;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = max_u64(x, dpp_u64<kDppQuadXor1>(x));
  x = max_u64(x, dpp_u64<kDppQuadXor2>(x));
  x = max_u64(x, dpp_u64<kDppRowHalfMirror>(x));
  x = max_u64(x, dpp_u64<kDppRowMirror>(x));
  return max_u64(max_u64(readlane_u64(x, 0), readlane_u64(x, 16)),
                 max_u64(readlane_u64(x, 32), readlane_u64(x, 48)));
}

// Inclusive prefix sum over lanes (lane i gets x_0 + ... + x_i).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    uint32_t y = __shfl_up(x, s);
    if (lane >= s) x += y;
  }
  return x;
}

// ------------------------------------------------------------ top-k keys
// A key orders candidates by logit (larger first) and, among equal logits,
// by full token id (lower first): high word = order-preserving image of the
// fp32 logit, low word = ~full_id. Key 0 is below every real candidate and
// marks an empty slot.
__device__ __forceinline__ uint32_t ord_from_f32(float z) {
  if (z == 0.0f) z = 0.0f;  // -0 and +0 are the same logit
  uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_ord(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t make_key(float z, int32_t full_id) {
  return ((uint64_t)ord_from_f32(z) << 32) | (uint32_t)(~(uint32_t)full_id);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  return f32_from_ord((uint32_t)(key >> 32));
}
__device__ __forceinline__ int32_t key_id(uint64_t key) {
  return (int32_t)(~(uint32_t)key);
}

// ------------------------------------------------------------- sampling
// Counter-based uniforms: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011). Ten rounds of two
// 32 x 32 -> 64-bit products of words 0 and 2 with fixed odd multipliers,
// half swaps and key mixing; the key advances by two Weyl increments between
// rounds. Each product is formed whole (one v_mad_u64_u32 instead of a
// low and a high multiply; the same bits, and half the integer multiplies).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// Standard Gumbel variates of the draw keyed by (seed, offset): one Philox
// call with counter (j, m / 4, offset) and key seed serves trimmed index j of
// the four draft rows 4 (m / 4) .. 4 (m / 4) + 3, row m taking word m % 4.
// The top 24 bits x of the word give u = (x + 1/2) / 2^24 in (0, 1) (exact
// in fp32), and the variate is -log(-log u).
__device__ __forceinline__ u32x4 gumbel_words(uint32_t seed_lo, uint32_t seed_hi,
                                              uint32_t off_lo, uint32_t off_hi, int mblock,
                                              int j) {
  return philox4x32_10((uint32_t)j, (uint32_t)mblock, off_lo, off_hi, seed_lo, seed_hi);
}
__device__ __forceinline__ float gumbel_from_word(uint32_t x) {
  const float u = ((float)(x >> 8) + 0.5f) * 0x1p-24f;
  return -logf(-logf(u));
}
__device__ __forceinline__ float gumbel(uint32_t seed_lo, uint32_t seed_hi, uint32_t off_lo,
                                        uint32_t off_hi, int m, int j) {
  const u32x4 x = gumbel_words(seed_lo, seed_hi, off_lo, off_hi, m >> 2, j);
  const int w = m & 3;
  return gumbel_from_word(w == 0 ? x[0] : w == 1 ? x[1] : w == 2 ? x[2] : x[3]);
}

// -------------------------------------------------- cross-workgroup order
// Workgroups hand partial results to the last one to finish without any
// cache-wide maintenance. On gfx950 each XCD has its own L2; an agent-scope
// release/acquire would write back (buffer_wbl2) and invalidate (buffer_inv)
// a whole L2 in every workgroup, which costs far more than the data moved
// here. Instead every value that crosses workgroups is written and read
// with agent-scope atomic stores and loads (global_store/load ... sc1),
// which are coherent across XCDs by themselves:
//   writer: publish_u64() stores, then arrive(): s_waitcnt vmcnt(0) makes
//           this wave's sc1 stores complete, the barrier extends that to
//           the workgroup, then one relaxed agent-scope atomic add takes a
//           ticket;
//   reader: the workgroup that draws the last ticket reads the data with
//           fetch_u64(); its loads are issued only after the ticket returns.
// Nothing else may be used to pass data between workgroups.
__device__ __forceinline__ void publish_u64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch_u64(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Takes a ticket after this workgroup's published stores have completed;
// returns how many workgroups arrived before it. Every thread of the
// workgroup must call it (it contains barriers); the result is uniform.
__device__ __forceinline__ uint32_t arrive(uint32_t *counter, uint32_t *s_slot) {
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt/lgkmcnt/expcnt = 0: stores done
  __syncthreads();
  if (threadIdx.x == 0)
    *s_slot = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_slot;
}

// Returns a ticket counter to zero for the next call (by its last holder).
__device__ __forceinline__ void reset_counter(uint32_t *counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace vt

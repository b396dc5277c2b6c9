// Plain streaming read of a device buffer: the practical ceiling of the
// draft head, which reads W_trim once with 16-byte non-temporal loads. The
// access pattern is the head kernel's: one 16-wave workgroup per CU over a
// contiguous slab, each wave reading 8 KiB per step with 8 loads per lane in
// flight. The data is folded into one word so that no load can be dropped.
#include "vt_internal.hpp"

namespace vt {
namespace {

constexpr int kSrWaves = 16;
constexpr int kSrLoads = 8;                              // 16-byte loads per lane per step
constexpr int kSrStep = kWave * kSrLoads;                // chunks per wave step (8 KiB)
constexpr int kSrBlocks = 256;

__global__ __launch_bounds__(kSrWaves *kWave) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                                      size_t n16,
                                                                      uint64_t *sink) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = min(n16, (size_t)blockIdx.x * per), hi = min(n16, lo + per);
  uint32_t acc = 0;
#pragma unroll 1
  for (size_t base = lo + (size_t)wave * kSrStep; base < hi; base += (size_t)kSrWaves * kSrStep) {
    u32x4 v[kSrLoads];
#pragma unroll
    for (int i = 0; i < kSrLoads; ++i) {
      const size_t c = base + (size_t)i * kWave + lane;
      v[i] = c < hi ? load_stream16(p + c) : u32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kSrLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  // A store that depends on every loaded word but (almost) never happens.
  if (acc == 0x9E3779B9u) sink[0] = (uint64_t)acc | ((uint64_t)blockIdx.x << 32);
}

}  // namespace

hipError_t launch_stream_read(const void *p, size_t bytes, uint64_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kSrBlocks), dim3(kSrWaves * kWave), 0, stream,
                     static_cast<const u32x4 *>(p), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace vt

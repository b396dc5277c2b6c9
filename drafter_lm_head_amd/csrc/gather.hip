// Trimmed-head row gather (VocabTrim page, Implementation, Step 3: keep the
// head rows of the kept ids; FR-Spec notes, key design: the head shrinks
// from d x 128k to d x 32k), for gfx950.
//
// W_trim[i, :] = W[t2f[i], :]. A workgroup copies kGatherRows rows with
// 16-byte loads and stores; each thread keeps kUnroll loads in flight before
// storing. Reads and writes are streaming: neither array is reused here.
// A head with a bias keeps the bias entries of the kept ids the same way
// (the page's reconstruction copies them alongside the rows).
#include "vt_internal.hpp"

namespace vt {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherRows = 4;

__global__ void gather_clear_kernel(uint32_t *n_bad) { *n_bad = 0; }

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const u32x4 *__restrict__ W, int32_t V, int32_t c16,
    const int32_t *__restrict__ t2f, int32_t V_high, u32x4 *__restrict__ out,
    uint32_t *__restrict__ n_bad) {
  const int32_t row0 = blockIdx.x * kGatherRows;
  const int32_t rows = min(kGatherRows, V_high - row0);
  __shared__ int32_t s_src[kGatherRows];
  if (threadIdx.x < rows) {
    const int32_t src = t2f[row0 + threadIdx.x];
    const bool ok = src >= 0 && src < V;
    s_src[threadIdx.x] = ok ? src : -1;
    if (!ok && n_bad) atomicAdd(n_bad, 1u);
  }
  __syncthreads();
  const int32_t total = rows * c16;  // 16-byte chunks this workgroup writes
  constexpr int kUnroll = 8;
  for (int32_t base = 0; base < total; base += kUnroll * kGatherThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t f = base + u * kGatherThreads + threadIdx.x;
      v[u] = u32x4{0, 0, 0, 0};
      if (f < total) {
        const int32_t r = f / c16, i = f - r * c16;
        const int32_t src = s_src[r];
        if (src >= 0) v[u] = load_stream16(W + (size_t)src * c16 + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t f = base + u * kGatherThreads + threadIdx.x;
      if (f < total) {
        const int32_t r = f / c16, i = f - r * c16;
        __builtin_nontemporal_store(v[u], out + (size_t)(row0 + r) * c16 + i);
      }
    }
  }
}

// Bias of the trimmed head: b_trim[i] = b[t2f[i]], zero for an entry
// outside [0, V) (counted like a bad row).
__global__ __launch_bounds__(kGatherThreads) void gather_bias_kernel(
    const uint16_t *__restrict__ b, int32_t V, const int32_t *__restrict__ t2f,
    int32_t V_high, uint16_t *__restrict__ out, uint32_t *__restrict__ n_bad) {
  const int32_t i = blockIdx.x * kGatherThreads + threadIdx.x;
  if (i >= V_high) return;
  const int32_t src = t2f[i];
  const bool ok = src >= 0 && src < V;
  if (!ok && n_bad) atomicAdd(n_bad, 1u);
  out[i] = ok ? b[src] : (uint16_t)0;
}

}  // namespace

hipError_t launch_gather_bias(const uint16_t *b, int32_t V, const int32_t *t2f,
                              int32_t V_high, uint16_t *b_trim, uint32_t *n_bad,
                              hipStream_t stream) {
  if (n_bad) {
    hipLaunchKernelGGL(gather_clear_kernel, dim3(1), dim3(1), 0, stream, n_bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int32_t blocks = (V_high + kGatherThreads - 1) / kGatherThreads;
  hipLaunchKernelGGL(gather_bias_kernel, dim3(blocks), dim3(kGatherThreads), 0, stream, b, V,
                     t2f, V_high, b_trim, n_bad);
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t *W, int32_t V, int32_t d,
                         const int32_t *t2f, int32_t V_high, uint16_t *W_trim,
                         uint32_t *n_bad, hipStream_t stream) {
  if (n_bad) {
    hipLaunchKernelGGL(gather_clear_kernel, dim3(1), dim3(1), 0, stream, n_bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int32_t c16 = d / 8;
  const int32_t blocks = (V_high + kGatherRows - 1) / kGatherRows;
  hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(kGatherThreads), 0,
                     stream, reinterpret_cast<const u32x4 *>(W), V, c16, t2f,
                     V_high, reinterpret_cast<u32x4 *>(W_trim), n_bad);
  return hipGetLastError();
}

}  // namespace vt

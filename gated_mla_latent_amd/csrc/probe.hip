// Read-bandwidth probe (diagnostic, not part of the attention path): streams
// a device buffer with 16-byte loads and folds it into one word per
// workgroup, so the loads cannot be dropped. Its rate is the measured
// read-only HBM ceiling that the HBM-bound kernels are compared against.
#include "common.h"
#include "kernels.h"

namespace gmla {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                   unsigned* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  unsigned r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  // one word per workgroup (vector store from lane 0 of the first wave)
  __shared__ unsigned red[kProbeThreads / 64];
  for (int off = 32; off > 0; off >>= 1) r ^= __shfl_xor(r, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) t ^= red[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_probe_read(const void* src, size_t bytes, unsigned* sink, int blocks, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  return launch(probe_read_kernel, dim3(blocks), dim3(kProbeThreads), 0, st, (const u32x4*)src,
                (int64_t)(bytes / 16), sink);
}

}  // namespace gmla

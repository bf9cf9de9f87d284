// Streaming-read probe for gfx950: every byte of a buffer is read once with 16-byte loads and the XOR of
// all 32-bit words is written out, so that no load can be dropped.  It measures the read rate that bounds
// the HBM-bound calls of the library (the merge, the salience pass, the acceptance scans, the gathers).
//
// A grid of a few work-groups per CU strides over the buffer; each thread keeps four independent 16-byte
// loads in flight per iteration.  Work-group partial XORs go to a per-work-group slot of the sink array
// and a second one-work-group launch folds them (no atomics).
#include "spec_internal.h"

namespace spec {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__device__ __forceinline__ uint32_t block_xor(uint32_t v) {
  __shared__ uint32_t part[kProbeThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v ^= __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < kProbeThreads / 64; ++w) r ^= part[w];
  return r;
}

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* data, int64_t n16, uint32_t* partial) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(data + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= data[i];
  const uint32_t r = block_xor(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (threadIdx.x == 0) partial[blockIdx.x] = r;
}

__global__ __launch_bounds__(kProbeThreads) void probe_fold_kernel(const uint32_t* partial, int n, uint32_t* out) {
  uint32_t v = 0;
  for (int i = threadIdx.x; i < n; i += kProbeThreads) v ^= partial[i];
  const uint32_t r = block_xor(v);
  if (threadIdx.x == 0) *out = r;
}

}  // namespace

hipError_t launch_read_probe(const void* data, int64_t bytes, uint32_t* sink, int grid, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, s, static_cast<const u32x4*>(data),
                     bytes / 16, sink + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_fold_kernel, dim3(1), dim3(kProbeThreads), 0, s, sink + 1, grid, sink);
  return hipGetLastError();
}

}  // namespace spec

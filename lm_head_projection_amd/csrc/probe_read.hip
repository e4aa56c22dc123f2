// probe_read.hip - the achievable HBM read rate of the box, for the
// benchmark's roofline: a plain streaming read of a large buffer with the
// scorer's access pattern (one 16-byte non-temporal load per lane, so each
// wave instruction reads 1 KiB contiguous), eight loads in flight per lane,
// grid-stride.  Not part of liblmtopk; built into its own library.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void k_probe_read(const u32x4* __restrict__ p, int64_t n_vec,
                                                     u32x4* __restrict__ sink) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = tid;
  for (; i + 7 * stride < n_vec; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n_vec; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  // keeps the loads; a data-dependent store that the probe's buffer never triggers
  if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u) sink[tid & 255] = acc;
}

extern "C" int probe_read(const void* p, int64_t bytes, void* sink, int grid, void* stream) {
  hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(1024), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(p), bytes / 16, static_cast<u32x4*>(sink));
  return (int)hipGetLastError();
}

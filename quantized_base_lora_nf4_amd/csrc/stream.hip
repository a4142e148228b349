// Measurement helper: a read-only stream over a device buffer, the HBM read
// ceiling that the few-token forward's weight stream is compared with.
// Every lane reads 16-byte words (grid-stride, four loads in flight, marked
// non-temporal), and each workgroup writes one XOR fold of what it read.
#include "kernels.hpp"

namespace qn {

namespace {

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one word per workgroup: the XOR of its lanes' folds
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int t = 0; t < 256; ++t) x ^= red[t];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace qn

// sa_stream.hip - a plain streaming read of device memory, the bandwidth a
// pure HBM read reaches on this device: the second denominator the decode
// step's effective bandwidth is quoted against ("SequenceO1" explainer,
// bottleneck analysis: decode is bound by memory bandwidth; "Quest 完全拆解",
// read-volume formula: the step's cost is the bytes it reads).
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;  // 16-byte loads in flight per thread and round

// Grid-stride read of n16 16-byte words.  Each thread folds its words into one
// XOR; a workgroup writes its word only if it equals a value no realistic input
// produces, which keeps every load live without a store per workgroup.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                                    size_t n16,
                                                                    uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    uint4 w[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) w[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 w = src[i];
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, st,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace sa

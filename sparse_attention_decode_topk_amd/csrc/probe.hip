// Streaming-read reference for the bandwidth figures of the decode step: a
// kernel that reads a buffer once, 16 bytes per lane per load with four
// loads in flight per lane, and folds what it read into one word per
// work-group (so the loads cannot be dropped).  It is the measured ceiling
// that the indexer scan's paged reads are compared with, next to the HBM
// datasheet figure.
#include "common.hpp"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const v4u* __restrict__ src,
                                                                    int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    v4u v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const v4u v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one word per work-group: XOR over the block through LDS
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) a ^= red[w];
    out[blockIdx.x] = a;
  }
}

}  // namespace

extern "C" int dsa_probe_stream_read(const void* src, size_t bytes, uint32_t* out, int32_t grid,
                                     void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16 != 0 || grid < 1) return DSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0,
                     dsa_host::as_stream(stream), static_cast<const v4u*>(src),
                     (int64_t)(bytes / 16), out);
  return dsa_host::launch_status(hipGetLastError());
}

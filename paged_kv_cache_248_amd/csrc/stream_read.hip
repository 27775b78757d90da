// Device read stream: the practical HBM read ceiling that the decode kernels
// (which read K/V and write almost nothing) are compared with.  Every byte
// of the buffer is loaded once with non-temporal 16-byte loads (the kind the
// decode kernels issue), sixteen in flight per lane, over a one-shot grid of
// 128 work-groups per CU (the fastest of the shapes measured on MI355X:
// 7.1 TB/s for 4 GiB, against 6.0 TB/s with plain loads).  Each work-group
// writes the XOR of the words it read to one sink entry (4 bytes per
// work-group, so the loads cannot be dropped and the writes are negligible).
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 16;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4 *__restrict__ src,
                                                                      int64_t n16,
                                                                      uint32_t *__restrict__ sink) {
  __shared__ uint32_t red[kStreamThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t sink_words,
                              hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + (int64_t)kStreamThreads * kStreamUnroll - 1) /
                       ((int64_t)kStreamThreads * kStreamUnroll);
  int64_t cap = (int64_t)device_cu_count() * 128;
  if (cap > sink_words) cap = sink_words;
  const int grid = (int)(want < 1 ? 1 : (want < cap ? want : cap));
  profile_begin(stream);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4 *>(src), n16, sink);
  profile_end(stream);
  return hipGetLastError();
}

}  // namespace pa

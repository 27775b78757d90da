// Plain device read stream: the practical HBM read ceiling that the decode
// kernels (which read K/V and write almost nothing) are compared with.
// Every byte of the buffer is loaded once with plain 16-byte loads (the
// kind the decode kernels issue), eight in flight per lane; the loaded words
// are folded into an XOR that is stored only if it equals a value the
// caller passes (so the loads cannot be dropped, and nothing is written in
// practice).
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4 *__restrict__ src,
                                                                      int64_t n16,
                                                                      uint32_t *__restrict__ sink,
                                                                      uint32_t magic) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == magic) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, uint32_t magic,
                              hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + (int64_t)kStreamThreads * kStreamUnroll - 1) /
                       ((int64_t)kStreamThreads * kStreamUnroll);
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int grid = (int)(want < 1 ? 1 : (want < cap ? want : cap));
  profile_begin(stream);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4 *>(src), n16, sink, magic);
  profile_end(stream);
  return hipGetLastError();
}

}  // namespace pa

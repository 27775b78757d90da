// Device read stream: the practical HBM read ceiling that the decode kernels
// (which read K/V and write almost nothing) are compared with; a device copy
// stream, the read+write ceiling of the block copy and the KV append; and a
// matrix-core stream, the practical MFMA ceiling the prefill is set beside.  Every byte
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

// Copy stream: every 16-byte piece is loaded and stored once with
// non-temporal accesses (the kind the block copy and the append issue).
// Default shape: one 4 KiB chunk per work-group, each lane loading one
// piece and then storing it (the fastest of the shapes measured on MI355X:
// 6.41-6.44 TB/s of reads plus writes for 2 GiB against 6.18-6.25 for
// 16 KiB chunks of four pieces per lane, 4.1 for 32 KiB or 64 KiB chunks and
// 5.1-5.2 for grid-stride loops of four pieces per lane, which stay
// available for comparison).
constexpr int kCopyChunkPieces = 1;   // pieces per lane, chunked form
constexpr int kCopyUnroll = 4;        // pieces per lane and step, grid-stride form

__global__ __launch_bounds__(kStreamThreads) void stream_copy_chunk_kernel(
    const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * kStreamThreads * kCopyChunkPieces + threadIdx.x;
  u32x4 v[kCopyChunkPieces];
#pragma unroll
  for (int u = 0; u < kCopyChunkPieces; ++u) {
    const int64_t i = base + (int64_t)u * kStreamThreads;
    if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyChunkPieces; ++u) {
    const int64_t i = base + (int64_t)u * kStreamThreads;
    if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
  }
}

__global__ __launch_bounds__(kStreamThreads) void stream_copy_kernel(const u32x4 *__restrict__ src,
                                                                      u32x4 *__restrict__ dst,
                                                                      int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * stride < n16; i += kCopyUnroll * stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Matrix-core stream: every wavefront runs `iters` rounds of 32
// back-to-back v_mfma_f32_32x32x16 on operands it read once (eight A and
// eight B fragments per lane, taken from the operand buffer, random 16-bit
// data), into four independent accumulators — the matrix cores' issue rate
// with no memory, LDS or softmax work beside it, at whatever clock the power
// limit allows for such data.  Work-group i writes the sum of its
// accumulators to sink[i], so nothing can be dropped.
template <class E>
__device__ __forceinline__ f32x16 mfma_32x32x16(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  if constexpr (__is_same(typename E::storage, _Float16))
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <class E>
__global__ __launch_bounds__(kStreamThreads) void mfma_stream_kernel(const u32x4 *__restrict__ ops,
                                                                      int64_t n16,
                                                                      float *__restrict__ sink,
                                                                      int iters) {
  __shared__ float red[kStreamThreads / 64];
  const int64_t g = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  u32x4 a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = ops[(g * 16 + k) % n16];
    b[k] = ops[(g * 16 + 8 + k) % n16];
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 32; ++u) acc[u & 3] = mfma_32x32x16<E>(a[u & 7], b[(u >> 2) & 7], acc[u & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kStreamThreads / 64; ++w) t += red[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, int32_t wgs_per_cu,
                              hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = (int64_t)kStreamThreads * kCopyUnroll;
  if (wgs_per_cu <= 0) {
    const int64_t per_chunk = (int64_t)kStreamThreads * kCopyChunkPieces;
    const int64_t grid = (n16 + per_chunk - 1) / per_chunk;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    return launch_main(stream_copy_chunk_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0,
                       stream, static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n16);
  }
  const int64_t want = (n16 + per_wg - 1) / per_wg;
  const int64_t cap = (int64_t)device_cu_count() * wgs_per_cu;
  const int grid = (int)(want < 1 ? 1 : (want < cap ? want : cap));
  return launch_main(stream_copy_kernel, dim3(grid), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n16);
}

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t sink_words,
                              hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + (int64_t)kStreamThreads * kStreamUnroll - 1) /
                       ((int64_t)kStreamThreads * kStreamUnroll);
  int64_t cap = (int64_t)device_cu_count() * 128;
  if (cap > sink_words) cap = sink_words;
  const int grid = (int)(want < 1 ? 1 : (want < cap ? want : cap));
  return launch_main(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4 *>(src), n16, sink);
}

hipError_t launch_mfma_stream(const void *ops, int64_t ops_bytes, float *sink, int32_t sink_words,
                              int32_t wgs_per_cu, int32_t iters, DType dtype, hipStream_t stream) {
  const int64_t want = (int64_t)device_cu_count() * wgs_per_cu;
  const int grid = (int)(want < sink_words ? want : sink_words);
  const int64_t n16 = ops_bytes / 16;
  if (dtype == DType::F16)
    return launch_main(mfma_stream_kernel<F16>, dim3(grid), dim3(kStreamThreads), 0, stream,
                       static_cast<const u32x4 *>(ops), n16, sink, iters);
  return launch_main(mfma_stream_kernel<BF16>, dim3(grid), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4 *>(ops), n16, sink, iters);
}

}  // namespace pa

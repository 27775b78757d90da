// Block copy by mapping for gfx950.
//
// src_to_dst[i] = j copies source block i into destination block j, -1 marks
// an unused entry ("vLLM中FlashAttention与KVCache交换机制解析", swap_blocks
// signature, argument list and simplified CPU implementation).  For each
// destination the lowest i naming it is the candidate and is copied only if it
// is a valid source block.  The same mapping is applied to the K pool and to
// the V pool ("vLLM中FlashAttention与KVCache优化解析", Swap Blocks 机制).
//
// Three short kernels, all on the caller's stream:
//   1. fill:    first_src[d] = INT32_MAX for every destination block;
//   2. resolve: first_src[src_to_dst[i]] = min(i) with an atomic min, so the
//               answer does not depend on execution order;
//   3. copy:    one work-group per 4 KiB slice of a destination block of
//               one pool moves it with 16-byte non-temporal loads and stores
//               (data is touched once; keeping it out of the caches leaves
//               them to the attention kernels).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 1;
constexpr int64_t kSliceBytes = (int64_t)kCopyThreads * 16 * kCopyUnroll;   // 4 KiB
static_assert(kSliceBytes == kCopySliceBytes, "the argument checks size the grid by this slice");

__global__ __launch_bounds__(256) void copy_fill_kernel(int32_t *first_src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) first_src[i] = 0x7fffffff;
}

__global__ __launch_bounds__(256) void copy_resolve_kernel(const int64_t *src_to_dst, int64_t nm,
                                                           int64_t num_dst, int32_t *first_src) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nm) return;
  const int64_t j = src_to_dst[i];
  if (j >= 0 && j < num_dst) atomicMin(first_src + j, (int32_t)i);
}

__device__ __forceinline__ u32x4 ldnt(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void stnt(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// One work-group per (pool, destination block, 4 KiB slice): each lane
// loads one 16-byte piece, then stores it.  Smaller work-groups copied
// faster on MI355X: on the 483 MB copy workload, slices of 4 / 8 / 16 KiB
// (one, two, four pieces per lane) moved 5.94 / 5.63 / 5.70 TB/s, two
// slices per work-group 5.18, and 1 / 2 / 8 KiB slices of one piece per
// lane (64, 128, 512 threads) 5.92 / 5.87 / 5.85; an earlier 2 GiB copy
// measured 4.1 TB/s at 32 KiB per work-group against 6.1 at 16 KiB.
__global__ __launch_bounds__(256) void copy_kernel(const char *src_k, const char *src_v,
                                                   char *dst_k, char *dst_v,
                                                   const int32_t *first_src, int64_t num_src,
                                                   int64_t block_bytes, uint32_t slices) {
  // blockIdx.x = destination block * slices + slice (below 2^31, checked by
  // the caller), blockIdx.y = pool (0: K, 1: V): one 32-bit division.
  const uint32_t x = blockIdx.x;
  const uint32_t d = x / slices;
  const uint32_t slice = x - d * slices;
  const int32_t i = first_src[d];
  if ((int64_t)i >= num_src) return;    // no valid source (INT32_MAX if nobody named d)
  const char *src = blockIdx.y == 0 ? src_k : src_v;
  char *dst = blockIdx.y == 0 ? dst_k : dst_v;
  const int64_t base = (int64_t)slice * kSliceBytes;
  const size_t so = (size_t)i * block_bytes, dof = (size_t)d * block_bytes;
  u32x4 r[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t off = base + ((int64_t)u * kCopyThreads + threadIdx.x) * 16;
    if (off < block_bytes) r[u] = ldnt(reinterpret_cast<const u32x4 *>(src + so + off));
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t off = base + ((int64_t)u * kCopyThreads + threadIdx.x) * 16;
    if (off < block_bytes) stnt(reinterpret_cast<u32x4 *>(dst + dof + off), r[u]);
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyLaunch &a, hipStream_t stream) {
  if (a.num_mappings == 0 || a.num_dst == 0) return hipSuccess;
  const int64_t fill_blocks = (a.num_dst + 255) / 256;
  hipLaunchKernelGGL(copy_fill_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, stream,
                     a.first_src, a.num_dst);
  const int64_t res_blocks = (a.num_mappings + 255) / 256;
  hipLaunchKernelGGL(copy_resolve_kernel, dim3((unsigned)res_blocks), dim3(256), 0, stream,
                     a.src_to_dst, a.num_mappings, a.num_dst, a.first_src);
  const int64_t slices = (a.block_bytes + kSliceBytes - 1) / kSliceBytes;
  const int64_t grid = slices * a.num_dst;            // below 2^31 (argument checks)
  return launch_main(copy_kernel, dim3((unsigned)grid, a.src_v ? 2 : 1), dim3(kCopyThreads), 0,
                     stream, static_cast<const char *>(a.src_k), static_cast<const char *>(a.src_v),
                     static_cast<char *>(a.dst_k), static_cast<char *>(a.dst_v),
                     static_cast<const int32_t *>(a.first_src), a.num_src, a.block_bytes,
                     (uint32_t)slices);
}

}  // namespace pa

// Pieces shared by the two causal paged prefill kernels (prefill.hip, the
// ping-pong schedule, and prefill_halftile.hip): work-group shape, kernel
// parameters, the matrix-core and maximum helpers, the phase barrier, the
// block-id scalar load and the host-side parameter and grid setup.
//
// Method (pages cited by title): softmax(Q K^T / sqrt(d)) V in tiles with the
// online (M, L, O) update — "vLLM中FlashAttention与KVCache交换机制解析",
// Kernel Fusion + Tiling + OnlineSoftmax; keys through the block table —
// "大模型长文本推理基座…PagedAttention 显存物理布局深度剖析" §二.2.
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kRows = 32;      // query rows per wavefront
constexpr int kWaves = 8;      // wavefronts per work-group (one work-group per CU)
constexpr int kStages = 4;     // LDS stages per K and per V tile stream
constexpr int kXcds = 8;       // XCDs of an MI355X; work-group ids are dealt to them round-robin

struct PrefillParams {
  void *out;
  const void *query;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start_loc;
  int32_t num_heads, num_kv_heads, group, heads_per_wg, subgroups, pos_per_wg;
  int32_t bs_log2, max_blocks_per_seq, num_blocks, ctx_cap, num_seqs;
  int32_t num_pairs, num_qtiles;
  float scale_log2e;
};

template <class E>
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  if constexpr (__is_same(typename E::storage, _Float16))
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Maximum over a lane's 32 scores and those of the lane 32 apart (the two
// halves of one query's keys), as a depth-4 tree of 3-input maxima; the
// halves are exchanged with v_permlane32_swap.  NaN-propagating maximum:
// lowers to v_maximum3_f32 without the per-operand canonicalisation of IEEE
// fmax.
__device__ __forceinline__ float row_max(const f32x16 (&s)[2]) {
  float a[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int x = 3 * i, y = 3 * i + 1, z = 3 * i + 2;
    a[i] = max3(s[x >> 4][x & 15], s[y >> 4][y & 15], s[z >> 4][z & 15]);
  }
  a[10] = __builtin_elementwise_maximum(s[1][14], s[1][15]);
  const float b0 = max3(a[0], a[1], a[2]), b1 = max3(a[3], a[4], a[5]);
  const float b2 = max3(a[6], a[7], a[8]), b3 = __builtin_elementwise_maximum(a[9], a[10]);
  const float r = __builtin_elementwise_maximum(max3(b0, b1, b2), b3);
  const f32x2 sw = pair_xor32(r);
  return __builtin_elementwise_maximum(sw[0], sw[1]);
}

// Raise the running maximum (and rescale O and L) only when a tile's maximum
// exceeds it by more than 2^kLazy; weights then stay within [0, 2^kLazy].
constexpr float kLazy = 8.0f;

// Work-group barrier between phases.  It keeps the compiler from moving
// memory accesses or any other instruction across it and waits for nothing:
// every LDS read of the loop is consumed (so complete) before its phase ends,
// LDS is written only by the direct-to-LDS tile loads, whose completion is
// awaited explicitly with exact counts before the barrier that publishes a
// tile, and block-id scalar loads may stay in flight across it.
__device__ __forceinline__ void phase_sync() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Scalar load of base[idx] (idx uniform), issued where it stands; its value
// may be used only after an lgkmcnt(0) wait tied to it.  Block-table entries
// are read this way so that the compiler can neither move the load next to
// its use (where the wait would also stall the in-flight LDS reads) nor wait
// on it early.
__device__ __forceinline__ int sload(const int32_t *base, int idx) {
  int v;
  asm volatile("s_load_dword %0, %1, %2" : "=s"(v) : "s"(base), "s"(idx * 4) : "memory");
  return v;
}

// Host side.  Work items are (sequence, kv head, head subgroup) pairs times
// query tiles of kRows * kWaves / heads_per_wg rows; the grid is persistent,
// a multiple of 8 work-groups, at most one per CU.  Returns the device in
// `dev` and the grid size in `grid`.
inline hipError_t prefill_setup(const PrefillLaunch &a, PrefillParams &p, long long &grid,
                                int &dev) {
  p.out = a.out;
  p.query = a.query;
  p.k_cache = a.k_cache;
  p.v_cache = a.v_cache;
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.query_start_loc = a.query_start_loc;
  p.num_heads = a.num_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_heads / a.num_kv_heads;
  p.heads_per_wg = (p.group % 4 == 0) ? 4 : (p.group % 2 == 0) ? 2 : 1;
  p.subgroups = p.group / p.heads_per_wg;
  p.pos_per_wg = kRows * (kWaves / p.heads_per_wg);
  int bl = 0;
  while ((1 << bl) < a.block_size) ++bl;
  p.bs_log2 = bl;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.ctx_cap = a.ctx_cap;
  p.num_seqs = a.num_seqs;
  p.scale_log2e = a.scale * kLog2e;
  const long long pairs = (long long)a.num_seqs * a.num_kv_heads * p.subgroups;
  const long long qtiles = (a.max_query_len + p.pos_per_wg - 1) / p.pos_per_wg;
  // Items of the XCD with the most; one work-group per CU at most.
  const long long xcd_items = ((pairs + kXcds - 1) / kXcds) * qtiles;
  if (xcd_items > 0x7fffffffLL) return hipErrorInvalidValue;
  int cus = 0;
  dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  grid = kXcds * std::min<long long>(std::max(cus / kXcds, 1), xcd_items);
  p.num_pairs = (int32_t)pairs;
  p.num_qtiles = (int32_t)qtiles;
  return hipSuccess;
}

// Allows `fn` lds_bytes of dynamic LDS on device `dev`.  The attribute
// belongs to the function on one device: bit d of the caller's
// per-instantiation mask records that device d has it (devices past 63 set
// it on every call).
inline hipError_t prefill_allow_lds(const void *fn, size_t lds_bytes, int dev,
                                    std::atomic<uint64_t> &attr_devices) {
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
  if (bit == 0 || (attr_devices.load(std::memory_order_relaxed) & bit) == 0) {
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
    attr_devices.fetch_or(bit, std::memory_order_relaxed);
  }
  return hipSuccess;
}

}  // namespace

}  // namespace pa

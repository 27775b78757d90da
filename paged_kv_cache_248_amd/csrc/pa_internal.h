// Internal launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

struct DecodeLaunch {
  void *out;
  const void *query;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int32_t num_seqs, num_heads, num_kv_heads, head_dim;
  int32_t block_size, num_blocks, max_blocks_per_seq;
  int32_t ctx_cap;      // min(max_context_len, max_blocks_per_seq * block_size)
  int32_t partition;    // tokens per partition (multiple of 64)
  int32_t max_parts;    // ceil(ctx_cap / partition)
  float scale;
  DType dtype;
  void *workspace;
};

// Workspace layout of the decode path, shared by size query and launcher.
struct DecodeWorkspace {
  size_t count_off, work_off, arrive_off, part_o_off, part_ml_off, total;
};
DecodeWorkspace decode_workspace_layout(int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads,
                                        int64_t head_dim, int64_t max_parts);

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream);

// Device address of this device's copy of the decode scratch array
// (PA_DECODE_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned), looked up once
// per device; nullptr if no device is current or the lookup fails.
void *decode_noalloc_scratch();

struct PrefillLaunch {
  void *out;
  const void *query;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start_loc;
  int32_t num_seqs, total_query_tokens, max_query_len, ctx_cap;
  int32_t num_heads, num_kv_heads, head_dim;
  int32_t block_size, num_blocks, max_blocks_per_seq;
  float scale;
  DType dtype;
};

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream);
// The same prefill with the half-tile schedule (prefill_halftile.hip).
hipError_t launch_prefill_halftile(const PrefillLaunch &a, hipStream_t stream);

// Bytes of a destination block one copy work-group moves (one 16-byte piece
// per lane of 256); the grid is one work-group per (pool, destination block,
// slice), so the argument checks bound it with the same figure.
constexpr int64_t kCopySliceBytes = 4096;

struct CopyLaunch {
  const void *src_k, *src_v;
  void *dst_k, *dst_v;
  const int64_t *src_to_dst;
  int64_t num_mappings, num_src, num_dst, block_bytes;
  int32_t *first_src;  // workspace, num_dst entries
};

hipError_t launch_copy_blocks(const CopyLaunch &a, hipStream_t stream);

struct AppendLaunch {
  void *k_cache, *v_cache;       // v_cache NULL: K only
  const void *key, *value;
  const int32_t *block_tables, *context_lens, *query_start_loc;
  int32_t num_seqs, total_tokens, num_kv_heads, head_dim, elem_bytes;
  int32_t block_size, num_blocks, max_blocks_per_seq;
};

hipError_t launch_append(const AppendLaunch &a, hipStream_t stream);

// Unfused (S and P in HBM) causal prefill, the baseline of the fused kernel.
struct UnfusedLaunch {
  void *out;
  const void *query;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;          // device
  const int32_t *context_lens;          // host
  const int32_t *query_start_loc;       // host
  int32_t num_seqs, max_q, max_ctx;     // max_q / max_ctx over the sequences
  int32_t num_heads, num_kv_heads, head_dim;
  int32_t block_size, num_blocks, max_blocks_per_seq;
  float scale;
  DType dtype;
  void *workspace;
};

// Scratch regions of one sequence (reused by the next): gathered K and V,
// grouped Q and O, S (fp32) and P with rows padded to 8 elements, and the
// matrix library's own workspace.
struct UnfusedWorkspace {
  size_t kg_off, vg_off, qg_off, og_off, s_off, p_off, blas_off, blas_bytes, total;
};
constexpr size_t kUnfusedBlasWorkspace = 64u << 20;
// Longest context the unfused softmax keeps in registers (1024 x 32 keys).
constexpr int32_t kUnfusedMaxContext = 32768;
UnfusedWorkspace unfused_workspace_layout(int64_t max_q, int64_t max_ctx, int64_t num_heads,
                                          int64_t num_kv_heads, int64_t head_dim,
                                          int64_t elem_bytes);

enum pa_gemm_status { PA_GEMM_OK = 0, PA_GEMM_NO_HANDLE, PA_GEMM_UNSUPPORTED, PA_GEMM_FAILED };
pa_gemm_status launch_prefill_unfused(const UnfusedLaunch &a, hipStream_t stream);

// Reads `bytes` (a multiple of 16) at src once; work-group i writes the XOR
// of the words it read to sink[i] (at most sink_words work-groups).
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t sink_words,
                              hipStream_t stream);

// Copies `bytes` (a multiple of 16) from src to dst once: one 4 KiB chunk
// per work-group (wgs_per_cu <= 0), or a grid-stride loop over at most
// wgs_per_cu work-groups per CU.
hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, int32_t wgs_per_cu,
                              hipStream_t stream);

// Matrix-core stream: min(CUs x wgs_per_cu, sink_words) work-groups of four
// wavefronts, each wavefront `iters` rounds of 32 v_mfma_f32_32x32x16 on
// operands read once from `ops` (ops_bytes, a multiple of 16); work-group i
// writes the sum of its accumulators to sink[i].
hipError_t launch_mfma_stream(const void *ops, int64_t ops_bytes, float *sink, int32_t sink_words,
                              int32_t wgs_per_cu, int32_t iters, DType dtype, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

// The caller's measurement events (pa_set_profile_events), or nullptr.
hipEvent_t profile_start_event();
hipEvent_t profile_stop_event();

// Launches a main kernel.  With measurement events set, the runtime records
// them as part of the kernel's own dispatch (start and end of its
// execution, the span a kernel trace reports), with no separate event
// packets in the stream; without them it is a plain launch.
template <class F, class... Args>
hipError_t launch_main(F kernel, dim3 grid, dim3 block, uint32_t lds_bytes, hipStream_t stream,
                       Args... args) {
  hipEvent_t start = profile_start_event(), stop = profile_stop_event();
  if (start && stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
  return hipGetLastError();
}

}  // namespace pa

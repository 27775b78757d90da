// C ABI entry points: host-side validation, workspace sizing and dispatch to
// the kernel launchers.  Declarations and the argument contract are in
// include/paged_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>

#include "../../include/paged_attn.h"
#include "pa_internal.h"

namespace pa {

int device_cu_count() {
  static std::atomic<int> cache[64];   // per device; 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {
hipEvent_t g_prof_start = nullptr;
hipEvent_t g_prof_stop = nullptr;
}  // namespace

hipEvent_t profile_start_event() { return g_prof_start; }
hipEvent_t profile_stop_event() { return g_prof_stop; }

}  // namespace pa

namespace {

bool pow2_in(int32_t v, int32_t lo, int32_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Partition length actually used (multiple of 64 tokens) and partition count.
bool decode_partition(int32_t ctx_cap, int32_t partition_size, int32_t group, int32_t *part,
                      int32_t *nparts) {
  int64_t P;
  if (partition_size == 0) P = group >= 4 ? PA_DEFAULT_PARTITION_GQA : PA_DEFAULT_PARTITION;
  else if (partition_size == -1) P = std::max<int64_t>(64, ((int64_t)ctx_cap + 63) / 64 * 64);
  else if (partition_size > 0 && partition_size % 64 == 0) P = partition_size;
  else return false;
  *part = (int32_t)P;
  *nparts = (int32_t)std::max<int64_t>(1, ((int64_t)ctx_cap + P - 1) / P);
  return true;
}

pa_status_t launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

bool device_ok() {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0;
}

}  // namespace

extern "C" {

pa_status_t pa_set_profile_events(void *start, void *stop) {
  if ((start == nullptr) != (stop == nullptr)) return PA_ERR_NULL;
  pa::g_prof_start = static_cast<hipEvent_t>(start);
  pa::g_prof_stop = static_cast<hipEvent_t>(stop);
  return PA_OK;
}

const char *pa_status_string(int32_t s) {
  // an int, not the enum: callers may pass any integer, and a C++ enum
  // object may not hold values outside its enumerators' range
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: dtype unknown or not supported by this operation";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid or inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim, block_size, partition or alignment not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing, too small or not 16-byte aligned";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: HIP reported an error while enqueueing";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE: no usable HIP device";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: no free physical block";
    case PA_ERR_REQUEST: return "PA_ERR_REQUEST: unknown or duplicate request id";
  }
  return "PA_ERR_UNKNOWN";
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_context_len,
                                        int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return 0;
  int32_t part = 0, nparts = 0;
  if (!decode_partition(std::max(max_context_len, 1), partition_size, num_heads / num_kv_heads,
                        &part, &nparts))
    return 0;
  return pa::decode_workspace_layout(num_seqs, num_heads, num_kv_heads, head_dim, nparts).total;
}

// Shared by paged_attn_decode (caller workspace) and paged_attn_decode_noalloc
// (noalloc: the library's static scratch array, workspace arguments unused).
static pa_status_t decode_call(void *out, const void *query, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, float scale, int32_t dtype,
                               int32_t partition_size, bool noalloc, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!pow2_in(block_size, 8, 256)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * num_heads * head_dim > INT32_MAX ||
      (int64_t)num_seqs * max_blocks_per_seq > INT32_MAX)
    return PA_ERR_SHAPE;
  const int32_t ctx_cap =
      (int32_t)std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size);
  int32_t part = 0, nparts = 0;
  if (!decode_partition(std::max(ctx_cap, 1), partition_size, num_heads / num_kv_heads, &part,
                        &nparts))
    return PA_ERR_UNSUPPORTED;
  if (nparts > PA_MAX_PARTITIONS) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || ctx_cap == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const pa::DecodeWorkspace ws =
      pa::decode_workspace_layout(num_seqs, num_heads, num_kv_heads, head_dim, nparts);
  if (noalloc) {
    if (ws.total > PA_DECODE_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  } else if (!workspace || !aligned16(workspace) || workspace_bytes < ws.total) {
    return PA_ERR_WORKSPACE;
  }
  if (!device_ok()) return PA_ERR_DEVICE;
  if (noalloc) {
    workspace = pa::decode_noalloc_scratch();
    if (!workspace) return PA_ERR_DEVICE;
  }
  pa::DecodeLaunch a;
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.ctx_cap = ctx_cap;
  a.partition = part;
  a.max_parts = nparts;
  a.scale = scale;
  a.dtype = (pa::DType)dtype;
  a.workspace = workspace;
  return launch_status(pa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

pa_status_t paged_attn_decode(void *out, const void *query, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables,
                              const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale, int32_t dtype,
                              int32_t partition_size, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return decode_call(out, query, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, dtype, partition_size, false,
                     workspace, workspace_bytes, stream);
}

pa_status_t paged_attn_decode_noalloc(void *out, const void *query, const void *k_cache,
                                      const void *v_cache, const int32_t *block_tables,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t dtype, int32_t partition_size,
                                      void *stream) {
  return decode_call(out, query, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, dtype, partition_size, true,
                     nullptr, 0, stream);
}

namespace {

pa_status_t prefill_call(void *out, const void *query, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *query_start_loc, int32_t num_seqs,
                         int32_t total_query_tokens, int32_t max_query_len,
                         int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, float scale, int32_t dtype, bool halftile,
                         void *stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_query_tokens < 0 || max_query_len < 0 || max_context_len < 0 ||
      num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_query_len > max_context_len)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!pow2_in(block_size, 8, 256)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)total_query_tokens * num_heads * head_dim > INT32_MAX ||
      (int64_t)num_seqs * max_blocks_per_seq > INT32_MAX)
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_query_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens ||
      !query_start_loc)
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  if (!device_ok()) return PA_ERR_DEVICE;
  pa::PrefillLaunch a;
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.total_query_tokens = total_query_tokens;
  a.max_query_len = max_query_len;
  a.ctx_cap =
      (int32_t)std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size);
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale = scale;
  a.dtype = (pa::DType)dtype;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return launch_status(halftile ? pa::launch_prefill_halftile(a, st) : pa::launch_prefill(a, st));
}

}  // namespace

pa_status_t paged_attn_prefill(void *out, const void *query, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, const int32_t *query_start_loc,
                               int32_t num_seqs, int32_t total_query_tokens,
                               int32_t max_query_len, int32_t max_context_len, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                               int32_t dtype, void *stream) {
  return prefill_call(out, query, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      num_seqs, total_query_tokens, max_query_len, max_context_len, num_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                      dtype, false, stream);
}

pa_status_t paged_attn_prefill_halftile(void *out, const void *query, const void *k_cache,
                                        const void *v_cache, const int32_t *block_tables,
                                        const int32_t *context_lens,
                                        const int32_t *query_start_loc, int32_t num_seqs,
                                        int32_t total_query_tokens, int32_t max_query_len,
                                        int32_t max_context_len, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks,
                                        int32_t max_blocks_per_seq, float scale, int32_t dtype,
                                        void *stream) {
  return prefill_call(out, query, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      num_seqs, total_query_tokens, max_query_len, max_context_len, num_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, scale,
                      dtype, true, stream);
}

size_t paged_attn_prefill_unfused_workspace_size(int32_t max_query_len, int32_t max_context_len,
                                                 int32_t num_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t dtype) {
  if ((dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) || max_query_len < 0 ||
      max_context_len < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return 0;
  return pa::unfused_workspace_layout(max_query_len, max_context_len, num_heads, num_kv_heads,
                                      head_dim, 2)
      .total;
}

pa_status_t paged_attn_prefill_unfused(void *out, const void *query, const void *k_cache,
                                       const void *v_cache, const int32_t *block_tables,
                                       const int32_t *context_lens_host,
                                       const int32_t *query_start_loc_host, int32_t num_seqs,
                                       int32_t total_query_tokens, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                                       int32_t dtype, void *workspace, size_t workspace_bytes,
                                       void *stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_query_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!pow2_in(block_size, 8, 256)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)total_query_tokens * num_heads * head_dim > INT32_MAX ||
      (int64_t)num_seqs * max_blocks_per_seq > INT32_MAX)
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_query_tokens == 0) return PA_OK;
  if (!context_lens_host || !query_start_loc_host) return PA_ERR_NULL;
  // The lengths are host arrays here (the library GEMMs take host-side
  // shapes), so their contents are checked, not clamped.
  if (query_start_loc_host[0] != 0 || query_start_loc_host[num_seqs] != total_query_tokens)
    return PA_ERR_SHAPE;
  int32_t max_q = 0, max_ctx = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t q = query_start_loc_host[b + 1] - query_start_loc_host[b];
    const int32_t n = context_lens_host[b];
    if (q < 0 || n < q || (int64_t)n > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
    if (q > 0 && n > pa::kUnfusedMaxContext) return PA_ERR_UNSUPPORTED;
    max_q = std::max(max_q, q);
    if (q > 0) max_ctx = std::max(max_ctx, n);
  }
  if (max_q == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < paged_attn_prefill_unfused_workspace_size(max_q, max_ctx, num_heads,
                                                                  num_kv_heads, head_dim, dtype))
    return PA_ERR_WORKSPACE;
  if (!device_ok()) return PA_ERR_DEVICE;
  pa::UnfusedLaunch a;
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens_host;
  a.query_start_loc = query_start_loc_host;
  a.num_seqs = num_seqs;
  a.max_q = max_q;
  a.max_ctx = max_ctx;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale = scale;
  a.dtype = (pa::DType)dtype;
  a.workspace = workspace;
  switch (pa::launch_prefill_unfused(a, static_cast<hipStream_t>(stream))) {
    case pa::PA_GEMM_OK: return PA_OK;
    case pa::PA_GEMM_NO_HANDLE: return PA_ERR_DEVICE;
    case pa::PA_GEMM_UNSUPPORTED: return PA_ERR_UNSUPPORTED;
    default: return PA_ERR_LAUNCH;
  }
}

pa_status_t paged_kv_append(void *k_cache, void *v_cache, const void *key, const void *value,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const int32_t *query_start_loc, int32_t num_seqs,
                            int32_t total_tokens, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t dtype, void *stream) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  const int32_t elem = dtype == PA_DTYPE_F32 ? 4 : 2;
  if (num_seqs < 0 || total_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if ((head_dim * elem) % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (!pow2_in(block_size, 8, 256)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * max_blocks_per_seq > INT32_MAX ||
      (int64_t)max_blocks_per_seq * block_size > INT32_MAX ||
      (int64_t)num_kv_heads * head_dim * elem > INT32_MAX / 2)
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_tokens == 0) return PA_OK;
  if (!k_cache || !key || !block_tables || !context_lens || !query_start_loc) return PA_ERR_NULL;
  if ((v_cache == nullptr) != (value == nullptr)) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(key) || (v_cache && (!aligned16(v_cache) || !aligned16(value))))
    return PA_ERR_UNSUPPORTED;
  if (!device_ok()) return PA_ERR_DEVICE;
  pa::AppendLaunch a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.key = key;
  a.value = value;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.elem_bytes = elem;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  return launch_status(pa::launch_append(a, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t sink_words,
                           void *stream) {
  if (bytes < 0 || sink_words <= 0) return PA_ERR_SHAPE;
  if (bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return PA_ERR_NULL;
  if (!aligned16(src)) return PA_ERR_UNSUPPORTED;
  if (!device_ok()) return PA_ERR_DEVICE;
  return launch_status(
      pa::launch_stream_read(src, bytes, sink, sink_words, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_stream_copy(const void *src, void *dst, int64_t bytes, int32_t wgs_per_cu,
                           void *stream) {
  if (bytes < 0) return PA_ERR_SHAPE;
  if (bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (bytes == 0) return PA_OK;
  if (!src || !dst) return PA_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return PA_ERR_UNSUPPORTED;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return PA_ERR_SHAPE;   // overlap
  if (!device_ok()) return PA_ERR_DEVICE;
  return launch_status(
      pa::launch_stream_copy(src, dst, bytes, wgs_per_cu, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_mfma_stream(const void *operands, int64_t operand_bytes, float *sink,
                           int32_t sink_words, int32_t wgs_per_cu, int32_t iters, int32_t dtype,
                           void *stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (operand_bytes < 4096 || sink_words <= 0 || wgs_per_cu < 1 || wgs_per_cu > 8 || iters <= 0)
    return PA_ERR_SHAPE;
  if (operand_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (!operands || !sink) return PA_ERR_NULL;
  if (!aligned16(operands)) return PA_ERR_UNSUPPORTED;
  if (!device_ok()) return PA_ERR_DEVICE;
  return launch_status(pa::launch_mfma_stream(operands, operand_bytes, sink, sink_words,
                                              wgs_per_cu, iters, (pa::DType)dtype,
                                              static_cast<hipStream_t>(stream)));
}

pa_status_t pa_host_device_pointer(void *host_ptr, void **device_ptr) {
  if (!host_ptr || !device_ptr) return PA_ERR_NULL;
  *device_ptr = nullptr;
  void *d = nullptr;
  if (hipHostGetDevicePointer(&d, host_ptr, 0) != hipSuccess || !d) {
    (void)hipGetLastError();    // leave no sticky error for the next call
    return PA_ERR_UNSUPPORTED;
  }
  *device_ptr = d;
  return PA_OK;
}

size_t paged_kv_copy_blocks_workspace_size(int64_t num_dst_blocks) {
  if (num_dst_blocks < 0) return 0;
  return (size_t)std::max<int64_t>(num_dst_blocks, 1) * sizeof(int32_t);
}

pa_status_t paged_kv_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                                 const int64_t *src_to_dst, int64_t num_mappings,
                                 int64_t num_src_blocks, int64_t num_dst_blocks,
                                 int64_t block_bytes, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  if (num_mappings < 0 || num_mappings >= (int64_t)INT32_MAX || num_src_blocks < 0 ||
      num_dst_blocks < 0 || block_bytes <= 0)
    return PA_ERR_SHAPE;
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  const int64_t slices = (block_bytes + pa::kCopySliceBytes - 1) / pa::kCopySliceBytes;
  // one work-group per (pool, destination block, slice)
  if (num_dst_blocks > 0 && slices > (int64_t)(INT32_MAX / 2) / num_dst_blocks) return PA_ERR_SHAPE;
  if (num_mappings == 0 || num_dst_blocks == 0 || num_src_blocks == 0) return PA_OK;
  if (!src_k || !dst_k || !src_to_dst) return PA_ERR_NULL;
  if ((src_v == nullptr) != (dst_v == nullptr)) return PA_ERR_NULL;
  if (!aligned16(src_k) || !aligned16(dst_k) || (src_v && (!aligned16(src_v) || !aligned16(dst_v))))
    return PA_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < paged_kv_copy_blocks_workspace_size(num_dst_blocks))
    return PA_ERR_WORKSPACE;
  if (!device_ok()) return PA_ERR_DEVICE;
  pa::CopyLaunch a;
  a.src_k = src_k;
  a.src_v = src_v;
  a.dst_k = dst_k;
  a.dst_v = dst_v;
  a.src_to_dst = src_to_dst;
  a.num_mappings = num_mappings;
  a.num_src = num_src_blocks;
  a.num_dst = num_dst_blocks;
  a.block_bytes = block_bytes;
  a.first_src = static_cast<int32_t *>(workspace);
  return launch_status(pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

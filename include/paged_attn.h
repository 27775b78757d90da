/*
 * paged_attn.h — C ABI of the MI355X (gfx950) paged-attention library.
 *
 * Three operations, on one GPU:
 *   paged_attn_decode     one query token per sequence attends to its cached
 *                         keys/values, read through a block table;
 *   paged_attn_prefill    the new tokens of each sequence attend causally to
 *                         the cached prefix and to each other;
 *   paged_kv_copy_blocks  copies whole cache blocks between two pools by a
 *                         src_to_dst mapping.
 * Beside them: paged_kv_append (writes new tokens' K/V into their slots), a
 * host block manager (pa_bm_*) that produces block tables,
 * paged_attn_prefill_unfused, the unfused baseline of prefill, and
 * paged_attn_prefill_halftile, the same prefill with a second kernel
 * schedule for comparison.
 *
 * Pages the operations follow (cited by title):
 *   [P-swap] "vLLM中FlashAttention与KVCache交换机制解析"
 *   [P-wall] "大模型长文本推理基座从 FlashAttention 硬件加速机制到 vLLM 核心
 *             PagedAttention 显存物理布局深度剖析"
 *   [P-opt]  "vLLM中FlashAttention与KVCache优化解析"
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers on the current HIP device,
 *     allocated and owned by the caller.  The library allocates and frees
 *     nothing and keeps no pointer after a call returns.  (Exceptions, stated
 *     where they are declared: the block manager lives in host memory it
 *     allocates, the unfused baseline takes host length arrays and creates a
 *     matrix-library handle, and the copy accepts pinned host pools.)
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream);
 *     it belongs to the current HIP device, like the arrays.  The library's
 *     per-device state (CU count, kernel attributes, the matrix-library
 *     handle) is keyed by the current device.  Calls only enqueue work:
 *     they return before the GPU finishes, never synchronise, and are safe
 *     to call from several host threads on different streams.  Calls that
 *     share a workspace must not overlap.
 *   - Every call validates its host-side arguments first and returns a
 *     pa_status_t; nothing is launched unless the result is PA_OK.  Errors
 *     never abort or throw.  A launch failure reported by HIP is PA_ERR_LAUNCH.
 *   - Arrays are dense and row-major with the shapes given below (no strides).
 *   - Device-side contents are not validated (that would need a device read):
 *     out-of-range block ids are clamped into the pool and context lengths are
 *     clamped to [0, min(max_context_len, max_blocks_per_seq*block_size)], so
 *     a bad table gives a meaningless result but never a memory fault.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,         /* a required pointer is NULL                       */
  PA_ERR_DTYPE = -2,        /* unknown dtype, or a dtype the operation lacks    */
  PA_ERR_SHAPE = -3,        /* a size is negative/zero where it must not be, or
                               sizes are inconsistent (e.g. heads % kv_heads)   */
  PA_ERR_UNSUPPORTED = -4,  /* valid but not built: head_dim, block_size,
                               partition size, alignment                        */
  PA_ERR_WORKSPACE = -5,    /* workspace NULL, smaller than the query says, or
                               not 16-byte aligned                              */
  PA_ERR_LAUNCH = -6,       /* HIP reported an error while enqueueing           */
  PA_ERR_DEVICE = -7,       /* no usable HIP device is current                  */
  PA_ERR_NO_BLOCKS = -8,    /* block manager: no free physical block            */
  PA_ERR_REQUEST = -9       /* block manager: unknown or duplicate request id   */
} pa_status_t;

/* Element types.  Entry points take the dtype as an int32_t holding one of
 * these values; any other integer gives PA_ERR_DTYPE. */
typedef enum { PA_DTYPE_F32 = 0, PA_DTYPE_F16 = 1, PA_DTYPE_BF16 = 2 } pa_dtype_t;

/* Library default KV partition length, in tokens, for split-KV decode:
 * PA_DEFAULT_PARTITION_GQA when num_heads / num_kv_heads >= 4 (each K/V
 * tile then feeds several heads, and longer partitions cut the per-item
 * overhead; measured fastest on the GQA workload), else PA_DEFAULT_PARTITION. */
#define PA_DEFAULT_PARTITION 512
#define PA_DEFAULT_PARTITION_GQA 4096
/* Most partitions one decode sequence may be split into
 * (ceil(min(max_context_len, max_blocks_per_seq*block_size) / partition)). */
#define PA_MAX_PARTITIONS 2048

/* Human-readable name of a status code (static string, never NULL).  Any
 * integer is accepted: values that are not a pa_status_t give
 * "PA_ERR_UNKNOWN". */
const char *pa_status_string(int32_t status);

/* --------------------------------------------------------------------------
 * Paged decode.
 *
 * Computes, for every sequence b and query head h,
 *   out[b,h,:] = softmax(scale * q[b,h,:] . K_b^T) V_b
 * where K_b/V_b are the first context_lens[b] cached rows of kv head
 * g = h / (num_heads/num_kv_heads), gathered in logical order: row j lives in
 * physical block block_tables[b, j / block_size], slot j % block_size.
 * This is scaled dot-product attention (formula at the top of [P-swap]) over
 * the PagedAttention cache ([P-wall] §二.2; [P-opt] "Block Table 管理"), with
 * query heads of a GQA group sharing one kv head by indexing, not by copying
 * ([P-swap], the MQA/GQA remarks).  Long contexts are cut into partitions of
 * `partition_size` tokens whose partial (M, L, O) states are merged with the
 * rescaling of the OnlineSoftmax update ([P-swap], M_new/L_new/O_new).
 *
 *   out          [num_seqs, num_heads, head_dim]                 dtype, written
 *   query        [num_seqs, num_heads, head_dim]                 dtype
 *   k_cache      [num_blocks, num_kv_heads, block_size, head_dim] dtype
 *   v_cache      [num_blocks, num_kv_heads, block_size, head_dim] dtype
 *   block_tables [num_seqs, max_blocks_per_seq] int32 physical block ids;
 *                entries past ceil(context_len/block_size) are never read
 *   context_lens [num_seqs] int32, keys attended per sequence (the current
 *                token's own K/V included), 1 <= context_lens[b] <= max_context_len
 *   max_context_len  host-side upper bound of context_lens (sizes the work)
 *   scale        softmax scale (normally 1/sqrt(head_dim))
 *   partition_size  tokens per split-KV partition: 0 = the library default,
 *                a positive multiple of 64, or -1 = never split; at most
 *                PA_MAX_PARTITIONS partitions per sequence (else
 *                PA_ERR_UNSUPPORTED)
 *   workspace    device scratch of at least
 *                paged_attn_decode_workspace_size(...) bytes, 16-byte aligned
 *                (else PA_ERR_WORKSPACE: the kernels read its work list with
 *                scalar loads and update its counter atomically); contents on
 *                entry are ignored and are clobbered
 *
 * Supported: dtype f32/f16/bf16 (query, caches and out share it; arithmetic
 * is fp32), head_dim 64 or 128, block_size a power of two in [8, 256],
 * num_heads % num_kv_heads == 0.  A sequence with context_lens[b] < 1 leaves
 * out[b] unwritten.
 * ------------------------------------------------------------------------ */
size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t partition_size);

pa_status_t paged_attn_decode(void *out, const void *query, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables,
                              const int32_t *context_lens, int32_t num_seqs,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len,
                              float scale, int32_t dtype, int32_t partition_size,
                              void *workspace, size_t workspace_bytes, void *stream);

/* --------------------------------------------------------------------------
 * Paged decode that allocates nothing.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, arguments, kernels and result as paged_attn_decode, bit for bit,
 * but without a workspace argument.  The work list, counters and split-KV
 * partials live in a static device array of PA_DECODE_NOALLOC_SCRATCH_BYTES
 * bytes inside the library; each GPU the library runs on holds its own copy
 * from the first call on it until the process ends.  A call whose
 * paged_attn_decode_workspace_size(...) exceeds that size returns
 * PA_ERR_WORKSPACE before launching anything (64 MiB holds, e.g., 128
 * sequences x 32 heads x 16 partitions of head_dim 128).  The array keeps the
 * last call's contents; every call re-initialises what it reads.  All calls
 * on one GPU share the array: calls that may overlap in time on one GPU (two
 * streams, two host threads) race and must be serialised by the caller.
 * The call performs no hipMalloc/hipFree and calls no allocating library
 * routine; the first call on a device looks up the array's device address.
 * ------------------------------------------------------------------------ */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

pa_status_t paged_attn_decode_noalloc(void *out, const void *query, const void *k_cache,
                                      const void *v_cache, const int32_t *block_tables,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t dtype, int32_t partition_size,
                                      void *stream);

/* --------------------------------------------------------------------------
 * Causal paged prefill / append.
 *
 * The new tokens of sequence b are rows query_start_loc[b] ..
 * query_start_loc[b+1]-1 of the packed `query`; with q_b of them and
 * n = context_lens[b] keys in the cache (prefix + new, all already written),
 * new token t sits at position n - q_b + t and attends to keys 0..n-q_b+t
 * (bottom-right causal alignment).  This is the prefill step of the serving
 * flow in [P-swap] (prefill through FlashAttention over the paged cache),
 * computed with tiled QK^T and PV and the OnlineSoftmax update, with S and P
 * never leaving the chip ([P-swap] Kernel Fusion + Tiling + OnlineSoftmax).
 *
 *   out, query       [total_query_tokens, num_heads, head_dim] dtype
 *   k_cache, v_cache [num_blocks, num_kv_heads, block_size, head_dim] dtype
 *   block_tables     [num_seqs, max_blocks_per_seq] int32
 *   context_lens     [num_seqs] int32, prefix + new keys
 *   query_start_loc  [num_seqs + 1] int32, non-decreasing, [0] = 0,
 *                    [num_seqs] = total_query_tokens, and
 *                    q_b <= context_lens[b] for every b
 *   max_query_len    host-side upper bound of q_b
 *   max_context_len  host-side upper bound of context_lens
 *
 * Supported: dtype f16/bf16 (matrix-core arithmetic with fp32 accumulation;
 * f32 returns PA_ERR_DTYPE), head_dim 64 or 128, block_size a power of two
 * in [8, 256], num_heads % num_kv_heads == 0, scale finite and > 0 (else
 * PA_ERR_UNSUPPORTED).  The softmax weights P enter the PV product rounded to
 * the input dtype; the normaliser L sums them in fp32.  Needs no workspace.
 * ------------------------------------------------------------------------ */
pa_status_t paged_attn_prefill(void *out, const void *query, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, const int32_t *query_start_loc,
                               int32_t num_seqs, int32_t total_query_tokens,
                               int32_t max_query_len, int32_t max_context_len,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, float scale, int32_t dtype,
                               void *stream);

/* --------------------------------------------------------------------------
 * The same causal paged prefill with a second kernel schedule.
 *
 * Computes exactly what paged_attn_prefill computes (same arguments, same
 * layouts, same validation and status codes, no workspace) with the
 * half-tile schedule: each wavefront interleaves tile j+1's QK^T with tile
 * j's softmax and PV, instead of paged_attn_prefill's ping-pong of two
 * wavefront groups.  Kept so that the two schedules can be measured against
 * each other on one GPU; paged_attn_prefill, the faster of the two on
 * MI355X, is the one to call.
 * ------------------------------------------------------------------------ */
pa_status_t paged_attn_prefill_halftile(void *out, const void *query, const void *k_cache,
                                        const void *v_cache, const int32_t *block_tables,
                                        const int32_t *context_lens,
                                        const int32_t *query_start_loc, int32_t num_seqs,
                                        int32_t total_query_tokens, int32_t max_query_len,
                                        int32_t max_context_len, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks,
                                        int32_t max_blocks_per_seq, float scale, int32_t dtype,
                                        void *stream);

/* --------------------------------------------------------------------------
 * Unfused causal paged prefill (baseline).
 *
 * Computes exactly what paged_attn_prefill computes (same arguments, same
 * causal alignment, same result within rounding) the way plain attention
 * does it, which [P-wall] section 二.1 contrasts with FlashAttention: per
 * sequence the full score matrix S = scale * Q K^T (fp32) is written to HBM,
 * a row softmax with the causal mask reads it and writes P (input dtype),
 * and O = P V reads P back; the [P-opt] FlashAttention table lists the
 * stored P and the separate kernels as what fusion removes.  K and V are
 * first gathered through the block table into contiguous scratch.  The two
 * products are hipBLASLt GEMMs (fp32 accumulation).  It exists to measure
 * the fused kernel against; it is not meant for serving.
 *
 *   out, query, k_cache, v_cache, block_tables  as for paged_attn_prefill
 *                    (device)
 *   context_lens_host    [num_seqs] int32, HOST memory: prefix + new keys
 *   query_start_loc_host [num_seqs + 1] int32, HOST memory
 *   workspace        device scratch of at least
 *                    paged_attn_prefill_unfused_workspace_size(max q_b,
 *                    max context_lens over sequences with q_b > 0, ...)
 *                    bytes, 16-byte aligned; about
 *                    Hq*q*n*(4 + e) + 2*Hkv*n*D*e + 2*q*Hq*D*e + 64 MiB
 *                    (e = 2).  Calls sharing it must not overlap.
 *
 * The lengths live on the host because the library GEMMs take host-side
 * shapes; their contents are validated (query_start_loc_host[0] = 0, last
 * entry = total_query_tokens, 0 <= q_b <= context_lens_host[b] <=
 * max_blocks_per_seq*block_size; else PA_ERR_SHAPE).  Supported: f16/bf16,
 * head_dim 64 or 128, block_size a power of two in [8, 256], contexts of
 * sequences with new tokens up to 32768 keys (else PA_ERR_UNSUPPORTED, as
 * when the matrix library finds no kernel for a shape).  The first call on a
 * device creates a hipBLASLt handle there, which lives until the process
 * ends; a failure to create it is PA_ERR_DEVICE.  Work is enqueued on
 * `stream` one sequence after another; if an error is returned after the
 * first sequence was enqueued, the rows of the earlier sequences may already
 * be written.
 * ------------------------------------------------------------------------ */
size_t paged_attn_prefill_unfused_workspace_size(int32_t max_query_len, int32_t max_context_len,
                                                 int32_t num_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t dtype);
pa_status_t paged_attn_prefill_unfused(void *out, const void *query, const void *k_cache,
                                       const void *v_cache, const int32_t *block_tables,
                                       const int32_t *context_lens_host,
                                       const int32_t *query_start_loc_host, int32_t num_seqs,
                                       int32_t total_query_tokens, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                                       int32_t dtype, void *workspace, size_t workspace_bytes,
                                       void *stream);

/* --------------------------------------------------------------------------
 * Block copy by mapping.
 *
 * src_to_dst[i] = j asks for source block i to be copied into destination
 * block j ([P-swap], swap_blocks and its mapping argument); -1 (or any value
 * outside [0, num_dst_blocks)) is ignored.  When several i name the same j,
 * only the lowest such i is considered, and it is copied only if
 * i < num_src_blocks.  Destination blocks nobody names keep their bytes.  The
 * K pool pair and the V pool pair are copied with the same mapping in one
 * call ([P-opt] "Swap Blocks 机制": K and V swapped separately, same map).
 * Copies are bytewise (NaN payloads and -0 survive).
 *
 *   src_k, src_v  [num_src_blocks, block_bytes] bytes (any element type)
 *   dst_k, dst_v  [num_dst_blocks, block_bytes] bytes; src_v and dst_v may
 *                 both be NULL to copy one pool only
 *   src_to_dst    [num_mappings] int64
 *   block_bytes   bytes per block, a positive multiple of 16; every pool
 *                 pointer 16-byte aligned
 *   workspace     device scratch of at least
 *                 paged_kv_copy_blocks_workspace_size(num_dst_blocks) bytes,
 *                 16-byte aligned (else PA_ERR_WORKSPACE)
 *
 * Source and destination pools must not overlap.  num_mappings may be 0
 * (nothing is launched) and must be below 2^31.  The copy runs one
 * work-group per 4 KiB slice of each destination block of each pool, so
 * num_dst_blocks * ceil(block_bytes / 4096) must not exceed 2^30 - 1
 * (else PA_ERR_SHAPE).
 * ------------------------------------------------------------------------ */
size_t paged_kv_copy_blocks_workspace_size(int64_t num_dst_blocks);

/* Device-accessible address of pinned host memory allocated with
 * hipHostMalloc (torch's pin_memory=True): with it, either pool pair of
 * paged_kv_copy_blocks may live in host memory, which turns the block copy
 * into the host<->device swap of [P-wall] §四.1 (swap out: device -> host
 * pool; swap in: host -> device pool), the kernel reading or writing host
 * memory over the host link.  Returns PA_ERR_NULL for NULL arguments and
 * PA_ERR_UNSUPPORTED when host_ptr is not such memory (*device_ptr is then
 * NULL). */
pa_status_t pa_host_device_pointer(void *host_ptr, void **device_ptr);

pa_status_t paged_kv_copy_blocks(const void *src_k, const void *src_v, void *dst_k,
                                 void *dst_v, const int64_t *src_to_dst, int64_t num_mappings,
                                 int64_t num_src_blocks, int64_t num_dst_blocks,
                                 int64_t block_bytes, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* --------------------------------------------------------------------------
 * Paged KV append: write the K and V rows of newly computed tokens into the
 * slots their block tables give them ([P-opt], the PagedKVCache sketch of the
 * PagedAttention section: append adds a sequence's new KV rows after its
 * cached ones through its block table; [P-wall] §二.2: logical token j lives
 * in block block_tables[b][j / block_size] at row j % block_size).
 *
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_dim]
 *                 pools, written in place; v_cache and value may both be
 *                 NULL to append K only
 *   key, value    [total_tokens, num_kv_heads, head_dim] rows of the new
 *                 tokens, packed by sequence: sequence b owns rows
 *                 query_start_loc[b] .. query_start_loc[b + 1] - 1
 *   block_tables  [num_seqs, max_blocks_per_seq] int32, entries for every
 *                 block the new tokens reach already allocated
 *   context_lens  [num_seqs] int32, tokens cached AFTER the append (prefix +
 *                 new, as for paged_attn_prefill): new token i of sequence b,
 *                 with q_b new tokens, is logical token context_lens[b] - q_b + i
 *   query_start_loc  [num_seqs + 1] int32, non-decreasing from 0 to
 *                 total_tokens
 *   head_dim      head_dim * element bytes a multiple of 16; block_size a
 *                 power of two in [8, 256]; every pool and row pointer
 *                 16-byte aligned
 *
 * Bytes are copied unchanged.  A token whose position is negative or at or
 * past max_blocks_per_seq * block_size, or whose table entry is outside
 * [0, num_blocks), is skipped; no other slot is written.  Two new tokens that
 * name the same slot leave either one's row there.  The call is asynchronous
 * on `stream`; total_tokens == 0 or num_seqs == 0 launches nothing.
 * ------------------------------------------------------------------------ */
pa_status_t paged_kv_append(void *k_cache, void *v_cache, const void *key, const void *value,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const int32_t *query_start_loc, int32_t num_seqs,
                            int32_t total_tokens, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t dtype, void *stream);

/* --------------------------------------------------------------------------
 * Host block manager ([P-wall] §三, the allocator simulator; §四.2, prefix
 * sharing and copy-on-write): the producer of the block tables the kernels
 * read.  Host memory only; no HIP call.  Not thread-safe: one manager is used
 * by one thread at a time.
 *
 * Physical blocks 0 .. num_blocks-1 start free.  An allocation takes the
 * lowest free id and gives it a reference count of 1; a release lowers the
 * count and frees the block at 0.  A request's table lists its blocks in
 * logical order and always holds ceil(tokens / block_size) of them.
 *
 *   pa_bm_create      num_blocks >= 1, block_size >= 1; *out receives the
 *                     manager (free with pa_bm_destroy)
 *   pa_bm_register    a new request with prompt_len tokens: allocates
 *                     ceil(prompt_len / block_size) blocks.  PA_ERR_NO_BLOCKS
 *                     (nothing kept) if they are not all free;
 *                     PA_ERR_REQUEST if the id is in use
 *   pa_bm_append_token  one more token: when the request's blocks are full a
 *                     block is added; when its last block is partly filled
 *                     and shared (count > 1) it is copied first: a new block
 *                     replaces it in the table, the old one is released, and
 *                     *cow_src / *cow_dst receive (old, new) so the caller can
 *                     copy the block's K and V (paged_kv_copy_blocks); else
 *                     both receive -1.  PA_ERR_NO_BLOCKS leaves the request
 *                     unchanged
 *   pa_bm_append_tokens  one decode step: one more token for each of the
 *                     num_requests listed requests, in list order, exactly
 *                     as that many pa_bm_append_token calls; cow_src[i] /
 *                     cow_dst[i] (arrays of num_requests, may be NULL)
 *                     receive request i's pair.  All or nothing: an unknown
 *                     or repeated id (PA_ERR_REQUEST) or too few free blocks
 *                     for the whole batch (PA_ERR_NO_BLOCKS) changes nothing
 *   pa_bm_fork        child_id shares every block of parent_id (each count
 *                     + 1) and starts with its token count (prefix sharing)
 *   pa_bm_finish      releases every block of the request and forgets it
 *   pa_bm_free_count  number of free blocks (or -1 for NULL)
 *   pa_bm_block_table  copies up to `capacity` block ids of the request into
 *                     blocks[], its block count into *num_blocks and its token
 *                     count into *num_tokens (either may be NULL);
 *                     PA_ERR_SHAPE if capacity is smaller than the count
 *   pa_bm_free_list   the free block ids in increasing order (same contract)
 *   pa_bm_ref_count   reference count of one block
 *   pa_bm_fill_batch  the kernels' block_tables [n, max_blocks_per_seq]
 *                     (unused entries -1) and context_lens [n] for a batch of
 *                     requests, host arrays; PA_ERR_SHAPE if a request holds
 *                     more than max_blocks_per_seq blocks
 * ------------------------------------------------------------------------ */
typedef struct pa_block_manager pa_block_manager;

pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager **out);
void pa_bm_destroy(pa_block_manager *bm);
pa_status_t pa_bm_register(pa_block_manager *bm, int64_t request_id, int64_t prompt_len);
pa_status_t pa_bm_append_token(pa_block_manager *bm, int64_t request_id, int32_t *cow_src,
                               int32_t *cow_dst);
pa_status_t pa_bm_append_tokens(pa_block_manager *bm, const int64_t *request_ids,
                                int32_t num_requests, int32_t *cow_src, int32_t *cow_dst);
pa_status_t pa_bm_fork(pa_block_manager *bm, int64_t parent_id, int64_t child_id);
pa_status_t pa_bm_finish(pa_block_manager *bm, int64_t request_id);
int32_t pa_bm_free_count(const pa_block_manager *bm);
pa_status_t pa_bm_block_table(const pa_block_manager *bm, int64_t request_id, int32_t *blocks,
                              int32_t capacity, int32_t *num_blocks, int64_t *num_tokens);
pa_status_t pa_bm_free_list(const pa_block_manager *bm, int32_t *blocks, int32_t capacity,
                            int32_t *num_blocks);
pa_status_t pa_bm_ref_count(const pa_block_manager *bm, int32_t block, int32_t *count);
pa_status_t pa_bm_fill_batch(const pa_block_manager *bm, const int64_t *request_ids,
                             int32_t num_requests, int32_t max_blocks_per_seq,
                             int32_t *block_tables, int32_t *context_lens);

/* --------------------------------------------------------------------------
 * Measurement hook.
 *
 * With non-NULL events (hipEvent_t passed as void*, created by the caller
 * with timing enabled), every later call has the runtime record `start` and
 * `stop` as part of its main kernel's dispatch (decode: the attention
 * kernel; prefill: the attention kernel; copy: the copy kernel; append: the
 * append kernel): the two events bracket that kernel's execution, the span a
 * kernel trace reports, and add no packets of their own to the stream, so
 * the caller can read the kernel's duration with hipEventElapsedTime.  Pass
 * NULL, NULL to stop recording (calls then launch plainly); leave them
 * unset while capturing a HIP graph, whose launches must be plain.  The
 * setting is process-wide and not synchronised: set it from the thread that
 * issues the calls being measured.  Returns PA_ERR_NULL if exactly one event
 * is NULL.
 * ------------------------------------------------------------------------ */
pa_status_t pa_set_profile_events(void *start, void *stop);

/* --------------------------------------------------------------------------
 * Read-stream probe (measurement only).
 *
 * Reads the `bytes` bytes at `src` (device, 16-byte aligned, bytes a
 * multiple of 16, else PA_ERR_UNSUPPORTED) once with non-temporal 16-byte
 * loads spread over the whole GPU.  Work-group i writes the XOR of the 32-bit
 * words it read to sink[i] (device, `sink_words` > 0 entries; at most that
 * many work-groups run, and entries past the grid are left untouched), so
 * the XOR of a zeroed sink after the call is the XOR of the whole buffer.
 * Its achieved GB/s is the practical HBM read ceiling that the
 * read-dominated decode kernels are set beside (decode moves K/V once; the
 * pages give an HBM figure only for an older GPU, [P-wall] section 二, the
 * HBM/SRAM diagram).  Recorded by pa_set_profile_events like a main kernel.
 * ------------------------------------------------------------------------ */
pa_status_t pa_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t sink_words,
                           void *stream);

/* --------------------------------------------------------------------------
 * Copy-stream probe (measurement only).
 *
 * Copies the `bytes` bytes at `src` to `dst` (device, both 16-byte aligned,
 * bytes a multiple of 16, else PA_ERR_UNSUPPORTED; overlapping ranges are
 * PA_ERR_SHAPE) with the non-temporal 16-byte loads and stores the block
 * copy and the KV append issue.  wgs_per_cu <= 0: one 4 KiB chunk per
 * work-group (the fastest shape measured); > 0: a grid-stride loop over at
 * most wgs_per_cu work-groups per CU.  Its achieved GB/s (bytes read plus
 * bytes written) is the practical read+write ceiling those two kernels are
 * set beside (the block copy of [P-swap] swap_blocks moves every byte once
 * in each direction).  Recorded by pa_set_profile_events like a main kernel.
 * ------------------------------------------------------------------------ */
pa_status_t pa_stream_copy(const void *src, void *dst, int64_t bytes, int32_t wgs_per_cu,
                           void *stream);

/* --------------------------------------------------------------------------
 * Matrix-core stream probe (measurement only).
 *
 * Runs min(CUs x wgs_per_cu, sink_words) work-groups of four wavefronts
 * (wgs_per_cu in [1, 8]); every wavefront performs `iters` (> 0) rounds of
 * 32 back-to-back v_mfma_f32_32x32x16 (dtype PA_DTYPE_F16 or PA_DTYPE_BF16)
 * on eight A and eight B operand fragments per lane that it reads once from
 * `operands` (device, 16-byte aligned, operand_bytes >= 4096 and a multiple
 * of 16; fragments are taken modulo the buffer, which should hold random
 * data of the dtype), into four independent fp32 accumulators.  Work-group
 * i writes the sum of its accumulators to sink[i] (device fp32).  Each
 * work-group does 4 x iters x 32 x 32768 flops.  Its achieved TFLOP/s is the
 * matrix cores' practical rate under the power limit for such data, with no
 * memory or softmax work beside it: the ceiling the prefill (a dense
 * contraction, [P-opt] 核心思想) is set beside.  Errors: PA_ERR_DTYPE,
 * PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (size or alignment), PA_ERR_NULL,
 * PA_ERR_DEVICE.  Recorded by pa_set_profile_events like a main kernel.
 * ------------------------------------------------------------------------ */
pa_status_t pa_mfma_stream(const void *operands, int64_t operand_bytes, float *sink,
                           int32_t sink_words, int32_t wgs_per_cu, int32_t iters, int32_t dtype,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */

// Paged KV append for gfx950: the K and V rows of newly computed tokens are
// written into the slots their sequences' block tables give them.
//
// Method (pages cited by title):
//   * the PagedKVCache sketch of "vLLM中FlashAttention与KVCache优化解析"
//     (PagedAttention section): append adds a sequence's new KV rows after
//     its cached ones, in pool blocks reached through its block table;
//   * logical token j of a sequence lives in physical block
//     block_table[j / block_size] at row j % block_size —
//     "大模型长文本推理基座…PagedAttention 显存物理布局深度剖析" §二.2;
//   * context_lens counts the tokens cached after the append (as prefill
//     does), so new token i of a sequence with q_b new tokens is logical token
//     context_lens[b] - q_b + i.
//
// Design for CDNA4 (HBM-bound scatter: every byte is read once and written
// once):
//   * a work-group owns a run of 8 consecutive new tokens (rows of the
//     packed [tokens, kv_heads, head_dim] inputs); each lane moves one
//     16-byte piece of every one of them (the K and V rows of a token are
//     2 * kv_heads * head_dim * elem / 16 pieces).  A lane first issues its
//     8 loads (they depend on nothing); meanwhile lanes 0-7 of the first
//     wavefront find the 8 destinations side by side, one token each (a
//     binary search of query_start_loc, then context_lens and the block
//     table), and publish them in LDS; after one barrier every lane stores.
//     The destinations cost a handful of dependent loads; one lane walking
//     the 8 tokens through scalar loads took some thirty, and the stores,
//     which wait for them, started that much later (4.6 against 5.1 TB/s on
//     the 134 MB append workload).  Rows are read and written once, with
//     non-temporal accesses;
//   * a token with no valid destination (position before 0 or past the table
//     row, or a table entry outside the pool) is skipped: nothing outside the
//     named slots is ever written.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kTokensPerGroup = 8;    // tokens per work-group (loads in flight per lane)

struct AppendParams {
  char *k_cache, *v_cache;
  const char *key, *value;
  const int32_t *block_tables, *context_lens, *query_start_loc;
  int32_t num_seqs, total_tokens, num_kv_heads, bs_log2, num_blocks, max_blocks_per_seq;
  int32_t head_bytes;     // one (token, kv head) row
  int32_t pieces;         // 16-byte pieces of one token in one tensor
  int32_t tensors;        // 2 (K and V) or 1 (K only)
};

__device__ __forceinline__ u32x4 ldnt(const char *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void stnt(char *p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  constexpr int NT = kTokensPerGroup;
  __shared__ long long s_row[NT];
  const int t_begin = blockIdx.x * NT;
  const int n_tok = min(NT, p.total_tokens - t_begin);
  const int bs = 1 << p.bs_log2;
  const int per_token = p.pieces * p.tensors;
  const int head_pieces = p.head_bytes >> 4;
  const size_t row_bytes = (size_t)p.pieces * 16;

  // Piece c of a token: tensor c / pieces, kv head (c mod pieces) /
  // head_pieces, 16-byte piece (c mod pieces) mod head_pieces of that row.
  auto piece_src = [&](int c) {
    const int tensor = c >= p.pieces;
    return (tensor ? p.value : p.key) + (size_t)t_begin * row_bytes + (size_t)(c - tensor * p.pieces) * 16;
  };
  auto piece_dst = [&](int c) {
    const int tensor = c >= p.pieces;
    const int within = c - tensor * p.pieces;
    const int h = within / head_pieces;
    return (tensor ? p.v_cache : p.k_cache) +
           ((size_t)h * bs * p.head_bytes + (size_t)(within - h * head_pieces) * 16);
  };
  // Loads of one piece for all NT tokens (a short last run re-reads its
  // last row, so the loads stay unconditional and all in flight), then its
  // stores.
  auto load = [&](int c, u32x4 (&v)[NT]) {
    const char *src = piece_src(c);
#pragma unroll
    for (int k = 0; k < NT; ++k) v[k] = ldnt(src + (size_t)min(k, n_tok - 1) * row_bytes);
  };
  auto store = [&](int c, const u32x4 (&v)[NT]) {
    char *dst = piece_dst(c);
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const long long row = s_row[k];
      if (k < n_tok && row >= 0) stnt(dst + (size_t)row * p.head_bytes, v[k]);
    }
  };

  u32x4 v[NT];
  const int c0 = threadIdx.x;
  if (c0 < per_token) load(c0, v);
  // Destinations: row index (block, kv head 0, slot) in units of head rows,
  // or -1 for none.
  if (threadIdx.x < 64) {
    // lane k < NT: token t_begin + k, its sequence by a binary search of
    // query_start_loc, then its slot; the NT searches run side by side
    const int lane = threadIdx.x;
    const int t = t_begin + min(lane, NT - 1);
    const int32_t *qsl = p.query_start_loc;
    int lo = 0, hi = p.num_seqs;                // qsl[lo] <= t < qsl[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (qsl[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int b = lo;
    const int cap = p.max_blocks_per_seq << p.bs_log2;
    const int q0 = qsl[b], q1 = qsl[b + 1];
    const int pos = p.context_lens[b] - (q1 - q0) + (t - q0);
    long long row = -1;
    if (lane < n_tok && pos >= 0 && pos < cap) {
      const int blk = p.block_tables[(size_t)b * p.max_blocks_per_seq + (pos >> p.bs_log2)];
      if (blk >= 0 && blk < p.num_blocks)
        row = (long long)blk * p.num_kv_heads * bs + (pos & (bs - 1));
    }
    if (lane < NT) s_row[lane] = row;
  }
  __syncthreads();
  if (c0 < per_token) store(c0, v);
  for (int c = c0 + 256; c < per_token; c += 256) {
    load(c, v);
    store(c, v);
  }
}

}  // namespace

hipError_t launch_append(const AppendLaunch &a, hipStream_t stream) {
  AppendParams p;
  p.k_cache = static_cast<char *>(a.k_cache);
  p.v_cache = static_cast<char *>(a.v_cache);
  p.key = static_cast<const char *>(a.key);
  p.value = static_cast<const char *>(a.value);
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.query_start_loc = a.query_start_loc;
  p.num_seqs = a.num_seqs;
  p.total_tokens = a.total_tokens;
  p.num_kv_heads = a.num_kv_heads;
  int bl = 0;
  while ((1 << bl) < a.block_size) ++bl;
  p.bs_log2 = bl;
  p.num_blocks = a.num_blocks;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.head_bytes = a.head_dim * a.elem_bytes;
  p.pieces = a.num_kv_heads * p.head_bytes / 16;
  p.tensors = a.v_cache ? 2 : 1;
  const int grid = (a.total_tokens + kTokensPerGroup - 1) / kTokensPerGroup;
  return launch_main(append_kernel, dim3(grid), dim3(256), 0, stream, p);
}

}  // namespace pa

// Host block manager of the paged KV cache: physical block allocation with
// reference counts, per-request block tables, growth one token at a time,
// prefix sharing and copy-on-write.
//
// Method (page cited by title): "大模型长文本推理基座…PagedAttention 显存物理
// 布局深度剖析" §三 — blocks carry a reference count; the free list is kept
// in increasing order and an allocation takes its lowest id; a request is
// registered with ceil(prompt / block_size) blocks and gains a block when a
// token arrives with every block full; finishing releases its blocks, which
// return to the free list when their count reaches 0 — and §四.2, where
// requests share prefix blocks by reference count and a request that writes
// into a shared block first gets its own copy.
//
// Host design: the free list is an ordered set (lowest id in O(log n), no
// re-sort on release); tables are vectors in a hash map keyed by request id.
// Every operation checks before it changes anything, so a failure leaves
// the manager as it was.
#include <algorithm>
#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "paged_attn.h"

struct pa_block_manager {
  struct Request {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  int32_t block_size = 1;
  std::vector<int32_t> ref;
  std::set<int32_t> free_ids;
  std::unordered_map<int64_t, Request> requests;

  int32_t allocate() {               // caller has checked free_ids is non-empty
    const int32_t b = *free_ids.begin();
    free_ids.erase(free_ids.begin());
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (ref[b] > 0 && --ref[b] == 0) free_ids.insert(b);
  }
};

extern "C" {

pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager **out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1) return PA_ERR_SHAPE;
  pa_block_manager *bm = new (std::nothrow) pa_block_manager;
  if (!bm) return PA_ERR_NO_BLOCKS;
  try {
    bm->block_size = block_size;
    bm->ref.assign((size_t)num_blocks, 0);
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_ids.insert(bm->free_ids.end(), b);
  } catch (...) {
    delete bm;
    return PA_ERR_NO_BLOCKS;
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

pa_status_t pa_bm_register(pa_block_manager *bm, int64_t request_id, int64_t prompt_len) {
  if (!bm) return PA_ERR_NULL;
  if (prompt_len < 0) return PA_ERR_SHAPE;
  if (bm->requests.count(request_id)) return PA_ERR_REQUEST;
  const int64_t need = (prompt_len + bm->block_size - 1) / bm->block_size;
  if (need > (int64_t)bm->free_ids.size()) return PA_ERR_NO_BLOCKS;
  pa_block_manager::Request r;
  r.blocks.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) r.blocks.push_back(bm->allocate());
  r.tokens = prompt_len;
  bm->requests.emplace(request_id, std::move(r));
  return PA_OK;
}

pa_status_t pa_bm_append_token(pa_block_manager *bm, int64_t request_id, int32_t *cow_src,
                               int32_t *cow_dst) {
  if (!bm) return PA_ERR_NULL;
  if (cow_src) *cow_src = -1;
  if (cow_dst) *cow_dst = -1;
  auto it = bm->requests.find(request_id);
  if (it == bm->requests.end()) return PA_ERR_REQUEST;
  pa_block_manager::Request &r = it->second;
  if (r.tokens % bm->block_size == 0) {            // every block full (or none yet)
    if (bm->free_ids.empty()) return PA_ERR_NO_BLOCKS;
    r.blocks.push_back(bm->allocate());
  } else if (bm->ref[r.blocks.back()] > 1) {      // partly filled and shared
    if (bm->free_ids.empty()) return PA_ERR_NO_BLOCKS;
    const int32_t old = r.blocks.back();
    const int32_t fresh = bm->allocate();
    bm->release(old);
    r.blocks.back() = fresh;
    if (cow_src) *cow_src = old;
    if (cow_dst) *cow_dst = fresh;
  }
  ++r.tokens;
  return PA_OK;
}

pa_status_t pa_bm_append_tokens(pa_block_manager *bm, const int64_t *request_ids,
                                int32_t num_requests, int32_t *cow_src, int32_t *cow_dst) {
  if (!bm) return PA_ERR_NULL;
  if (num_requests < 0) return PA_ERR_SHAPE;
  if (num_requests == 0) return PA_OK;
  if (!request_ids) return PA_ERR_NULL;
  // Check the whole batch first: every id known and listed once, and enough
  // free blocks for the appends in list order (a copy-on-write lowers the
  // count of the shared block, which a later request of the batch may share).
  std::unordered_map<int64_t, char> seen;
  std::unordered_map<int32_t, int32_t> dropped;     // block -> references given up so far
  seen.reserve((size_t)num_requests);
  int64_t need = 0;
  for (int32_t i = 0; i < num_requests; ++i) {
    auto it = bm->requests.find(request_ids[i]);
    if (it == bm->requests.end() || !seen.emplace(request_ids[i], 1).second) return PA_ERR_REQUEST;
    const pa_block_manager::Request &r = it->second;
    if (r.tokens % bm->block_size == 0) {
      ++need;
    } else {
      const int32_t last = r.blocks.back();
      auto d = dropped.find(last);
      const int32_t refs = bm->ref[last] - (d == dropped.end() ? 0 : d->second);
      if (refs > 1) {
        ++need;
        ++dropped[last];
      }
    }
  }
  if (need > (int64_t)bm->free_ids.size()) return PA_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < num_requests; ++i)
    (void)pa_bm_append_token(bm, request_ids[i], cow_src ? cow_src + i : nullptr,
                             cow_dst ? cow_dst + i : nullptr);
  return PA_OK;
}

pa_status_t pa_bm_fork(pa_block_manager *bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->requests.find(parent_id);
  if (it == bm->requests.end() || bm->requests.count(child_id)) return PA_ERR_REQUEST;
  pa_block_manager::Request child = it->second;
  for (int32_t b : child.blocks) ++bm->ref[b];
  bm->requests.emplace(child_id, std::move(child));
  return PA_OK;
}

pa_status_t pa_bm_finish(pa_block_manager *bm, int64_t request_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->requests.find(request_id);
  if (it == bm->requests.end()) return PA_ERR_REQUEST;
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->requests.erase(it);
  return PA_OK;
}

int32_t pa_bm_free_count(const pa_block_manager *bm) {
  return bm ? (int32_t)bm->free_ids.size() : -1;
}

pa_status_t pa_bm_block_table(const pa_block_manager *bm, int64_t request_id, int32_t *blocks,
                              int32_t capacity, int32_t *num_blocks, int64_t *num_tokens) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->requests.find(request_id);
  if (it == bm->requests.end()) return PA_ERR_REQUEST;
  const auto &r = it->second;
  if (num_blocks) *num_blocks = (int32_t)r.blocks.size();
  if (num_tokens) *num_tokens = r.tokens;
  if ((int64_t)r.blocks.size() > capacity) return PA_ERR_SHAPE;
  if (!blocks && !r.blocks.empty()) return PA_ERR_NULL;
  for (size_t i = 0; i < r.blocks.size(); ++i) blocks[i] = r.blocks[i];
  return PA_OK;
}

pa_status_t pa_bm_free_list(const pa_block_manager *bm, int32_t *blocks, int32_t capacity,
                            int32_t *num_blocks) {
  if (!bm) return PA_ERR_NULL;
  if (num_blocks) *num_blocks = (int32_t)bm->free_ids.size();
  if ((int64_t)bm->free_ids.size() > capacity) return PA_ERR_SHAPE;
  if (!blocks && !bm->free_ids.empty()) return PA_ERR_NULL;
  int32_t i = 0;
  for (int32_t b : bm->free_ids) blocks[i++] = b;
  return PA_OK;
}

pa_status_t pa_bm_ref_count(const pa_block_manager *bm, int32_t block, int32_t *count) {
  if (!bm || !count) return PA_ERR_NULL;
  if (block < 0 || block >= (int32_t)bm->ref.size()) return PA_ERR_SHAPE;
  *count = bm->ref[block];
  return PA_OK;
}

pa_status_t pa_bm_fill_batch(const pa_block_manager *bm, const int64_t *request_ids,
                             int32_t num_requests, int32_t max_blocks_per_seq,
                             int32_t *block_tables, int32_t *context_lens) {
  if (!bm) return PA_ERR_NULL;
  if (num_requests < 0 || max_blocks_per_seq < 1) return PA_ERR_SHAPE;
  if (num_requests == 0) return PA_OK;
  if (!request_ids || !block_tables || !context_lens) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_requests; ++i) {    // check everything before writing
    auto it = bm->requests.find(request_ids[i]);
    if (it == bm->requests.end()) return PA_ERR_REQUEST;
    if ((int64_t)it->second.blocks.size() > max_blocks_per_seq ||
        it->second.tokens > INT32_MAX)
      return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < num_requests; ++i) {
    const auto &r = bm->requests.find(request_ids[i])->second;
    int32_t *row = block_tables + (size_t)i * max_blocks_per_seq;
    std::copy(r.blocks.begin(), r.blocks.end(), row);
    std::fill(row + r.blocks.size(), row + max_blocks_per_seq, -1);
    context_lens[i] = (int32_t)r.tokens;
  }
  return PA_OK;
}

}  // extern "C"

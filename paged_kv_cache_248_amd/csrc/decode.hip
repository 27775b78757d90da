// Paged decode for gfx950: one query token per sequence attends to its cached
// keys/values through the block table.
//
// Method (pages cited by title):
//   * scaled dot-product attention, softmax(q K^T / sqrt(d)) V — formula at
//     the top of "vLLM中FlashAttention与KVCache交换机制解析";
//   * K/V tiles streamed through on-chip storage with the OnlineSoftmax
//     update of M (running max), L (normaliser) and O — same page, the
//     M_new / L_new / O_new equations; O is kept unnormalised here and divided
//     by L once at the end (algebraically the same recurrence);
//   * PagedAttention indirection: token j of a sequence lives in physical
//     block block_table[j / block_size] at slot j % block_size —
//     "大模型长文本推理基座…PagedAttention 显存物理布局深度剖析" §二.2;
//   * GQA: the query heads of one group share a single K/V read, addressed by
//     index — the MQA/GQA remarks of the swap-mechanism page;
//   * long contexts are cut into partitions processed in parallel, each
//     leaving (M, L, O~) partials that are merged with the same rescaling
//     (block-level parallelism, "vLLM中FlashAttention与KVCache优化解析",
//     FlashAttention advantages table).
//
// Design for CDNA4 (HBM-bound path, ~1-4 flop per byte):
//   * one work-group of 4 wavefronts = one work item (sequence, kv head,
//     partition, head chunk); wavefront w takes tiles w, w+4, ... of the
//     partition and the four partial states are combined in LDS.  The grid is
//     persistent and items are handed out through an atomic counter from a
//     compact list built on device (full partitions first, the shorter last
//     partitions at the end), so the kernel drains evenly whatever the mix of
//     context lengths;
//   * a sequence that spans several partitions leaves (M, L, O~) partials;
//     the work-group that stores the last partition of a (sequence, kv head,
//     head chunk) — counted with an atomic arrival counter, the partials
//     written and read through the device-coherent path — merges them in the
//     same kernel, so the merge costs no extra launch and overlaps the other
//     work-groups' partitions;
//   * a token row (D * elem bytes) is split into 16-byte pieces, one per lane:
//     each load instruction moves 1 KiB fully coalesced; the lanes of one
//     token reduce their partial dot products with DPP row exchanges;
//   * the next tile's K and V are in flight while the current tile is
//     consumed; block ids, work items and context lengths are read through the
//     constant address space, i.e. with scalar loads whose counter is separate
//     from the vector loads, and the ids run one tile further ahead, so the
//     id -> data dependency never drains the K/V pipeline;
//   * reductions only depend on a token's logical position, never on its
//     physical block, so permuting the pool leaves results bit-identical.
#include <atomic>

#include "../../include/paged_attn.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <class E, int D, int GT>
struct Geom {
  static constexpr int kRowBytes = D * E::bytes;   // one token row of K or V
  static constexpr int kLPT = kRowBytes / 16;      // lanes per token
  static constexpr int kTPL = 64 / kLPT;           // tokens per load instruction
  // load instructions per tile per tensor (two tiles of K and V are held in
  // registers).  One head per wave keeps the large tile (more bytes in
  // flight per wave); with 4+ heads the vector work per byte is 4x higher
  // and more resident waves hide it better: 2 loads per tile lets 4 waves
  // per SIMD fit (measured ~20% faster than 8 loads at 2 waves per SIMD).
  static constexpr int kNL = GT >= 4 ? 2 : 8;
  static constexpr int kTile = kNL * kTPL;         // tokens per tile
  static constexpr int kEPL = 16 / E::bytes;       // elements per lane per load
  static_assert(kLPT >= 8 && kLPT <= 32, "row must span 8..32 lanes");
};

struct DecodeParams {
  void *out;
  const void *query;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *work;        // (seq, partition) pairs
  const int32_t *work_count;  // number of pairs
  int32_t *next_item;         // dynamic work counter (zeroed by the plan kernel)
  float *part_o;              // [B, Hq, max_parts, D] unnormalised O
  float *part_ml;             // [B, Hq, max_parts, 2] (M in log2 units, L)
  int32_t *arrive;            // [B, Hkv, head_chunks] partitions finished (zeroed by the plan kernel)
  int32_t num_heads, num_kv_heads, group, head_chunks;
  int32_t bs_log2, max_blocks_per_seq, num_blocks;
  int32_t partition, max_parts, ctx_cap;
  // 1: every sequence fits one partition; work-group i takes item i (items
  // numbered (sequence, kv head, head chunk)) and there is no work list.
  int32_t direct;
  float scale_log2e;
};

// Partial dot product of one 16-byte piece of q with one of k.
template <class E>
__device__ __forceinline__ float dot16(const u32x4 &q, const u32x4 &k) {
  if constexpr (E::bytes == 4) {
    float s = __uint_as_float(q[0]) * __uint_as_float(k[0]);
    s = fmaf(__uint_as_float(q[1]), __uint_as_float(k[1]), s);
    s = fmaf(__uint_as_float(q[2]), __uint_as_float(k[2]), s);
    return fmaf(__uint_as_float(q[3]), __uint_as_float(k[3]), s);
  } else if constexpr (sizeof(typename E::storage) == 2 && E::bytes == 2 &&
                       __is_same(typename E::storage, _Float16)) {
    // Elements are copied to scalars before the bit cast: a bit cast of an
    // indexed vector element miscompiles (every index reads element 0).
    const uint32_t qa[4] = {q.x, q.y, q.z, q.w};
    const uint32_t ka[4] = {k.x, k.y, k.z, k.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qa[i]),
                                 __builtin_bit_cast(f16x2, ka[i]), s, false);
    return s;
  } else {
    const uint32_t qa[4] = {q.x, q.y, q.z, q.w};
    const uint32_t ka[4] = {k.x, k.y, k.z, k.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qa[i]),
                                          __builtin_bit_cast(bf16x2, ka[i]), s, false);
    return s;
  }
}

// Unpack one 16-byte piece into fp32 values.
template <class E>
__device__ __forceinline__ void unpack16(const u32x4 &v, float *f) {
  if constexpr (E::bytes == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  } else if constexpr (__is_same(typename E::storage, _Float16)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_lo(v[i]);
      f[2 * i + 1] = f16_hi(v[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v[i]);
      f[2 * i + 1] = bf16_hi(v[i]);
    }
  }
}

// Pack fp32 values (round to nearest even) into one 16-byte piece.
template <class E>
__device__ __forceinline__ u32x4 pack16(const float *f) {
  u32x4 r;
  if constexpr (E::bytes == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
  } else if constexpr (__is_same(typename E::storage, _Float16)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_f16(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
  }
  return r;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read-only int32 data addressed with wave-uniform indices: through the
// constant address space the compiler emits scalar loads.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ cint32 *as_const(const int32_t *p) {
  return (cint32 *)(p);
}
__device__ __forceinline__ float uniformf(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}


template <class E>
__device__ __forceinline__ void store_elem(void *out, size_t idx, float v) {
  if constexpr (E::bytes == 4) static_cast<float *>(out)[idx] = v;
  else if constexpr (__is_same(typename E::storage, _Float16))
    static_cast<uint16_t *>(out)[idx] = f32_to_f16_bits(v);
  else static_cast<uint16_t *>(out)[idx] = f32_to_bf16(v);
}

constexpr int kWaves = 4;

// Device-coherent store and load of split-KV partials (agent-scope relaxed
// atomics: the write-through / coherent-read cache policy), so that a
// work-group on any XCD reads what another one wrote without a device-wide
// cache write-back or invalidate.
__device__ __forceinline__ void coherent_store(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-KV merge of one (sequence, kv head, head chunk), run inside the
// decode kernel by the work-group that stores its last partition's partials:
// M = max_p M_p, L = sum_p L_p 2^(M_p - M), O = sum_p O~_p 2^(M_p - M) / L —
// the OnlineSoftmax rescaling applied across partitions.  Wavefront w forms
// M and 1/L of heads w, w + 4, ... by wave-level reductions (kept in
// s_mm / s_il); then each thread takes (head, dim) pairs and reads their
// partials a few at a time, recomputing each weight from (M_p, L).
template <class E, int D, int GT>
__device__ __forceinline__ void merge_partials(const DecodeParams &p, int b, int h0, int nh,
                                               int nparts, float *s_mm, float *s_il) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int j = wave; j < nh; j += kWaves) {
    const float *ml = p.part_ml + ((size_t)b * p.num_heads + h0 + j) * p.max_parts * 2;
    float mx = -__builtin_inff();
    for (int q = lane; q < nparts; q += 64) mx = fmaxf(mx, coherent_load(&ml[2 * q]));
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
    float ls = 0.f;
    for (int q = lane; q < nparts; q += 64)
      ls = fmaf(fast_exp2(coherent_load(&ml[2 * q]) - mx), coherent_load(&ml[2 * q + 1]), ls);
    for (int off = 32; off > 0; off >>= 1) ls += shfl_xor(ls, off);
    if (lane == 0) {
      s_mm[j] = mx;
      s_il[j] = 1.0f / ls;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nh * D; idx += kWaves * 64) {
    const int j = idx / D, d = idx % D;
    const size_t row = (size_t)b * p.num_heads + h0 + j;
    const float *po = p.part_o + row * p.max_parts * D + d;
    const float *ml = p.part_ml + row * p.max_parts * 2;
    const float M = s_mm[j];
    // kBatch partials per round, all loads in flight together; past the
    // last partition the index is clamped (a cached re-read) and the weight
    // is 0
    constexpr int kBatch = 4;
    float acc = 0.f;
    for (int q0 = 0; q0 < nparts; q0 += kBatch) {
      float v[kBatch], mq[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int q = min(q0 + u, nparts - 1);
        v[u] = coherent_load(&po[(size_t)q * D]);
        mq[u] = coherent_load(&ml[2 * q]);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        acc = fmaf(q0 + u < nparts ? fast_exp2(mq[u] - M) : 0.f, v[u], acc);
    }
    store_elem<E>(p.out, row * D + d, acc * s_il[j]);
  }
}

// After a work-group has stored the partials of a partition of a
// multi-partition sequence (coherent stores): every wavefront waits until
// its stores are complete, then one thread counts the partition; the
// work-group that counts the last partition of a (sequence, kv head, head
// chunk) merges, reading the partials coherently after it saw the count.
// Called by every thread of the work-group (it synchronises).
template <class E, int D, int GT>
__device__ __forceinline__ void finish_partition(const DecodeParams &p, int b, int g, int hc, int h0,
                                                 int nh, int nparts, int *s_flag, float *s_mm,
                                                 float *s_il) {
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = atomicAdd(p.arrive + ((size_t)b * p.num_kv_heads + g) * p.head_chunks + hc, 1) ==
              nparts - 1;
  __syncthreads();
  if (*s_flag) merge_partials<E, D, GT>(p, b, h0, nh, nparts, s_mm, s_il);
}

template <class E, int D, int GT>
__global__ __launch_bounds__(256, GT == 4 ? 4 : 2) void decode_kernel(DecodeParams p) {
  using G = Geom<E, D, GT>;
  constexpr int NL = G::kNL, TPL = G::kTPL, LPT = G::kLPT, EPL = G::kEPL, TILE = G::kTile;
  __shared__ int s_item, s_flag;
  __shared__ float s_m[kWaves][GT], s_l[kWaves][GT];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][GT][D];

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);   // wave-uniform: keeps tile/page math scalar
  const int lane = tid & 63;
  const int tok = lane / LPT;     // token of each load this lane holds
  const int chunk = lane % LPT;   // 16-byte piece of the row this lane holds
  const int bs = 1 << p.bs_log2;
  const int Hq = p.num_heads, Hkv = p.num_kv_heads;
  const char *kbase = static_cast<const char *>(p.k_cache);
  const char *vbase = static_cast<const char *>(p.v_cache);
  const size_t head_stride = (size_t)bs * G::kRowBytes;          // one (block, head) page
  const size_t block_stride = head_stride * (size_t)Hkv;
  const int total = p.direct ? (int)gridDim.x : as_const(p.work_count)[0] * Hkv * p.head_chunks;

  for (int round = 0;; ++round) {
    int item;
    if (p.direct) {
      if (round > 0) break;
      item = blockIdx.x;
    } else {
      if (tid == 0) s_item = atomicAdd(p.next_item, 1);
      __syncthreads();
      item = s_item;
    }
    if (item >= total) break;
    const int hc = item % p.head_chunks;
    const int rest = item / p.head_chunks;
    const int g = rest % Hkv;
    const int wi = rest / Hkv;
    const int b = p.direct ? wi : as_const(p.work)[2 * wi];
    const int part = p.direct ? 0 : as_const(p.work)[2 * wi + 1];
    const int ctx = min(max(as_const(p.context_lens)[b], 0), p.ctx_cap);
    if (ctx == 0) break;            // direct items only (the work list holds no empty sequence)
    const int start = part * p.partition;
    const int end = min(start + p.partition, ctx);
    const int nparts = (ctx + p.partition - 1) / p.partition;
    const int h0 = g * p.group + hc * GT;
    const int nh = min(GT, p.group - hc * GT);
    const int npages = (ctx + bs - 1) >> p.bs_log2;
    cint32 *tbl = as_const(p.block_tables) + (size_t)b * p.max_blocks_per_seq;
    // Wave-uniform bases; the per-lane part (slot row, 16-byte piece) is a
    // 32-bit offset, so each load is a scalar page address plus one VGPR.
    const char *kpage_base = kbase + (size_t)g * head_stride;
    const char *vpage_base = vbase + (size_t)g * head_stride;

    // Query pieces of the GT heads (raw storage; exact).
    u32x4 q[GT];
#pragma unroll
    for (int j = 0; j < GT; ++j) {
      if (j < nh) {
        const char *qp = static_cast<const char *>(p.query) +
                         ((size_t)(b * Hq + h0 + j) * D) * E::bytes + (size_t)chunk * 16;
        q[j] = ld16(qp);
      } else {
        q[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    float m[GT], l[GT], o[GT][EPL];
#pragma unroll
    for (int j = 0; j < GT; ++j) {
      m[j] = -__builtin_inff();
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
    }

    // This wavefront's tiles: wave, wave + 4, ... of the partition.
    const int ntiles_all = (end - start + TILE - 1) / TILE;
    const int ntiles = ntiles_all > wave ? (ntiles_all - wave + kWaves - 1) / kWaves : 0;
    auto tile_start = [&](int t) { return start + (wave + t * kWaves) * TILE; };

    // Tokens past the end of the partition are read as copies of its last
    // token (same page, as pages hold a multiple of TPL tokens): their
    // weight is exactly 0 and the copy is finite, so V needs no zeroing and
    // the loads no branches.  Block ids of the pages each load of a tile
    // touches (wave-uniform).
    auto fetch_ids = [&](int t, int *ids) {
      const int ts = tile_start(t);
#pragma unroll
      for (int L = 0; L < NL; ++L) {
        const int page = min(ts + L * TPL, end - 1) >> p.bs_log2;
        int id = 0;
        if (t < ntiles) id = tbl[page];
        ids[L] = (int)min((unsigned)id, (unsigned)(p.num_blocks - 1));
      }
    };
    auto issue = [&](int t, const int *ids, u32x4 *kr, u32x4 *vr) {
      const int ts = tile_start(t);
#pragma unroll
      for (int L = 0; L < NL; ++L) {
        const int slot = min(ts + L * TPL + tok, end - 1) & (bs - 1);
        const size_t page_off = (size_t)ids[L] * block_stride;
        const uint32_t lane_off = (uint32_t)(slot * G::kRowBytes + chunk * 16);
        kr[L] = ld16_nt(kpage_base + page_off + lane_off);
        vr[L] = ld16_nt(vpage_base + page_off + lane_off);
      }
    };
    const float c = p.scale_log2e;
    auto consume = [&](int t, const u32x4 *kr, const u32x4 *vr) {
      const int ts = tile_start(t);
      const bool tail = ts + TILE > end;     // only the last tile can hold rows past the end
      // Scores in log2 units.  (Subtracting the running maximum from the
      // scaled score keeps a lone maximal key's weight exactly 1.)
      float x[GT][NL];
#pragma unroll
      for (int L = 0; L < NL; ++L)
#pragma unroll
        for (int j = 0; j < GT; ++j) x[j][L] = group_sum<LPT>(dot16<E>(q[j], kr[L])) * c;
      if (tail) {
#pragma unroll
        for (int L = 0; L < NL; ++L)
          if (ts + L * TPL + tok >= end) {
#pragma unroll
            for (int j = 0; j < GT; ++j) x[j][L] = -__builtin_inff();
          }
      }
#pragma unroll
      for (int j = 0; j < GT; ++j) {
        float mx = x[j][0];
#pragma unroll
        for (int L = 1; L < NL; ++L) mx = vmax(mx, x[j][L]);
        mx = uniformf(across_groups_max<LPT>(mx));
        if (mx > m[j]) {                     // wave-uniform branch
          const float alpha = fast_exp2(m[j] - mx);
          l[j] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[j][e] *= alpha;
          m[j] = mx;
        }
#pragma unroll
        for (int L = 0; L < NL; ++L) {
          x[j][L] = fast_exp2(x[j][L] - m[j]);
          l[j] += x[j][L];
        }
      }
#pragma unroll
      for (int L = 0; L < NL; ++L) {
        float vf[EPL];
        unpack16<E>(vr[L], vf);
#pragma unroll
        for (int j = 0; j < GT; ++j)
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(x[j][L], vf[e], o[j][e]);
      }
    };

    if (ntiles > 0) {
      int ids_a[NL], ids_b[NL];
      u32x4 ka[NL], va[NL], kb[NL], vb[NL];
      fetch_ids(0, ids_a);
      issue(0, ids_a, ka, va);
      fetch_ids(1, ids_b);
      for (int t = 0; t < ntiles; t += 2) {
        if (t + 1 < ntiles) {
          issue(t + 1, ids_b, kb, vb);
          fetch_ids(t + 2, ids_a);
        }
        consume(t, ka, va);
        if (t + 1 < ntiles) {
          if (t + 2 < ntiles) {
            issue(t + 2, ids_a, ka, va);
            fetch_ids(t + 3, ids_b);
          }
          consume(t + 1, kb, vb);
        }
      }
    }

    // Combine the lane groups (different tokens, same dims), then the waves.
#pragma unroll
    for (int j = 0; j < GT; ++j) {
      l[j] = across_groups_sum<LPT>(l[j]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] = across_groups_sum<LPT>(o[j][e]);
    }
    if (tok == 0) {
#pragma unroll
      for (int j = 0; j < GT; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_o[wave][j][chunk * EPL + e] = o[j][e];
        if (chunk == 0) {
          s_m[wave][j] = m[j];
          s_l[wave][j] = l[j];
        }
      }
    }
    __syncthreads();

    // State of the whole partition, one (head, dim) per thread.
    for (int idx = tid; idx < GT * D; idx += 256) {
      const int j = idx / D, d = idx % D;
      if (j >= nh) continue;
      float M = s_m[0][j];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][j]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float c = fast_exp2(s_m[w][j] - M);     // idle waves: 2^-inf = 0
        L = fmaf(c, s_l[w][j], L);
        O = fmaf(c, s_o[w][j][d], O);
      }
      const size_t row = (size_t)(b * Hq + h0 + j);
      if (nparts <= 1) {
        store_elem<E>(p.out, row * D + d, O / L);
      } else {
        // partials go through the device-coherent path (another work-group,
        // possibly on another XCD, merges them)
        const size_t slot = row * p.max_parts + part;
        coherent_store(&p.part_o[slot * D + d], O);
        if (d == 0) {
          coherent_store(&p.part_ml[slot * 2], M);
          coherent_store(&p.part_ml[slot * 2 + 1], L);
        }
      }
    }
    if (nparts > 1)
      finish_partition<E, D, GT>(p, b, g, hc, h0, nh, nparts, &s_flag, s_m[0], s_l[0]);
    __syncthreads();   // LDS and s_item are reused by the next item
  }
}

// ---- Matrix-core decode for grouped-query attention ----------------------
// The GT query heads of a kv-head group (GT >= 4) share every K/V tile, so
// the dot products are a small dense contraction per tile and run on the
// matrix cores, which leaves the vector ALU only the softmax (about two
// instructions per token instead of some twenty):
//   S^T (16 tokens x 16 heads) = K (16 x D) Q^T (D x 16): D/32 MFMA
//     16x16x32.  K goes from the cache straight into the operand layout
//     (lane l: token l % 16, the 16 bytes at d = 32 ks + 8 (l / 16));
//   O^T (D x 16 heads) += V^T (D x 16 tokens) P^T (16 tokens x 16 heads):
//     D/16 MFMA 16x16x16.  V goes cache -> LDS by direct loads and is read
//     back transposed (ds_read_b64_tr_b16).
// Heads past the group are zero columns of Q^T.  The S^T accumulator gives
// lane l head l % 16 for tokens 4 (l / 16) .. +3, which is exactly the P^T
// operand layout of the PV step, so the softmax output feeds it directly.
// Each wavefront keeps four tiles in flight (K in registers, V in its own
// LDS stages: 64 KiB per work-group, two work-groups per CU at D = 128) and
// waits for each with an exact vmcnt count.  Three tiles (48 KiB, three
// work-groups per CU at 167 VGPRs) held fewer bytes in flight per CU and
// read 2% slower.
// 16-byte non-temporal global load at sbase + voff + OFF (K is streamed
// once), issued as inline assembly: the
// compiler does not track it, so it inserts no wait of its own; the kernel
// waits with an exact vmcnt and then ties the registers (tie_regs) before any
// use.
template <int OFF>
__device__ __forceinline__ u32x4 gload16(const char *sbase, uint32_t voff) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 nt"
               : "=v"(v) : "v"(voff), "s"(sbase), "i"(OFF) : "memory");
  return v;
}
template <class E>
__device__ __forceinline__ f32x4 mfma_k32(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  if constexpr (__is_same(typename E::storage, _Float16))
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <class E>
__device__ __forceinline__ f32x4 mfma_k16(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
  if constexpr (__is_same(typename E::storage, _Float16))
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Weights stay within [0, 2^kLazyDecode]: the running maximum is raised only
// when a tile's maximum exceeds it by more than that.
constexpr float kLazyDecode = 8.0f;

template <class E, int D, int GT>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeParams p) {
  constexpr int T = 16;                  // tokens per tile
  constexpr int KS = D / 32;             // QK k-steps
  constexpr int DB = D / 16;             // PV d-blocks
  constexpr int ROWB = D * 2;            // bytes of one token row
  constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;       // rows per direct-to-LDS instruction
  constexpr int VI = T / RPI;            // direct-to-LDS instructions per V tile
  constexpr int TILEB = T * ROWB;        // LDS bytes of one V tile
  constexpr int NST = 4;                 // tiles in flight per wavefront
  constexpr int PER_TILE = KS + VI;      // vector-memory operations per tile
  static_assert(GT >= 4 && GT <= 16, "one 16-column MFMA block of heads");
  static_assert(kWaves * GT * D * 4 <= kWaves * NST * TILEB, "partials fit the V stages");
  __shared__ __attribute__((aligned(1024))) char s_v[kWaves * NST * TILEB];
  __shared__ int s_item, s_flag;
  __shared__ float s_m[kWaves][GT], s_l[kWaves][GT];
  float(*s_o)[GT][D] = reinterpret_cast<float(*)[GT][D]>(s_v);   // after the key loop

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane & 15;         // head column of this lane
  const int G = lane >> 4;          // token group: tokens 4G .. 4G+3 of a tile
  const int bs = 1 << p.bs_log2;
  const int Hq = p.num_heads, Hkv = p.num_kv_heads;
  const size_t head_stride = (size_t)bs * ROWB;
  const size_t block_stride = head_stride * (size_t)Hkv;
  const int total = p.direct ? (int)gridDim.x : as_const(p.work_count)[0] * Hkv * p.head_chunks;

  // V stages: row r of a tile holds its 16-byte chunk c at position
  // c ^ vsw(r), vsw(r) = 2 (r mod 8) for 256-byte rows and 2 ((r / 2) mod 4)
  // for 128-byte rows.  The transposing read of d-block db: lane l reads row
  // l / 4, the 8 bytes at d = 16 db + 4 (l mod 4); the swizzle puts the 32
  // lanes of each half-wave on distinct banks.  As the swizzle only moves
  // 32-byte pairs, the address of d-block db is the d-block-0 address XOR 32 db.
  auto vsw = [](int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };
  char *const my_v = s_v + wave * (NST * TILEB);
  const uint32_t my_v_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)my_v;
  uint32_t tr_addr[DB];
  {
    const int r = lane >> 2;
    const uint32_t a0 = (uint32_t)(r * ROWB + 16 * vsw(r) + 8 * (lane & 3));
#pragma unroll
    for (int db = 0; db < DB; ++db) tr_addr[db] = my_v_addr + (a0 ^ (uint32_t)(32 * db));
  }
  // Direct-to-LDS lane mapping: instruction q, lane i fills row
  // q RPI + i / CPR at chunk position i mod CPR, i.e. reads the row's global
  // chunk (i mod CPR) ^ vsw(row).
  int v_row[VI], v_chunk[VI];
#pragma unroll
  for (int q = 0; q < VI; ++q) {
    v_row[q] = q * RPI + lane / CPR;
    v_chunk[q] = ((lane % CPR) ^ vsw(v_row[q])) * 16;
  }

  for (int round = 0;; ++round) {
    int item;
    if (p.direct) {
      if (round > 0) break;
      item = blockIdx.x;
    } else {
      if (tid == 0) s_item = atomicAdd(p.next_item, 1);
      __syncthreads();
      item = s_item;
    }
    if (item >= total) break;
    const int hc = item % p.head_chunks;
    const int rest = item / p.head_chunks;
    const int g = rest % Hkv;
    const int wi = rest / Hkv;
    const int b = p.direct ? wi : as_const(p.work)[2 * wi];
    const int part = p.direct ? 0 : as_const(p.work)[2 * wi + 1];
    const int ctx = min(max(as_const(p.context_lens)[b], 0), p.ctx_cap);
    if (ctx == 0) break;            // direct items only (the work list holds no empty sequence)
    const int start = part * p.partition;
    const int end = min(start + p.partition, ctx);
    const int nparts = (ctx + p.partition - 1) / p.partition;
    const int h0 = g * p.group + hc * GT;
    const int nh = min(GT, p.group - hc * GT);
    cint32 *tbl = as_const(p.block_tables) + (size_t)b * p.max_blocks_per_seq;
    const char *kpage_base = static_cast<const char *>(p.k_cache) + (size_t)g * head_stride;
    const char *vpage_base = static_cast<const char *>(p.v_cache) + (size_t)g * head_stride;

    // Q^T operand: lane l holds head h0 + l % 16, d = 32 ks + 8 (l / 16) .. +7.
    u32x4 qf[KS];
    {
      const char *qp = static_cast<const char *>(p.query) +
                       ((size_t)(b * Hq + h0 + hl) * D) * 2 + G * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = hl < nh ? ld16(qp + ks * 64) : u32x4{0u, 0u, 0u, 0u};
    }

    // Tiles w, w + 4, ... of the partition.  Tiles start at multiples of 16
    // tokens and pages hold at least 16, so a tile lies in one page; tokens
    // past the partition end are read as copies of its last token (weight
    // exactly 0, finite), so loads carry no branches.
    const int ntiles_all = (end - start + T - 1) / T;
    const int ntiles = ntiles_all > wave ? (ntiles_all - wave + kWaves - 1) / kWaves : 0;
    auto tile_start = [&](int t) { return start + (wave + t * kWaves) * T; };
    auto fetch_id = [&](int t) {
      const int page = min(tile_start(t), end - 1) >> p.bs_log2;
      int id = 0;
      if (t < ntiles) id = tbl[page];
      return (int)min((unsigned)id, (unsigned)(p.num_blocks - 1));
    };
    u32x4 kr[NST][KS];
    auto issue = [&](int t, int id, auto buf_tag) {
      constexpr int buf = decltype(buf_tag)::value;
      const int ts = tile_start(t);
      const size_t page_off = (size_t)id * block_stride;
      const char *kp = kpage_base + page_off;
      const char *vp = vpage_base + page_off;
      const uint32_t koff = (uint32_t)((min(ts + hl, end - 1) & (bs - 1)) * ROWB + G * 16);
      for_each_index(std::make_integer_sequence<int, KS>{}, [&](auto ks_tag) {
        constexpr int ks = decltype(ks_tag)::value;
        kr[buf][ks] = gload16<ks * 64>(kp, koff);
      });
#pragma unroll
      for (int q = 0; q < VI; ++q) {
        const uint32_t voff = (uint32_t)((min(ts + v_row[q], end - 1) & (bs - 1)) * ROWB + v_chunk[q]);
        dma16_nt(vp + voff, my_v + buf * TILEB + q * 1024);
      }
    };
    // Tile loads still allowed in flight when tile t must have landed: the
    // tiles issued after it (at most NST - 1; fewer near the end).
    auto wait_tile = [&](int t) {
      const int later = ntiles - 1 - t;
      if (later >= 3) wait_vm<3 * PER_TILE>();
      else if (later == 2) wait_vm<2 * PER_TILE>();
      else if (later == 1) wait_vm<PER_TILE>();
      else wait_vm<0>();
    };

    float m = -__builtin_inff(), l = 0.f;
    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float c = p.scale_log2e;
    int id_next = 0;

    auto step = [&](int t, auto buf_tag) {
      constexpr int buf = decltype(buf_tag)::value;
      constexpr int nbuf = (buf + NST - 1) % NST;
      // Tile t + NST - 1 goes into the buffers tile t - 1 used (consumed last step).
      if (t + NST - 1 < ntiles) issue(t + NST - 1, id_next, std::integral_constant<int, nbuf>{});
      id_next = fetch_id(t + NST);
      wait_tile(t);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(kr[buf][ks]));
      u32x2 vt[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) vt[db] = lds_tr16<buf * TILEB>(tr_addr[db]);
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc = mfma_k32<E>(kr[buf][ks], qf[ks], sc);
      // Softmax on S^T: lane (head l % 16) holds tokens ts + 4G + r, in log2
      // units after scaling.
      const int ts = tile_start(t);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = sc[r] * c;
      if (ts + T > end) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (ts + 4 * G + r >= end) x[r] = -__builtin_inff();
      }
      float mx = vmax(vmax(x[0], x[1]), vmax(x[2], x[3]));
      const f32x2 m16 = pair_xor16(mx);
      mx = vmax(m16[0], m16[1]);
      const f32x2 m32 = pair_xor32(mx);
      mx = vmax(m32[0], m32[1]);
      if (__any(mx > m + kLazyDecode)) {
        const float m_new = vmax(m, mx);
        const float alpha = fast_exp2(m - m_new);        // 0 when m was -inf
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m = m_new;
      }
      float e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) e[r] = fast_exp2(x[r] - m);
      l += (e[0] + e[1]) + (e[2] + e[3]);
      const u32x2 pt = {pack2<E>(e[0], e[1]), pack2<E>(e[2], e[3])};
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vt[0]), "+v"(vt[DB - 1]));
#pragma unroll
      for (int db = 1; db < DB - 1; ++db) asm volatile("" : "+v"(vt[db]));
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mfma_k16<E>(vt[db], pt, o[db]);
    };

    if (ntiles > 0) {
      issue(0, fetch_id(0), std::integral_constant<int, 0>{});
      if (ntiles > 1) issue(1, fetch_id(1), std::integral_constant<int, 1>{});
      if (ntiles > 2) issue(2, fetch_id(2), std::integral_constant<int, 2>{});
      id_next = fetch_id(3);
      // Q, the first three tiles and whatever the previous work item stored
      // (stores and loads do not complete in one order, so the exact counts
      // below start from an empty queue).
      wait_vm<0>();
      for (int t = 0; t < ntiles; t += NST) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
        if (t + 2 < ntiles) step(t + 2, std::integral_constant<int, 2>{});
        if (t + 3 < ntiles) step(t + 3, std::integral_constant<int, 3>{});
      }
    }

    // L of a head is spread over the four token groups; O^T is complete.
    {
      const f32x2 a = pair_xor16(l);
      const float l2 = a[0] + a[1];
      const f32x2 b2 = pair_xor32(l2);
      l = b2[0] + b2[1];
    }
    __syncthreads();          // every wavefront is done with its V stages
    if (hl < nh) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4 *>(&s_o[wave][hl][16 * db + 4 * G]) = o[db];
      if (G == 0) {
        s_m[wave][hl] = m;
        s_l[wave][hl] = l;
      }
    }
    __syncthreads();

    for (int idx = tid; idx < GT * D; idx += 256) {
      const int j = idx / D, d = idx % D;
      if (j >= nh) continue;
      float M = s_m[0][j];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][j]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float cw = fast_exp2(s_m[w][j] - M);     // idle waves: 2^-inf = 0
        L = fmaf(cw, s_l[w][j], L);
        O = fmaf(cw, s_o[w][j][d], O);
      }
      const size_t row = (size_t)(b * Hq + h0 + j);
      if (nparts <= 1) {
        store_elem<E>(p.out, row * D + d, O / L);
      } else {
        // partials go through the device-coherent path (another work-group,
        // possibly on another XCD, merges them)
        const size_t slot = row * p.max_parts + part;
        coherent_store(&p.part_o[slot * D + d], O);
        if (d == 0) {
          coherent_store(&p.part_ml[slot * 2], M);
          coherent_store(&p.part_ml[slot * 2 + 1], L);
        }
      }
    }
    if (nparts > 1)
      finish_partition<E, D, GT>(p, b, g, hc, h0, nh, nparts, &s_flag, s_m[0], s_l[0]);
    __syncthreads();   // LDS and s_item are reused by the next item
  }
}

// Builds the compact list of (sequence, partition) work items — full-length
// partitions first, then the shorter last partitions — and clears the
// dynamic work counter and the merge arrival counters.  With long
// partitions (lpt set: 1024 tokens or more, a few items per work-group) the
// last partitions go longest first (in 32 length classes), so that
// work-groups taking items in list order end on short ones (GQA workload,
// 2048-token partitions: +5.5% kernel bandwidth); with short partitions
// (many items per work-group) they stay in sequence order (the headline MHA
// workload, 512-token partitions, measured 0.7% slower in length order).
// Inclusive prefix sum and total over one wavefront (shuffles, no barrier).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

__global__ __launch_bounds__(256) void decode_plan_kernel(const int32_t *context_lens, int num_seqs,
                                                          int partition, int ctx_cap, int lpt,
                                                          int32_t *work, int32_t *work_count,
                                                          int32_t *next_item, int32_t *arrive,
                                                          int n_arrive) {
  constexpr int kClasses = 32, kT = 256;
  __shared__ int s_wave[kT / 64][2];     // per-wavefront totals (full, last partitions)
  __shared__ int s_total_full;
  __shared__ int s_class[kClasses];      // last partitions per length class, then their next slot
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto tail_class = [&](int tail) { return (int)((long long)tail * kClasses / partition); };
  for (int i = tid; i < n_arrive; i += kT) arrive[i] = 0;   // merge arrival counters
  if (tid < kClasses) s_class[tid] = 0;
  __syncthreads();
  // pass 1: number of full partitions over all sequences, and the last
  // partitions per length class
  int full_sum = 0;
  for (int b = tid; b < num_seqs; b += kT) {
    const int ctx = min(max(context_lens[b], 0), ctx_cap);
    full_sum += ctx / partition;
    if (lpt && ctx % partition) atomicAdd(&s_class[tail_class(ctx % partition)], 1);
  }
  full_sum = wave_incl_scan(full_sum);
  if (lane == 63) s_wave[wave][0] = full_sum;
  __syncthreads();
  if (tid == 0) {
    int tf = 0;
    for (int w = 0; w < kT / 64; ++w) tf += s_wave[w][0];
    s_total_full = tf;
    // first slot of each class, longest class first
    int acc = 0;
    for (int k = kClasses - 1; k >= 0; --k) {
      const int nk = s_class[k];
      s_class[k] = acc;
      acc += nk;
    }
  }
  __syncthreads();
  const int total_full = s_total_full;
  // pass 2: place items, 256 sequences at a time
  int base_full = 0, base_tail = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += kT) {
    const int b = c0 + tid;
    int nf = 0, nt = 0, tail = 0;
    if (b < num_seqs) {
      const int ctx = min(max(context_lens[b], 0), ctx_cap);
      nf = ctx / partition;
      tail = ctx % partition;
      nt = tail != 0;
    }
    const int sf = wave_incl_scan(nf), st = wave_incl_scan(nt);
    __syncthreads();                      // s_wave of the previous chunk is read
    if (lane == 63) {
      s_wave[wave][0] = sf;
      s_wave[wave][1] = st;
    }
    __syncthreads();
    int pf = 0, pt = 0, tf = 0, tt = 0;
    for (int w = 0; w < kT / 64; ++w) {
      if (w < wave) pf += s_wave[w][0], pt += s_wave[w][1];
      tf += s_wave[w][0];
      tt += s_wave[w][1];
    }
    const int f0 = base_full + pf + sf - nf;
    for (int k = 0; k < nf; ++k) {
      work[2 * (f0 + k)] = b;
      work[2 * (f0 + k) + 1] = k;
    }
    if (nt) {
      const int t0 = total_full + (lpt ? atomicAdd(&s_class[tail_class(tail)], 1)
                                       : base_tail + pt + st - 1);
      work[2 * t0] = b;
      work[2 * t0 + 1] = nf;
    }
    base_full += tf;
    base_tail += tt;
  }
  if (tid == 0) {
    *work_count = total_full + base_tail;
    *next_item = 0;
  }
}


size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

template <class E, int D, int GT, bool MF>
hipError_t launch_typed(const DecodeLaunch &a, const DecodeWorkspace &ws, hipStream_t stream) {
  char *w = static_cast<char *>(a.workspace);
  DecodeParams p;
  p.out = a.out;
  p.query = a.query;
  p.k_cache = a.k_cache;
  p.v_cache = a.v_cache;
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.work = reinterpret_cast<const int32_t *>(w + ws.work_off);
  p.work_count = reinterpret_cast<const int32_t *>(w + ws.count_off);
  p.next_item = reinterpret_cast<int32_t *>(w + ws.count_off + 4);
  p.part_o = reinterpret_cast<float *>(w + ws.part_o_off);
  p.part_ml = reinterpret_cast<float *>(w + ws.part_ml_off);
  p.arrive = reinterpret_cast<int32_t *>(w + ws.arrive_off);
  p.num_heads = a.num_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_heads / a.num_kv_heads;
  p.head_chunks = (p.group + GT - 1) / GT;
  int bl = 0;
  while ((1 << bl) < a.block_size) ++bl;
  p.bs_log2 = bl;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.partition = a.partition;
  p.max_parts = a.max_parts;
  p.ctx_cap = a.ctx_cap;
  p.scale_log2e = a.scale * kLog2e;
  // A single partition per sequence needs neither the work list nor the
  // dynamic counter: one work-group per item, launched directly.
  p.direct = a.max_parts == 1;

  if (!p.direct)
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(256), 0, stream, a.context_lens,
                       a.num_seqs, a.partition, a.ctx_cap, a.partition >= 1024 ? 1 : 0,
                       reinterpret_cast<int32_t *>(w + ws.work_off),
                       reinterpret_cast<int32_t *>(w + ws.count_off), p.next_item, p.arrive,
                       a.num_seqs * a.num_kv_heads * p.head_chunks);

  // Resident work-groups per CU; items are fetched dynamically, so a grid
  // larger than what fits only queues (it cannot unbalance the work).
  auto kernel = [] {
    if constexpr (MF) return decode_mfma_kernel<E, D, GT>;
    else return decode_kernel<E, D, GT>;
  }();
  static std::atomic<int> occ_cache[64];   // per instantiation and device; 0 = not queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cached = dev >= 0 && dev < 64;
  int occ = cached ? occ_cache[dev].load(std::memory_order_relaxed) : 0;
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, 0) != hipSuccess || occ < 1)
      occ = 2;
    if (cached) occ_cache[dev].store(occ, std::memory_order_relaxed);
  }
  const long long upper =
      (long long)a.num_seqs * a.max_parts * a.num_kv_heads * p.head_chunks;
  const long long resident = (long long)device_cu_count() * occ;
  const int grid = p.direct ? (int)std::max(1LL, upper)
                            : (int)std::max(1LL, std::min(upper, resident));
  return launch_main(kernel, dim3(grid), dim3(256), 0, stream, p);
}

template <class E, int D>
hipError_t launch_group(const DecodeLaunch &a, const DecodeWorkspace &ws, hipStream_t s) {
  const int group = a.num_heads / a.num_kv_heads;
  // 16-bit caches with a group of 4 or more heads per kv head and pages of
  // at least 16 tokens take the matrix-core kernel (one 16-column block of
  // heads per work item).
  if constexpr (E::bytes == 2) {
    if (group >= 4 && a.block_size >= 16) {
      if (group == 4) return launch_typed<E, D, 4, true>(a, ws, s);
      if (group <= 8) return launch_typed<E, D, 8, true>(a, ws, s);
      return launch_typed<E, D, 16, true>(a, ws, s);
    }
  }
  if (group == 1) return launch_typed<E, D, 1, false>(a, ws, s);
  if (group == 2) return launch_typed<E, D, 2, false>(a, ws, s);
  if (group <= 4) return launch_typed<E, D, 4, false>(a, ws, s);
  return launch_typed<E, D, 8, false>(a, ws, s);
}

template <class E>
hipError_t launch_dim(const DecodeLaunch &a, const DecodeWorkspace &ws, hipStream_t s) {
  if (a.head_dim == 64) return launch_group<E, 64>(a, ws, s);
  return launch_group<E, 128>(a, ws, s);
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads,
                                        int64_t head_dim, int64_t max_parts) {
  // counts (work_count, next_item) | work list | merge arrival counters
  // (one per sequence and query head: at least one per (sequence, kv head,
  // head chunk)) | partials
  (void)num_kv_heads;
  DecodeWorkspace w;
  w.count_off = 0;
  w.work_off = 256;
  size_t off = align_up(w.work_off + (size_t)num_seqs * max_parts * 2 * sizeof(int32_t), 256);
  w.arrive_off = off;
  off = align_up(off + (size_t)num_seqs * num_heads * sizeof(int32_t), 256);
  w.part_o_off = off;
  w.part_ml_off = off;
  if (max_parts > 1) {
    off = align_up(off + (size_t)num_seqs * num_heads * max_parts * head_dim * sizeof(float), 256);
    w.part_ml_off = off;
    off = align_up(off + (size_t)num_seqs * num_heads * max_parts * 2 * sizeof(float), 256);
  }
  w.total = off;
  return w;
}

// ---- Scratch of the allocation-free entry point --------------------------
// paged_attn_decode_noalloc keeps the work list, the counters and the
// split-KV partials of a call here instead of in a caller workspace.  Every
// GPU the library runs on holds its own copy of this array, at its own
// address, from the first use until the process ends; every call on that GPU
// uses the same copy, so calls that overlap on one GPU race.  The host-side
// name is only a stand-in: kernels get the device address looked up below.
static __device__ __align__(256) char scratch[PA_DECODE_NOALLOC_SCRATCH_BYTES];

void *decode_noalloc_scratch() {
  static std::atomic<void *> per_device[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void *ptr = per_device[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  // Once per device, with that device current (two threads racing here
  // store the same address).
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();     // leave no sticky error for the next call
    return nullptr;
  }
  per_device[dev].store(ptr, std::memory_order_release);
  return ptr;
}

hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream) {
  const DecodeWorkspace ws = decode_workspace_layout(a.num_seqs, a.num_heads, a.num_kv_heads,
                                                     a.head_dim, a.max_parts);
  switch (a.dtype) {
    case DType::F32: return launch_dim<F32>(a, ws, stream);
    case DType::F16: return launch_dim<F16>(a, ws, stream);
    default: return launch_dim<BF16>(a, ws, stream);
  }
}

}  // namespace pa

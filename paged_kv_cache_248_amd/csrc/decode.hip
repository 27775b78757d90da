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
//     leaving (M, L, O~) partials that a second kernel merges with the same
//     rescaling (block-level parallelism, "vLLM中FlashAttention与KVCache优化解析",
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
//   * a sequence that spans several partitions leaves (M, L, O~) partials that
//     a short merge kernel combines; the weights of a (sequence, head) are
//     computed once in LDS and every partial is then read with independent
//     loads, so the merge costs a few memory latencies, not one per partial;
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
  int32_t num_heads, num_kv_heads, group, head_chunks;
  int32_t bs_log2, max_blocks_per_seq, num_blocks;
  int32_t partition, max_parts, ctx_cap;
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

template <class E, int D, int GT>
__global__ __launch_bounds__(256, GT == 4 ? 4 : 2) void decode_kernel(DecodeParams p) {
  using G = Geom<E, D, GT>;
  constexpr int NL = G::kNL, TPL = G::kTPL, LPT = G::kLPT, EPL = G::kEPL, TILE = G::kTile;
  __shared__ int s_item;
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
  const int total = as_const(p.work_count)[0] * Hkv * p.head_chunks;

  for (;;) {
    if (tid == 0) s_item = atomicAdd(p.next_item, 1);
    __syncthreads();
    const int item = s_item;
    if (item >= total) break;
    const int hc = item % p.head_chunks;
    const int rest = item / p.head_chunks;
    const int g = rest % Hkv;
    const int wi = rest / Hkv;
    const int b = as_const(p.work)[2 * wi];
    const int part = as_const(p.work)[2 * wi + 1];
    const int ctx = min(max(as_const(p.context_lens)[b], 0), p.ctx_cap);
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
        kr[L] = ld16(kpage_base + page_off + lane_off);
        vr[L] = ld16(vpage_base + page_off + lane_off);
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
        const size_t slot = row * p.max_parts + part;
        p.part_o[slot * D + d] = O;
        if (d == 0) {
          p.part_ml[slot * 2] = M;
          p.part_ml[slot * 2 + 1] = L;
        }
      }
    }
    __syncthreads();   // LDS and s_item are reused by the next item
  }
}

// Builds the compact list of (sequence, partition) work items — full-length
// partitions first, each sequence's shorter last partition after them — and
// clears the dynamic work counter.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t *context_lens, int num_seqs,
                                                           int partition, int ctx_cap,
                                                           int32_t *work, int32_t *work_count,
                                                           int32_t *next_item) {
  __shared__ int s_full[1024], s_tail[1024];
  __shared__ int s_total_full;
  const int tid = threadIdx.x;
  // pass 1: number of full partitions over all sequences
  int full_sum = 0;
  for (int b = tid; b < num_seqs; b += 1024) {
    const int ctx = min(max(context_lens[b], 0), ctx_cap);
    full_sum += ctx / partition;
  }
  s_full[tid] = full_sum;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) s_full[tid] += s_full[tid + off];
    __syncthreads();
  }
  if (tid == 0) s_total_full = s_full[0];
  __syncthreads();
  const int total_full = s_total_full;
  __syncthreads();
  // pass 2: place items, chunk by chunk of 1024 sequences
  int base_full = 0, base_tail = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += 1024) {
    const int b = c0 + tid;
    int nf = 0, nt = 0;
    if (b < num_seqs) {
      const int ctx = min(max(context_lens[b], 0), ctx_cap);
      nf = ctx / partition;
      nt = (ctx % partition) != 0;
    }
    s_full[tid] = nf;
    s_tail[tid] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int a = tid >= off ? s_full[tid - off] : 0;
      const int c = tid >= off ? s_tail[tid - off] : 0;
      __syncthreads();
      s_full[tid] += a;
      s_tail[tid] += c;
      __syncthreads();
    }
    const int f0 = base_full + s_full[tid] - nf;
    for (int k = 0; k < nf; ++k) {
      work[2 * (f0 + k)] = b;
      work[2 * (f0 + k) + 1] = k;
    }
    if (nt) {
      const int t0 = total_full + base_tail + s_tail[tid] - 1;
      work[2 * t0] = b;
      work[2 * t0 + 1] = nf;
    }
    base_full += s_full[1023];
    base_tail += s_tail[1023];
    __syncthreads();
  }
  if (tid == 0) {
    *work_count = total_full + base_tail;
    *next_item = 0;
  }
}


// Merges the partition partials of one (sequence, kv head, head chunk):
// M = max_p M_p, L = sum_p L_p 2^(M_p - M), O = sum_p O~_p 2^(M_p - M) / L —
// the OnlineSoftmax rescaling applied across partitions.  Wavefront w forms
// the weights 2^(M_p - M) / L of heads w, w+4, ... in LDS with wave-level
// reductions; then every (head, dim) sum reads its partials 32 at a time, so
// a sequence of many partitions costs a few memory round trips.
template <class E, int D, int GT>
__global__ __launch_bounds__(256) void decode_merge_kernel(void *out, const float *part_o,
                                                          const float *part_ml,
                                                          const int32_t *context_lens,
                                                          int num_heads, int group,
                                                          int head_chunks, int partition,
                                                          int max_parts, int ctx_cap) {
  extern __shared__ float s_w[];                  // [GT][max_parts]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.y;
  const int hc = blockIdx.x % head_chunks;
  const int g = blockIdx.x / head_chunks;
  const int ctx = min(max(context_lens[b], 0), ctx_cap);
  const int nparts = (ctx + partition - 1) / partition;
  if (nparts <= 1) return;
  const int h0 = g * group + hc * GT;
  const int nh = min(GT, group - hc * GT);
  for (int j = wave; j < nh; j += 4) {
    const float *ml = part_ml + ((size_t)b * num_heads + h0 + j) * max_parts * 2;
    float mx = -__builtin_inff();
    for (int q = lane; q < nparts; q += 64) mx = fmaxf(mx, ml[2 * q]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
    float ls = 0.f;
    for (int q = lane; q < nparts; q += 64) {
      const float c = fast_exp2(ml[2 * q] - mx);
      s_w[j * max_parts + q] = c;
      ls = fmaf(c, ml[2 * q + 1], ls);
    }
    for (int off = 32; off > 0; off >>= 1) ls += shfl_xor(ls, off);
    const float inv = 1.0f / ls;
    for (int q = lane; q < nparts; q += 64) s_w[j * max_parts + q] *= inv;
  }
  __syncthreads();
  for (int idx = tid; idx < nh * D; idx += 256) {
    const int j = idx / D, d = idx % D;
    const size_t row = (size_t)b * num_heads + h0 + j;
    const float *po = part_o + row * max_parts * D + d;
    const float *w = s_w + j * max_parts;
    // 32 partials per round, all loads in flight together; past the last
    // partition the index is clamped (a cached re-read) and the weight is 0
    float acc = 0.f;
    for (int q0 = 0; q0 < nparts; q0 += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = po[(size_t)min(q0 + u, nparts - 1) * D];
#pragma unroll
      for (int u = 0; u < 32; ++u) acc = fmaf(q0 + u < nparts ? w[q0 + u] : 0.f, v[u], acc);
    }
    store_elem<E>(out, row * D + d, acc);
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

template <class E, int D, int GT>
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

  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, a.context_lens,
                     a.num_seqs, a.partition, a.ctx_cap, reinterpret_cast<int32_t *>(w + ws.work_off),
                     reinterpret_cast<int32_t *>(w + ws.count_off), p.next_item);

  // Resident work-groups per CU; items are fetched dynamically, so a grid
  // larger than what fits only queues (it cannot unbalance the work).
  static int occ_cache[3][2][4] = {};
  const int ti = (int)a.dtype, di = D == 128, gi = GT == 1 ? 0 : GT == 2 ? 1 : GT == 4 ? 2 : 3;
  int occ = occ_cache[ti][di][gi];
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_kernel<E, D, GT>, 256, 0) !=
            hipSuccess || occ < 1)
      occ = 2;
    occ_cache[ti][di][gi] = occ;
  }
  const long long upper =
      (long long)a.num_seqs * a.max_parts * a.num_kv_heads * p.head_chunks;
  const long long resident = (long long)device_cu_count() * occ;
  const int grid = (int)std::max(1LL, std::min(upper, resident));
  profile_begin(stream);
  hipLaunchKernelGGL((decode_kernel<E, D, GT>), dim3(grid), dim3(256), 0, stream, p);
  profile_end(stream);
  if (a.max_parts > 1) {
    hipLaunchKernelGGL((decode_merge_kernel<E, D, GT>),
                       dim3(a.num_kv_heads * p.head_chunks, a.num_seqs), dim3(256),
                       (size_t)GT * a.max_parts * sizeof(float), stream, a.out, p.part_o,
                       p.part_ml, a.context_lens, a.num_heads, p.group, p.head_chunks,
                       a.partition, a.max_parts, a.ctx_cap);
  }
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_group(const DecodeLaunch &a, const DecodeWorkspace &ws, hipStream_t s) {
  const int group = a.num_heads / a.num_kv_heads;
  if (group == 1) return launch_typed<E, D, 1>(a, ws, s);
  if (group == 2) return launch_typed<E, D, 2>(a, ws, s);
  if (group <= 4) return launch_typed<E, D, 4>(a, ws, s);
  return launch_typed<E, D, 8>(a, ws, s);
}

template <class E>
hipError_t launch_dim(const DecodeLaunch &a, const DecodeWorkspace &ws, hipStream_t s) {
  if (a.head_dim == 64) return launch_group<E, 64>(a, ws, s);
  return launch_group<E, 128>(a, ws, s);
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads,
                                        int64_t head_dim, int64_t max_parts) {
  // counts (work_count, next_item) | work list | partials
  (void)num_kv_heads;
  DecodeWorkspace w;
  w.count_off = 0;
  w.work_off = 256;
  size_t off = align_up(w.work_off + (size_t)num_seqs * max_parts * 2 * sizeof(int32_t), 256);
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

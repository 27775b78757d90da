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
//   * one wavefront = one work item (sequence, kv head, partition, head
//     chunk).  The grid is persistent: (#CU x resident waves) wavefronts walk
//     a compact work list built on device, so no wavefront is launched for an
//     empty partition and all partitions have equal size;
//   * a token row (D * elem bytes) is split into 16-byte pieces, one per lane:
//     each load instruction moves 1 KiB fully coalesced; the lanes of one
//     token reduce their partial dot products with DPP row exchanges;
//   * the next tile's K and V (16 KiB for fp16/D128) are in flight while the
//     current tile is consumed; block ids are fetched one tile further ahead
//     through the scalar cache so the dependent id -> data load chain never
//     stalls the vector pipe;
//   * reductions only depend on a token's logical position, never on its
//     physical block, so permuting the pool leaves results bit-identical.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <class E, int D>
struct Geom {
  static constexpr int kRowBytes = D * E::bytes;   // one token row of K or V
  static constexpr int kLPT = kRowBytes / 16;      // lanes per token
  static constexpr int kTPL = 64 / kLPT;           // tokens per load instruction
  static constexpr int kNL = 8;                    // load instructions per tile per tensor
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
__device__ __forceinline__ float uniformf(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

template <class E, int D, int GT>
__global__ __launch_bounds__(64) void decode_kernel(DecodeParams p) {
  using G = Geom<E, D>;
  constexpr int NL = G::kNL, TPL = G::kTPL, LPT = G::kLPT, EPL = G::kEPL, TILE = G::kTile;
  const int lane = threadIdx.x;
  const int tok = lane / LPT;     // token of each load this lane holds
  const int chunk = lane % LPT;   // 16-byte piece of the row this lane holds
  const int bs = 1 << p.bs_log2;
  const int Hq = p.num_heads, Hkv = p.num_kv_heads;
  const char *kbase = static_cast<const char *>(p.k_cache);
  const char *vbase = static_cast<const char *>(p.v_cache);
  const size_t head_stride = (size_t)bs * G::kRowBytes;          // one (block, head) page
  const size_t block_stride = head_stride * (size_t)Hkv;
  const int total = uniform(*p.work_count) * Hkv * p.head_chunks;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int hc = item % p.head_chunks;
    const int rest = item / p.head_chunks;
    const int g = rest % Hkv;
    const int wi = rest / Hkv;
    const int b = uniform(p.work[2 * wi]);
    const int part = uniform(p.work[2 * wi + 1]);
    const int ctx = min(max(uniform(p.context_lens[b]), 0), p.ctx_cap);
    const int start = part * p.partition;
    const int end = min(start + p.partition, ctx);
    const int nparts = (ctx + p.partition - 1) / p.partition;
    const int h0 = g * p.group + hc * GT;
    const int nh = min(GT, p.group - hc * GT);
    const int npages = (ctx + bs - 1) >> p.bs_log2;
    const int32_t *tbl = p.block_tables + (size_t)b * p.max_blocks_per_seq;
    const char *kpage_base = kbase + (size_t)g * head_stride + (size_t)chunk * 16;
    const char *vpage_base = vbase + (size_t)g * head_stride + (size_t)chunk * 16;

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

    const int ntiles = (end - start + TILE - 1) / TILE;

    // Block ids of the pages each load of a tile touches (wave-uniform).
    auto fetch_ids = [&](int tile, int *ids) {
      const int ts = start + tile * TILE;
#pragma unroll
      for (int L = 0; L < NL; ++L) {
        const int page = (ts + L * TPL) >> p.bs_log2;
        int id = 0;
        if (tile < ntiles && page < npages) id = tbl[page];
        ids[L] = (int)min((unsigned)id, (unsigned)(p.num_blocks - 1));
      }
    };
    auto issue = [&](int tile, const int *ids, u32x4 *kr, u32x4 *vr) {
      const int ts = start + tile * TILE;
#pragma unroll
      for (int L = 0; L < NL; ++L) {
        const int page = (ts + L * TPL) >> p.bs_log2;
        if (page < npages) {
          const int slot = (ts + L * TPL + tok) & (bs - 1);
          const size_t off = (size_t)ids[L] * block_stride + (size_t)slot * G::kRowBytes;
          kr[L] = ld16(kpage_base + off);
          vr[L] = ld16(vpage_base + off);
        } else {
          kr[L] = u32x4{0u, 0u, 0u, 0u};
          vr[L] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto consume = [&](int tile, const u32x4 *kr, const u32x4 *vr) {
      const int ts = start + tile * TILE;
      float x[GT][NL];
#pragma unroll
      for (int L = 0; L < NL; ++L) {
        const bool valid = ts + L * TPL + tok < end;
#pragma unroll
        for (int j = 0; j < GT; ++j) {
          const float s = group_sum<LPT>(dot16<E>(q[j], kr[L]));
          x[j][L] = valid ? s * p.scale_log2e : -__builtin_inff();
        }
      }
#pragma unroll
      for (int j = 0; j < GT; ++j) {
        float mx = x[j][0];
#pragma unroll
        for (int L = 1; L < NL; ++L) mx = fmaxf(mx, x[j][L]);
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
      const bool tail = ts + TILE > end;     // only the last tile can hold rows past the end
#pragma unroll
      for (int L = 0; L < NL; ++L) {
        float vf[EPL];
        unpack16<E>(vr[L], vf);
        if (tail && ts + L * TPL + tok >= end) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) vf[e] = 0.f;   // slots past the context may hold anything
        }
#pragma unroll
        for (int j = 0; j < GT; ++j)
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(x[j][L], vf[e], o[j][e]);
      }
    };

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

    // Combine the lane groups (different tokens, same dims).
#pragma unroll
    for (int j = 0; j < GT; ++j) {
      l[j] = across_groups_sum<LPT>(l[j]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] = across_groups_sum<LPT>(o[j][e]);
    }

    if (tok == 0 && end > start) {
      if (nparts <= 1) {
#pragma unroll
        for (int j = 0; j < GT; ++j) {
          if (j < nh) {
            const float inv = 1.0f / l[j];
            float r[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) r[e] = o[j][e] * inv;
            char *op = static_cast<char *>(p.out) +
                       ((size_t)(b * Hq + h0 + j) * D) * E::bytes + (size_t)chunk * 16;
            st16(op, pack16<E>(r));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < GT; ++j) {
          if (j < nh) {
            const size_t slot = ((size_t)(b * Hq + h0 + j) * p.max_parts + part);
            float *po = p.part_o + slot * D + chunk * EPL;
#pragma unroll
            for (int e = 0; e < EPL; e += 4)
              *reinterpret_cast<f32x4 *>(po + e) = f32x4{o[j][e], o[j][e + 1], o[j][e + 2], o[j][e + 3]};
            if (chunk == 0) {
              p.part_ml[slot * 2] = m[j];
              p.part_ml[slot * 2 + 1] = l[j];
            }
          }
        }
      }
    }
  }
}

// Builds the compact list of (sequence, partition) work items.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t *context_lens, int num_seqs,
                                                           int partition, int ctx_cap,
                                                           int32_t *work, int32_t *work_count) {
  __shared__ int s[1024];
  const int tid = threadIdx.x;
  int base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += 1024) {
    const int b = c0 + tid;
    int n = 0;
    if (b < num_seqs) {
      const int ctx = min(max(context_lens[b], 0), ctx_cap);
      n = (ctx + partition - 1) / partition;
    }
    s[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int t = tid >= off ? s[tid - off] : 0;
      __syncthreads();
      s[tid] += t;
      __syncthreads();
    }
    const int excl = base + s[tid] - n;
    for (int k = 0; k < n; ++k) {
      work[2 * (excl + k)] = b;
      work[2 * (excl + k) + 1] = k;
    }
    base += s[1023];
    __syncthreads();
  }
  if (tid == 0) *work_count = base;
}

// Merges the partition partials of each (sequence, head): M = max M_p,
// L = sum L_p 2^(M_p - M), O = sum O~_p 2^(M_p - M) / L.
template <class E, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(void *out, const float *part_o,
                                                          const float *part_ml,
                                                          const int32_t *context_lens,
                                                          int num_heads, int partition,
                                                          int max_parts, int ctx_cap) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int ctx = min(max(context_lens[b], 0), ctx_cap);
  const int nparts = (ctx + partition - 1) / partition;
  if (nparts <= 1) return;
  const size_t slot0 = (size_t)(b * num_heads + h) * max_parts;
  const float *ml = part_ml + slot0 * 2;
  float M = -__builtin_inff();
  for (int q = 0; q < nparts; ++q) M = fmaxf(M, ml[2 * q]);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float L = 0.f;
  for (int q = 0; q < nparts; ++q) {
    const float w = fast_exp2(ml[2 * q] - M);
    L = fmaf(w, ml[2 * q + 1], L);
    const float *po = part_o + (slot0 + q) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, po[threadIdx.x + 64 * i], acc[i]);
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = threadIdx.x + 64 * i;
    const float r = acc[i] * inv;
    const size_t idx = (size_t)(b * num_heads + h) * D + d;
    if constexpr (E::bytes == 4) {
      static_cast<float *>(out)[idx] = r;
    } else if constexpr (__is_same(typename E::storage, _Float16)) {
      static_cast<uint16_t *>(out)[idx] = f32_to_f16_bits(r);
    } else {
      static_cast<uint16_t *>(out)[idx] = f32_to_bf16(r);
    }
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
                     reinterpret_cast<int32_t *>(w + ws.count_off));

  static int occ_cache[3][2][4] = {};
  const int ti = (int)a.dtype, di = D == 128, gi = GT == 1 ? 0 : GT == 2 ? 1 : GT == 4 ? 2 : 3;
  int occ = occ_cache[ti][di][gi];
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_kernel<E, D, GT>, 64, 0) !=
            hipSuccess || occ < 1)
      occ = 4;
    occ_cache[ti][di][gi] = occ;
  }
  const long long upper =
      (long long)a.num_seqs * a.max_parts * a.num_kv_heads * p.head_chunks;
  const long long resident = (long long)device_cu_count() * occ;
  const int grid = (int)std::max(1LL, std::min(upper, resident));
  profile_begin(stream);
  hipLaunchKernelGGL((decode_kernel<E, D, GT>), dim3(grid), dim3(64), 0, stream, p);
  profile_end(stream);
  if (a.max_parts > 1) {
    hipLaunchKernelGGL((decode_merge_kernel<E, D>), dim3(a.num_heads, a.num_seqs), dim3(64), 0,
                       stream, a.out, p.part_o, p.part_ml, a.context_lens, a.num_heads,
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

DecodeWorkspace decode_workspace_layout(int64_t num_seqs, int64_t num_heads, int64_t head_dim,
                                        int64_t max_parts) {
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
  const DecodeWorkspace ws =
      decode_workspace_layout(a.num_seqs, a.num_heads, a.head_dim, a.max_parts);
  switch (a.dtype) {
    case DType::F32: return launch_dim<F32>(a, ws, stream);
    case DType::F16: return launch_dim<F16>(a, ws, stream);
    default: return launch_dim<BF16>(a, ws, stream);
  }
}

}  // namespace pa

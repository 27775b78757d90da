// Causal paged prefill / append for gfx950 on the matrix cores.
//
// Method (pages cited by title):
//   * Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V, computed FlashAttention
//     style: Q/K/V in tiles, QK^T -> softmax -> PV fused in one kernel, S and P
//     never written to HBM, softmax state (M, L, O) carried across key tiles by
//     the OnlineSoftmax update — "vLLM中FlashAttention与KVCache交换机制解析",
//     Kernel Fusion + Tiling + OnlineSoftmax and the M_new / L_new / O_new
//     equations (O kept unnormalised, divided by L once at the end);
//   * keys are read through the per-sequence block table of the paged cache
//     ("大模型长文本推理基座…PagedAttention 显存物理布局深度剖析" §二.2);
//   * prefill of new tokens over the cached prefix is the prefill step of the
//     serving flow on the swap-mechanism page; the new token t of a sequence
//     with q_b new tokens and n keys is at position n - q_b + t and sees keys
//     0..n - q_b + t (bottom-right causal alignment).
//
// Design for CDNA4:
//   * one work-group = 4 wavefronts; each wavefront owns 32 query rows of one
//     head; the heads of a GQA group sharing a kv head sit in the same
//     work-group, so each K/V tile staged in LDS serves all of them;
//   * per 64-key tile a wavefront computes S^T = K Q^T (2 x D/16 MFMA
//     32x32x16), so each lane holds one query's scores: the softmax max/sum
//     stay in-lane except one exchange with the lane 32 apart;
//   * P^T (bf16/fp16) feeds O^T += V^T P^T (D/32 x 4 MFMA) directly from the
//     S^T accumulator layout: the MFMA reduction order of the 16 keys of a
//     k-step is permuted identically in both operands, so no shuffle is needed;
//   * V is staged transposed in LDS (4-key x 8-dim register transpose with
//     v_perm), K row-major; both with XOR swizzles that make the MFMA operand
//     reads and the staging writes bank-conflict free;
//   * LDS is double buffered: the next tile's global loads are in flight while
//     the current tile is on the matrix cores; block ids run two tiles ahead;
//   * grid order: (sequence, kv head) fastest, query tiles from the last
//     (most keys) to the first; the (sequence, kv head) of a work-group fixes
//     its XCD, so the K/V of one head stays in one L2.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kRows = 32;      // query rows per wavefront
constexpr int kWaves = 4;

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

template <class E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (__is_same(typename E::storage, _Float16)) return pack_f16(a, b);
  else return pack_bf16(a, b);
}

template <class E>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (__is_same(typename E::storage, _Float16)) return f16_lo(w);
  else return bf16_lo(w);
}
template <class E>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (__is_same(typename E::storage, _Float16)) return f16_hi(w);
  else return bf16_hi(w);
}

// V^T row swizzle: 8-byte chunk c of row d is stored at c ^ vt_swz(d).
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 3) & 15) ^ (((d & 7) >> 1) << 2); }

template <class E, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  constexpr int KCH = D / 8;                    // 16-byte chunks per K row
  constexpr int K_BYTES = kBN * D * 2;          // K tile in LDS
  constexpr int VT_ROW = kBN * 2;               // bytes per V^T row
  constexpr int BUF = 2 * K_BYTES;              // K tile + V^T tile
  constexpr int UNITS = (kBN / 4) * KCH;        // (4 keys x 1 chunk) staging units
  constexpr int KS = D / 16;                    // MFMA k-steps over head_dim
  constexpr int DT = D / 32;                    // 32-wide output sub-tiles
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;      // query column owned by this lane
  const int half = lane >> 5;

  // Work-group coordinates.
  const int bg = blockIdx.x;                      // (sequence, kv head, head subgroup)
  const int hs = bg % p.subgroups;
  const int g = (bg / p.subgroups) % p.num_kv_heads;
  const int b = bg / (p.subgroups * p.num_kv_heads);
  const int qt = gridDim.y - 1 - blockIdx.y;      // last query tile first
  const int q0 = p.query_start_loc[b];
  const int qb = p.query_start_loc[b + 1] - q0;
  if (qt * p.pos_per_wg >= qb) return;
  const int ctx = min(max(p.context_lens[b], 0), p.ctx_cap);
  const int prefix = ctx - qb;
  const int bs = 1 << p.bs_log2;
  const int npages = (ctx + bs - 1) >> p.bs_log2;
  const int32_t *tbl = p.block_tables + (size_t)b * p.max_blocks_per_seq;

  const int hpw = p.heads_per_wg;
  const int h = g * p.group + hs * hpw + (wave % hpw);
  const int t0 = qt * p.pos_per_wg + (wave / hpw) * kRows;     // first row of this wavefront
  const int t = t0 + col;                                      // this lane's query row
  const bool row_ok = t < qb;
  const int pos = prefix + t;

  const int wg_last_t = min(qb, qt * p.pos_per_wg + p.pos_per_wg) - 1;
  const int kend = max(0, min(ctx, prefix + wg_last_t + 1));
  const int ntiles = (kend + kBN - 1) / kBN;
  const int wave_last_t = min(qb - 1, t0 + kRows - 1);
  const int wave_kend = max(0, min(ctx, prefix + wave_last_t + 1));
  const int wave_tiles = t0 < qb ? (wave_kend + kBN - 1) / kBN : 0;

  // Query fragment (B operand of S^T = K Q^T): lane holds d = 16ks + 8half .. +7.
  u32x4 qf[KS];
  {
    const char *qp = static_cast<const char *>(p.query) +
                     ((size_t)(q0 + t) * p.num_heads + h) * D * 2 + half * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? ld16(qp + ks * 32) : u32x4{0u, 0u, 0u, 0u};
  }

  // Staging unit of this thread: keys 4kg..4kg+3 of the tile, 16-byte chunk dc.
  const bool stager = tid < UNITS;
  const int kg = tid / KCH;
  const int dc = tid % KCH;
  const size_t head_stride = (size_t)bs * D * 2;
  const size_t block_stride = head_stride * p.num_kv_heads;
  const char *kb = static_cast<const char *>(p.k_cache) + (size_t)g * head_stride + dc * 16;
  const char *vb = static_cast<const char *>(p.v_cache) + (size_t)g * head_stride + dc * 16;

  auto fetch_id = [&](int tile) -> int {
    const int page = (tile * kBN + 4 * kg) >> p.bs_log2;
    int id = 0;
    if (stager && tile < ntiles && page < npages) id = tbl[page];
    return (int)min((unsigned)id, (unsigned)(p.num_blocks - 1));
  };
  u32x4 kr[4], vr[4];
  auto stage = [&](int tile, int id) {
    const int key0 = tile * kBN + 4 * kg;
    const bool page_ok = stager && (key0 >> p.bs_log2) < npages;
    const size_t base = (size_t)id * block_stride + (size_t)(key0 & (bs - 1)) * D * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (page_ok && key0 + i < ctx) {
        kr[i] = ld16(kb + base + (size_t)i * D * 2);
        vr[i] = ld16(vb + base + (size_t)i * D * 2);
      } else {
        kr[i] = u32x4{0u, 0u, 0u, 0u};
        vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto commit = [&](int buf) {
    if (!stager) return;
    char *kl = lds + buf * BUF;
    char *vl = kl + K_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * kg + i;
      st16(kl + row * (D * 2) + ((dc ^ (row & (KCH - 1))) * 16), kr[i]);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a0 = vr[0][w], a1 = vr[1][w], a2 = vr[2][w], a3 = vr[3][w];
      const u32x2 even = {__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                          __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
      const u32x2 odd = {__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                         __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
      const int d0 = dc * 8 + 2 * w;
      *reinterpret_cast<u32x2 *>(vl + d0 * VT_ROW + ((kg ^ vt_swz(d0)) * 8)) = even;
      *reinterpret_cast<u32x2 *>(vl + (d0 + 1) * VT_ROW + ((kg ^ vt_swz(d0 + 1)) * 8)) = odd;
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  float m = -__builtin_inff();
  float l = 0.f;

  int id_next = fetch_id(0);
  stage(0, id_next);
  id_next = fetch_id(1);
  int id_after = fetch_id(2);
  commit(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int cur = j & 1;
    if (j + 1 < ntiles) {
      stage(j + 1, id_next);
      id_next = id_after;
      id_after = fetch_id(j + 3);
    }
    if (j < wave_tiles) {
      const char *kl = lds + cur * BUF;
      const char *vl = kl + K_BYTES;
      // S^T = K Q^T for two 32-key sub-tiles.
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 acc = f32x16{};
        const int row = kt * 32 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = 2 * ks + half;
          const u32x4 a = ld16(kl + row * (D * 2) + ((c ^ (row & (KCH - 1))) * 16));
          acc = mfma32<E>(a, qf[ks], acc);
        }
        s[kt] = acc;
      }
      // Scale to log2 units and apply the causal mask where the tile can
      // reach past this wavefront's first position.
      const int key_base = j * kBN + 4 * half;
      const bool diag = j * kBN + kBN - 1 > prefix + t0;
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = s[kt][i] * p.scale_log2e;
          if (diag) {
            const int key = key_base + kt * 32 + 8 * (i >> 2) + (i & 3);
            if (key > pos) x = -__builtin_inff();
          }
          s[kt][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      if (__any(m_new > m)) {
        const float alpha = m_new > m ? fast_exp2(m - m_new) : 1.0f;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) o[i] *= alpha;
      }
      m = m_new;
      // A row with every key so far masked keeps m = -inf; use 0 as its
      // reference so its weights come out 0 instead of NaN.
      const float mref = m == -__builtin_inff() ? 0.f : m;
      // P^T fragments: k-step ks2 = 2kt + hh takes accumulator entries 8hh..8hh+7.
      u32x4 pf[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 w;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float e0 = fast_exp2(s[kt][8 * hh + 2 * q] - mref);
            const float e1 = fast_exp2(s[kt][8 * hh + 2 * q + 1] - mref);
            const uint32_t pk = pack2<E>(e0, e1);
            l += lo16<E>(pk) + hi16<E>(pk);     // normaliser of the rounded weights
            w[q] = pk;
          }
          pf[2 * kt + hh] = w;
        }
      // O^T += V^T P^T.
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 32 + col;
        const char *vrow = vl + d * VT_ROW;
        const int sw = vt_swz(d);
#pragma unroll
        for (int ks2 = 0; ks2 < 4; ++ks2) {
          const int c0 = 4 * ks2 + half;        // keys 16ks2 + 4half .. +3
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + ((c0 ^ sw) * 8));
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + (((c0 + 2) ^ sw) * 8));
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          o[dt] = mfma32<E>(a, pf[ks2], o[dt]);
        }
      }
    }
    if (j + 1 < ntiles) commit(cur ^ 1);
    __syncthreads();
  }

  if (!row_ok || wave_tiles == 0) return;
  const float lt = l + shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  char *op = static_cast<char *>(p.out) + ((size_t)(q0 + t) * p.num_heads + h) * D * 2;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = dt * 32 + 8 * r + 4 * half;
      const u32x2 v = {pack2<E>(o[dt][4 * r] * inv, o[dt][4 * r + 1] * inv),
                       pack2<E>(o[dt][4 * r + 2] * inv, o[dt][4 * r + 3] * inv)};
      *reinterpret_cast<u32x2 *>(op + d * 2) = v;
    }
}

template <class E, int D>
hipError_t launch_typed(const PrefillLaunch &a, hipStream_t stream) {
  PrefillParams p;
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
  const long long gx = (long long)a.num_seqs * a.num_kv_heads * p.subgroups;
  const int gy = (a.max_query_len + p.pos_per_wg - 1) / p.pos_per_wg;
  if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidValue;
  profile_begin(stream);
  hipLaunchKernelGGL((prefill_kernel<E, D>), dim3((unsigned)gx, gy), dim3(256), 0, stream, p);
  profile_end(stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream) {
  if (a.dtype == DType::F16)
    return a.head_dim == 64 ? launch_typed<F16, 64>(a, stream) : launch_typed<F16, 128>(a, stream);
  return a.head_dim == 64 ? launch_typed<BF16, 64>(a, stream) : launch_typed<BF16, 128>(a, stream);
}

}  // namespace pa

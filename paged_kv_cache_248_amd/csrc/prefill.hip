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
//   * grid order is XCD-aware: the ids an XCD receives walk one (sequence,
//     kv head) pair at a time through all its query tiles (the last, with the
//     most keys, first), so the tiles sharing K/V run together in one L2.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kRows = 32;      // query rows per wavefront
constexpr int kWaves = 4;
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

template <class E>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (__is_same(typename E::storage, _Float16))
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

template <class E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (__is_same(typename E::storage, _Float16)) return pack_f16(a, b);
  else return pack_bf16(a, b);
}

// V^T tile layout.  Row d holds the tile's 64 keys; inside every group of 16
// keys the key order is k -> (k & 3) | bit3(k) << 2 | bit2(k) << 3, which puts
// the 8 keys one lane feeds to a PV k-step (keys 4h..4h+3 and 8+4h..8+4h+3
// for lane half h) in one contiguous 16-byte chunk.  Chunk c of row d is
// stored at c ^ vt_swz(d); the swizzle depends on d mod 32 only, so the
// operand reads of every 32-row sub-tile share one set of per-lane offsets,
// and is conflict-free for those reads.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) & 7) ^ ((d >> 4) & 1); }

// Raise the running maximum (and rescale O and L) only when a tile's maximum
// exceeds it by more than 2^kLazy; weights then stay within [0, 2^kLazy].
constexpr float kLazy = 8.0f;

template <class E, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  constexpr int KCH = D / 8;                    // 16-byte chunks per K row
  constexpr int K_BYTES = kBN * D * 2;          // K tile in LDS
  constexpr int VT_ROW = kBN * 2;               // bytes per V^T row
  constexpr int BUF = 2 * K_BYTES;              // K tile + V^T tile
  constexpr int UNITS = (kBN / 4) * KCH;        // (4 keys x 1 chunk) staging units
  constexpr int KS = D / 16;                    // MFMA k-steps over head_dim
  constexpr int DT = D / 32;                    // 32-wide output sub-tiles
  static_assert(2 * BUF <= 65536, "LDS offsets must fit the 16-bit immediate");
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;      // query column owned by this lane
  const int half = lane >> 5;

  // Work-group coordinates.  Work-group ids are dealt round-robin to the 8
  // XCDs; id -> (xcd, local) -> (pair, query tile) makes each XCD run all the
  // query tiles of one (sequence, kv head, head subgroup) pair together, so
  // they stream the same K/V tiles through that XCD's L2 close in time.
  int pair, qt;
  {
    const int n_qt = p.num_qtiles, n_pairs = p.num_pairs;
    const int id = blockIdx.x;
    const int xcd = id % kXcds, local = id / kXcds;
    const int xcd_pairs = (n_pairs - xcd + kXcds - 1) / kXcds;   // pairs xcd, xcd+8, ...
    if (local < xcd_pairs * n_qt) {
      pair = xcd + kXcds * (local / n_qt);
      qt = n_qt - 1 - local % n_qt;               // last query tile (most keys) first
    } else {
      return;                                     // padding of the grid to a multiple of 8
    }
  }
  const int hs = pair % p.subgroups;
  const int g = (pair / p.subgroups) % p.num_kv_heads;
  const int b = pair / (p.subgroups * p.num_kv_heads);
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

  // Per-lane LDS read offsets (the sub-tile / buffer parts are immediates).
  int k_rd[KS], v_rd[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_rd[ks] = col * (D * 2) + (((2 * ks + half) ^ (col & (KCH - 1))) * 16);
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2)
    v_rd[ks2] = K_BYTES + col * VT_ROW + (((2 * ks2 + half) ^ vt_swz(col)) * 16);

  // Staging unit of this thread: keys 4kg..4kg+3 of the tile, 16-byte chunk dc.
  const bool stager = tid < UNITS;
  const int kg = tid / KCH;
  const int dc = tid % KCH;
  int k_wr[4], v_wr[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * kg + i;
    k_wr[i] = row * (D * 2) + ((dc ^ (row & (KCH - 1))) * 16);
  }
  {
    // the 4 keys land at 16-byte chunk vchunk, byte offset vsub, of each row
    const int vchunk = 2 * (kg >> 2) + (kg & 1);
    const int vsub = 8 * ((kg >> 1) & 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dc * 8 + e;
      v_wr[e] = K_BYTES + d * VT_ROW + ((vchunk ^ vt_swz(d)) * 16) + vsub;
    }
  }
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
  auto commit = [&](char *buf) {
    if (!stager) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(buf + k_wr[i], kr[i]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a0 = vr[0][w], a1 = vr[1][w], a2 = vr[2][w], a3 = vr[3][w];
      const u32x2 even = {__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                          __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
      const u32x2 odd = {__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                         __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
      *reinterpret_cast<u32x2 *>(buf + v_wr[2 * w]) = even;
      *reinterpret_cast<u32x2 *>(buf + v_wr[2 * w + 1]) = odd;
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  float m = -__builtin_inff();
  float l = 0.f;
  const float c = p.scale_log2e;
  // packed pair of 1.0 in the storage type
  const uint32_t ones2 = __is_same(typename E::storage, _Float16) ? 0x3C003C00u : 0x3F803F80u;

  // One key tile on the matrix cores: S^T = K Q^T, softmax update, O^T += V^T P^T.
  auto compute = [&](const char *buf, int j) {
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 acc = mfma32<E>(ld16(buf + k_rd[0] + kt * 32 * D * 2), qf[0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < KS; ++ks)
        acc = mfma32<E>(ld16(buf + k_rd[ks] + kt * 32 * D * 2), qf[ks], acc);
      s[kt] = acc;
    }
    // Causal mask where the tile can reach past this wavefront's first
    // position: key (tile offset kt*32 + 8*(i/4) + 4*half + i%4) > position.
    if (j * kBN + kBN - 1 > prefix + t0) {
      const int lim = pos - (j * kBN + 4 * half);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kt][i] = (kt * 32 + 8 * (i >> 2) + (i & 3)) > lim ? -__builtin_inff() : s[kt][i];
    }
    // Row maximum on raw scores (scale > 0); the scale is folded into the
    // exponent: p = 2^(s*c - m).
    // (NaN-propagating maximum: lowers to v_maximum3_f32 without the
    // per-operand canonicalisation an IEEE fmax needs)
    float rmx = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = (kt == 0 ? 2 : 0); i < 16; i += 2)
        rmx = __builtin_elementwise_maximum(rmx, __builtin_elementwise_maximum(s[kt][i], s[kt][i + 1]));
    rmx = __builtin_elementwise_maximum(rmx, shfl_xor(rmx, 32));
    const float cand = rmx * c;
    if (__any(cand > m + kLazy)) {
      const float m_new = fmaxf(m, cand);
      const float alpha = m_new > m ? fast_exp2(m - m_new) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) o[i] *= alpha;
      m = m_new;
    }
    // A row with every key so far masked keeps m = -inf; use 0 as its
    // reference so its weights come out 0 instead of NaN.
    const float nm = m == -__builtin_inff() ? 0.f : -m;
    // P^T fragments: k-step ks2 = 2kt + hh takes accumulator entries 8hh..8hh+7.
    u32x4 pf[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e0 = fast_exp2(fmaf(s[kt][8 * hh + 2 * q], c, nm));
          const float e1 = fast_exp2(fmaf(s[kt][8 * hh + 2 * q + 1], c, nm));
          const uint32_t pk = pack2<E>(e0, e1);
          l = dot2<E>(pk, ones2, l);     // L sums the rounded weights PV uses
          w[q] = pk;
        }
        pf[2 * kt + hh] = w;
      }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2)
        o[dt] = mfma32<E>(ld16(buf + v_rd[ks2] + dt * 32 * VT_ROW), pf[ks2], o[dt]);
  };

  int id_next = fetch_id(0);
  stage(0, id_next);
  id_next = fetch_id(1);
  int id_after = fetch_id(2);
  commit(lds);
  __syncthreads();

  // Tile j uses buffer j % 2; the loop is unrolled by two so every LDS
  // offset is a compile-time immediate.
  auto step = [&](auto cur_tag, int j) {
    constexpr int CUR = decltype(cur_tag)::value;
    if (j + 1 < ntiles) {
      stage(j + 1, id_next);
      id_next = id_after;
      id_after = fetch_id(j + 3);
    }
    if (j < wave_tiles) compute(lds + CUR * BUF, j);
    if (j + 1 < ntiles) commit(lds + (CUR ^ 1) * BUF);
    __syncthreads();
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) step(std::integral_constant<int, 1>{}, j + 1);
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
  const long long pairs = (long long)a.num_seqs * a.num_kv_heads * p.subgroups;
  const long long qtiles = (a.max_query_len + p.pos_per_wg - 1) / p.pos_per_wg;
  // each XCD gets ceil(pairs / 8) pairs' worth of slots
  const long long grid = kXcds * ((pairs + kXcds - 1) / kXcds) * qtiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  p.num_pairs = (int32_t)pairs;
  p.num_qtiles = (int32_t)qtiles;
  profile_begin(stream);
  hipLaunchKernelGGL((prefill_kernel<E, D>), dim3((unsigned)grid), dim3(256), 0, stream, p);
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

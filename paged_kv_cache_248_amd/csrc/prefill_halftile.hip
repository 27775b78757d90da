// Causal paged prefill for gfx950, second schedule: every wavefront
// interleaves its own softmax with its own matrix work (the alternative to
// the ping-pong schedule of prefill.hip, which stays the default; the
// library exports both so that they can be compared on one GPU).
//
// Method (pages cited by title): the same computation as prefill.hip —
// Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V fused per tile with the
// OnlineSoftmax (M, L, O) update ("vLLM中FlashAttention与KVCache交换机制解析",
// Kernel Fusion + Tiling + OnlineSoftmax), keys through the block table
// ("大模型长文本推理基座…PagedAttention 显存物理布局深度剖析" §二.2), the new
// token t of a sequence with q_b new tokens and n keys at position
// n - q_b + t seeing keys 0..n - q_b + t.
//
// Schedule:
//   * one work-group = 8 wavefronts (two per SIMD), each owning 32 query
//     rows of one head; the heads of a GQA group share the work-group and so
//     every K/V tile in LDS;
//   * K and V tiles go from the paged cache straight into LDS
//     (global_load_lds_dwordx4), four stages each; every wavefront loads 8
//     rows of each tile, so all of them issue loads;
//   * iteration j, after one work-group barrier, runs four segments of
//     MFMAs: QK^T of tile j+1's first 32 keys, PV of tile j's first 32 keys,
//     QK^T of tile j+1's second 32 keys, PV of tile j's second 32 keys.
//     While tile j+1's scores accumulate, the same wavefront turns tile j's
//     scores into weights (the exps ride along unit by unit), and in the
//     last segment it takes tile j+1's row maximum and decides its
//     reference, so the vector work of a tile hides behind the MFMAs of its
//     neighbour.  Tile j's first half is consumed before tile j+1's second
//     half is computed, so the scores need one and a half tiles of
//     registers;
//   * tiles that cross the causal diagonal take a sequential iteration
//     (mask, maximum, exps, then the MFMAs);
//   * the grid is the same persistent, XCD-aware one as prefill.hip's.
#include "prefill_common.h"

namespace pa {

namespace {

constexpr int kHalfReadAhead = 3;  // MFMAs whose operand reads are in flight ahead of the current one

// Segment plans of one iteration: the four interleaved segments, or one
// segment alone (0 QK^T first half, 1 PV first half, 2 QK^T second half,
// 3 PV second half).
enum : int { kPlanFull = 0, kPlanQk0 = 10, kPlanPv0 = 11, kPlanQk1 = 12, kPlanPv1 = 13 };
constexpr int plan_segments(int plan) { return plan == kPlanFull ? 4 : 1; }
constexpr int plan_segment(int plan, int i) { return plan == kPlanFull ? i : plan - 10; }

template <class E, int D>
__global__ __launch_bounds__(512, 1) void prefill_halftile_kernel(PrefillParams p) {
  constexpr int KCH = D / 8;                    // 16-byte chunks per row
  constexpr int ROWB = D * 2;                   // bytes per K or V row in LDS
  constexpr int TILE = kBN * ROWB;              // one K or V tile
  constexpr int RPI = 1024 / ROWB;              // rows per 1 KB load instruction
  constexpr int WROWS = kBN / kWaves;           // rows of each tile a wavefront loads
  constexpr int IPW = WROWS / RPI;              // load instructions per wavefront, tile and stream
  constexpr int KS = D / 16;                    // MFMA k-steps over head_dim
  constexpr int DT = D / 32;                    // 32-wide output sub-tiles
  constexpr int SEG = KS;                       // MFMAs per segment (QK^T and PV alike)
  constexpr int NS = kStages;
  constexpr int AHEAD = kHalfReadAhead;
  static_assert(KS == 2 * DT, "QK^T and PV segments of equal length");
  static_assert(IPW >= 1, "one load per wavefront and stream at least");
  extern __shared__ __attribute__((aligned(1024))) char lds[];   // K stages, then V stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;      // query column owned by this lane
  const int half = lane >> 5;

  // One work item: the query tile qt of one (sequence, kv head, head
  // subgroup) pair.
  auto process = [&](const int pair, const int qt) {
  const int hs = pair % p.subgroups;
  const int g = (pair / p.subgroups) % p.num_kv_heads;
  const int b = pair / (p.subgroups * p.num_kv_heads);
  const int q0 = p.query_start_loc[b];
  const int qb = p.query_start_loc[b + 1] - q0;
  if (qt * p.pos_per_wg >= qb) return;            // uniform over the work-group
  const int ctx = min(max(p.context_lens[b], 0), p.ctx_cap);
  const int prefix = ctx - qb;
  const int bs = 1 << p.bs_log2;
  const int npages = (ctx + bs - 1) >> p.bs_log2;
  const int32_t *tbl = p.block_tables + (size_t)b * p.max_blocks_per_seq;

  // This wavefront's 32 query rows: head (wave mod hpw) of the work-group's
  // heads, position block wave / hpw.
  const int hpw = p.heads_per_wg;
  const int h = g * p.group + hs * hpw + wave % hpw;
  const int t0 = qt * p.pos_per_wg + (wave / hpw) * kRows;
  const int t = t0 + col;                                  // this lane's query row
  const bool row_ok = t < qb;
  const int pos = prefix + t;
  const int last_t = min(qb - 1, t0 + kRows - 1);
  const int kend = max(0, min(ctx, prefix + last_t + 1));
  const int n = t0 < qb ? (kend + kBN - 1) / kBN : 0;      // this wavefront's key tiles
  const int wg_last_t = min(qb, qt * p.pos_per_wg + p.pos_per_wg) - 1;
  const int wg_kend = max(0, min(ctx, prefix + wg_last_t + 1));
  const int N = (wg_kend + kBN - 1) / kBN;                 // the work-group's key tiles

  // Query fragment (B operand of S^T = K Q^T): lane holds d = 16ks + 8half .. +7.
  u32x4 qf[KS];
  {
    const char *qp = static_cast<const char *>(p.query) +
                     ((size_t)(q0 + t) * p.num_heads + h) * D * 2 + half * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? ld16(qp + ks * 32) : u32x4{0u, 0u, 0u, 0u};
  }

  // LDS layouts and operand reads as in prefill.hip: K row-major with chunk
  // c of row r at c ^ (r mod KCH), read as the A operand with one
  // ds_read_b128 per MFMA; V row-major with chunk c at c ^ vsw(r), read
  // transposed with two ds_read_b64_tr_b16 per MFMA.
  int k_rd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_rd[ks] = col * ROWB + (((2 * ks + half) ^ (col & (KCH - 1))) * 16);
  auto vsw = [](int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  int v_tr[DT];
  {
    const int G = lane >> 4, tt = lane & 15;
    const int row = 4 * (G >> 1) + (tt >> 2);
    const int c0 = 2 * (G & 1) + ((tt & 3) >> 1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      v_tr[dt] = row * ROWB + (((4 * dt + c0) ^ vsw(row)) * 16) + 8 * (tt & 1);
  }

  // Tile loads: wavefront w loads rows WROWS w .. WROWS w + WROWS - 1 of
  // every K and V tile; they lie in one page (pages hold at least 8 keys),
  // whose block id is one scalar load.  Keys past the context are read as
  // copies of the last key (same page), which every query row masks.
  const size_t head_stride = (size_t)bs * D * 2;
  const size_t block_stride = head_stride * p.num_kv_heads;
  const char *ksrc = static_cast<const char *>(p.k_cache) + (size_t)g * head_stride;
  const char *vsrc = static_cast<const char *>(p.v_cache) + (size_t)g * head_stride;
  const int klast = max(ctx - 1, 0);
  const int lrow = lane / KCH;
  int lchunk[2][IPW], lane_off[2][IPW];
  const int rmask = min(bs, kBN) - 1;
#pragma unroll
  for (int q = 0; q < IPW; ++q) {
    const int r = WROWS * wave + RPI * q + lrow;
    lchunk[0][q] = ((lane % KCH) ^ (r & (KCH - 1))) * 16;
    lchunk[1][q] = ((lane % KCH) ^ vsw(r)) * 16;
    lane_off[0][q] = (r & rmask) * ROWB + lchunk[0][q];
    lane_off[1][q] = (r & rmask) * ROWB + lchunk[1][q];
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
  auto fetch_id = [&](int tile) -> int {
    return sload(tbl, min((tile * kBN + WROWS * wave) >> p.bs_log2, max(npages - 1, 0)));
  };
  auto id_tie = [](int &v) { asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v)); };
  auto load_tile = [&](int tile, int id, int vstream) {
    const char *src = (vstream ? vsrc : ksrc) +
                      (size_t)min((unsigned)id, (unsigned)(p.num_blocks - 1)) * block_stride;
    char *dst = lds + (vstream ? NS * TILE : 0) + (tile % NS) * TILE + (WROWS * wave) * ROWB;
    if (tile * kBN + kBN <= ctx) {                // every key of the tile exists
      const uint32_t toff = (uint32_t)((tile * kBN) & (bs - 1)) * ROWB;
#pragma unroll
      for (int q = 0; q < IPW; ++q) dma16(src + (toff + lane_off[vstream][q]), dst + RPI * q * ROWB);
    } else {
#pragma unroll
      for (int q = 0; q < IPW; ++q) {
        const int key = min(tile * kBN + WROWS * wave + RPI * q + lrow, klast);
        dma16(src + ((uint32_t)(key & (bs - 1)) * ROWB + lchunk[vstream][q]), dst + RPI * q * ROWB);
      }
    }
  };

  const float c = p.scale_log2e;
  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  f32x16 s[2];            // tile j's scores (32-key halves)
  f32x16 sn[2];           // tile j+1's
  u32x4 pf[4];            // tile j's weights, one P^T operand per PV k-step
  float m = -__builtin_inff(), l = 0.f, nm = 0.f, alpha = 1.f;
  bool need = false;
  float amax[4], ls[4];
  // Empty volatile statements that pin each softmax step to the MFMA unit it
  // rides with (the scheduler would otherwise sink the arithmetic).
  auto pin = [](float &x) { asm volatile("" : "+v"(x)); };
  auto pinu = [](uint32_t &x) { asm volatile("" : "+v"(x)); };

  // Weights of pair q (entries 2q, 2q+1) of tile j's scores: p = 2^(s c - m),
  // packed into the P^T operand of k-step 2 (q / 8) + (q mod 8) / 4; L adds
  // the fp32 weights in four partial sums.
  auto exp_pair = [&](auto q_tag) {
    constexpr int q = decltype(q_tag)::value;
    constexpr int kt = q / 8, i0 = (2 * q) % 16;
    float x0 = s[kt][i0], x1 = s[kt][i0 + 1];
    pin(x0);
    pin(x1);
    const float w0 = fast_exp2(fmaf(x0, c, nm));
    const float w1 = fast_exp2(fmaf(x1, c, nm));
    if constexpr (q < 2) ls[2 * q] = w0, ls[2 * q + 1] = w1;
    else ls[(2 * q) & 3] += w0, ls[(2 * q + 1) & 3] += w1;
    uint32_t pk = pack2<E>(w0, w1);
    pinu(pk);
    pf[2 * kt + (i0 >> 3)][(i0 & 7) >> 1] = pk;
    pin(ls[(2 * q) & 3]);
    pin(ls[(2 * q + 1) & 3]);
  };
  auto lsum = [&]() {
    l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    pin(l);
  };
  // Causal mask of tile jn's scores in sn, where the tile reaches past this
  // wavefront's first position: key (tile offset kt*32 + 8*(i/4) + 4*half +
  // i%4) > position.
  auto mask_next = [&](int jn) {
    const int lim = pos - (jn * kBN + 4 * half);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sn[kt][i] = (kt * 32 + 8 * (i >> 2) + (i & 3)) > lim ? -__builtin_inff() : sn[kt][i];
  };
  // Maximum of 8 of tile j+1's scores (step k of 4).
  auto max_step = [&](auto k_tag) {
    constexpr int k = decltype(k_tag)::value;
    if constexpr (k % 2 == 0) asm volatile("" : "+v"(sn[k / 2]));
    float v[8];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int e = 8 * k + e8;
      v[e8] = sn[e / 16][e % 16];
    }
    amax[k] = __builtin_elementwise_maximum(
        max3(v[0], v[1], v[2]),
        max3(v[3], v[4], __builtin_elementwise_maximum(v[5], __builtin_elementwise_maximum(v[6], v[7]))));
    pin(amax[k]);
  };
  // Reference for tile j+1: raised when its maximum (both lane halves)
  // exceeds the current one by more than 2^kLazy; L is rescaled now, O after
  // tile j's PV.  A row with every key so far masked keeps m = -inf and uses
  // 0 as its reference, so its weights come out 0 instead of NaN.
  auto decide = [&]() {
    const float r = __builtin_elementwise_maximum(max3(amax[0], amax[1], amax[2]), amax[3]);
    const f32x2 sw = pair_xor32(r);
    const float cand = __builtin_elementwise_maximum(sw[0], sw[1]) * c;
    need = __any(cand > m + kLazy);
    const float m_new = need ? fmaxf(m, cand) : m;
    alpha = m_new > m ? fast_exp2(m - m_new) : 1.0f;
    l *= alpha;
    m = m_new;
    nm = m_new == -__builtin_inff() ? 0.f : -m_new;
    pin(nm);
    pin(l);
  };

  // One plan: its MFMAs in order, each preceded by the LDS operand read of
  // the MFMA AHEAD later (an explicit lgkmcnt wait ties each operand to its
  // MFMA).  In the full plan the softmax steps ride along: tile j's exps
  // over segments 0-1, its row sum at the start of segment 2, tile j+1's
  // maximum and reference in segment 3.
  auto iteration = [&](auto plan_tag, uint32_t kb, uint32_t vb) {
    constexpr int PLAN = decltype(plan_tag)::value;
    constexpr int NU = plan_segments(PLAN) * SEG;
    u32x4 R[AHEAD + 1];
    auto issue = [&](auto u_tag) {
      constexpr int u = decltype(u_tag)::value;
      constexpr int seg = plan_segment(PLAN, u / SEG), w = u % SEG;
      u32x4 &r = R[u % (AHEAD + 1)];
      if constexpr (seg == 0 || seg == 2) {
        constexpr int kt = seg / 2;
        r = lds_b128<kt * 32 * ROWB>(kb + k_rd[w]);
      } else {
        constexpr int kt = seg / 2, ks2 = 2 * kt + w / DT, dt = w % DT;
        const uint32_t ad = vb + v_tr[dt];
        const u32x2 lo = lds_tr16<(16 * ks2) * ROWB>(ad), hi = lds_tr16<(16 * ks2 + 8) * ROWB>(ad);
        r = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    auto consume = [&](auto u_tag) {
      constexpr int u = decltype(u_tag)::value;
      constexpr int seg = plan_segment(PLAN, u / SEG), w = u % SEG;
      u32x4 &r = R[u % (AHEAD + 1)];
      if constexpr (seg == 0 || seg == 2) {
        constexpr int kt = seg / 2;
        sn[kt] = mfma32<E>(r, qf[w], w == 0 ? f32x16{} : sn[kt]);
      } else {
        constexpr int kt = seg / 2, ks2 = 2 * kt + w / DT, dt = w % DT;
        o[dt] = mfma32<E>(r, pf[ks2], o[dt]);
      }
    };
    auto softmax_at = [&](auto u_tag) {
      if constexpr (PLAN == kPlanFull) {
        constexpr int u = decltype(u_tag)::value;
        for_each_index(std::make_integer_sequence<int, 16>{}, [&](auto q_tag) {
          if constexpr ((decltype(q_tag)::value * 2 * SEG) / 16 == u) exp_pair(q_tag);
        });
        if constexpr (u == 2 * SEG) lsum();
        if constexpr (u == 3 * SEG) max_step(std::integral_constant<int, 0>{});
        if constexpr (u == 3 * SEG + 1) max_step(std::integral_constant<int, 1>{});
        if constexpr (u == 3 * SEG + SEG / 2) max_step(std::integral_constant<int, 2>{});
        if constexpr (u == 3 * SEG + SEG / 2 + 1) max_step(std::integral_constant<int, 3>{});
        if constexpr (u == 4 * SEG - 1) decide();
      }
    };
    constexpr auto ops = [](int v) { return (plan_segment(PLAN, v / SEG) & 1) ? 2 : 1; };
    for_each_index(std::make_integer_sequence<int, (AHEAD < NU ? AHEAD : NU)>{},
                   [&](auto u_tag) { issue(u_tag); });
    for_each_index(std::make_integer_sequence<int, NU>{}, [&](auto u_tag) {
      constexpr int u = decltype(u_tag)::value;
      if constexpr (u + AHEAD < NU) issue(std::integral_constant<int, u + AHEAD>{});
      constexpr int later = [&] {
        int nn = 0;
        for (int v = u + 1; v <= u + AHEAD && v < NU; ++v) nn += ops(v);
        return nn;
      }();
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(R[u % (AHEAD + 1)]) : "i"(later < 15 ? later : 15));
      consume(u_tag);
      softmax_at(u_tag);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto all_exps = [&]() {
    for_each_index(std::make_integer_sequence<int, 16>{}, [&](auto q_tag) { exp_pair(q_tag); });
    lsum();
  };
  auto next_max = [&](int jn) {
    if (jn * kBN + kBN - 1 > prefix + t0) mask_next(jn);
    for_each_index(std::make_integer_sequence<int, 4>{}, [&](auto k_tag) { max_step(k_tag); });
    decide();
  };
  auto rescale = [&]() {
    if (need) {
#pragma unroll
      for (int i = 0; i < DT; ++i) o[i] *= alpha;
      need = false;
    }
  };
  constexpr auto QK0 = std::integral_constant<int, kPlanQk0>{};
  constexpr auto QK1 = std::integral_constant<int, kPlanQk1>{};
  constexpr auto PV0 = std::integral_constant<int, kPlanPv0>{};
  constexpr auto PV1 = std::integral_constant<int, kPlanPv1>{};

  // Loads issued after the ones awaited at the end of iteration j (K_{j+2},
  // V_{j+1}): K_{j+3}, V_{j+2}, K_{j+4}, V_{j+3}, those that exist.
  auto wait_after = [&](int j) {
    if (j + 4 < N) wait_vm<4 * IPW>();
    else if (j + 3 < N) wait_vm<3 * IPW>();
    else if (j + 2 < N) wait_vm<IPW>();
    else wait_vm<0>();
  };

  // Prologue: K_0, K_1, V_0, K_2, V_1, K_3, V_2 (iteration j continues with
  // K_{j+4}, V_{j+3}); wait for K_0 (and the query loads before it).
  {
    int id[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) id[tt] = fetch_id(tt);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) id_tie(id[tt]);
    int after0 = 0;
    if (N > 0) load_tile(0, id[0], 0);
    if (N > 1) { load_tile(1, id[1], 0); ++after0; }
    if (N > 0) { load_tile(0, id[0], 1); ++after0; }
    if (N > 2) { load_tile(2, id[2], 0); ++after0; }
    if (N > 1) { load_tile(1, id[1], 1); ++after0; }
    if (N > 3) { load_tile(3, id[3], 0); ++after0; }
    if (N > 2) { load_tile(2, id[2], 1); ++after0; }
    switch (after0) {
      case 6: wait_vm<6 * IPW>(); break;
      case 5: wait_vm<5 * IPW>(); break;
      case 4: wait_vm<4 * IPW>(); break;
      case 3: wait_vm<3 * IPW>(); break;
      case 2: wait_vm<2 * IPW>(); break;
      case 1: wait_vm<IPW>(); break;
      default: wait_vm<0>(); break;
    }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  phase_sync();
  if (n > 0) {                                        // S_0, its mask and reference
    iteration(QK0, lds0, 0u);
    iteration(QK1, lds0, 0u);
    next_max(0);
    s[0] = sn[0];
    s[1] = sn[1];
    need = false;                                     // O is still zero
  }
  // Block ids of iteration 0's loads.  Scalar loads issued at the end of an
  // iteration are awaited after the next barrier, so none is in flight under
  // the LDS operand waits of the MFMAs (scalar and LDS loads share a counter).
  int id_k = fetch_id(4), id_v = fetch_id(3);
  wait_after(-1);

  // Iteration j: PV of tile j (V_j) and QK^T of tile j+1 (K_{j+1}); the
  // barrier that starts it publishes both; after it no wavefront reads K_j
  // or V_{j-1} any more, so their stages take K_{j+4} and V_{j+3}.
  auto begin = [&](int j, uint32_t &kb, uint32_t &vb) {
    phase_sync();
    id_tie(id_k);
    id_tie(id_v);
    if (j + 4 < N) load_tile(j + 4, id_k, 0);
    if (j + 3 < N) load_tile(j + 3, id_v, 1);
    kb = lds0 + ((j + 1) % NS) * TILE;
    vb = lds0 + (NS + j % NS) * TILE;
  };
  auto finish = [&](int j) {
    id_k = fetch_id(j + 5);
    id_v = fetch_id(j + 4);
    wait_after(j);
  };
  // Interleaved iterations while tile j+1 exists and needs no mask; then
  // sequential ones (the same barrier count in every wavefront: one per
  // work-group tile).
  const int jm = (prefix + t0 + 1) / kBN;           // first tile that needs the mask
  const int J1 = max(0, min(n - 1, jm - 1));
  int j = 0;
  for (; j < J1; ++j) {
    uint32_t kb, vb;
    begin(j, kb, vb);
    iteration(std::integral_constant<int, kPlanFull>{}, kb, vb);
    rescale();
    s[0] = sn[0];
    s[1] = sn[1];
    finish(j);
  }
  for (; j < N; ++j) {
    uint32_t kb, vb;
    begin(j, kb, vb);
    if (j < n) {
      all_exps();
      if (j + 1 < n) {
        iteration(QK0, kb, vb);
        iteration(QK1, kb, vb);
      }
      iteration(PV0, kb, vb);
      iteration(PV1, kb, vb);
      if (j + 1 < n) {
        next_max(j + 1);
        rescale();
        s[0] = sn[0];
        s[1] = sn[1];
      }
    }
    finish(j);
  }
  // No tile load may still be writing this work-group's LDS when it exits.
  wait_vm<0>();

  if (row_ok && n > 0) {
    const float lt = l + shfl_xor(l, 32);
    const float inv = 1.0f / lt;
    char *op = static_cast<char *>(p.out) + ((size_t)(q0 + t) * p.num_heads + h) * D * 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = dt * 32 + 8 * r4 + 4 * half;
        const u32x2 v = {pack2<E>(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv),
                         pack2<E>(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv)};
        *reinterpret_cast<u32x2 *>(op + d * 2) = v;
      }
  }
  // Every wavefront's tile loads have landed (each waited for all of its
  // own); the next item's prologue may refill any stage.
  phase_sync();
  };

  // Persistent, XCD-aware walk over the work items, as in prefill.hip.
  {
    const int n_qt = p.num_qtiles;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int per_xcd = gridDim.x / kXcds;
    const int xcd_pairs = (p.num_pairs - xcd + kXcds - 1) / kXcds;
    const int n_local = xcd_pairs * n_qt;
    for (int r = 0; r * per_xcd < n_local; ++r) {
      const int local = r * per_xcd + ((r & 1) ? per_xcd - 1 - slot : slot);
      if (local < n_local) process(xcd + kXcds * (local / n_qt), n_qt - 1 - local % n_qt);
    }
  }
}

template <class E, int D>
hipError_t launch_typed(const PrefillLaunch &a, hipStream_t stream) {
  PrefillParams p;
  long long grid = 0;
  int dev = 0;
  hipError_t e = prefill_setup(a, p, grid, dev);
  if (e != hipSuccess) return e;
  const size_t lds_bytes = (size_t)2 * kStages * kBN * D * 2;
  static std::atomic<uint64_t> attr_devices{0};
  e = prefill_allow_lds(reinterpret_cast<const void *>(&prefill_halftile_kernel<E, D>), lds_bytes,
                        dev, attr_devices);
  if (e != hipSuccess) return e;
  return launch_main(prefill_halftile_kernel<E, D>, dim3((unsigned)grid), dim3(64 * kWaves),
                     (uint32_t)lds_bytes, stream, p);
}

}  // namespace

hipError_t launch_prefill_halftile(const PrefillLaunch &a, hipStream_t stream) {
  if (a.dtype == DType::F16)
    return a.head_dim == 64 ? launch_typed<F16, 64>(a, stream) : launch_typed<F16, 128>(a, stream);
  return a.head_dim == 64 ? launch_typed<BF16, 64>(a, stream) : launch_typed<BF16, 128>(a, stream);
}

}  // namespace pa

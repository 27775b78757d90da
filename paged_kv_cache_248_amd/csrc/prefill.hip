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
//   * one work-group = 8 wavefronts in two groups of four; a CU runs one
//     work-group, so each SIMD holds one wavefront of each group.  Each
//     wavefront owns 32 query rows of one head; the heads of a GQA group
//     sharing a kv head sit in the same work-group, so each K/V tile in LDS
//     serves all of them;
//   * ping-pong schedule: the key loop runs in phases separated by
//     work-group barriers.  In every phase one group issues matrix work (QK of
//     tile j, then PV of tile j-1) while the other group does the softmax of
//     its last scores; the groups swap roles each phase.  The matrix cores and
//     the vector ALU of a SIMD are separate units, so the two wavefronts
//     sharing a SIMD keep both busy;
//   * K and V tiles go from the paged cache straight into LDS
//     (global_load_lds_dwordx4, no registers, no LDS write instructions), four
//     stages each, issued by each group in its softmax phase (the matrix
//     phases carry only MFMAs and their operand reads); completion is
//     awaited with exact vmcnt counts before the barrier that publishes a
//     tile, so loads of the next tiles stay in flight across phases;
//   * per 64-key tile a wavefront computes S^T = K Q^T (2 x D/16 MFMA
//     32x32x16), so each lane holds one query's scores: the softmax max/sum
//     stay in-lane except one exchange with the lane 32 apart;
//   * P^T (bf16/fp16) feeds O^T += V^T P^T (D/32 x 4 MFMA) directly from the
//     S^T accumulator layout: the MFMA reduction order of the 16 keys of a
//     k-step is permuted identically in both operands, so no shuffle is needed;
//   * K and V are row-major in LDS with XOR swizzles of the 16-byte chunks;
//     the V^T operand is read with the transposing ds_read_b64_tr_b16; the
//     operand reads of the seven MFMAs after the current one are in flight
//     while it executes;
//   * the grid is persistent (one work-group per CU, each taking several
//     work items), which removes the idle time between one work-group's end
//     and the next one's start on a CU; the item order is XCD-aware: the
//     work-groups of an XCD walk one (sequence, kv head) pair at a time
//     through all its query tiles (the last, with the most keys, first), so
//     the tiles sharing K/V run together in one L2.
#include "prefill_common.h"

namespace pa {

namespace {

constexpr int kReadAhead = 7;  // MFMAs whose operand reads are in flight ahead of the current one

template <class E, int D>
__global__ __launch_bounds__(512, 1) void prefill_kernel(PrefillParams p) {
  constexpr int KCH = D / 8;                    // 16-byte chunks per row
  constexpr int ROWB = D * 2;                   // bytes per K or V row in LDS
  constexpr int TILE = kBN * ROWB;              // one K or V tile
  constexpr int RPI = 1024 / ROWB;              // rows per 1 KB load instruction
  constexpr int IPW = 16 / RPI;                 // load instructions per wavefront and tile
  constexpr int KS = D / 16;                    // MFMA k-steps over head_dim
  constexpr int DT = D / 32;                    // 32-wide output sub-tiles
  constexpr int NS = kStages;
  // Outstanding vector-memory operations allowed when the tile issued
  // NS - 2 steps ago must be complete: each step issues IPW tile loads (and
  // no other vector-memory operation).
  constexpr int kWaitSteady = (NS - 2) * IPW;
  extern __shared__ __attribute__((aligned(1024))) char lds[];   // K stages, then V stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;      // 0: matrix work in even phases, loads K; 1: odd, loads V
  const int wi = wave & 3;        // wave within its group; waves wi and wi + 4 share a SIMD
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

  // Rows: the 32-row blocks of a head alternate between the groups, so both
  // groups reach the causal diagonal at about the same tile.
  const int hpw = p.heads_per_wg;
  const int h = g * p.group + hs * hpw + (wi % hpw);
  const int t0 = qt * p.pos_per_wg + ((wi / hpw) * 2 + grp) * kRows;
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

  // K tile in LDS: row r (key), 16-byte chunk c at position c ^ (r mod KCH).
  // K operand (A of S^T = K Q^T) read offsets; the 32-key sub-tile is an
  // immediate.
  int k_rd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_rd[ks] = col * ROWB + (((2 * ks + half) ^ (col & (KCH - 1))) * 16);
  // V tile in LDS: row r (key), chunk c at position c ^ vsw(r), vsw(r) =
  // 4 (r mod 4) for 256-byte rows and 4 ((r / 2) mod 2) for 128-byte rows.
  // The V^T operand of O^T += V^T P^T is read with ds_read_b64_tr_b16: in
  // each group of 16 lanes, output lane i takes element j from source lane
  // 4j + i/4, element i mod 4.  Source lane (G, tt) = (lane / 16, lane % 16)
  // therefore reads row 4 (G / 2) + tt / 4 of the 8-key half-step at
  // d = 16 (G mod 2) + 4 (tt mod 4), so that output lane l receives
  // V[4 (l / 32) + j][l mod 32] for j = 0..3: the four keys MFMA lane l
  // feeds (the second read, 8 keys later, gives the other four).  The
  // swizzle makes each 32-lane half of a read hit 16 distinct 16-byte bank
  // groups; one offset per 32-wide d sub-tile (the key offsets are
  // immediates).
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

  // Tile loads: group 0 loads K tiles, group 1 V tiles.  Wave wi of a group
  // loads rows 16 wi .. 16 wi + 15 of a tile with IPW instructions of RPI
  // rows; lane i of an instruction fills row i / KCH, position i mod KCH, so
  // it reads the global chunk (i mod KCH) ^ swizzle(row).  Keys past the
  // context are read as copies of the last key (same page, as pages hold a
  // multiple of RPI keys): such keys are masked for every query row, so their
  // P is 0 and the finite copy adds nothing.
  const size_t head_stride = (size_t)bs * D * 2;
  const size_t block_stride = head_stride * p.num_kv_heads;
  const char *src = static_cast<const char *>(grp == 0 ? p.k_cache : p.v_cache) +
                    (size_t)g * head_stride;
  const int klast = max(ctx - 1, 0);
  const int lrow = lane / KCH;                    // row of this lane within an instruction
  // Per instruction q: the global chunk byte offset of this lane, and its
  // byte offset within the page for tiles that lie inside the context (row
  // r of tile t is key 64 t + r, in slot (64 t mod bs) + (r mod min(bs, 64))).
  int lchunk[IPW], lane_off[IPW];
  const int rmask = min(bs, kBN) - 1;
#pragma unroll
  for (int q = 0; q < IPW; ++q) {
    const int r = 16 * wi + RPI * q + lrow;       // row within the tile
    const int sw = grp == 0 ? (r & (KCH - 1)) : vsw(r);
    lchunk[q] = ((lane % KCH) ^ sw) * 16;
    lane_off[q] = (r & rmask) * ROWB + lchunk[q];
  }
  char *const kbase = lds;
  char *const vbase = lds + NS * TILE;
  char *const mybase = grp == 0 ? kbase : vbase;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

  // Block ids of a tile for this wavefront, one per load instruction (the
  // page of its first row, clamped into the table row), as scalar loads:
  // they are issued at the start of the softmax phase before the matrix
  // phase that uses them and awaited at the start of that matrix phase,
  // before any of its LDS reads (scalar and LDS loads share one counter and
  // scalar loads complete out of order, so the wait is for all of them).
  // A wavefront's 16 rows of a tile lie in at most two pages (rows 0-7 and
  // 8-15 of its part share a page, as pages hold at least 8 keys): ids.v[h]
  // is the entry of the page of row 16 wi + 8 h.
  struct Ids { int v[2]; };
  auto fetch_ids = [&](int tile) -> Ids {
    Ids r;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      r.v[hh] = sload(tbl, min((tile * kBN + 16 * wi + 8 * hh) >> p.bs_log2, max(npages - 1, 0)));
    return r;
  };
  auto ids_tie = [](Ids &r) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(r.v[0]), "+s"(r.v[1]));
  };
  // Issue instructions [q_lo, q_hi) of the loads of a tile into its stage.
  auto load_tile = [&](int tile, const Ids &ids, int q_lo, int q_hi) {
    char *dst = mybase + (tile % NS) * TILE + (16 * wi) * ROWB;
    const char *base[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      base[hh] = src + (size_t)min((unsigned)ids.v[hh], (unsigned)(p.num_blocks - 1)) * block_stride;
    if (tile * kBN + kBN <= ctx) {                // every key of the tile exists
      const uint32_t toff = (uint32_t)((tile * kBN) & (bs - 1)) * ROWB;
#pragma unroll
      for (int q = 0; q < IPW; ++q) {
        if (q < q_lo || q >= q_hi) continue;
        dma16(base[RPI * q / 8] + (toff + lane_off[q]), dst + RPI * q * ROWB);
      }
    } else {
#pragma unroll
      for (int q = 0; q < IPW; ++q) {
        if (q < q_lo || q >= q_hi) continue;
        const int key = min(tile * kBN + 16 * wi + RPI * q + lrow, klast);
        dma16(base[RPI * q / 8] + ((uint32_t)(key & (bs - 1)) * ROWB + lchunk[q]),
              dst + RPI * q * ROWB);
      }
    }
  };

  const float c = p.scale_log2e;

  // The whole key loop of one group, specialised on the group so that each
  // wavefront runs straight-line code with its own register allocation.
  auto run = [&](auto grp_tag) {
    constexpr int GRP = decltype(grp_tag)::value;
    f32x16 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] = f32x16{};
    f32x16 s[2];
    u32x4 pf[4];
    float m = -__builtin_inff();
    float l = 0.f;

    // Matrix phase: S^T = K_j Q^T, then O^T += V^T_{j-1} P^T_{j-1}.
    auto matrix_phase = [&](uint32_t kb, uint32_t vb, bool do_pv) {
      // One unit = one MFMA; the operand reads of unit u + AHEAD are issued
      // before the MFMA of unit u (same-box A/B: 7 ahead, one MFMA per unit,
      // +0.9% over groups of four MFMAs read one group ahead; 5 ahead +0.7%;
      // 9 ahead runs out of registers and loses 1.3%).
      constexpr int AHEAD = kReadAhead;
      constexpr int QN = 2 * KS;                  // QK MFMAs, (kt, ks) with kt major
      constexpr int PN = 4 * DT;                  // PV MFMAs, (dt, ks2) with dt major
      u32x4 R[AHEAD + 1];
      auto issue = [&](auto u_tag) {
        constexpr int u = decltype(u_tag)::value;
        u32x4 &r = R[u % (AHEAD + 1)];
        if constexpr (u < QN) {
          constexpr int kt = u / KS, ks = u % KS;
          r = lds_b128<kt * 32 * ROWB>(kb + k_rd[ks]);
        } else {
          constexpr int dt = (u - QN) / 4, ks2 = (u - QN) % 4;
          const uint32_t ad = vb + v_tr[dt];
          const u32x2 lo = lds_tr16<(16 * ks2) * ROWB>(ad), hi = lds_tr16<(16 * ks2 + 8) * ROWB>(ad);
          r = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      };
      auto consume = [&](auto u_tag) {
        constexpr int u = decltype(u_tag)::value;
        u32x4 &r = R[u % (AHEAD + 1)];
        if constexpr (u < QN) {
          constexpr int kt = u / KS, ks = u % KS;
          s[kt] = mfma32<E>(r, qf[ks], ks == 0 ? f32x16{} : s[kt]);
        } else {
          constexpr int dt = (u - QN) / 4, ks2 = (u - QN) % 4;
          o[dt] = mfma32<E>(r, pf[ks2], o[dt]);
        }
      };
      auto pipeline = [&](auto n_tag) {
        constexpr int N = decltype(n_tag)::value;   // units run: QN (QK only) or QN + PN
        constexpr auto ops = [](int v) { return v < QN ? 1 : 2; };
        for_each_index(std::make_integer_sequence<int, (AHEAD < N ? AHEAD : N)>{},
                       [&](auto u_tag) { issue(u_tag); });
        for_each_index(std::make_integer_sequence<int, N>{}, [&](auto u_tag) {
            constexpr int u = decltype(u_tag)::value;
            if constexpr (u + AHEAD < N) issue(std::integral_constant<int, u + AHEAD>{});
            constexpr int later = [&] {
              int n = 0;
              for (int v = u + 1; v <= u + AHEAD && v < N; ++v) n += ops(v);
              return n;
            }();
            asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(R[u % (AHEAD + 1)]) : "i"(later < 15 ? later : 15));
            consume(std::integral_constant<int, u>{});
        });
      };
      if (do_pv) pipeline(std::integral_constant<int, QN + PN>{});
      else pipeline(std::integral_constant<int, QN>{});
    };

    // Softmax of tile j's scores: online update of (m, l, O) and the P^T
    // fragments for the next matrix phase.
    auto softmax = [&](int j) {
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
      const float rmx = row_max(s);
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
      // L adds the fp32 weights in four partial sums (plain VALU adds: the
      // dot2 instructions would not overlap with the other wavefront's MFMAs
      // on this SIMD); rounding P to 16 bits for PV is unbiased, so the
      // normalised output differs from summing the rounded weights only by
      // that rounding noise.
      float ls[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 w;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float e0 = fast_exp2(fmaf(s[kt][8 * hh + 2 * q], c, nm));
            const float e1 = fast_exp2(fmaf(s[kt][8 * hh + 2 * q + 1], c, nm));
            ls[q] = kt == 0 && hh == 0 ? e0 + e1 : ls[q] + (e0 + e1);
            w[q] = pack2<E>(e0, e1);
          }
          pf[2 * kt + hh] = w;
        }
      l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };

    // Prologue.  Group 0 loads K_0 .. K_{NS-2} and waits for K_0; group 1
    // loads V_0 .. V_{NS-3}.
    wait_vm<0>();                                 // query fragments in registers
    if constexpr (GRP == 0) {
#pragma unroll
      for (int tt = 0; tt < NS - 1; ++tt) {
        Ids pre = fetch_ids(tt);
        ids_tie(pre);
        load_tile(tt, pre, 0, IPW);
      }
      wait_vm<IPW * (NS - 2)>();
    } else {
#pragma unroll
      for (int tt = 0; tt < NS - 2; ++tt) {
        Ids pre = fetch_ids(tt);
        ids_tie(pre);
        load_tile(tt, pre, 0, IPW);
      }
    }
    phase_sync();

    // Step j = phases 2j and 2j+1.  In both, the matrix group reads K_j (K
    // stage j % NS) and V_{j-1} (V stage (j-1) % NS).  Each group issues its
    // tile loads in its softmax phase, so the matrix phases carry only MFMAs
    // and their operand reads: group 0 loads K_{j+NS-1} in phase 2j+1 and
    // waits for K_{j+1} before the barrier that ends it; group 1 loads
    // V_{j+NS-2} in phase 2j and waits for V_j before the barrier that ends
    // phase 2j+1.  A stage is refilled only after the barrier that ends the
    // last phase reading it.  The block ids of a load are fetched with scalar
    // loads at the start of the softmax phase and awaited after the softmax
    // (no LDS read is in flight there: scalar and LDS loads share a counter).
    for (int j = 0; j <= ntiles; ++j) {
      const uint32_t kb = lds0 + (j % NS) * TILE;
      const uint32_t vb = lds0 + (NS + (j + NS - 1) % NS) * TILE;
      const bool qk = j < wave_tiles;
      const bool pv = j >= 1 && j - 1 < wave_tiles;
      const int lt = GRP == 0 ? j + NS - 1 : j + NS - 2;     // tile loaded this step
      // The wavefront in its matrix phase runs at raised issue priority, so
      // that its operand reads and MFMAs win the SIMD's arbitration against
      // the softmax wavefront beside it.
      if constexpr (GRP == 0) {
        __builtin_amdgcn_s_setprio(1);                    // phase 2j
        matrix_phase(kb, vb, pv);
        __builtin_amdgcn_s_setprio(0);
        phase_sync();
        Ids ids = fetch_ids(lt);                          // phase 2j+1
        if (qk) softmax(j);
        ids_tie(ids);
        load_tile(lt, ids, 0, IPW);
        wait_vm<kWaitSteady>();
        phase_sync();
      } else {
        Ids ids = fetch_ids(lt);                          // phase 2j
        if (pv) softmax(j - 1);
        ids_tie(ids);
        load_tile(lt, ids, 0, IPW);
        phase_sync();
        __builtin_amdgcn_s_setprio(1);                    // phase 2j+1
        matrix_phase(kb, vb, pv);
        __builtin_amdgcn_s_setprio(0);
        wait_vm<kWaitSteady>();
        phase_sync();
      }
    }
    // No tile load may still be writing this work-group's LDS when it exits.
    wait_vm<0>();

    if (!row_ok || wave_tiles == 0) return;
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
  };
  if (grp == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
  // Every wavefront's tile loads have landed (each waited for all of its
  // own); the next item's prologue may refill any stage.
  phase_sync();
  };

  // The grid is persistent: a multiple of 8 work-groups, at most one per
  // CU.  Work-group ids are dealt round-robin to the 8 XCDs; XCD x owns the
  // pairs x, x + 8, ...  and its work-groups take that list of items (pair
  // by pair, the query tiles of a pair from the last, which has the most
  // keys, to the first) in rounds of one item each, so that the query tiles
  // of a pair run together and stream the same K/V tiles through that XCD's
  // L2.  The order within a round alternates between rounds: a work-group
  // that took one of the longer tiles of a pair takes one of the shorter
  // ones of the next pair.
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
  e = prefill_allow_lds(reinterpret_cast<const void *>(&prefill_kernel<E, D>), lds_bytes, dev,
                        attr_devices);
  if (e != hipSuccess) return e;
  return launch_main(prefill_kernel<E, D>, dim3((unsigned)grid), dim3(64 * kWaves),
                     (uint32_t)lds_bytes, stream, p);
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream) {
  if (a.dtype == DType::F16)
    return a.head_dim == 64 ? launch_typed<F16, 64>(a, stream) : launch_typed<F16, 128>(a, stream);
  return a.head_dim == 64 ? launch_typed<BF16, 64>(a, stream) : launch_typed<BF16, 128>(a, stream);
}

}  // namespace pa

// Block-sparse flash attention over per-query-block key-block lists.
//
// DFSAttn (Significance): block-wise execution over reordered tokens;
// DynamicRad (section 2.2): a shared candidate set aggregated block-wise for a
// FlashAttention-style kernel. Each workgroup owns one (head, query block);
// key blocks not in its list are never loaded.
//
// bf16 kernel (gfx950 matrix cores, wave64):
//  - one wave per 32 query rows (or 64 with two query tiles per wave); Q
//    stays in registers as the B operand;
//  - each listed key block is consumed in stages of 64 keys; K and V stages
//    go HBM/L2 -> LDS with direct (register-free) 16-byte loads into
//    XOR-swizzled, double-buffered layouts, requested one iteration (V) or
//    two (K) before they are read, so one barrier and one wait per stage;
//  - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 so each lane holds 32-key runs
//    of ONE query: the row max is in-lane plus one half-wave lane swap; the
//    next stage's S is computed in the same scheduling region as the current
//    stage's softmax and value product, so matrix and vector work overlap;
//  - online softmax in the log2 domain (scale folded into one FMA), keys
//    beyond a ragged block's real length masked to -inf;
//  - deferred values: a stage's exponentials are taken against the running
//    reference without the stage's own row max, the rounded row sums (every
//    weight is at most its row's sum) show when the reference is stale, and
//    only then is the max taken, O rescaled and the stage redone; P.V of a
//    stage runs beside the next stage's exponentials (fewer vector
//    instructions per stage than taking each stage's max first);
//  - P is rounded to bf16 straight from the accumulator layout and used as
//    the B operand of O^T += V^T P^T; V^T comes from the row-major V tile via
//    ds_read_b64_tr_b16 (no transpose pass) in the accumulator's key order;
//    the normalising row sum adds the rounded weights (v_dot2 with ones), so
//    output rows are convex combinations of V rows even under rounding;
//  - the list of key blocks and their real lengths is held in lanes and read
//    with v_readlane, keeping scalar memory round trips out of the loop;
//  - epilogue divides by the row sum, rounds to bf16, zeroes pad rows and
//    writes the natural-log log-sum-exp (from an unrounded fp32 sum).
// Token-layout I/O: Q rows are read from, and output rows written to, the
// token-major tensors through the slot -> token map, so the reorder of Q and
// the inverse reorder of O happen inside this kernel's first loads and last
// stores; pad slots take zero query rows and store nothing. With gathered
// K/V the direct LDS loads also fetch key/value rows from the token-major
// tensors (each lane's source rows for a stage are looked up in the map one
// iteration ahead), so no reordered copy of Q, K or V is made at all.
// f32 kernel: the same block-sparse online softmax on the float32 matrix
// cores (16x16x4 products, a wave per 16 queries), for float inputs.
#include <type_traits>

#include "common.h"

namespace hsa {


// tok[i] = max(lane i of this lane's 16-lane row of v, 0) for i < N (DPP
// row broadcast; the control must be a constant, hence the recursion).
template <int N, int I = 0>
__device__ __forceinline__ void row_bcast_clamped(int v, int (&tok)[N]) {
  if constexpr (I < N) {
    tok[I] = max(__builtin_amdgcn_update_dpp(0, v, 0x150 + I, 0xF, 0xF, false), 0);
    row_bcast_clamped<N, I + 1>(v, tok);
  }
}

// Software-pipelined variant. Each listed key block is processed in stages
// of ST keys (ST = 64 splits a 128-key block in two). K and V stages are
// double-buffered in LDS so that S(c+1) = K(c+1) Q^T is computed in the same
// scheduling region as the softmax and value product of stage c: the matrix
// core works on one stage while the vector ALU exponentiates the other.
// Loads for K(c+2) and V(c+1) are issued at the start of iteration c and
// have a whole iteration to land.
// A wave owns QT tiles of 32 queries. With QT = 2 every K or V fragment read
// from LDS feeds two matrix instructions, halving LDS read traffic per flop;
// the wave then needs about 400 registers, so each SIMD runs one wave and the
// overlap of matrix and vector work comes from the pipelining alone. With
// QT = 1 two workgroups of four waves share a CU, two waves per SIMD.
// IO: 0 reordered Q/K/V/O; 1 token-major Q and O; 2 token-major Q, K, V, O.
// WK: walk the stages, leaving out empty ones (below).
template <int D, int BK, int ST, int QT, bool LSE, int IO, bool WK = false>
__global__ void __launch_bounds__(BK * 2 / QT, QT == 1 ? 2 : 1)
attn_bf16_pipe_kernel(const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp,
                      const uint16_t *__restrict__ vp, uint16_t *__restrict__ op,
                      float *__restrict__ lse, const int32_t *__restrict__ blk_len,
                      const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt,
                      const int32_t *__restrict__ order, int max_kv, int kv_shared, int nh,
                      int nb, float scale_log2, const int32_t *__restrict__ perm,
                      int64_t q_stride, int64_t kv_stride, int64_t o_stride) {
  constexpr bool TOK = IO >= 1, GKV = IO == 2;
  constexpr int NW = BK / (32 * QT);
  constexpr int CPR = D / 8;
  constexpr int NS = BK / ST;   // stages per key block
  constexpr int MT = ST / 32;
  constexpr int DK = D / 16;
  constexpr int DM = D / 32;
  constexpr int PK = ST / 16;
  constexpr int TILE = ST * D;  // elements per stage buffer
  static_assert(BK % ST == 0 && ST % 32 == 0, "stage size");
  static_assert(NW >= 1 && BK % (32 * QT) == 0, "query tiles per wave");
  __shared__ __attribute__((aligned(1024))) uint16_t sK[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2 * TILE];

  int h, I;
  block_of(blockIdx.x, order, kv_shared, nh, nb, h, I);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ln = lane & 31;
  const int64_t head_off = static_cast<int64_t>(h) * nb * BK * D;
  const int qrow0 = w * 32 * QT + ln;  // row of query tile 0 within the block
  const uint32_t ldsK = lds_addr(sK), ldsV = lds_addr(sV);
  lds_char_t *const vl = to_lds(sV);
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    koff[i] = GKV ? tile_lane_chunk<D, false>(i, lane) : tile_lane_offset<D, false>(i, lane);
    voff[i] = GKV ? tile_lane_chunk<D, true>(i, lane) : tile_lane_offset<D, true>(i, lane);
  }
  const int64_t lrow = kv_shared ? static_cast<int64_t>(I) : static_cast<int64_t>(h) * nb + I;
  // caller lists: lengths clamped to [0, max_kv], entries to [0, nb)
  const int cnt = min(max(kv_cnt[lrow], 0), max_kv);
  const int32_t *list = kv_idx + lrow * max_kv;
  const uint16_t *kbase = GKV ? kp + h * D : kp + head_off;
  const uint16_t *vbase = GKV ? vp + h * D : vp + head_off;
  const uint32_t kv_row_bytes = static_cast<uint32_t>(kv_stride * 2);
  // Stage t covers keys (t % NS)*ST .. +ST of listed block t / NS. The
  // listed blocks and their real lengths sit in lanes, packed as
  // (J << 8) | L (lane i of the lo/hi pair holds entry mbase + i / mbase +
  // 64 + i), so a stage's address and length cost two lane reads instead of
  // dependent scalar loads. The window slides by 64 entries when the list is
  // longer than 128. (J < 2^24 and L <= BK <= 128 are checked on the host /
  // clamped here.)
  const int nst = cnt * NS;
  int mbase = 0, lo_E, hi_E;
  auto fetch = [&](int b0, int &mE) {
    const int i = b0 + lane;
    const int J = i < cnt ? min(max(list[i], 0), nb - 1) : 0;
    const int L = i < cnt ? min(max(blk_len[J], 0), BK) : 0;
    mE = static_cast<int>((static_cast<uint32_t>(J) << 8) | static_cast<uint32_t>(L));
  };
  fetch(0, lo_E);
  fetch(64, hi_E);
  wait_vmcnt<0>();
  auto entry_packed = [&](int b) {  // b in [mbase, mbase + 128), wave-uniform
    const int r = b - mbase;
    const int rl = r & 63;
    const int el = __builtin_amdgcn_readlane(lo_E, rl), eh = __builtin_amdgcn_readlane(hi_E, rl);
    return r < 64 ? el : eh;
  };
  auto entry = [&](int b, int &J, int &L) {
    const uint32_t e = static_cast<uint32_t>(entry_packed(b));
    J = static_cast<int>(e >> 8);
    L = static_cast<int>(e & 255u);
  };
  auto ofs_of = [&](int e, int half) {  // element offset of half `half` of packed entry e
    return static_cast<int64_t>(static_cast<uint32_t>(e) >> 8) * BK * D + static_cast<int64_t>(half) * ST * D;
  };
  auto valid_of = [&](int e, int half) { return min(max(static_cast<int>(e & 255) - half * ST, 0), ST); };
  auto stage_ofs = [&](int t) { return ofs_of(entry_packed(t / NS), t % NS); };
  auto stage_valid = [&](int t) { return valid_of(entry_packed(t / NS), t % NS); };
  // WK, with two stages per block and contiguous tiles: the stages are
  // walked block by block, and a block's second stage is left out when its
  // real keys fit in the first (a frame's last tile). That stage would only
  // add masked keys, i.e. zero weights and an unchanged O, so the outputs
  // are those of the full stage sequence. At the start of iteration c the
  // walk holds stage c (entry wE0, half wH0; wX0: it exists) and stage c+1
  // (wE1, wH1 at list position wB1; wX1); each iteration steps once, to
  // stage c+2, reading at most one new entry. The walk costs each stage a
  // few scalar instructions, so it is compiled only where such tiles are
  // expected (the launch picks it for lists shared by all heads, the frame
  // masks, and when the caller says the blocks are often short).
  constexpr bool kWalk = WK && NS == 2 && !GKV;
  int wE0 = 0, wH0 = 0, wE1 = 0, wH1 = 0, wB1 = 0;
  bool wX0 = false, wX1 = false;
  // the stage after (e, half) at list position b: its entry, half and
  // position; false if there is none
  auto walk_next = [&](int e, int half, int b, int &e2, int &h2, int &b2) {
    const bool second = half == 0 && (e & 255) > ST;
    const int en = entry_packed(b + 1);  // past the list: unused
    e2 = second ? e : en;
    h2 = second ? 1 : 0;
    b2 = second ? b : b + 1;
    return second || b + 1 < cnt;
  };
  // Otherwise, with two stages per block and contiguous tiles, iteration c
  // only needs the entries of blocks c/2 and c/2 + 1 (ea, eb): read once per
  // block, at even iterations, instead of once per use.
  constexpr bool kPair = NS == 2 && !GKV && !kWalk;
  int ea = 0, eb = 0;
  // Gathered K/V: the token rows this lane's loads of stage t read. With
  // D = 128 a 16-lane row of the wave fills one tile row per load, so each
  // lane fetches the map entry of load (lane mod NI) of its row and load i
  // takes lane i of the row by a DPP row broadcast: one lookup per stage.
  // Otherwise every load's entry is fetched. Raw entries are clamped to >= 0
  // when expanded (pad keys read token 0 and are masked).
  using TL = TileLoads<D, ST, NW>;
  constexpr bool kRowBcast = TL::CPR == 16 && 16 % TL::NI == 0;
  constexpr int RAW = kRowBcast ? 1 : TL::NI;
  uint32_t prow[RAW];
#pragma unroll
  for (int r = 0; r < RAW; ++r)
    prow[r] = static_cast<uint32_t>(kRowBcast ? TL::row(w, lane % TL::NI, lane) : TL::row(w, r, lane));
  auto stage_rows = [&](int t, int (&raw)[RAW]) {
    int J, L;
    entry(t / NS, J, L);
    const int32_t *pr = perm + (J * BK + (t % NS) * ST);
#pragma unroll
    for (int r = 0; r < RAW; ++r) raw[r] = pr[prow[r]];
  };
  auto expand_rows = [&](const int (&raw)[RAW], int (&tok)[TL::NI]) {
    if constexpr (kRowBcast) {
      row_bcast_clamped<TL::NI>(raw[0], tok);
    } else {
#pragma unroll
      for (int i = 0; i < TL::NI; ++i) tok[i] = max(raw[i], 0);
    }
  };
  // keep entries c / NS .. (c + 2) / NS inside the window
  auto slide = [&](int c) {
    if (c / NS - mbase >= 64) {
      mbase += 64;
      lo_E = hi_E;
      fetch(mbase + 64, hi_E);
      wait_vmcnt<0>();  // settle the window here, not at its first lane read
    }
  };
  // (kWalk) keep list positions b .. b + 1 inside the window
  auto slide_to = [&](int b) {
    if (b - mbase >= 64) {
      mbase += 64;
      lo_E = hi_E;
      fetch(mbase + 64, hi_E);
      wait_vmcnt<0>();
    }
  };

  // Q rows: reordered layout, or the token-major tensor through perm
  int qtok[QT];
  bf16x8 qf[QT][DK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qslot = I * BK + qrow0 + qt * 32;
    const uint16_t *qrow;
    if constexpr (TOK) {
      qtok[qt] = perm[qslot];
      qrow = qp + static_cast<int64_t>(max(qtok[qt], 0)) * q_stride + h * D + g * 8;
    } else {
      qtok[qt] = 0;
      qrow = qp + head_off + static_cast<int64_t>(qslot) * D + g * 8;
    }
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) qf[qt][ks] = *reinterpret_cast<const bf16x8 *>(qrow + ks * 16);
    // Pad query rows are zero, as in the reordered layout: their scores then
    // never trigger the wave-wide lazy rescale, so real rows round exactly as
    // they do there.
    if (TOK && qtok[qt] < 0) {
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) qf[qt][ks] = bf16x8{};
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) asm volatile("" ::"v"(qf[qt][ks]));
  int kofs[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) kofs[ks] = ln * CPR + ((2 * ks + g) ^ (ln & (CPR - 1)));
  const int q16 = lane >> 4, jj = lane & 15;
  int vofs[DM];
#pragma unroll
  for (int md = 0; md < DM; ++md) {
    const int col = md * 32 + (q16 & 1) * 16 + 4 * (jj & 3);
    const int chunk = (col >> 3) ^ ((jj & 12) & (CPR - 1));
    vofs[md] = ((g * 4 + (jj >> 2)) * CPR + chunk) * 16 + ((col >> 2) & 1) * 8;
  }

  f32x16 oacc[QT][DM];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int md = 0; md < DM; ++md)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qt][md][i] = 0.f;
  // Softmax reference m_ref (log2 units): the score buffers hold raw q.k
  // and each weight is exp2(s * scale_log2 - m_ref). noref: no stage with a
  // real key seen yet (then the first real max becomes the reference).
  float m_ref[QT], l_run[QT], e_run[QT];
  bool noref = true;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_ref[qt] = 0.f;
    l_run[qt] = 0.f;
    e_run[qt] = 0.f;
  }
  // a score as a log2 weight relative to the reference
  auto rel = [&](float x, int qt) { return fmaf(x, scale_log2, -m_ref[qt]); };
  // row max of a buffer relative to the reference (the two half-waves' runs
  // of the same query combined by a lane swap)
  auto rel_max = [&](const f32x16 (&sacc)[MT][QT], int qt) {
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mt][qt][i]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    return mx * scale_log2 - m_ref[qt];
  };

  auto compute_s = [&](f32x16 (&sacc)[MT][QT], int buf) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      bf16x8 kf[DK];
#pragma unroll
      for (int ks = 0; ks < DK; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8 *>(&sK[buf * TILE + (mt * 32 * CPR + kofs[ks]) * 8]);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[mt][qt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[mt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[qt][ks], sacc[mt][qt], 0, 0, 0);
    }
  };
  // Deferred-value pipeline: the exponentials of stage c are taken against
  // the current reference max without looking at the stage's own max first;
  // their rounded row sums decide afterwards whether the reference is stale
  // (a sum above 2^20, which bounds every weight, or not finite), and only
  // then is the max taken, O rescaled and the stage recomputed. Weights up
  // to 2^20 lose nothing in bf16 or in the float sums, and the high bound
  // makes the recomputation rare (with 2^8 it ran often enough to cost ~3
  // stages per workgroup). P.V of stage c runs one iteration later, beside
  // the next stage's exponentials.
  constexpr float kSumCap = 1048576.f;
  auto mask_tail = [&](f32x16 (&sacc)[MT][QT], int kvalid) {
    if (kvalid < ST) {
      const int lim = kvalid - g * 4;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (mt * 32 + (i >> 2) * 8 + (i & 3) >= lim) sacc[mt][qt][i] = -INFINITY;
    }
  };
  auto exps = [&](const f32x16 (&sacc)[MT][QT], bf16x8 (&pf)[QT][PK], float (&rs)[QT], float (&es)[QT]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      rs[qt] = 0.f;
      es[qt] = 0.f;
#pragma unroll
      for (int ks2 = 0; ks2 < PK; ++ks2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(rel(sacc[ks2 >> 1][qt][(ks2 & 1) * 8 + j], qt));
          if constexpr (LSE) es[qt] += p;
          pf[qt][ks2][j] = static_cast<__bf16>(p);
        }
        const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        const bf16x2 p01 = {pf[qt][ks2][0], pf[qt][ks2][1]}, p23 = {pf[qt][ks2][2], pf[qt][ks2][3]},
                     p45 = {pf[qt][ks2][4], pf[qt][ks2][5]}, p67 = {pf[qt][ks2][6], pf[qt][ks2][7]};
        rs[qt] = __builtin_amdgcn_fdot2_f32_bf16(p01, ones, rs[qt], false);
        rs[qt] = __builtin_amdgcn_fdot2_f32_bf16(p23, ones, rs[qt], false);
        rs[qt] = __builtin_amdgcn_fdot2_f32_bf16(p45, ones, rs[qt], false);
        rs[qt] = __builtin_amdgcn_fdot2_f32_bf16(p67, ones, rs[qt], false);
      }
    }
  };
  auto pv_only = [&](const bf16x8 (&pf)[QT][PK], int buf) {
#pragma unroll
    for (int ks2 = 0; ks2 < PK; ++ks2) {
      bf16x8 va[DM];
#pragma unroll
      for (int md = 0; md < DM; ++md) {
        lds_i16x4_t *a0 = (lds_i16x4_t *)(vl + buf * TILE * 2 + vofs[md] + ks2 * 16 * CPR * 16);
        lds_i16x4_t *a1 = (lds_i16x4_t *)(vl + buf * TILE * 2 + vofs[md] + (ks2 * 16 + 8) * CPR * 16);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(a0);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(a1);
        const i16x8_t both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        va[md] = __builtin_bit_cast(bf16x8, both);
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int md = 0; md < DM; ++md)
          oacc[qt][md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[md], pf[qt][ks2], oacc[qt][md], 0, 0, 0);
    }
  };
  // After the exponentials of a stage: rescale if any row's weights outgrew
  // the cap, then fold the stage's sums into the running ones.
  auto settle = [&](const f32x16 (&sacc)[MT][QT], bf16x8 (&pf)[QT][PK], float (&rs)[QT], float (&es)[QT]) {
    bool stale = noref;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) stale |= !(rs[qt] <= kSumCap);
    if (__any(stale)) {
      bool found = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float tm = m_ref[qt] + rel_max(sacc, qt);
        const bool fin = tm > -INFINITY;
        const float m_new = noref ? (fin ? tm : m_ref[qt]) : fmaxf(m_ref[qt], tm);
        const float alpha = noref ? 1.f : __builtin_amdgcn_exp2f(m_ref[qt] - m_new);
        l_run[qt] *= alpha;
        e_run[qt] *= alpha;
#pragma unroll
        for (int md = 0; md < DM; ++md)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qt][md][i] *= alpha;
        m_ref[qt] = m_new;
        found |= fin;
      }
      if (__any(found)) noref = false;
      exps(sacc, pf, rs, es);
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      l_run[qt] += rs[qt];
      if constexpr (LSE) e_run[qt] += es[qt];
    }
  };

  // Gathered K/V: byte offsets of this lane's loads for the V stage issued
  // next (ov) and the K stage issued next (ok), the source rows of that K
  // stage (rk, which the V stage after it reuses), and the raw entries of
  // the stage after it (rn, in flight). Offsets are formed at the end of
  // the previous iteration, so the loads issue without waiting on
  // arithmetic.
  int rk[TL::NI], rn[RAW], r0[RAW], r1[RAW];
  uint32_t ok[TL::NI], ov[TL::NI];
#pragma unroll
  for (int i = 0; i < TL::NI; ++i) {
    rk[i] = 0;
    ok[i] = ov[i] = 0;
  }
  auto offsets = [&](const int (&tok)[TL::NI], const uint32_t (&coff)[4], uint32_t (&off)[TL::NI]) {
#pragma unroll
    for (int i = 0; i < TL::NI; ++i) off[i] = __umul24(static_cast<uint32_t>(tok[i]), kv_row_bytes) + coff[i & 3];
  };
#pragma unroll
  for (int r = 0; r < RAW; ++r) rn[r] = r0[r] = r1[r] = 0;

  // Prologue: K(0) and K(1) in flight, S(0) once both landed. Gathered
  // K/V: at the start of iteration c, ok holds K(c+2)'s offsets and rk its
  // rows, rk1 the rows of K(c+1) (which V(c+1) reuses), ov V(c)'s offsets
  // and rn the raw entries of K(c+3) (in flight).
  f32x16 sA[MT][QT], sB[MT][QT];
  bf16x8 pX[QT][PK], pY[QT][PK];
  int rk1[TL::NI];
#pragma unroll
  for (int i = 0; i < TL::NI; ++i) rk1[i] = 0;
  if (nst > 0) {
    if constexpr (GKV) {
      stage_rows(0, r0);
      if (nst > 1) stage_rows(1, r1);
      wait_vmcnt<0>();
      int t0[TL::NI];
      expand_rows(r0, t0);
      expand_rows(r1, rk1);
      offsets(t0, koff, ok);
      issue_tile_offs<D, ST, NW>(kbase, ldsK, w, ok);
      offsets(rk1, koff, ok);
      if (nst > 1) issue_tile_offs<D, ST, NW>(kbase, ldsK + TILE * 2, w, ok);
      offsets(t0, voff, ov);  // V(0)
      if (nst > 2) stage_rows(2, rn);
    } else {
      if constexpr (kWalk) {
        wE0 = entry_packed(0);
        wX0 = true;
        wX1 = walk_next(wE0, 0, 0, wE1, wH1, wB1);
        issue_tile<D, ST, NW>(kbase + ofs_of(wE0, 0), ldsK, w, koff);
        if (wX1) issue_tile<D, ST, NW>(kbase + ofs_of(wE1, wH1), ldsK + TILE * 2, w, koff);
      } else {
        if constexpr (kPair) eb = entry_packed(0);  // the first even iteration shifts it to ea
        issue_tile<D, ST, NW>(kbase + stage_ofs(0), ldsK, w, koff);
        if (nst > 1) issue_tile<D, ST, NW>(kbase + stage_ofs(1), ldsK + TILE * 2, w, koff);
      }
    }
    wait_vmcnt<0>();
    if constexpr (GKV) {
      expand_rows(rn, rk);  // K(2)
      offsets(rk, koff, ok);
    }
    __syncthreads();
    compute_s(sA, 0);
    if constexpr (kWalk) mask_tail(sA, valid_of(wE0, 0));
    else mask_tail(sA, stage_valid(0));
    // the first stage's own row max as the reference (no recomputation);
    // a stage without a real key leaves noref set
    bool found = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float tm = rel_max(sA, qt);  // m_ref = 0 so far
      if (tm > -INFINITY) {
        m_ref[qt] = tm;
        found = true;
      }
    }
    if (__any(found)) noref = false;
  }
  // Iteration c: issue K(c+2) and V(c); S(c+1), the exponentials of stage c
  // and P.V of stage c-1 in one region; then settle stage c.
  int last = 0;  // (kWalk) the last stage run
  auto body2 = [&](auto with_pv, auto par, int c, f32x16 (&cur)[MT][QT], f32x16 (&nxt)[MT][QT],
                   bf16x8 (&pprev)[QT][PK], bf16x8 (&pcur)[QT][PK]) {
    constexpr int P = decltype(par)::value;  // c & 1
    bool has1 = c + 1 < nst, has2 = c + 2 < nst;
    __syncthreads();  // K(c) and V(c-2) buffers are free, K(c+1) and V(c-1) visible
    int wE2 = 0, wH2 = 0, wB2 = 0;  // (kWalk) stage c+2
    if constexpr (kWalk) {
      slide_to(wB1);
      has1 = wX1;
      has2 = wX1 && walk_next(wE1, wH1, wB1, wE2, wH2, wB2);
    } else {
      slide(c);
    }
    // (kPair) K(c+2) is half P of block c/2 + 1, V(c) half P of block c/2;
    // the length of stage c+1 is half 1 of block c/2 (P = 0) or half 0 of
    // block c/2 + 1 (P = 1)
    if constexpr (kPair && P == 0) {
      ea = eb;
      eb = entry_packed((c >> 1) + 1);
    }
    if constexpr (GKV) {
      if (c + 3 < nst) stage_rows(c + 3, rn);
      if (has2) issue_tile_offs<D, ST, NW>(kbase, ldsK + P * TILE * 2, w, ok);
      issue_tile_offs<D, ST, NW>(vbase, ldsV + P * TILE * 2, w, ov);
    } else if constexpr (kWalk) {
      if (has2) issue_tile<D, ST, NW>(kbase + ofs_of(wE2, wH2), ldsK + P * TILE * 2, w, koff);
      issue_tile<D, ST, NW>(vbase + ofs_of(wE0, wH0), ldsV + P * TILE * 2, w, voff);
    } else if constexpr (kPair) {
      if (has2) issue_tile<D, ST, NW>(kbase + ofs_of(eb, P), ldsK + P * TILE * 2, w, koff);
      issue_tile<D, ST, NW>(vbase + ofs_of(ea, P), ldsV + P * TILE * 2, w, voff);
    } else {
      if (has2) issue_tile<D, ST, NW>(kbase + stage_ofs(c + 2), ldsK + P * TILE * 2, w, koff);
      issue_tile<D, ST, NW>(vbase + stage_ofs(c), ldsV + P * TILE * 2, w, voff);
    }
    compute_s(nxt, P ^ 1);
    float rs[QT], es[QT];
    exps(cur, pcur, rs, es);
    if constexpr (decltype(with_pv)::value) pv_only(pprev, P ^ 1);
    // No interleave directive here: LLVM's default schedule reads the K and
    // V fragments ahead of their products and ran 0.5-3.9 % faster than
    // its strategies 0-3 on every workload's lists (identical bits). With
    // the log-sum-exp sums the register budget is tighter: without a
    // directive that variant spills 20-30 registers into the loop, with
    // strategy 3 seven, so it keeps strategy 3.
    if constexpr (LSE) __builtin_amdgcn_iglp_opt(3);
    settle(cur, pcur, rs, es);
    int v1 = 0;
    if constexpr (kWalk) v1 = valid_of(wE1, wH1);
    else if constexpr (kPair) v1 = valid_of(P == 0 ? ea : eb, P ^ 1);
    else if (has1) v1 = stage_valid(c + 1);
    mask_tail(nxt, has1 ? v1 : 0);
    wait_vmcnt<0>();
    if constexpr (kWalk) {
      wE0 = wE1;
      wH0 = wH1;
      wX0 = wX1;
      wE1 = wE2;
      wH1 = wH2;
      wB1 = wB2;
      wX1 = has2;
      last = c;
    }
    if constexpr (GKV) {
      offsets(rk1, voff, ov);  // V(c+1) reads K(c+1)'s rows
#pragma unroll
      for (int i = 0; i < TL::NI; ++i) rk1[i] = rk[i];
      expand_rows(rn, rk);     // K(c+3)
      offsets(rk, koff, ok);
    }
  };
  // stage c exists (at the top of iteration c): c < nst, or the walk's flag
  auto more = [&](int c) {
    if constexpr (kWalk) return wX0;
    else return c < nst;
  };
  if (nst > 0) body2(std::false_type{}, std::integral_constant<int, 0>{}, 0, sA, sB, pY, pX);
  for (int c = 1; more(c); c += 2) {
    body2(std::true_type{}, std::integral_constant<int, 1>{}, c, sB, sA, pX, pY);
    if (more(c + 1)) body2(std::true_type{}, std::integral_constant<int, 0>{}, c + 1, sA, sB, pY, pX);
  }
  if (nst > 0) {
    __syncthreads();  // V of the last stage visible
    if constexpr (kWalk) {
      if (last & 1) pv_only(pY, 1);
      else pv_only(pX, 0);
    } else {
      if ((nst - 1) & 1) pv_only(pY, (nst - 1) & 1);
      else pv_only(pX, (nst - 1) & 1);
    }
  }

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = qrow0 + qt * 32;
    const int qslot = I * BK + row;
    const float l_tot = l_run[qt] + __shfl_xor(l_run[qt], 32, 64);
    const bool real = row < blk_len[I];
    const float inv = (real && l_tot > 0.f) ? 1.f / l_tot : 0.f;
    uint16_t *orow = TOK ? op + static_cast<int64_t>(max(qtok[qt], 0)) * o_stride + h * D
                         : op + head_off + static_cast<int64_t>(qslot) * D;
    // the token layout has no pad rows: only real slots store
    if (!TOK || (real && qtok[qt] >= 0)) {
#pragma unroll
      for (int md = 0; md < DM; ++md)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = md * 32 + i4 * 8 + g * 4;
          const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(oacc[qt][md][i4 * 4 + 0] * inv)) |
                              (static_cast<uint32_t>(f32_to_bf16(oacc[qt][md][i4 * 4 + 1] * inv)) << 16);
          const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(oacc[qt][md][i4 * 4 + 2] * inv)) |
                              (static_cast<uint32_t>(f32_to_bf16(oacc[qt][md][i4 * 4 + 3] * inv)) << 16);
          *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(w0, w1);
        }
    }
    if constexpr (LSE) {
      const float e_tot = e_run[qt] + __shfl_xor(e_run[qt], 32, 64);
      if (g == 0) {
        const float ln2 = 0.6931471805599453f;
        lse[static_cast<int64_t>(h) * nb * BK + qslot] =
            (real && e_tot > 0.f) ? (m_ref[qt] + log2f(e_tot)) * ln2 : 0.f;
      }
    }
  }
}

// Float kernel on the float32 matrix cores (v_mfma_f32_16x16x4_f32). A wave
// owns 16 queries; K and V of each listed block pass through LDS in chunks of
// KC keys (K row-major with its 16-byte chunks XOR-swizzled by row, V stored
// transposed with padded rows, so both operand reads are conflict-free).
// Per 16-key tile: S^T = K Q^T (Q pre-scaled to log2 units and held in
// registers, lane group g owning dimensions 16m + 4g .. + 3), each lane then
// holds keys 4g .. 4g + 3 of its query; online softmax in the log2 domain
// with O rescaled only when a query's max grows by more than 2^8; O^T +=
// V^T P^T in four steps whose keys are 4g + r (r = the step), so every lane
// feeds its own weights. Chunks past a block's real keys are skipped.
template <int D, int BK>
__global__ void __launch_bounds__(BK * 4)
attn_f32_kernel(const float *__restrict__ qp, const float *__restrict__ kp,
                const float *__restrict__ vp, float *__restrict__ op, float *__restrict__ lse,
                const int32_t *__restrict__ blk_len, const int32_t *__restrict__ kv_idx,
                const int32_t *__restrict__ kv_cnt, const int32_t *__restrict__ order, int max_kv,
                int kv_shared, int nh, int nb, float scale_log2, const int32_t *__restrict__ perm,
                int64_t q_stride, int64_t kv_stride, int64_t o_stride) {
  constexpr int NT = BK * 4;    // BK / 16 waves
  constexpr int KC = 32;        // keys per LDS chunk
  constexpr int DQ = D / 4;     // MFMA k-steps of S
  constexpr int DT = D / 16;    // 16-wide d tiles of O
  constexpr int VS = KC + 4;    // V^T row stride (floats): rows 144 B apart hit distinct banks
  constexpr float kLazy = 8.f;
  static_assert(BK % KC == 0 && D % 16 == 0, "tile shapes");
  __shared__ __attribute__((aligned(16))) float sK[KC * D];
  __shared__ __attribute__((aligned(16))) float sVt[D * VS];
  int h, I;
  block_of(blockIdx.x, order, kv_shared, nh, nb, h, I);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ul = lane & 15, g = lane >> 4;
  const int64_t head_off = static_cast<int64_t>(h) * nb * BK * D;
  const int qrow = w * 16 + ul;
  const int qslot = I * BK + qrow;
  // token-layout I/O when perm is given (pad slots: zero query, no store)
  const int tok = perm ? perm[qslot] : 0;
  const int64_t qofs = perm ? static_cast<int64_t>(max(tok, 0)) * q_stride + h * D
                            : head_off + static_cast<int64_t>(qslot) * D;
  const int64_t oofs = perm ? static_cast<int64_t>(max(tok, 0)) * o_stride + h * D
                            : head_off + static_cast<int64_t>(qslot) * D;
  float qreg[DQ];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const float4 t = *reinterpret_cast<const float4 *>(qp + qofs + 16 * m + 4 * g);
    const float z = (perm && tok < 0) ? 0.f : scale_log2;
    qreg[4 * m] = t.x * z; qreg[4 * m + 1] = t.y * z; qreg[4 * m + 2] = t.z * z; qreg[4 * m + 3] = t.w * z;
  }
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // this lane's query; l over this lane's keys
  const int64_t lrow = kv_shared ? static_cast<int64_t>(I) : static_cast<int64_t>(h) * nb + I;
  const int cnt = min(max(kv_cnt[lrow], 0), max_kv);
  const int32_t *list = kv_idx + lrow * max_kv;
  for (int c = 0; c < cnt; ++c) {
    const int J = min(max(list[c], 0), nb - 1);
    const int kvalid = min(max(blk_len[J], 0), BK);
    for (int k0 = 0; k0 < kvalid; k0 += KC) {
      __syncthreads();  // the previous chunk's reads are done
      for (int i = tid; i < KC * D / 4; i += NT) {
        const int r = i / (D / 4), c4 = i - r * (D / 4);
        int64_t src;
        if (perm && kv_stride > 0)  // K/V rows gathered from the token-major tensors
          src = static_cast<int64_t>(max(perm[J * BK + k0 + r], 0)) * kv_stride + h * D + c4 * 4;
        else
          src = head_off + static_cast<int64_t>(J * BK + k0 + r) * D + c4 * 4;
        const float4 kv4 = *reinterpret_cast<const float4 *>(kp + src);
        const float4 vv4 = *reinterpret_cast<const float4 *>(vp + src);
        *reinterpret_cast<float4 *>(&sK[r * D + ((c4 ^ (r & 15)) * 4)]) = kv4;
        sVt[(4 * c4 + 0) * VS + r] = vv4.x;
        sVt[(4 * c4 + 1) * VS + r] = vv4.y;
        sVt[(4 * c4 + 2) * VS + r] = vv4.z;
        sVt[(4 * c4 + 3) * VS + r] = vv4.w;
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < KC / 16; ++t) {
        const int kt0 = k0 + 16 * t;
        if (kt0 >= kvalid) break;
        float kreg[DQ];
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
          const float4 k4 = *reinterpret_cast<const float4 *>(&sK[(16 * t + ul) * D + (((4 * m + g) ^ ul) * 4)]);
          kreg[4 * m] = k4.x; kreg[4 * m + 1] = k4.y; kreg[4 * m + 2] = k4.z; kreg[4 * m + 3] = k4.w;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < DQ; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kreg[j], qreg[j], acc, 0, 0, 0);
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = (kt0 + 4 * g + r < kvalid) ? acc[r] : -INFINITY;
        // the tile's max for this query (its keys sit in the four lane groups)
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (mx > m_run + kLazy) {  // (always on the first tile: m_run = -inf)
          const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
          m_run = mx;
        }
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(sv[r] - m_run);
          l_run += pv[r];
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const float4 vf = *reinterpret_cast<const float4 *>(&sVt[(16 * dt + ul) * VS + 16 * t + 4 * g]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.x, pv[0], oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.y, pv[1], oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.z, pv[2], oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf.w, pv[3], oacc[dt], 0, 0, 0);
        }
      }
    }
  }
  // the four lane groups' sums, added in the same order on every lane of a query
  const float l_pair = l_run + __shfl_xor(l_run, 16, 64);
  const float l_tot = l_pair + __shfl_xor(l_pair, 32, 64);
  const bool real = qrow < blk_len[I];
  const float inv = (real && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (!perm || (real && tok >= 0)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4 *>(op + oofs + 16 * dt + 4 * g) =
          make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
  }
  if (lse != nullptr && g == 0)
    lse[static_cast<int64_t>(h) * nb * BK + qslot] =
        (real && l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.6931471805599453f : 0.f;
}

// Counting sort of each head's list rows by length, longest first (one
// workgroup per head; heads stay in order so a head's key/value blocks are
// read by workgroups that run together): a histogram of lengths, a scan from
// the longest length down, then every row takes the next free position of
// its length.
constexpr int kOrderThreads = 1024;
constexpr int kOrderBins = 4096;

__global__ void __launch_bounds__(kOrderThreads)
attn_order_kernel(const int32_t *__restrict__ kv_cnt, int nb, int max_kv, int32_t *__restrict__ order) {
  __shared__ int next[kOrderBins];
  __shared__ int part[kOrderThreads];
  const int tid = threadIdx.x;
  const int base_row = blockIdx.x * nb;
  const int32_t *cnt = kv_cnt + base_row;
  for (int c = tid; c < kOrderBins; c += kOrderThreads) next[c] = 0;
  __syncthreads();
  for (int e = tid; e < nb; e += kOrderThreads) atomicAdd(&next[min(max(cnt[e], 0), max_kv)], 1);
  __syncthreads();
  // exclusive scan over lengths max, max-1, ..., 0: each thread owns a run
  // of bins, sums it, the run totals are scanned, then each run is expanded
  constexpr int kPer = kOrderBins / kOrderThreads;
  int run[kPer], tot = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    run[j] = next[kOrderBins - 1 - (tid * kPer + j)];
    tot += run[j];
  }
  part[tid] = tot;
  __syncthreads();
  for (int off = 1; off < kOrderThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int pos = part[tid] - tot;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    next[kOrderBins - 1 - (tid * kPer + j)] = pos;
    pos += run[j];
  }
  __syncthreads();
  for (int e = tid; e < nb; e += kOrderThreads) {
    const int p = atomicAdd(&next[min(max(cnt[e], 0), max_kv)], 1);
    order[base_row + p] = base_row + e;
  }
}

}  // namespace hsa

namespace hsa_host {

hsa_status_t launch_attn_order(const int32_t *kv_cnt, int G, int nb, int max_kv, int32_t *order,
                               hipStream_t stream) {
  hipLaunchKernelGGL(hsa::attn_order_kernel, dim3(G), dim3(hsa::kOrderThreads), 0, stream, kv_cnt, nb,
                     max_kv, order);
  return check_launch("hsa_attn_order");
}

template <typename K, typename... A>
static void launch_k(K kernel, dim3 grid, dim3 block, hipStream_t stream, A... args) {
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

hsa_status_t launch_attn(const void *qp, const void *kp, const void *vp, void *op, float *lse,
                         const int32_t *blk_len, const int32_t *kv_idx, const int32_t *kv_cnt,
                         const int32_t *order, int max_kv, int kv_shared, int nh, int nb, int B,
                         int D, int dtype, float scale, const int32_t *perm, int64_t q_stride,
                         int64_t kv_stride, int64_t o_stride, hipStream_t stream) {
  // list entries are packed as (block << 8) | length in the bf16 kernel
  if (nb > (1 << 24)) return fail(HSA_ERR_UNSUPPORTED, "hsa_attn: nb %d > 2^24 blocks", nb);
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(nh * nb);
  const int shared = kv_shared & 1;  // bit 1 only picks the stage walk
  if (dtype == HSA_BF16) {
    const uint16_t *q = static_cast<const uint16_t *>(qp), *k = static_cast<const uint16_t *>(kp),
                   *v = static_cast<const uint16_t *>(vp);
    uint16_t *o = static_cast<uint16_t *>(op);
    const dim3 block(B * 2);
#define HSA_ATTN_BF16(DD, BB, QQ, L, IO, WK)                                                    \
  launch_k(hsa::attn_bf16_pipe_kernel<DD, BB, (QQ == 2 ? 32 : 64), QQ, L, IO, WK>, grid, dim3(BB * 2 / QQ), stream, \
           q, k, v, o, lse, blk_len, kv_idx, kv_cnt, order, max_kv, shared, nh, nb, scale_log2, perm, q_stride, \
           kv_stride, o_stride)
#define HSA_ATTN_BF16_IO(DD, BB)                                      \
  do {                                                                \
    if (io == 2) { if (L) HSA_ATTN_BF16(DD, BB, 1, true, 2, false); else HSA_ATTN_BF16(DD, BB, 1, false, 2, false); } \
    else if (io == 1) {                                               \
      if (L) HSA_ATTN_BF16(DD, BB, 1, true, 1, false);                \
      else if (walk) HSA_ATTN_BF16(DD, BB, 1, false, 1, BB == 128);   \
      else HSA_ATTN_BF16(DD, BB, 1, false, 1, false);                 \
    } else {                                                          \
      if (L) HSA_ATTN_BF16(DD, BB, 1, true, 0, false);                \
      else if (walk) HSA_ATTN_BF16(DD, BB, 1, false, 0, BB == 128);   \
      else HSA_ATTN_BF16(DD, BB, 1, false, 0, false);                 \
    }                                                                 \
  } while (0)
    const int io = perm == nullptr ? 0 : (kv_stride > 0 ? 2 : 1);
    const bool L = lse != nullptr;
    // Lists shared by all heads come from the frame masks, whose frame
    // tiles end in short tiles: those launches, and those whose caller says
    // the blocks are often short (bit 1), walk the stages and leave out the
    // empty ones (same outputs).
    const bool walk = kv_shared != 0;
    if (D == 128 && B == 128) HSA_ATTN_BF16_IO(128, 128);
    else if (D == 64 && B == 128) HSA_ATTN_BF16_IO(64, 128);
    else if (D == 128 && B == 64) HSA_ATTN_BF16_IO(128, 64);
    else HSA_ATTN_BF16_IO(64, 64);
#undef HSA_ATTN_BF16_IO
#undef HSA_ATTN_BF16
  } else {
    const float *q = static_cast<const float *>(qp), *k = static_cast<const float *>(kp),
                *v = static_cast<const float *>(vp);
    float *o = static_cast<float *>(op);
    const dim3 block(B * 4);  // B / 16 waves of 16 queries
    if (D == 128 && B == 128) launch_k(hsa::attn_f32_kernel<128, 128>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, order, max_kv, shared, nh, nb, scale_log2, perm, q_stride, kv_stride, o_stride);
    else if (D == 64 && B == 128) launch_k(hsa::attn_f32_kernel<64, 128>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, order, max_kv, shared, nh, nb, scale_log2, perm, q_stride, kv_stride, o_stride);
    else if (D == 128 && B == 64) launch_k(hsa::attn_f32_kernel<128, 64>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, order, max_kv, shared, nh, nb, scale_log2, perm, q_stride, kv_stride, o_stride);
    else launch_k(hsa::attn_f32_kernel<64, 64>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, order, max_kv, shared, nh, nb, scale_log2, perm, q_stride, kv_stride, o_stride);
  }
  return check_launch("hsa_attn");
}

}  // namespace hsa_host

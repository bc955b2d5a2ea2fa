// Block-sparse attention backward: dQ, dK, dV over the forward's lists.
//
// VMoBA (abstract) trains video diffusion models natively with block-sparse
// attention; this is the gradient of hsa_attn for the same attended key set
// per query block (DFSAttn, Significance; DynamicRad, section 2 item 2: the
// shared candidate set consumed block-wise). With P = softmax(scale q K^T)
// over the real keys of the listed blocks and D_i = dO_i . O_i:
//   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . V_j - D_i),
//   dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i.
// P is rebuilt from the forward's log-sum-exp, so nothing quadratic is
// stored. Three kernels keep every sum in a fixed order (bit-reproducible):
//  - dQ: one workgroup per (head, query block), over its list (as the
//    forward), S^T = K Q^T and dP^T = V dO^T with one query per lane
//    column, dQ^T += K^T dS^T with K^T read by ds_read_b64_tr_b16;
//  - dV and dK: one workgroup per (head, key block), over the query blocks
//    whose list holds it (a transposed list built first), S = Q K^T (and
//    dP = dO V^T) with one key per lane column so P (dS) feeds
//    dV^T += dO^T P (dK^T += Q^T dS) straight from the accumulators.
// Each is software-pipelined and sized for two waves per SIMD; workgroups
// take their rows longest list first.
// bf16 runs on 32x32x16 matrix cores with float accumulation; P and dS are
// rounded to bf16 for the products, as the forward rounds P. Float inputs use
// plain one-thread-per-row loops. Pad query rows and pad keys get zero
// gradient.
#include "common.h"

namespace hsa {

constexpr float kLog2e = 1.4426950408889634f;

// D_i = dO_i . O_i in float, zero for pad slots; and the log-sum-exp in
// log2 units, +inf for pad slots (their weights then come out as 0 with no
// per-element select in the dK / dV kernels).
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_delta_kernel(const T *__restrict__ op, const T *__restrict__ dop, const int32_t *__restrict__ blk_len,
                 int n_pad, int B, int64_t total, const float *__restrict__ lse, float *__restrict__ delta,
                 float *__restrict__ lse2) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int slot = static_cast<int>(idx % n_pad);
  const bool real = (slot % B) < blk_len[slot / B];
  float s = 0.f;
  if (real) {
    const T *o = op + idx * D;
    const T *d = dop + idx * D;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < D; c += 8) {
        const uint4 a = *reinterpret_cast<const uint4 *>(o + c);
        const uint4 b = *reinterpret_cast<const uint4 *>(d + c);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s = fmaf(__uint_as_float(aw[j] << 16), __uint_as_float(bw[j] << 16), s);
          s = fmaf(__uint_as_float(aw[j] & 0xFFFF0000u), __uint_as_float(bw[j] & 0xFFFF0000u), s);
        }
      }
    } else {
#pragma unroll 8
      for (int c = 0; c < D; ++c) s = fmaf(o[c], d[c], s);
    }
  }
  delta[idx] = s;
  lse2[idx] = real ? lse[idx] * kLog2e : INFINITY;
}

// Transposed lists: for list set g and key block J, the query blocks I whose
// (ascending) list holds J, ascending. One wave per (g, J).
__global__ void __launch_bounds__(64)
bwd_transpose_kernel(const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt, int nb,
                     int max_kv, int32_t *__restrict__ t_idx, int32_t *__restrict__ t_cnt) {
  const int gJ = blockIdx.x;
  const int g = gJ / nb, J = gJ - g * nb;
  const int lane = lane_id();
  int32_t *out = t_idx + static_cast<int64_t>(gJ) * nb;
  int before = 0;
  for (int I0 = 0; I0 < nb; I0 += 64) {
    const int I = I0 + lane;
    bool found = false;
    if (I < nb) {
      const int32_t *list = kv_idx + (static_cast<int64_t>(g) * nb + I) * max_kv;
      int lo = 0, hi = min(max(kv_cnt[static_cast<int64_t>(g) * nb + I], 0), max_kv);
      const int cnt = hi;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (list[mid] < J) lo = mid + 1;
        else hi = mid;
      }
      found = lo < cnt && list[lo] == J;
    }
    const uint64_t b = __ballot(found);
    if (found) out[before + popc64(b & lanemask_lt())] = I;
    before += popc64(b);
  }
  if (lane == 0) t_cnt[gJ] = before;
}

// Per-lane fragment offsets, as in the forward kernel: b128 reads of a
// K-swizzled tile (row ln of a 32-row slice, 8-element chunk 2*ks + g) and
// ds_read_b64_tr_b16 reads of a V-swizzled tile.
template <int D>
struct FragOffsets {
  static constexpr int CPR = D / 8, DK = D / 16, DM = D / 32;
  int row[DK];  // element offset / 8 inside a 32-row slice
  int tr[DM];   // byte offset of the first transposed read
  __device__ __forceinline__ FragOffsets(int lane) {
    const int g = lane >> 5, ln = lane & 31;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) row[ks] = ln * CPR + ((2 * ks + g) ^ (ln & (CPR - 1)));
    const int q16 = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int md = 0; md < DM; ++md) {
      const int col = md * 32 + (q16 & 1) * 16 + 4 * (jj & 3);
      const int chunk = (col >> 3) ^ ((jj & 12) & (CPR - 1));
      tr[md] = ((g * 4 + (jj >> 2)) * CPR + chunk) * 16 + ((col >> 2) & 1) * 8;
    }
  }
};

// 8 bf16 of the transposed tile for k-step kk (16 rows) and d-slice md.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(lds_char_t *tile, int tr_ofs, int kk) {
  constexpr int CPR = D / 8;
  lds_i16x4_t *a0 = (lds_i16x4_t *)(tile + tr_ofs + kk * 16 * CPR * 16);
  lds_i16x4_t *a1 = (lds_i16x4_t *)(tile + tr_ofs + (kk * 16 + 8) * CPR * 16);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(a0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(a1);
  const i16x8_t both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}

template <int D>
__device__ __forceinline__ void load_row_frags(const uint16_t *row, int g, bf16x8 (&f)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) f[ks] = *reinterpret_cast<const bf16x8 *>(row + g * 8 + ks * 16);
}

// Write a d x 32 accumulator (one column per lane) as rows of the output.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t *row, const f32x16 (&acc)[D / 32], float mul, int g) {
#pragma unroll
  for (int md = 0; md < D / 32; ++md)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = md * 32 + i4 * 8 + g * 4;
      const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(acc[md][i4 * 4 + 0] * mul)) |
                          (static_cast<uint32_t>(f32_to_bf16(acc[md][i4 * 4 + 1] * mul)) << 16);
      const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(acc[md][i4 * 4 + 2] * mul)) |
                          (static_cast<uint32_t>(f32_to_bf16(acc[md][i4 * 4 + 3] * mul)) << 16);
      *reinterpret_cast<uint2 *>(row + d0) = make_uint2(w0, w1);
    }
}

// dQ, software-pipelined like the forward: stage c's dS and dQ products
// run in the same scheduling region as the next stage's S and dP products.
// K and V stages in row layout (b128 reads) are consumed an iteration
// before the transposed K copy, so iteration c issues K, V for stage c + 2
// and the transposed K for stage c + 1, each into the buffer freed by the
// barrier that opens the iteration.
constexpr int kDqStage = 32;

template <int D, int BK>
__global__ void __launch_bounds__(BK * 2, 2)
attn_bwd_dq_kernel(const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp,
                   const uint16_t *__restrict__ vp, const uint16_t *__restrict__ dop,
                   const float *__restrict__ lse, const float *__restrict__ delta,
                   const int32_t *__restrict__ blk_len, const int32_t *__restrict__ kv_idx,
                   const int32_t *__restrict__ kv_cnt, const int32_t *__restrict__ order, int max_kv,
                   int kv_shared, int nh, int nb, float scale_log2, float scale,
                   uint16_t *__restrict__ dqp) {
  // 32-key stages keep registers under 256 and LDS at 48 KB, so two
  // workgroups (two waves per SIMD) share a CU
  constexpr int ST = kDqStage, NS = BK / ST;
  constexpr int NW = BK / 32, CPR = D / 8, DK = D / 16, DM = D / 32, MT = ST / 32, TILE = ST * D;
  constexpr int NI = ST * CPR / (64 * NW);  // direct loads per wave per tile
  __shared__ __attribute__((aligned(1024))) uint16_t sK[2 * TILE];   // b128 rows (K swizzle)
  __shared__ __attribute__((aligned(1024))) uint16_t sKt[2 * TILE];  // transposed reads (V swizzle)
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2 * TILE];   // b128 rows (K swizzle)
  int h, I;  // longest lists first
  block_of(blockIdx.x, order, kv_shared, nh, nb, h, I);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ln = lane & 31;
  const int64_t n_pad = static_cast<int64_t>(nb) * BK;
  const int64_t head_off = static_cast<int64_t>(h) * n_pad * D;
  const int qslot = I * BK + w * 32 + ln;
  const FragOffsets<D> fo(lane);
  // lane offsets of this wave's NI direct loads (slice w*NI + i of the tile;
  // the swizzle key depends on the absolute slice)
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    koff[i] = tile_lane_offset<D, false>(w * NI + i, lane);
    voff[i] = tile_lane_offset<D, true>(w * NI + i, lane);
  }
  const uint32_t ldsK = lds_addr(sK), ldsKt = lds_addr(sKt), ldsV = lds_addr(sV);
  lds_char_t *const ktl = to_lds(sKt);

  bf16x8 qf[DK], dof[DK];
  load_row_frags<D>(qp + head_off + static_cast<int64_t>(qslot) * D, g, qf);
  load_row_frags<D>(dop + head_off + static_cast<int64_t>(qslot) * D, g, dof);
  const float lq2 = lse[static_cast<int64_t>(h) * n_pad + qslot] * kLog2e;
  const float dq_i = delta[static_cast<int64_t>(h) * n_pad + qslot];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(dof[ks]));
  asm volatile("" ::"v"(lq2), "v"(dq_i));

  f32x16 acc[DM];
#pragma unroll
  for (int md = 0; md < DM; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[md][i] = 0.f;

  const int64_t lrow = kv_shared ? static_cast<int64_t>(I) : static_cast<int64_t>(h) * nb + I;
  // caller lists: lengths clamped to [0, max_kv], entries to [0, nb)
  const int nst = min(max(kv_cnt[lrow], 0), max_kv) * NS;
  const int32_t *list = kv_idx + lrow * max_kv;
  auto entry = [&](int t) { return min(max(list[t / NS], 0), nb - 1); };
  auto stage_off = [&](int t) {
    return head_off + (static_cast<int64_t>(entry(t)) * BK + (t % NS) * ST) * D;
  };
  auto stage_valid = [&](int t) { return min(max(blk_len[entry(t)] - (t % NS) * ST, 0), ST); };
  auto issue = [&](const uint16_t *src, uint32_t lds_tile, const uint32_t (&off)[NI]) {
    issue_tile_slices<NI>(src, lds_tile, w, off);
  };
  auto issue_rows = [&](int t) {  // K and V in row layout, buffer t & 1
    const int64_t off = stage_off(t);
    const uint32_t b = static_cast<uint32_t>((t & 1) * TILE * 2);
    issue(kp + off, ldsK + b, koff);
    issue(vp + off, ldsV + b, koff);
  };
  auto issue_tr = [&](int t) {  // transposed K, buffer t & 1
    issue(kp + stage_off(t), ldsKt + static_cast<uint32_t>((t & 1) * TILE * 2), voff);
  };
  // S^T = K Q^T and dP^T = V dO^T of one stage (one query per lane column)
  auto compute_sdp = [&](f32x16 (&s)[MT], f32x16 (&dp)[MT], int buf) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[mt][i] = 0.f;
        dp[mt][i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&sK[buf * TILE + (mt * 32 * CPR + fo.row[ks]) * 8]);
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&sV[buf * TILE + (mt * 32 * CPR + fo.row[ks]) * 8]);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[mt], 0, 0, 0);
        dp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[ks], dp[mt], 0, 0, 0);
      }
    }
  };
  // dS = P (dP - D) from the stage's S, dP; dQ^T += K^T dS^T
  auto ds_dq = [&](const f32x16 (&s)[MT], const f32x16 (&dp)[MT], int buf, int kvalid) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // element i is key mt*32 + 8(i/4) + 4g + i%4 of the stage, query = lane column
      const int lim = kvalid - mt * 32 - g * 4;
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool real_key = (i >> 2) * 8 + (i & 3) < lim;
        // pad keys: exponent -inf, so p = 0 (computed, then selected)
        float arg = fmaf(s[mt][i], scale_log2, -lq2);
        arg = real_key ? arg : -INFINITY;
        const float p = __builtin_amdgcn_exp2f(arg);
        ds[i] = p * (dp[mt][i] - dq_i);
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8 dsf;
#pragma unroll
        for (int j = 0; j < 8; ++j) dsf[j] = static_cast<__bf16>(ds[ks2 * 8 + j]);
#pragma unroll
        for (int md = 0; md < DM; ++md)
          acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_frag<D>(ktl + buf * TILE * 2, fo.tr[md], mt * 2 + ks2), dsf, acc[md], 0, 0, 0);
      }
    }
  };

  f32x16 sA[MT], dA[MT], sB[MT], dB[MT];
  if (nst > 0) {
    issue_rows(0);
    issue_tr(0);
    if (nst > 1) issue_rows(1);
    wait_vmcnt<0>();
    __syncthreads();
    compute_sdp(sA, dA, 0);
  }
  // iteration c: issue K, V (c + 2) and K^T (c + 1); S, dP (c + 1) beside dS, dQ (c)
  auto body = [&](int c, f32x16 (&sc)[MT], f32x16 (&dc)[MT], f32x16 (&sn)[MT], f32x16 (&dn)[MT]) {
    __syncthreads();  // row buffer c & 1 and transposed buffer (c + 1) & 1 are free
    if (c + 2 < nst) issue_rows(c + 2);
    if (c + 1 < nst) issue_tr(c + 1);
    const int kvalid = stage_valid(c);
    // unconditional so it shares a scheduling region with ds_dq; on the last
    // stage it reads an idle buffer and the result is unused
    compute_sdp(sn, dn, (c + 1) & 1);
    ds_dq(sc, dc, c & 1, kvalid);
    __builtin_amdgcn_iglp_opt(3);
    wait_vmcnt<0>();
  };
  for (int c = 0; c < nst; c += 2) {
    body(c, sA, dA, sB, dB);
    if (c + 1 < nst) body(c + 1, sB, dB, sA, dA);
  }
  const bool real = (w * 32 + ln) < blk_len[I];
  store_rows<D>(dqp + head_off + static_cast<int64_t>(qslot) * D, acc, real ? scale : 0.f, g);
}

// dK and dV in two kernels over the transposed lists (one workgroup per
// (head, key block), one key per lane column): the dV kernel forms S and P
// and accumulates dV^T += dO^T P; the dK kernel forms S, dP and dS and
// accumulates dK^T += Q^T dS. Splitting recomputes S once more (5 products
// instead of 4) but halves the accumulators, so each kernel fits two waves
// per SIMD with 32-query stages and is software-pipelined like the forward:
// the next stage's S (and dP) products share a scheduling region with this
// stage's exponentials and accumulation. Tiles read in row layout (Q, dO)
// are consumed an iteration before the transposed ones (dO^T, Q^T) and the
// stage's lse / D rows.
// 64-query stages for dV (fewer barriers per product; registers allow it),
// 32 for dK (more live accumulators).
template <bool DK>
constexpr int dkv_stage() { return DK ? 32 : 64; }

template <int D, int BK, bool DK>
__global__ void __launch_bounds__(BK * 2, 2)
attn_bwd_dkv_kernel(const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp,
                    const uint16_t *__restrict__ vp, const uint16_t *__restrict__ dop,
                    const float *__restrict__ lse, const float *__restrict__ delta,
                    const int32_t *__restrict__ blk_len, const int32_t *__restrict__ t_idx,
                    const int32_t *__restrict__ t_cnt, const int32_t *__restrict__ order, int kv_shared,
                    int nh, int nb, float scale_log2, float scale, uint16_t *__restrict__ outp) {
  constexpr int ST = dkv_stage<DK>(), NS = BK / ST, QT = ST / 32;
  constexpr int NW = BK / 32, CPR = D / 8, DKS = D / 16, DM = D / 32, TILE = ST * D;
  constexpr int NI = ST * CPR / (64 * NW);  // direct loads per wave per tile
  // row-layout tiles: Q (and dO for dK); transposed: dO^T for dV, Q^T for dK
  __shared__ __attribute__((aligned(1024))) uint16_t sA[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sB[DK ? 2 * TILE : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sT[2 * TILE];
  // per wave and buffer: the stage's lse (and D) rows; each 1 KB load
  // fills ST * 4 bytes of data, the other lanes repeat it
  __shared__ __attribute__((aligned(1024))) float sLD[NW][2][2][256];
  // key blocks with the longest transposed lists first (uneven lists would
  // otherwise leave a tail of long workgroups)
  int h, J;
  block_of(blockIdx.x, order, kv_shared, nh, nb, h, J);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ln = lane & 31;
  const int64_t n_pad = static_cast<int64_t>(nb) * BK;
  const int64_t head_off = static_cast<int64_t>(h) * n_pad * D;
  const int kslot = J * BK + w * 32 + ln;
  const FragOffsets<D> fo(lane);
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    koff[i] = tile_lane_offset<D, false>(w * NI + i, lane);
    voff[i] = tile_lane_offset<D, true>(w * NI + i, lane);
  }
  const uint32_t ldsA = lds_addr(sA), ldsB = lds_addr(sB), ldsT = lds_addr(sT);
  const uint32_t ldsLD = __builtin_amdgcn_readfirstlane(lds_addr(&sLD[w][0][0][0]));
  lds_char_t *const ttl = to_lds(sT);

  bf16x8 kf[DKS], vf[DKS];
  load_row_frags<D>(kp + head_off + static_cast<int64_t>(kslot) * D, g, kf);
  if constexpr (DK) load_row_frags<D>(vp + head_off + static_cast<int64_t>(kslot) * D, g, vf);
#pragma unroll
  for (int ks = 0; ks < DKS; ++ks) {
    asm volatile("" ::"v"(kf[ks]));
    if constexpr (DK) asm volatile("" ::"v"(vf[ks]));
  }

  f32x16 acc[DM];
#pragma unroll
  for (int md = 0; md < DM; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[md][i] = 0.f;

  const int64_t lrow = kv_shared ? static_cast<int64_t>(J) : static_cast<int64_t>(h) * nb + J;
  const int nst = t_cnt[lrow] * NS;
  const int32_t *tl = t_idx + lrow * nb;
  const uint32_t ld_off = static_cast<uint32_t>((lane & (ST / 4 - 1)) * 16);  // ST floats
  auto stage_row0 = [&](int t) { return static_cast<int64_t>(tl[t / NS]) * BK + (t % NS) * ST; };
  auto issue = [&](const uint16_t *src, uint32_t lds_tile, const uint32_t (&off)[NI]) {
    issue_tile_slices<NI>(src, lds_tile, w, off);
  };
  auto issue_rows = [&](int t) {  // Q (and dO) in row layout, buffer t & 1
    const int64_t off = head_off + stage_row0(t) * D;
    const uint32_t b = static_cast<uint32_t>((t & 1) * TILE * 2);
    issue(qp + off, ldsA + b, koff);
    if constexpr (DK) issue(dop + off, ldsB + b, koff);
  };
  auto issue_tr = [&](int t) {  // dO^T (dV) or Q^T (dK), and the lse / D rows, buffer t & 1
    const int64_t row0 = stage_row0(t);
    issue((DK ? qp : dop) + head_off + row0 * D, ldsT + static_cast<uint32_t>((t & 1) * TILE * 2), voff);
    const int64_t r = static_cast<int64_t>(h) * n_pad + row0;
    const uint32_t lb = ldsLD + static_cast<uint32_t>((t & 1) * 2 * 256 * 4);
    load_lds16(lse + r, ld_off, lb);
    if constexpr (DK) load_lds16(delta + r, ld_off, lb + 256 * 4);
  };
  // S = Q K^T (and dP = dO V^T): element i of tile qt is query
  // qt*32 + 8(i/4) + 4g + i%4 of the stage, key = lane column
  auto compute_s = [&](f32x16 (&s)[QT], f32x16 (&dp)[QT], int buf) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[qt][i] = 0.f;
        dp[qt][i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(&sA[buf * TILE + (qt * 32 * CPR + fo.row[ks]) * 8]);
        s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s[qt], 0, 0, 0);
        if constexpr (DK) {
          const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(&sB[buf * TILE + (qt * 32 * CPR + fo.row[ks]) * 8]);
          dp[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[ks], dp[qt], 0, 0, 0);
        }
      }
    }
  };
  // P (and dS) of a stage, then dV^T += dO^T P or dK^T += Q^T dS
  auto accumulate = [&](const f32x16 (&s)[QT], const f32x16 (&dp)[QT], int buf) {
    const float *sL = &sLD[w][buf][0][0];
    const float *sD = &sLD[w][buf][1][0];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
    float x[16];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int q0 = qt * 32 + i4 * 8 + g * 4;
      const float4 l4 = *reinterpret_cast<const float4 *>(&sL[q0]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};  // log2 units, +inf on pad rows
      float dv4[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DK) {
        const float4 d4 = *reinterpret_cast<const float4 *>(&sD[q0]);
        dv4[0] = d4.x; dv4[1] = d4.y; dv4[2] = d4.z; dv4[3] = d4.w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i4 * 4 + r;
        // pad query rows: lse is +inf there, so the exponent is -inf and p = 0
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[qt][i], scale_log2, -lv[r]));
        x[i] = DK ? pv * (dp[qt][i] - dv4[r]) : pv;
      }
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      bf16x8 xf;
#pragma unroll
      for (int j = 0; j < 8; ++j) xf[j] = static_cast<__bf16>(x[ks2 * 8 + j]);
#pragma unroll
      for (int md = 0; md < DM; ++md)
        acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_frag<D>(ttl + buf * TILE * 2, fo.tr[md], qt * 2 + ks2), xf, acc[md], 0, 0, 0);
    }
    }
  };

  f32x16 s0[QT], d0[QT], s1[QT], d1[QT];
  if (nst > 0) {
    issue_rows(0);
    issue_tr(0);
    if (nst > 1) issue_rows(1);
    wait_vmcnt<0>();
    __syncthreads();
    compute_s(s0, d0, 0);
  }
  // iteration c: row tiles of stage c + 2, transposed tile and lse / D of
  // stage c + 1; S (dP) of stage c + 1 beside the accumulation of stage c
  auto body = [&](int c, f32x16 (&sc)[QT], f32x16 (&dc)[QT], f32x16 (&sn)[QT], f32x16 (&dn)[QT]) {
    __syncthreads();  // row buffer c & 1 and transposed buffer (c + 1) & 1 are free
    if (c + 2 < nst) issue_rows(c + 2);
    if (c + 1 < nst) issue_tr(c + 1);
    compute_s(sn, dn, (c + 1) & 1);  // on the last stage: an idle buffer, result unused
    accumulate(sc, dc, c & 1);
    __builtin_amdgcn_iglp_opt(3);
    wait_vmcnt<0>();
  };
  for (int c = 0; c < nst; c += 2) {
    body(c, s0, d0, s1, d1);
    if (c + 1 < nst) body(c + 1, s1, d1, s0, d0);
  }
  const bool real = (w * 32 + ln) < blk_len[J];
  store_rows<D>(outp + head_off + static_cast<int64_t>(kslot) * D, acc, real ? (DK ? scale : 1.f) : 0.f, g);
}

// Float inputs: one thread per query row (dQ) / per key row (dK, dV), tiles
// of the other side in LDS.
template <int D, int BK>
__global__ void __launch_bounds__(BK)
attn_bwd_dq_f32_kernel(const float *__restrict__ qp, const float *__restrict__ kp, const float *__restrict__ vp,
                       const float *__restrict__ dop, const float *__restrict__ lse,
                       const float *__restrict__ delta, const int32_t *__restrict__ blk_len,
                       const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt, int max_kv,
                       int kv_shared, int nh, int nb, float scale, float *__restrict__ dqp) {
  __shared__ __attribute__((aligned(16))) float sK[BK * D];
  __shared__ __attribute__((aligned(16))) float sV[BK * D];
  const int h = blockIdx.x / nb, I = blockIdx.x % nb;
  const int tid = threadIdx.x;
  const int64_t n_pad = static_cast<int64_t>(nb) * BK;
  const int64_t head_off = static_cast<int64_t>(h) * n_pad * D;
  const int qslot = I * BK + tid;
  float q[D], dq[D], dO[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qp[head_off + static_cast<int64_t>(qslot) * D + d];
    dO[d] = dop[head_off + static_cast<int64_t>(qslot) * D + d];
    dq[d] = 0.f;
  }
  const float L = lse[static_cast<int64_t>(h) * n_pad + qslot];
  const float Di = delta[static_cast<int64_t>(h) * n_pad + qslot];
  const int64_t lrow = kv_shared ? static_cast<int64_t>(I) : static_cast<int64_t>(h) * nb + I;
  const int cnt = min(max(kv_cnt[lrow], 0), max_kv);
  const int32_t *list = kv_idx + lrow * max_kv;
  for (int c = 0; c < cnt; ++c) {
    const int J = min(max(list[c], 0), nb - 1);
    const int kvalid = blk_len[J];
    const float4 *ks = reinterpret_cast<const float4 *>(kp + head_off + static_cast<int64_t>(J) * BK * D);
    const float4 *vs = reinterpret_cast<const float4 *>(vp + head_off + static_cast<int64_t>(J) * BK * D);
    __syncthreads();
    for (int e = tid; e < BK * D / 4; e += BK) {
      reinterpret_cast<float4 *>(sK)[e] = ks[e];
      reinterpret_cast<float4 *>(sV)[e] = vs[e];
    }
    __syncthreads();
    for (int key = 0; key < kvalid; ++key) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(q[d], sK[key * D + d], s);
        dp = fmaf(dO[d], sV[key * D + d], dp);
      }
      const float ds = expf(s * scale - L) * (dp - Di);
#pragma unroll
      for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, sK[key * D + d], dq[d]);
    }
  }
  const bool real = tid < blk_len[I];
#pragma unroll
  for (int d = 0; d < D; ++d) dqp[head_off + static_cast<int64_t>(qslot) * D + d] = real ? dq[d] * scale : 0.f;
}

template <int D, int BK>
__global__ void __launch_bounds__(BK)
attn_bwd_dkdv_f32_kernel(const float *__restrict__ qp, const float *__restrict__ kp, const float *__restrict__ vp,
                         const float *__restrict__ dop, const float *__restrict__ lse,
                         const float *__restrict__ delta, const int32_t *__restrict__ blk_len,
                         const int32_t *__restrict__ t_idx, const int32_t *__restrict__ t_cnt, int kv_shared,
                         int nh, int nb, float scale, float *__restrict__ dkp, float *__restrict__ dvp) {
  __shared__ __attribute__((aligned(16))) float sQ[BK * D];
  __shared__ __attribute__((aligned(16))) float sO[BK * D];
  __shared__ float sL[BK], sD[BK];
  const int h = blockIdx.x / nb, J = blockIdx.x % nb;
  const int tid = threadIdx.x;
  const int64_t n_pad = static_cast<int64_t>(nb) * BK;
  const int64_t head_off = static_cast<int64_t>(h) * n_pad * D;
  const int kslot = J * BK + tid;
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = kp[head_off + static_cast<int64_t>(kslot) * D + d];
    v[d] = vp[head_off + static_cast<int64_t>(kslot) * D + d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const int64_t lrow = kv_shared ? static_cast<int64_t>(J) : static_cast<int64_t>(h) * nb + J;
  const int cnt = t_cnt[lrow];
  const int32_t *tl = t_idx + lrow * nb;
  for (int c = 0; c < cnt; ++c) {
    const int I = tl[c];
    const int qvalid = blk_len[I];
    const float4 *qs = reinterpret_cast<const float4 *>(qp + head_off + static_cast<int64_t>(I) * BK * D);
    const float4 *os = reinterpret_cast<const float4 *>(dop + head_off + static_cast<int64_t>(I) * BK * D);
    __syncthreads();
    for (int e = tid; e < BK * D / 4; e += BK) {
      reinterpret_cast<float4 *>(sQ)[e] = qs[e];
      reinterpret_cast<float4 *>(sO)[e] = os[e];
    }
    sL[tid] = lse[static_cast<int64_t>(h) * n_pad + static_cast<int64_t>(I) * BK + tid];
    sD[tid] = delta[static_cast<int64_t>(h) * n_pad + static_cast<int64_t>(I) * BK + tid];
    __syncthreads();
    for (int qi = 0; qi < qvalid; ++qi) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(sQ[qi * D + d], k[d], s);
        dp = fmaf(sO[qi * D + d], v[d], dp);
      }
      const float p = expf(s * scale - sL[qi]);
      const float ds = p * (dp - sD[qi]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(p, sO[qi * D + d], dv[d]);
        dk[d] = fmaf(ds, sQ[qi * D + d], dk[d]);
      }
    }
  }
  const bool real = tid < blk_len[J];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    dkp[head_off + static_cast<int64_t>(kslot) * D + d] = real ? dk[d] * scale : 0.f;
    dvp[head_off + static_cast<int64_t>(kslot) * D + d] = real ? dv[d] : 0.f;
  }
}

}  // namespace hsa

namespace hsa_host {

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

hsa_status_t launch_attn_order(const int32_t *kv_cnt, int G, int nb, int max_kv, int32_t *order,
                               hipStream_t stream);

size_t attn_bwd_ws_bytes(int nh, int nb, int B, int G) {
  return 2 * align256(static_cast<size_t>(nh) * nb * B * sizeof(float)) +
         align256(static_cast<size_t>(G) * nb * nb * sizeof(int32_t)) +
         3 * align256(static_cast<size_t>(G) * nb * sizeof(int32_t));
}

hsa_status_t launch_attn_bwd(const void *qp, const void *kp, const void *vp, const void *op, const void *dop,
                             const float *lse, const int32_t *blk_len, const int32_t *kv_idx,
                             const int32_t *kv_cnt, int max_kv, int kv_shared, int nh, int nb, int B, int D,
                             int dtype, float scale, void *dqp, void *dkp, void *dvp, void *ws,
                             hipStream_t stream) {
  const int G = kv_shared ? 1 : nh;
  char *base = static_cast<char *>(ws);
  float *delta = reinterpret_cast<float *>(base);
  base += align256(static_cast<size_t>(nh) * nb * B * sizeof(float));
  float *lse2 = reinterpret_cast<float *>(base);  // log-sum-exp in log2 units, +inf on pads
  base += align256(static_cast<size_t>(nh) * nb * B * sizeof(float));
  int32_t *t_idx = reinterpret_cast<int32_t *>(base);
  base += align256(static_cast<size_t>(G) * nb * nb * sizeof(int32_t));
  int32_t *t_cnt = reinterpret_cast<int32_t *>(base);
  base += align256(static_cast<size_t>(G) * nb * sizeof(int32_t));
  int32_t *t_order = reinterpret_cast<int32_t *>(base);
  base += align256(static_cast<size_t>(G) * nb * sizeof(int32_t));
  int32_t *q_order = reinterpret_cast<int32_t *>(base);
  const int n_pad = nb * B;
  const int64_t total = static_cast<int64_t>(nh) * n_pad;
  const dim3 dgrid(static_cast<unsigned>((total + 255) / 256));
  const bool bf = dtype == HSA_BF16;
#define HSA_DELTA(TT, DD)                                                                          \
  hipLaunchKernelGGL((hsa::bwd_delta_kernel<TT, DD>), dgrid, dim3(256), 0, stream,                 \
                     static_cast<const TT *>(op), static_cast<const TT *>(dop), blk_len, n_pad, B, total, lse, \
                     delta, lse2)
  if (bf) { if (D == 128) HSA_DELTA(uint16_t, 128); else HSA_DELTA(uint16_t, 64); }
  else { if (D == 128) HSA_DELTA(float, 128); else HSA_DELTA(float, 64); }
#undef HSA_DELTA
  hipLaunchKernelGGL(hsa::bwd_transpose_kernel, dim3(G * nb), dim3(64), 0, stream, kv_idx, kv_cnt, nb,
                     max_kv, t_idx, t_cnt);
  // longest transposed lists first for the dK / dV kernels (the counting
  // sort takes lengths up to 4095; beyond that the natural order is kept)
  const int32_t *korder = nullptr, *qorder = nullptr;
  if (nb <= 4095) {
    launch_attn_order(t_cnt, G, nb, nb, t_order, stream);
    korder = t_order;
  }
  if (max_kv <= 4095) {  // and the query blocks' own lists for dQ
    launch_attn_order(kv_cnt, G, nb, max_kv, q_order, stream);
    qorder = q_order;
  }
  const dim3 grid(nh * nb);
  const float sl2 = scale * hsa::kLog2e;
  if (bf) {
    const uint16_t *q = static_cast<const uint16_t *>(qp), *k = static_cast<const uint16_t *>(kp),
                   *v = static_cast<const uint16_t *>(vp), *dO = static_cast<const uint16_t *>(dop);
    uint16_t *dq = static_cast<uint16_t *>(dqp), *dk = static_cast<uint16_t *>(dkp), *dv = static_cast<uint16_t *>(dvp);
#define HSA_BWD(DD, BB)                                                                                 \
  do {                                                                                                  \
    hipLaunchKernelGGL((hsa::attn_bwd_dq_kernel<DD, BB>), grid, dim3(BB * 2), 0, stream, q, k, v, dO, lse, \
                       delta, blk_len, kv_idx, kv_cnt, qorder, max_kv, kv_shared, nh, nb, sl2, scale, dq); \
    hipLaunchKernelGGL((hsa::attn_bwd_dkv_kernel<DD, BB, false>), grid, dim3(BB * 2), 0, stream, q, k, v, dO, \
                       lse2, delta, blk_len, t_idx, t_cnt, korder, kv_shared, nh, nb, sl2, scale, dv);    \
    hipLaunchKernelGGL((hsa::attn_bwd_dkv_kernel<DD, BB, true>), grid, dim3(BB * 2), 0, stream, q, k, v, dO, \
                       lse2, delta, blk_len, t_idx, t_cnt, korder, kv_shared, nh, nb, sl2, scale, dk);     \
  } while (0)
    if (D == 128 && B == 128) HSA_BWD(128, 128);
    else if (D == 64 && B == 128) HSA_BWD(64, 128);
    else if (D == 128 && B == 64) HSA_BWD(128, 64);
    else HSA_BWD(64, 64);
#undef HSA_BWD
  } else {
    const float *q = static_cast<const float *>(qp), *k = static_cast<const float *>(kp),
                *v = static_cast<const float *>(vp), *dO = static_cast<const float *>(dop);
    float *dq = static_cast<float *>(dqp), *dk = static_cast<float *>(dkp), *dv = static_cast<float *>(dvp);
#define HSA_BWD32(DD, BB)                                                                                  \
  do {                                                                                                     \
    hipLaunchKernelGGL((hsa::attn_bwd_dq_f32_kernel<DD, BB>), grid, dim3(BB), 0, stream, q, k, v, dO, lse,   \
                       delta, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale, dq);              \
    hipLaunchKernelGGL((hsa::attn_bwd_dkdv_f32_kernel<DD, BB>), grid, dim3(BB), 0, stream, q, k, v, dO, lse, \
                       delta, blk_len, t_idx, t_cnt, kv_shared, nh, nb, scale, dk, dv);                    \
  } while (0)
    if (D == 128 && B == 128) HSA_BWD32(128, 128);
    else if (D == 64 && B == 128) HSA_BWD32(64, 128);
    else if (D == 128 && B == 64) HSA_BWD32(128, 64);
    else HSA_BWD32(64, 64);
#undef HSA_BWD32
  }
  return check_launch("hsa_attn_bwd");
}

}  // namespace hsa_host

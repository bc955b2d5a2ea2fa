// Hierarchical block scoring.
//
// DFSAttn (Methodology, design 2): blocks are split into sub-blocks, scores
// are computed between sub-block summaries and aggregated into block
// importance. Two kernels:
//  1. pool: sub-block means of Qp and Kp over real tokens (float32). A pure
//     HBM stream: one wave per sub-block, 16-byte loads, a butterfly
//     reduction across the lanes that share a column group. Skipped when the
//     caller passes the means hsa_perm computed while reordering.
//  2. contract + aggregate: per head, a strip of 16 query sub-blocks against
//     all key sub-blocks on float32 matrix cores (v_mfma_f32_16x16x4_f32),
//     logits kept in registers; the MASS softmax (count-weighted: the log2
//     of each key sub-block's count is added to its logit, so a weight is
//     one exp2; max subtracted) and the per-block sums are reduced with lane
//     shuffles and a small LDS exchange between the waves; MAX takes maxima
//     instead. The block scores leave through each wave's idle key-tile
//     slot as runs of consecutive columns of a row.
//     Beyond 2048 sub-blocks per head the logits do not fit in registers and
//     a streaming variant passes over the key tiles twice (online maximum
//     and sum, then the normalised aggregation).
#include "common.h"

namespace hsa {

constexpr int kPoolWaves = 4;

template <typename T, int D>
__global__ void __launch_bounds__(kPoolWaves * 64)
pool_kernel(const T *__restrict__ qp, const T *__restrict__ kp, const int32_t *__restrict__ blk_len,
            int n_pad, int nsub, int s, int R, float *__restrict__ means /* [2][nh][nsub][D] */,
            int nh) {
  constexpr int kCols = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int kGroups = D / kCols;     // lanes per row
  constexpr int kRows = 64 / kGroups;    // rows per load instruction
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * kPoolWaves + (threadIdx.x >> 6);
  const int h = blockIdx.y;
  const int which = blockIdx.z;
  if (u >= nsub) return;
  const int I = u / R;
  const int c = min(max(blk_len[I] - (u - I * R) * s, 0), s);
  const T *__restrict__ src = (which ? kp : qp) + (static_cast<int64_t>(h) * n_pad + static_cast<int64_t>(u) * s) * D;
  const int cg = lane % kGroups;
  const int r0 = lane / kGroups;
  float acc[kCols];
#pragma unroll
  for (int j = 0; j < kCols; ++j) acc[j] = 0.f;
#pragma unroll 4
  for (int r = r0; r < c; r += kRows) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(r) * D + cg * kCols);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(w[j] << 16);
        acc[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
      }
    } else {
      acc[0] += __uint_as_float(v.x);
      acc[1] += __uint_as_float(v.y);
      acc[2] += __uint_as_float(v.z);
      acc[3] += __uint_as_float(v.w);
    }
  }
#pragma unroll
  for (int off = kGroups; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < kCols; ++j) acc[j] += __shfl_xor(acc[j], off, 64);
  }
  if (lane < kGroups) {
    const float inv = c > 0 ? 1.f / static_cast<float>(c) : 0.f;
    float *dst = means + ((static_cast<int64_t>(which) * nh + h) * nsub + u) * D + cg * kCols;
#pragma unroll
    for (int j = 0; j < kCols; j += 4) {
      *reinterpret_cast<float4 *>(dst + j) =
          make_float4(acc[j] * inv, acc[j + 1] * inv, acc[j + 2] * inv, acc[j + 3] * inv);
    }
  }
}

// Sum (or max) across the R lanes of a query block: lanes u0..u0+15 hold
// consecutive sub-blocks; R divides 16. The partners (lane ^ 1, 2, 4, 8) sit
// in the same 16-lane row, so DPP moves reach them: quad permutations for 1
// and 2, row rotations by 4 or 12 (chosen by bit 2) for 4, by 8 for 8.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float reduce_block_lanes(float v, int R, bool take_max) {
  const bool b2 = (lane_id() & 4) != 0;
  float o;
  if (R > 1) {
    o = dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]: lane ^ 1
    v = take_max ? fmaxf(v, o) : v + o;
  }
  if (R > 2) {
    o = dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]: lane ^ 2
    v = take_max ? fmaxf(v, o) : v + o;
  }
  if (R > 4) {
    const float a = dpp_f<0x124>(v), c = dpp_f<0x12C>(v);  // row rotations by 4 and 12: lane ^ 4
    o = b2 ? a : c;
    v = take_max ? fmaxf(v, o) : v + o;
  }
  if (R > 8) {
    o = dpp_f<0x128>(v);  // row rotation by 8: lane ^ 8
    v = take_max ? fmaxf(v, o) : v + o;
  }
  return v;
}

// Real tokens of sub-block v (real tokens are the first blk_len slots of a block).
__device__ __forceinline__ int sub_count(const int32_t *blk_len, int v, int R, int s) {
  const int I = v / R;
  return min(max(blk_len[I] - (v - I * R) * s, 0), s);
}

constexpr int kMaxSub = 2048;  // sub-blocks per head (validated at the boundary)

// Block scores of one strip from per-lane values z[t][r] (query sub-block
// u, key sub-block 16 (w VT + t) + 4g + r): MASS sums the R x R sub-block
// pairs of each block pair, each query sub-block's weights scaled by wu,
// the total by inv_c; MAX takes the largest. RR = R (sub-blocks per block,
// 2, 4 or 8), so block indices are shifts. A tile gives 16/RR rows x 16/RR
// columns of block scores; they are gathered in the wave's (now idle)
// key-tile slot and leave as runs of up to 64 consecutive columns of a row
// (stored tile by tile they would touch 16/RR rows per store).
template <int RR, int MAXT, bool MAXAGG>
__device__ __forceinline__ void store_block_scores(const float (&z)[MAXT][4], float wu, float inv_c, int w, int VT,
                                                   int U, int nb, int h, int u, int g, float *__restrict__ S,
                                                   float *slot) {
  static_assert(RR == 2 || RR == 4 || RR == 8, "sub-blocks per block");
  constexpr int BPT = 16 / RR;       // block rows (and columns) per tile
  constexpr int WC = MAXT * BPT;     // slot row length: the wave's block columns
  const int ul = u & 15, u0 = u - ul;
  const bool leader = (ul % RR) == 0 && u < U;
  const int ri = ul / RR;            // this lane's block row within the strip
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t < VT) {
      if constexpr (RR == 2) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float val = MAXAGG ? fmaxf(z[t][2 * p], z[t][2 * p + 1]) : (z[t][2 * p] + z[t][2 * p + 1]) * wu;
          val = reduce_block_lanes(val, RR, MAXAGG);
          if constexpr (!MAXAGG) val *= inv_c;
          if (leader) slot[ri * WC + t * BPT + 2 * g + p] = val;
        }
      } else {
        float val = MAXAGG ? fmaxf(fmaxf(z[t][0], z[t][1]), fmaxf(z[t][2], z[t][3]))
                           : ((z[t][0] + z[t][1]) + (z[t][2] + z[t][3])) * wu;
        if constexpr (RR == 8) {
          const float o = __shfl_xor(val, 16, 64);
          val = MAXAGG ? fmaxf(val, o) : val + o;
        }
        val = reduce_block_lanes(val, RR, MAXAGG);
        if constexpr (!MAXAGG) val *= inv_c;
        const bool writer = leader && (RR == 4 || (g & 1) == 0);
        if (writer) slot[ri * WC + t * BPT + (4 * g) / RR] = val;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int lane = lane_id();
  const int J0 = w * VT * BPT;                   // the wave's first block column
  const int ncol = min(VT * BPT, nb - J0);       // its block columns that exist
#pragma unroll
  for (int rho = 0; rho < BPT; ++rho) {
    if (u0 + rho * RR < U) {
      float *Srow = S + (static_cast<int64_t>(h) * nb + u0 / RR + rho) * nb + J0;
#pragma unroll
      for (int c = 0; c < WC; c += 64)
        if (c + lane < ncol) Srow[c + lane] = slot[rho * WC + c + lane];
    }
  }
}

// R = 1 (a sub-block per block): every score is a block score, 16 rows x
// 16 columns per tile, held one row per lane (columns 4g .. 4g + 3). Written
// as they are, each store would touch 16 rows; instead the wave's scores go
// through its (now idle) key-tile slot, TC tiles at a time, and leave as
// runs of 64 consecutive columns of one row.
template <int D, int MAXT, bool MAXAGG>
__device__ __forceinline__ void store_rows_r1(const float (&z)[MAXT][4], float wu, float inv_c, int w, int VT, int U,
                                              int nb, int h, int u, int g, float *__restrict__ S, float *slot) {
  constexpr int TC = D / 16;  // tiles per pass: 16 rows x 16 TC columns fill the 16 x D slot
  constexpr int W = TC * 16;  // columns per pass
  const int ul = u & 15, u0 = u - ul;
  const int lane = lane_id();
#pragma unroll
  for (int t0 = 0; t0 < MAXT; t0 += TC) {
    if (t0 >= VT) break;
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) {
      const int t = t0 + tt;
      if (t < MAXT && t < VT) {
        float4 o;
        o.x = MAXAGG ? z[t][0] : z[t][0] * wu * inv_c;
        o.y = MAXAGG ? z[t][1] : z[t][1] * wu * inv_c;
        o.z = MAXAGG ? z[t][2] : z[t][2] * wu * inv_c;
        o.w = MAXAGG ? z[t][3] : z[t][3] * wu * inv_c;
        *reinterpret_cast<float4 *>(slot + ul * W + tt * 16 + 4 * g) = o;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int c0 = (w * VT + t0) * 16;                 // first column of the pass
    const int cend = min(min((w * VT + VT) * 16, c0 + W), nb);  // this wave's columns end there
#pragma unroll
    for (int rho = 0; rho < 16; ++rho) {
      const int row = u0 + rho;
      if (row < U) {
        float *Srow = S + (static_cast<int64_t>(h) * nb + row) * nb;
#pragma unroll
        for (int c = 0; c < W; c += 64) {
          const int col = c0 + c + lane;
          if (col < cend) Srow[col] = slot[rho * W + c + lane];
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Each lane group g of an MFMA chain owns columns 16m + 4g .. +3 (m = 0 ..
// D/16 - 1) of its row, so a row's four lane groups read 64 contiguous bytes
// per load and the k-slots of Q and K line up.
template <int D, int NWV, int MAXT, bool MAXAGG>
__global__ void __launch_bounds__(NWV * 64, 3)
contract_kernel(const float *__restrict__ qbar, const float *__restrict__ kbar,
                const int32_t *__restrict__ blk_len, int s, int U, int R, int nb, float scale,
                float *__restrict__ S) {
  constexpr int DQ = D / 4;          // MFMA steps (k-slots per lane group)
  constexpr int CPR = D / 4;         // 16-byte chunks per fp32 row
  constexpr int NI = 16 * D * 4 / 1024;  // direct loads per 16-row tile
  __shared__ float red[NWV][16];
  // Per key sub-block: MASS the log2 of its real tokens (-inf when empty),
  // so a count-weighted exponential is one exp2 of logit + log2 count; MAX
  // the count itself. Past U: -inf (MASS) or 0, over every tile a wave may
  // index (NWV MAXT tiles).
  __shared__ float kv_s[kMaxSub + 16];
  __shared__ int cq[16];  // real tokens of the strip's query sub-blocks
  // One key tile per wave, chunk c of row r at slot c ^ (r mod 16): the 16
  // rows read by one MFMA operand load hit distinct banks.
  __shared__ __attribute__((aligned(1024))) float kt[NWV][16 * D];
  // MASS works in the log2 domain: logits carry scale * log2(e).
  const float zscale = MAXAGG ? scale : scale * 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ul = lane & 15;
  const int g = lane >> 4;
  const int h = blockIdx.y;
  const int u0 = blockIdx.x * 16;
  const int u = u0 + ul;
  const int tiles = (U + 15) / 16;
  const int VT = (tiles + NWV - 1) / NWV;  // tiles per wave (<= MAXT)
  const int nt = min(VT, max(tiles - w * VT, 0));  // tiles this wave owns
  const float *qb = qbar + static_cast<int64_t>(h) * U * D;
  const float *kb = kbar + static_cast<int64_t>(h) * U * D;
  const uint32_t slot = __builtin_amdgcn_readfirstlane(lds_addr(&kt[w][0]));
  const float *kslot = &kt[w][0];

  // Direct loads of tile t into this wave's slot; rows past U repeat row
  // U - 1 (their logits are discarded). (A lane's offsets are formed per
  // tile: kept across tiles they would cost the registers of a third
  // resident wave.)
  auto issue = [&](int t) {
    const int v0 = (w * VT + t) * 16;
    const float *base = kb + static_cast<int64_t>(v0) * D;
    if (v0 + 16 <= U) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int P = i * 64 + lane;
        const int row = P / CPR, c = (P % CPR) ^ (row & 15);
        load_lds16(base, static_cast<uint32_t>(row * D * 4 + c * 16), slot + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int P = i * 64 + lane;
        const int row = P / CPR, c = (P % CPR) ^ (row & 15);
        const int rowc = min(v0 + row, U - 1) - v0;
        load_lds16(base, static_cast<uint32_t>(rowc * D * 4 + c * 16), slot + i * 1024);
      }
    }
  };
  if (nt > 0) issue(0);

  float qreg[DQ];
  if (u < U) {
#pragma unroll
    for (int m = 0; m < DQ / 4; ++m) {
      const float4 t = *reinterpret_cast<const float4 *>(qb + static_cast<int64_t>(u) * D + 16 * m + 4 * g);
      qreg[4 * m] = t.x; qreg[4 * m + 1] = t.y; qreg[4 * m + 2] = t.z; qreg[4 * m + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < DQ; ++j) qreg[j] = 0.f;
  }
  // Key sub-block entries: one length load per block (U = nb R), a
  // thread's loads issued after the first key tile's and the Q rows', so
  // that one round trip covers them all; then the R sub-block entries of
  // each block, and the counts of the strip's own query sub-blocks.
  {
    constexpr int kPer = kMaxSub / (NWV * 64);
    int len[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int I = threadIdx.x + k * NWV * 64;
      len[k] = I < nb ? blk_len[I] : 0;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int I = threadIdx.x + k * NWV * 64;
      if (I < nb)
        for (int r = 0; r < R; ++r) {
          const int c = min(max(len[k] - r * s, 0), s);
          kv_s[I * R + r] = MAXAGG ? static_cast<float>(c) : (c > 0 ? __builtin_amdgcn_logf(static_cast<float>(c)) : -INFINITY);
          const int q = I * R + r - u0;
          if (q >= 0 && q < 16) cq[q] = c;
        }
    }
    for (int v = U + static_cast<int>(threadIdx.x); v < NWV * MAXT * 16; v += NWV * 64) kv_s[v] = MAXAGG ? 0.f : -INFINITY;
  }
  __syncthreads();  // kv_s, cq
  const int cu = (u < U) ? cq[ul] : 0;  // real tokens of query sub-block u

  // Logits z[t][r]: query sub-block u, key sub-block v = v0 + 4g + r.
  float z[MAXT][4];  // -inf marks an empty key sub-block
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) z[t][r] = -INFINITY;
    if (t < nt) {
      wait_vmcnt<0>();  // tile t is in the slot (and the Q loads are in)
      if (!MAXAGG && t == 0 && cu == 0) {
        // an empty query sub-block gets weight wu = 0; zero means keep its logits finite
#pragma unroll
        for (int j = 0; j < DQ; ++j) qreg[j] = 0.f;
      }
      float kreg[DQ];
      {
        // this lane's fragment addresses, formed per tile (kept across the
        // loop they would cost the registers of a third resident wave)
        int lt = lane;
        asm volatile("" : "+v"(lt));
        const int ult = lt & 15, gt = lt >> 4;
#pragma unroll
        for (int m = 0; m < DQ / 4; ++m) {
          const float4 k4 = *reinterpret_cast<const float4 *>(kslot + ult * D + (((gt + 4 * m) ^ ult) * 4));
          kreg[4 * m] = k4.x; kreg[4 * m + 1] = k4.y; kreg[4 * m + 2] = k4.z; kreg[4 * m + 3] = k4.w;
        }
      }
      // the slot is reused by the next tile's loads: its reads must be done
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      if (t + 1 < nt) issue(t + 1);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < DQ; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kreg[j], qreg[j], acc, 0, 0, 0);
      const int v0 = (w * VT + t) * 16;
      const float4 c4 = *reinterpret_cast<const float4 *>(&kv_s[v0 + 4 * g]);
      const float kv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (MAXAGG) {
          if (kv[r] > 0.f && cu > 0) z[t][r] = acc[r] * zscale;
        } else {
          z[t][r] = fmaf(acc[r], zscale, kv[r]);  // log2(count) + logit, -inf for an empty key sub-block
        }
      }
    }
  }

  if constexpr (!MAXAGG) {
    // Row maximum over every key sub-block of query sub-block u (the last
    // tiles first: a value held through the loop in scratch is then read
    // last).
    float m = -INFINITY;
#pragma unroll
    for (int t = MAXT - 1; t >= 0; --t)
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, z[t][r]);
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (g == 0) red[w][ul] = m;
    __syncthreads();
    m = red[0][ul];
#pragma unroll
    for (int i = 1; i < NWV; ++i) m = fmaxf(m, red[i][ul]);
    __syncthreads();
    // Count-weighted exponentials c_v 2^(z - m) = 2^(z + log2 c_v - m) and
    // their row sum; m is the largest count-weighted term's exponent (the
    // shift cancels in the normalisation). A row without real keys (m =
    // -inf) takes m = 0, so every weight is exactly zero.
    m = (m == -INFINITY) ? 0.f : m;
    float den = 0.f;
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(z[t][r] - m);
        z[t][r] = e;
        den += e;
      }
    den += __shfl_xor(den, 16, 64);
    den += __shfl_xor(den, 32, 64);
    if (g == 0) red[w][ul] = den;
    __syncthreads();
    den = 0.f;
#pragma unroll
    for (int i = 0; i < NWV; ++i) den += red[i][ul];
    // The query count and index are taken again here rather than kept across
    // the tile loop (where holding them spills at three waves per SIMD).
    int ue = u;
    asm volatile("" : "+v"(ue));
    const int cue = (ue < U) ? *static_cast<volatile int *>(&cq[ue & 15]) : 0;
    const float wu = (den > 0.f) ? static_cast<float>(cue) / den : 0.f;
    const float cblk = reduce_block_lanes(static_cast<float>(cue), R, false);
    const float inv_c = cblk > 0.f ? 1.f / cblk : 0.f;
    switch (R) {
      case 1: store_rows_r1<D, MAXT, false>(z, wu, inv_c, w, VT, U, nb, h, ue, g, S, &kt[w][0]); break;
      case 2: store_block_scores<2, MAXT, false>(z, wu, inv_c, w, VT, U, nb, h, ue, g, S, &kt[w][0]); break;
      case 4: store_block_scores<4, MAXT, false>(z, wu, inv_c, w, VT, U, nb, h, ue, g, S, &kt[w][0]); break;
      default: store_block_scores<8, MAXT, false>(z, wu, inv_c, w, VT, U, nb, h, ue, g, S, &kt[w][0]); break;
    }
  } else {
    // MAX: largest sub-block logit between the two blocks.
    switch (R) {
      case 1: store_rows_r1<D, MAXT, true>(z, 1.f, 1.f, w, VT, U, nb, h, u, g, S, &kt[w][0]); break;
      case 2: store_block_scores<2, MAXT, true>(z, 1.f, 1.f, w, VT, U, nb, h, u, g, S, &kt[w][0]); break;
      case 4: store_block_scores<4, MAXT, true>(z, 1.f, 1.f, w, VT, U, nb, h, u, g, S, &kt[w][0]); break;
      default: store_block_scores<8, MAXT, true>(z, 1.f, 1.f, w, VT, U, nb, h, u, g, S, &kt[w][0]); break;
    }
  }
}


// Any number of sub-blocks: the key tiles are streamed twice instead of
// being held in registers. Pass 1 keeps, per query sub-block, an online
// maximum and count-weighted exponential sum (combined across the lane
// groups and the waves at the end); pass 2 recomputes each tile's logits
// and aggregates the normalised mass (or, for MAX, the largest logit) per
// key block. Each wave streams its own contiguous range of key tiles.
template <int D, int NWV, bool MAXAGG>
__global__ void __launch_bounds__(NWV * 64)
contract_stream_kernel(const float *__restrict__ qbar, const float *__restrict__ kbar,
                       const int32_t *__restrict__ blk_len, int s, int U, int R, int nb, float scale,
                       float *__restrict__ S) {
  constexpr int DQ = D / 4;
  constexpr int CPR = D / 4;
  constexpr int NI = 16 * D * 4 / 1024;
  __shared__ float redm[NWV][16], redd[NWV][16];
  __shared__ __attribute__((aligned(1024))) float kt[NWV][16 * D];
  const float zscale = MAXAGG ? scale : scale * 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ul = lane & 15;
  const int g = lane >> 4;
  const int h = blockIdx.y;
  const int u0 = blockIdx.x * 16;
  const int u = u0 + ul;
  const int tiles = (U + 15) / 16;
  const int VT = (tiles + NWV - 1) / NWV;
  const int t0 = w * VT, t1 = min(tiles, t0 + VT);  // this wave's tiles
  const float *qb = qbar + static_cast<int64_t>(h) * U * D;
  const float *kb = kbar + static_cast<int64_t>(h) * U * D;
  const uint32_t slot = __builtin_amdgcn_readfirstlane(lds_addr(&kt[w][0]));
  const float *kslot = &kt[w][0];
  auto issue = [&](int t) {
    const int v0 = t * 16;
    const float *base = kb + static_cast<int64_t>(v0) * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int P = i * 64 + lane;
      const int row = P / CPR, c = (P % CPR) ^ (row & 15);
      const int rowc = min(v0 + row, U - 1) - v0;
      load_lds16(base, static_cast<uint32_t>(rowc * D * 4 + c * 16), slot + i * 1024);
    }
  };
  float qreg[DQ];
  if (u < U) {
#pragma unroll
    for (int m = 0; m < DQ / 4; ++m) {
      const float4 t = *reinterpret_cast<const float4 *>(qb + static_cast<int64_t>(u) * D + 16 * m + 4 * g);
      qreg[4 * m] = t.x; qreg[4 * m + 1] = t.y; qreg[4 * m + 2] = t.z; qreg[4 * m + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < DQ; ++j) qreg[j] = 0.f;
  }
  const int cu = (u < U) ? sub_count(blk_len, u, R, s) : 0;
  // logits of tile t (already in the slot): z[r] for key sub-block
  // 16t + 4g + r, -inf for an empty one; the next tile's loads are issued
  // once this one's operands are read
  auto tile_logits = [&](int t, int tnext, float (&z)[4], float (&cv)[4]) {
    wait_vmcnt<0>();
    float kreg[DQ];
#pragma unroll
    for (int m = 0; m < DQ / 4; ++m) {
      const float4 k4 = *reinterpret_cast<const float4 *>(kslot + ul * D + (((g + 4 * m) ^ ul) * 4));
      kreg[4 * m] = k4.x; kreg[4 * m + 1] = k4.y; kreg[4 * m + 2] = k4.z; kreg[4 * m + 3] = k4.w;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the slot may be refilled
    if (tnext >= 0) issue(tnext);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < DQ; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kreg[j], qreg[j], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int v = t * 16 + 4 * g + r;
      cv[r] = (v < U) ? static_cast<float>(sub_count(blk_len, v, R, s)) : 0.f;
      z[r] = (cv[r] > 0.f && cu > 0) ? acc[r] * zscale : -INFINITY;
    }
  };
  const int I = u / R;
  const bool leader = (ul % R) == 0 && u < U;
  float M = -INFINITY, wu = 0.f, inv_c = 0.f;
  if constexpr (!MAXAGG) {
    // pass 1: online max and count-weighted exponential sum
    float m = -INFINITY, den = 0.f;
    if (t0 < t1) issue(t0);
    for (int t = t0; t < t1; ++t) {
      float z[4], cv[4];
      tile_logits(t, t + 1 < t1 ? t + 1 : -1, z, cv);
      const float tm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      if (tm > m) {
        den *= __builtin_amdgcn_exp2f(m - tm);
        m = tm;
      }
      if (m > -INFINITY) {
#pragma unroll
        for (int r = 0; r < 4; ++r) den += cv[r] * __builtin_amdgcn_exp2f(z[r] - m);
      }
    }
    // combine the four lane groups of the query, then the waves
    auto combine = [](float &ma, float &da, float mb, float db) {
      const float mm = fmaxf(ma, mb);
      da = (mm > -INFINITY) ? da * __builtin_amdgcn_exp2f(ma - mm) + db * __builtin_amdgcn_exp2f(mb - mm) : 0.f;
      ma = mm;
    };
    combine(m, den, __shfl_xor(m, 16, 64), __shfl_xor(den, 16, 64));
    combine(m, den, __shfl_xor(m, 32, 64), __shfl_xor(den, 32, 64));
    if (g == 0) {
      redm[w][ul] = m;
      redd[w][ul] = den;
    }
    __syncthreads();
    M = redm[0][ul];
    float DEN = redd[0][ul];
#pragma unroll
    for (int i = 1; i < NWV; ++i) combine(M, DEN, redm[i][ul], redd[i][ul]);
    wu = (DEN > 0.f) ? static_cast<float>(cu) / DEN : 0.f;
    const float cblk = reduce_block_lanes(static_cast<float>(cu), R, false);
    inv_c = cblk > 0.f ? 1.f / cblk : 0.f;
  }
  // pass 2 (the only pass for MAX): per key block of each tile
  if (t0 < t1) issue(t0);
  for (int t = t0; t < t1; ++t) {
    float z[4], cv[4];
    tile_logits(t, t + 1 < t1 ? t + 1 : -1, z, cv);
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (MAXAGG) o[r] = z[r];
      else o[r] = (z[r] > -INFINITY) ? cv[r] * __builtin_amdgcn_exp2f(z[r] - M) * wu : 0.f;
    }
    const int v0 = t * 16;
    if (R == 1) {
      const int J0 = v0 + 4 * g;
      if (leader) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (J0 + r < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J0 + r] = MAXAGG ? o[r] : o[r] * inv_c;
      }
    } else if (R == 2) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float val = MAXAGG ? fmaxf(o[2 * p], o[2 * p + 1]) : o[2 * p] + o[2 * p + 1];
        val = reduce_block_lanes(val, R, MAXAGG);
        const int J = (v0 + 4 * g + 2 * p) / 2;
        if (leader && J < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J] = MAXAGG ? val : val * inv_c;
      }
    } else {
      // R = 4 or 8 (s >= 16 and B <= 128): a block's key sub-blocks are one
      // lane group (R = 4) or two neighbouring ones (R = 8)
      float val = MAXAGG ? fmaxf(fmaxf(o[0], o[1]), fmaxf(o[2], o[3])) : (o[0] + o[1]) + (o[2] + o[3]);
      if (R == 8) val = MAXAGG ? fmaxf(val, __shfl_xor(val, 16, 64)) : val + __shfl_xor(val, 16, 64);
      val = reduce_block_lanes(val, R, MAXAGG);
      const int J = (v0 + 4 * g) / R;
      const bool writer = leader && (R == 4 || (g & 1) == 0);
      if (writer && J < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J] = MAXAGG ? val : val * inv_c;
    }
  }
}

}  // namespace hsa

namespace hsa_host {

size_t score_ws_bytes(int nh, int n_pad, int s, int D) {
  const size_t U = static_cast<size_t>(n_pad / s);
  return 2ull * nh * U * D * sizeof(float);
}

template <int D, bool MAXAGG>
static void launch_contract(int U, dim3 grid, const float *qb, const float *kb,
                            const int32_t *blk_len, int s, int R, int nb, float scale, float *S,
                            hipStream_t stream) {
  // Each wave owns up to MAXT 16-wide key tiles of the strip. Sixteen tiles
  // per wave keep a wave's logits in registers within the 168 that let three
  // waves share a SIMD (the kernel's launch bounds ask for three): three
  // workgroups per CU, so a 1024-sub-block head's 64 strips x 12 heads run
  // in one round on 256 CUs (at two per CU the last third ran as a second,
  // half-empty round: 52 -> 39 us).
  const int tiles = (U + 15) / 16;
  if (tiles <= 16)
    hipLaunchKernelGGL((hsa::contract_kernel<D, 4, 4, MAXAGG>), grid, dim3(256), 0, stream, qb, kb, blk_len, s, U, R, nb, scale, S);
  else if (tiles <= 64)
    hipLaunchKernelGGL((hsa::contract_kernel<D, 4, 16, MAXAGG>), grid, dim3(256), 0, stream, qb, kb, blk_len, s, U, R, nb, scale, S);
  else
    hipLaunchKernelGGL((hsa::contract_kernel<D, 8, 16, MAXAGG>), grid, dim3(512), 0, stream, qb, kb, blk_len, s, U, R, nb, scale, S);
}

hsa_status_t launch_score(const void *qp, const void *kp, const float *pooled,
                          const int32_t *blk_len, int nh, int nb, int B, int s, int D, int dtype,
                          int agg, float scale, float *S, void *ws, hipStream_t stream) {
  const int n_pad = nb * B;
  const int U = n_pad / s;
  const int R = B / s;
  const float *means = pooled;
  if (means == nullptr) {
    float *m = static_cast<float *>(ws);
    const dim3 pgrid((U + hsa::kPoolWaves - 1) / hsa::kPoolWaves, nh, 2);
    const dim3 pblock(hsa::kPoolWaves * 64);
    if (dtype == HSA_BF16) {
      const uint16_t *q = static_cast<const uint16_t *>(qp), *k = static_cast<const uint16_t *>(kp);
      if (D == 128)
        hipLaunchKernelGGL((hsa::pool_kernel<uint16_t, 128>), pgrid, pblock, 0, stream, q, k, blk_len, n_pad, U, s, R, m, nh);
      else
        hipLaunchKernelGGL((hsa::pool_kernel<uint16_t, 64>), pgrid, pblock, 0, stream, q, k, blk_len, n_pad, U, s, R, m, nh);
    } else {
      const float *q = static_cast<const float *>(qp), *k = static_cast<const float *>(kp);
      if (D == 128)
        hipLaunchKernelGGL((hsa::pool_kernel<float, 128>), pgrid, pblock, 0, stream, q, k, blk_len, n_pad, U, s, R, m, nh);
      else
        hipLaunchKernelGGL((hsa::pool_kernel<float, 64>), pgrid, pblock, 0, stream, q, k, blk_len, n_pad, U, s, R, m, nh);
    }
    means = m;
  }
  const float *qb = means;
  const float *kb = means + static_cast<size_t>(nh) * U * D;
  const dim3 cgrid((U + 15) / 16, nh);
  if (U > hsa::kMaxSub) {  // logits do not fit in registers: stream the key tiles twice
    if (D == 128) {
      if (agg == HSA_AGG_MAX) hipLaunchKernelGGL((hsa::contract_stream_kernel<128, 4, true>), cgrid, dim3(256), 0, stream, qb, kb, blk_len, s, U, R, nb, scale, S);
      else hipLaunchKernelGGL((hsa::contract_stream_kernel<128, 4, false>), cgrid, dim3(256), 0, stream, qb, kb, blk_len, s, U, R, nb, scale, S);
    } else {
      if (agg == HSA_AGG_MAX) hipLaunchKernelGGL((hsa::contract_stream_kernel<64, 4, true>), cgrid, dim3(256), 0, stream, qb, kb, blk_len, s, U, R, nb, scale, S);
      else hipLaunchKernelGGL((hsa::contract_stream_kernel<64, 4, false>), cgrid, dim3(256), 0, stream, qb, kb, blk_len, s, U, R, nb, scale, S);
    }
    return check_launch("hsa_score");
  }
  if (D == 128) {
    if (agg == HSA_AGG_MAX) launch_contract<128, true>(U, cgrid, qb, kb, blk_len, s, R, nb, scale, S, stream);
    else launch_contract<128, false>(U, cgrid, qb, kb, blk_len, s, R, nb, scale, S, stream);
  } else {
    if (agg == HSA_AGG_MAX) launch_contract<64, true>(U, cgrid, qb, kb, blk_len, s, R, nb, scale, S, stream);
    else launch_contract<64, false>(U, cgrid, qb, kb, blk_len, s, R, nb, scale, S, stream);
  }
  return check_launch("hsa_score");
}

}  // namespace hsa_host

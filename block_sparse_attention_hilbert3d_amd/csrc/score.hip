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
//     logits kept in registers; the MASS softmax (count-weighted, max
//     subtracted) and the per-block sums are reduced with lane shuffles and
//     a small LDS exchange between the four waves; MAX takes maxima instead.
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
// consecutive sub-blocks; R divides 16.
__device__ __forceinline__ float reduce_block_lanes(float v, int R, bool take_max) {
  for (int off = 1; off < R; off <<= 1) {
    const float o = __shfl_xor(v, off, 64);
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

// Each lane group g of an MFMA chain owns columns 16m + 4g .. +3 (m = 0 ..
// D/16 - 1) of its row, so a row's four lane groups read 64 contiguous bytes
// per load and the k-slots of Q and K line up.
template <int D, int NWV, int MAXT, bool MAXAGG>
__global__ void __launch_bounds__(NWV * 64)
contract_kernel(const float *__restrict__ qbar, const float *__restrict__ kbar,
                const int32_t *__restrict__ blk_len, int s, int U, int R, int nb, float scale,
                float *__restrict__ S) {
  constexpr int DQ = D / 4;          // MFMA steps (k-slots per lane group)
  constexpr int CPR = D / 4;         // 16-byte chunks per fp32 row
  constexpr int NI = 16 * D * 4 / 1024;  // direct loads per 16-row tile
  __shared__ float red[NWV][16];
  __shared__ float cnt_s[kMaxSub];   // real tokens of every key sub-block
  // One key tile per wave, chunk c of row r at slot c ^ (r mod 16): the 16
  // rows read by one MFMA operand load hit distinct banks.
  __shared__ __attribute__((aligned(1024))) float kt[NWV][16 * D];
  for (int v = threadIdx.x; v < U; v += NWV * 64) cnt_s[v] = static_cast<float>(sub_count(blk_len, v, R, s));
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
  // U - 1 (their logits are discarded).
  auto issue = [&](int t) {
    const int v0 = (w * VT + t) * 16;
    const float *base = kb + static_cast<int64_t>(v0) * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int P = i * 64 + lane;
      const int row = P / CPR, c = (P % CPR) ^ (row & 15);
      const int rowc = min(v0 + row, U - 1) - v0;
      load_lds16(base, static_cast<uint32_t>(rowc * D * 4 + c * 16), slot + i * 1024);
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
  __syncthreads();  // cnt_s
  const int cu = (u < U) ? static_cast<int>(cnt_s[u]) : 0;

  // Logits z[t][r]: query sub-block u, key sub-block v = v0 + 4g + r.
  float z[MAXT][4];  // -inf marks an empty key sub-block
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) z[t][r] = -INFINITY;
    if (t < nt) {
      wait_vmcnt<0>();  // tile t is in the slot (and the Q loads are in)
      float kreg[DQ];
#pragma unroll
      for (int m = 0; m < DQ / 4; ++m) {
        const float4 k4 = *reinterpret_cast<const float4 *>(kslot + ul * D + (((g + 4 * m) ^ ul) * 4));
        kreg[4 * m] = k4.x; kreg[4 * m + 1] = k4.y; kreg[4 * m + 2] = k4.z; kreg[4 * m + 3] = k4.w;
      }
      // the slot is reused by the next tile's loads: its reads must be done
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      if (t + 1 < nt) issue(t + 1);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < DQ; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kreg[j], qreg[j], acc, 0, 0, 0);
      const int v0 = (w * VT + t) * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = v0 + 4 * g + r;
        const float c = (v < U) ? cnt_s[v] : 0.f;
        if (c > 0.f && cu > 0) z[t][r] = acc[r] * zscale;
      }
    }
  }

  if constexpr (!MAXAGG) {
    // Row maximum over every key sub-block of query sub-block u.
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
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
    // Count-weighted exponentials and their row sum.
    float den = 0.f;
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      const int v0 = (w * VT + t) * 16 + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float e = 0.f;
        if (t < VT && z[t][r] != -INFINITY) e = cnt_s[v0 + r] * __builtin_amdgcn_exp2f(z[t][r] - m);
        z[t][r] = e;
        den += e;
      }
    }
    den += __shfl_xor(den, 16, 64);
    den += __shfl_xor(den, 32, 64);
    if (g == 0) red[w][ul] = den;
    __syncthreads();
    den = 0.f;
#pragma unroll
    for (int i = 0; i < NWV; ++i) den += red[i][ul];
    const float wu = (den > 0.f) ? static_cast<float>(cu) / den : 0.f;
    const float cblk = reduce_block_lanes(static_cast<float>(cu), R, false);
    const float inv_c = cblk > 0.f ? 1.f / cblk : 0.f;
    const int I = u / R;
    const bool leader = (ul % R) == 0 && u < U;
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < VT) {
        const int v0 = (w * VT + t) * 16;
        if (v0 < U) {
          if (R == 1) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = z[t][r] * wu * inv_c;
            const int J0 = v0 + 4 * g;
            if (leader) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (J0 + r < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J0 + r] = o[r];
            }
          } else if (R == 2) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              float val = (z[t][2 * p] + z[t][2 * p + 1]) * wu;
              val = reduce_block_lanes(val, R, false) * inv_c;
              const int J = (v0 + 4 * g + 2 * p) / 2;
              if (leader && J < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J] = val;
            }
          } else {
            float val = ((z[t][0] + z[t][1]) + (z[t][2] + z[t][3])) * wu;
            if (R == 8) val += __shfl_xor(val, 16, 64);
            val = reduce_block_lanes(val, R < 16 ? R : 16, false) * inv_c;
            const int J = (v0 + 4 * g) / R;
            const bool writer = leader && (R == 4 || (g & 1) == 0);
            if (writer && J < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J] = val;
          }
        }
      }
    }
  } else {
    // MAX: largest sub-block logit between the two blocks.
    const int I = u / R;
    const bool leader = (ul % R) == 0 && u < U;
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < VT) {
        const int v0 = (w * VT + t) * 16;
        if (v0 < U) {
          if (R == 1) {
            const int J0 = v0 + 4 * g;
            if (leader) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (J0 + r < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J0 + r] = z[t][r];
            }
          } else if (R == 2) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              float val = fmaxf(z[t][2 * p], z[t][2 * p + 1]);
              val = reduce_block_lanes(val, R, true);
              const int J = (v0 + 4 * g + 2 * p) / 2;
              if (leader && J < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J] = val;
            }
          } else {
            float val = fmaxf(fmaxf(z[t][0], z[t][1]), fmaxf(z[t][2], z[t][3]));
            if (R == 8) val = fmaxf(val, __shfl_xor(val, 16, 64));
            val = reduce_block_lanes(val, R, true);
            const int J = (v0 + 4 * g) / R;
            const bool writer = leader && (R == 4 || (g & 1) == 0);
            if (writer && J < nb) S[(static_cast<int64_t>(h) * nb + I) * nb + J] = val;
          }
        }
      }
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
  // per wave keep a wave's logits in ~160 registers, so three waves share a
  // SIMD and several workgroups a CU: one's softmax phase overlaps another's
  // matrix work (measured 5-6 % faster than eight tiles per wave).
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

// Block-sparse flash attention over per-query-block key-block lists.
//
// DFSAttn (Significance): block-wise execution over reordered tokens;
// DynamicRad (section 2.2): a shared candidate set aggregated block-wise for a
// FlashAttention-style kernel. Each workgroup owns one (head, query block);
// key blocks not in its list are never loaded.
//
// bf16 kernel (gfx950 matrix cores, wave64):
//  - one wave per 32 query rows; Q stays in registers as the B operand;
//  - per listed key block: K tile staged row-major and V tile staged
//    transposed in LDS (padded strides), then S^T = K Q^T on
//    v_mfma_f32_32x32x16_bf16 so each lane holds 32-key runs of ONE query:
//    the row max / row sum are in-lane plus one cross-half exchange;
//  - online softmax in the log2 domain (scale folded with log2 e), keys
//    beyond the block's real length masked to -inf;
//  - P is rounded to bf16 straight from the accumulator layout and used as
//    the B operand of O^T += V^T P^T; the key order inside each 16-key slice
//    follows the accumulator layout and the V^T reads use the same order;
//  - epilogue divides by the row sum, rounds to bf16, zeroes pad rows and
//    writes the natural-log log-sum-exp.
// f32 kernel: a plain one-thread-per-query online-softmax loop with K/V tiles
// in LDS, for float inputs (small shapes).
#include "common.h"

namespace hsa {

template <int D, int BK>
__global__ void __launch_bounds__(BK * 2, 2)
attn_bf16_kernel(const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp,
                 const uint16_t *__restrict__ vp, uint16_t *__restrict__ op,
                 float *__restrict__ lse, const int32_t *__restrict__ blk_len,
                 const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt,
                 int max_kv, int kv_shared, int nh, int nb, float scale_log2) {
  constexpr int NW = BK / 32;  // waves per workgroup, 32 query rows each
  constexpr int NT = NW * 64;
  constexpr int KS = D + 8;    // LDS stride of a K row (elements)
  constexpr int VS = BK + 4;   // LDS stride of a V^T row (elements)
  constexpr int MT = BK / 32;  // 32-key slices of a tile
  constexpr int DK = D / 16;   // 16-wide k-steps over the head dim
  constexpr int DM = D / 32;   // 32-row slices of the head dim
  constexpr int PK = BK / 16;  // 16-key k-steps of the value product
  __shared__ __attribute__((aligned(16))) uint16_t sK[BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VS];

  const int total = nh * nb;
  const int bid = xcd_remap(blockIdx.x, total);
  const int h = bid / nb, I = bid - (bid / nb) * nb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;
  const int64_t head_off = static_cast<int64_t>(h) * nb * BK * D;
  const int qslot = I * BK + w * 32 + ln;

  bf16x8 qf[DK];
  {
    const uint16_t *qrow = qp + head_off + static_cast<int64_t>(qslot) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) qf[ks] = *reinterpret_cast<const bf16x8 *>(qrow + ks * 16);
  }

  f32x16 oacc[DM];
#pragma unroll
  for (int md = 0; md < DM; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[md][i] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  const int64_t lrow = kv_shared ? static_cast<int64_t>(I) : static_cast<int64_t>(h) * nb + I;
  const int cnt = kv_cnt[lrow];
  const int32_t *list = kv_idx + lrow * max_kv;

  for (int c = 0; c < cnt; ++c) {
    const int J = list[c];
    const int kvalid = blk_len[J];
    const uint16_t *kt = kp + head_off + static_cast<int64_t>(J) * BK * D;
    const uint16_t *vt = vp + head_off + static_cast<int64_t>(J) * BK * D;
    // K tile, row-major: 16-byte chunks, consecutive lanes along a row.
#pragma unroll
    for (int ch = tid; ch < BK * D / 8; ch += NT) {
      const int row = ch / (D / 8), col = (ch - row * (D / 8)) * 8;
      *reinterpret_cast<uint4 *>(&sK[row * KS + col]) =
          *reinterpret_cast<const uint4 *>(kt + row * D + col);
    }
    // V tile, transposed: each lane takes two consecutive keys of one
    // 8-wide column chunk and writes 8 key-pair words.
#pragma unroll
    for (int ch = tid; ch < (BK / 2) * (D / 8); ch += NT) {
      const int kpair = ch % (BK / 2), dc = ch / (BK / 2);
      const uint4 a = *reinterpret_cast<const uint4 *>(vt + (2 * kpair) * D + dc * 8);
      const uint4 b = *reinterpret_cast<const uint4 *>(vt + (2 * kpair + 1) * D + dc * 8);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
      const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (j & 1) ? (aw[j >> 1] >> 16) : (aw[j >> 1] & 0xFFFFu);
        const uint32_t hi = (j & 1) ? (bw[j >> 1] & 0xFFFF0000u) : (bw[j >> 1] << 16);
        *reinterpret_cast<uint32_t *>(&sV[(dc * 8 + j) * VS + 2 * kpair]) = lo | hi;
      }
    }
    __syncthreads();

    // S^T: rows = keys, columns = this wave's 32 queries.
    f32x16 sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[mt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sK[(mt * 32 + ln) * KS + ks * 16 + g * 8]);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[mt], 0, 0, 0);
      }
    }
    // Accumulator element i of slice mt is key mt*32 + (i/4)*8 + g*4 + i%4.
    float mx = -1e30f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = mt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        const float s = (key < kvalid) ? sacc[mt][i] * scale_log2 : -INFINITY;
        sacc[mt][i] = s;
        mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(sacc[mt][i] - m_new);
        sacc[mt][i] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int md = 0; md < DM; ++md)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[md][i] *= alpha;

    // O^T += V^T P^T over 16-key steps. Step ks2 takes accumulator elements
    // (ks2%2)*8 + j of slice ks2/2: keys ks2*16 + g*4 + {0..3} and
    // ks2*16 + 8 + g*4 + {0..3}; the V^T operand reads the same keys.
#pragma unroll
    for (int ks2 = 0; ks2 < PK; ++ks2) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = static_cast<__bf16>(sacc[ks2 >> 1][(ks2 & 1) * 8 + j]);
#pragma unroll
      for (int md = 0; md < DM; ++md) {
        const uint16_t *vr = &sV[(md * 32 + ln) * VS + ks2 * 16 + g * 4];
        const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 8);
        const uint4 packed = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8 a = __builtin_bit_cast(bf16x8, packed);
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, oacc[md], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Epilogue: lane holds query ln, head-dim rows md*32 + (i/4)*8 + g*4 + i%4.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool real = (w * 32 + ln) < blk_len[I];
  const float inv = (real && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  uint16_t *orow = op + head_off + static_cast<int64_t>(qslot) * D;
#pragma unroll
  for (int md = 0; md < DM; ++md)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = md * 32 + i4 * 8 + g * 4;
      const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(oacc[md][i4 * 4 + 0] * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16(oacc[md][i4 * 4 + 1] * inv)) << 16);
      const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(oacc[md][i4 * 4 + 2] * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16(oacc[md][i4 * 4 + 3] * inv)) << 16);
      *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(w0, w1);
    }
  if (lse != nullptr && g == 0) {
    const float ln2 = 0.6931471805599453f;
    lse[static_cast<int64_t>(h) * nb * BK + qslot] = real ? (m_run + log2f(l_tot)) * ln2 : 0.f;
  }
}

template <int D, int BK>
__global__ void __launch_bounds__(BK)
attn_f32_kernel(const float *__restrict__ qp, const float *__restrict__ kp,
                const float *__restrict__ vp, float *__restrict__ op, float *__restrict__ lse,
                const int32_t *__restrict__ blk_len, const int32_t *__restrict__ kv_idx,
                const int32_t *__restrict__ kv_cnt, int max_kv, int kv_shared, int nh, int nb,
                float scale_log2) {
  __shared__ __attribute__((aligned(16))) float sK[BK * D];
  __shared__ __attribute__((aligned(16))) float sV[BK * D];
  const int h = blockIdx.x / nb, I = blockIdx.x % nb;
  const int tid = threadIdx.x;
  const int64_t head_off = static_cast<int64_t>(h) * nb * BK * D;
  const int qslot = I * BK + tid;
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qp[head_off + static_cast<int64_t>(qslot) * D + d] * scale_log2;
    o[d] = 0.f;
  }
  float m = -1e30f, l = 0.f;
  const int64_t lrow = kv_shared ? static_cast<int64_t>(I) : static_cast<int64_t>(h) * nb + I;
  const int cnt = kv_cnt[lrow];
  const int32_t *list = kv_idx + lrow * max_kv;
  for (int c = 0; c < cnt; ++c) {
    const int J = list[c];
    const int kvalid = blk_len[J];
    const float4 *ks = reinterpret_cast<const float4 *>(kp + head_off + static_cast<int64_t>(J) * BK * D);
    const float4 *vs = reinterpret_cast<const float4 *>(vp + head_off + static_cast<int64_t>(J) * BK * D);
    for (int i = tid; i < BK * D / 4; i += BK) {
      reinterpret_cast<float4 *>(sK)[i] = ks[i];
      reinterpret_cast<float4 *>(sV)[i] = vs[i];
    }
    __syncthreads();
    for (int key = 0; key < kvalid; ++key) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], sK[key * D + d], s);
      if (s > m) {
        const float a = exp2f(m - s);
        l *= a;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= a;
        m = s;
      }
      const float p = exp2f(s - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, sV[key * D + d], o[d]);
    }
    __syncthreads();
  }
  const bool real = tid < blk_len[I];
  const float inv = (real && l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) op[head_off + static_cast<int64_t>(qslot) * D + d] = o[d] * inv;
  if (lse != nullptr) lse[static_cast<int64_t>(h) * nb * BK + qslot] = real ? (m + log2f(l)) * 0.6931471805599453f : 0.f;
}

}  // namespace hsa

namespace hsa_host {

template <typename K, typename... A>
static void launch_k(K kernel, dim3 grid, dim3 block, hipStream_t stream, A... args) {
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

hsa_status_t launch_attn(const void *qp, const void *kp, const void *vp, void *op, float *lse,
                         const int32_t *blk_len, const int32_t *kv_idx, const int32_t *kv_cnt,
                         int max_kv, int kv_shared, int nh, int nb, int B, int D, int dtype,
                         float scale, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(nh * nb);
  if (dtype == HSA_BF16) {
    const uint16_t *q = static_cast<const uint16_t *>(qp), *k = static_cast<const uint16_t *>(kp),
                   *v = static_cast<const uint16_t *>(vp);
    uint16_t *o = static_cast<uint16_t *>(op);
    const dim3 block(B * 2);
    if (D == 128 && B == 128) launch_k(hsa::attn_bf16_kernel<128, 128>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
    else if (D == 64 && B == 128) launch_k(hsa::attn_bf16_kernel<64, 128>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
    else if (D == 128 && B == 64) launch_k(hsa::attn_bf16_kernel<128, 64>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
    else launch_k(hsa::attn_bf16_kernel<64, 64>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
  } else {
    const float *q = static_cast<const float *>(qp), *k = static_cast<const float *>(kp),
                *v = static_cast<const float *>(vp);
    float *o = static_cast<float *>(op);
    const dim3 block(B);
    if (D == 128 && B == 128) launch_k(hsa::attn_f32_kernel<128, 128>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
    else if (D == 64 && B == 128) launch_k(hsa::attn_f32_kernel<64, 128>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
    else if (D == 128 && B == 64) launch_k(hsa::attn_f32_kernel<128, 64>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
    else launch_k(hsa::attn_f32_kernel<64, 64>, grid, block, stream, q, k, v, o, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, scale_log2);
  }
  return check_launch("hsa_attn");
}

}  // namespace hsa_host

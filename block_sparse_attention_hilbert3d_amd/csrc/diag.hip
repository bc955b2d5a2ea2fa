// Selection diagnostic: exact attention mass per key block, and recall.
//
// Block selection (DFSAttn, Methodology, designs 2-3; VMoBA abstract;
// DynamicRad section 2) estimates which key blocks carry a query block's
// attention. This kernel measures the truth for sampled query rows: the
// dense softmax over every real key, summed per key block, and the share of
// it that the selected list keeps (recall). It is off the hot path and
// favours plainness: fp32 vector arithmetic, one thread per query row, key
// blocks streamed through LDS and read by broadcast.
#include "common.h"

namespace hsa {

constexpr int kMassThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

// Two passes over all key blocks: (1) the row's exact maximum and sum in the
// log2 domain, (2) each block's share. rows[h][i] is a slot of head h.
template <typename T, int D>
__global__ void __launch_bounds__(kMassThreads)
block_mass_kernel(const T *__restrict__ qp, const T *__restrict__ kp, const int32_t *__restrict__ blk_len,
                  const int32_t *__restrict__ rows, int n_rows, int nb, int B, float scale_log2,
                  const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt, int max_kv,
                  int kv_shared, float *__restrict__ mass, float *__restrict__ recall) {
  extern __shared__ float ktile[];  // B x D
  const int h = blockIdx.y;
  const int i = blockIdx.x * kMassThreads + threadIdx.x;
  const bool live = i < n_rows;
  const int64_t n_pad = static_cast<int64_t>(nb) * B;
  const int r = live ? min(max(rows[static_cast<int64_t>(h) * n_rows + i], 0), static_cast<int>(n_pad - 1)) : 0;
  const T *kh = kp + static_cast<int64_t>(h) * n_pad * D;
  float q[D];
  {
    const T *qr = qp + (static_cast<int64_t>(h) * n_pad + r) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) q[d] = to_f32(qr[d]) * scale_log2;
  }
  auto load_tile = [&](int J, int len) {
    __syncthreads();
    const T *src = kh + static_cast<int64_t>(J) * B * D;
    for (int e = threadIdx.x; e < len * D; e += kMassThreads) ktile[e] = to_f32(src[e]);
    __syncthreads();
  };
  auto logit = [&](int k) {
    const float4 *kr = reinterpret_cast<const float4 *>(ktile + k * D);
    float s = 0.f;
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 kv = kr[d4];
      s = fmaf(q[4 * d4], kv.x, s);
      s = fmaf(q[4 * d4 + 1], kv.y, s);
      s = fmaf(q[4 * d4 + 2], kv.z, s);
      s = fmaf(q[4 * d4 + 3], kv.w, s);
    }
    return s;
  };
  float m = -INFINITY, l = 0.f;
  for (int J = 0; J < nb; ++J) {
    const int len = blk_len[J];
    if (len <= 0) continue;
    load_tile(J, len);
    for (int k = 0; k < len; ++k) {
      const float s = logit(k);
      if (s > m) {
        l = l * exp2f(m - s) + 1.f;
        m = s;
      } else {
        l += exp2f(s - m);
      }
    }
  }
  const int I = r / B;
  const int64_t lrow = kv_shared ? static_cast<int64_t>(I) : static_cast<int64_t>(h) * nb + I;
  const int cnt = (recall != nullptr) ? min(max(kv_cnt[lrow], 0), max_kv) : 0;
  const int32_t *list = (recall != nullptr) ? kv_idx + lrow * max_kv : nullptr;
  int p = 0;
  float rec = 0.f;
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  for (int J = 0; J < nb; ++J) {
    const int len = blk_len[J];
    float share = 0.f;
    if (len > 0) {
      load_tile(J, len);
      for (int k = 0; k < len; ++k) share += exp2f(logit(k) - m);
      share *= inv_l;
    }
    if (live && mass != nullptr) mass[(static_cast<int64_t>(h) * n_rows + i) * nb + J] = share;
    if (list != nullptr) {
      while (p < cnt && list[p] < J) ++p;
      if (p < cnt && list[p] == J) rec += share;
    }
  }
  if (live && recall != nullptr) recall[static_cast<int64_t>(h) * n_rows + i] = rec;
}

}  // namespace hsa

namespace hsa_host {

hsa_status_t launch_block_mass(const void *qp, const void *kp, const int32_t *blk_len, const int32_t *rows,
                               int n_rows, int nh, int nb, int B, int D, int dtype, float scale,
                               const int32_t *kv_idx, const int32_t *kv_cnt, int max_kv, int kv_shared,
                               float *mass, float *recall, hipStream_t stream) {
  const dim3 grid((n_rows + hsa::kMassThreads - 1) / hsa::kMassThreads, nh);
  const float sl2 = scale * 1.4426950408889634f;
  const size_t lds = static_cast<size_t>(B) * D * sizeof(float);
#define HSA_MASS(TT, DD)                                                                              \
  hipLaunchKernelGGL((hsa::block_mass_kernel<TT, DD>), grid, dim3(hsa::kMassThreads), lds, stream,      \
                     static_cast<const TT *>(qp), static_cast<const TT *>(kp), blk_len, rows, n_rows, nb, \
                     B, sl2, kv_idx, kv_cnt, max_kv, kv_shared, mass, recall)
  if (dtype == HSA_BF16) {
    if (D == 128) HSA_MASS(uint16_t, 128); else HSA_MASS(uint16_t, 64);
  } else {
    if (D == 128) HSA_MASS(float, 128); else HSA_MASS(float, 64);
  }
#undef HSA_MASS
  return check_launch("hsa_block_mass");
}

}  // namespace hsa_host

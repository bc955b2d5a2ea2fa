// Gather into / scatter out of the reordered head-major layout.
//
// DFSAttn (Methodology, design 1): tokens are reordered before attention so
// that blocks are spatiotemporal neighbourhoods; the inverse reorder follows
// attention. Both directions are pure HBM streams: every token row of every
// head moves once.
//
// A workgroup owns G consecutive slots. A token's row holds nh*D elements =
// P 16-byte chunks, contiguous in the token-major tensor; thread t owns
// chunk positions t, t+256, ... of every slot of its group, so a warp reads
// contiguous pieces of a token row and writes whole D-element rows of the
// reordered tensor. Because a thread keeps its positions across the group,
// the gather can also sum its chunks over each sub-block of s slots and emit
// the sub-block means of Q and K that hierarchical scoring pools (DFSAttn,
// Methodology, design 2) without reading Qp/Kp again.
#include "common.h"

namespace hsa {

// Streaming 16-byte load with the nontemporal hint: the token-major inputs
// are read once here, and the hint measured ~3-5 % faster for the gather
// (a nontemporal store of the reordered rows was slower: attention reads them
// right after).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr int kPermThreads = 256;
constexpr int kPermMaxPos = 4;  // chunk positions per thread: P <= 1024

struct PermArgs {
  const char *src[3];
  char *dst[3];
};

__device__ __forceinline__ void add_chunk(float *acc, uint4 v, bool bf16) {
  if (bf16) {
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

// x [token][nh][D] -> xp [nh][n_pad][D] (pads zero), optionally with the
// sub-block means of tensors 0 and 1 (pooled [2][nh][n_pad/s][D], float).
template <bool BF16, int NP>
__global__ void __launch_bounds__(kPermThreads)
perm_gather_kernel(PermArgs a, const int32_t *__restrict__ perm, int n_pad, int G, int P,
                   int cpr /* chunks per head row */, int D, int64_t tok_stride_bytes,
                   int64_t head_stride_bytes, int s, float *__restrict__ pooled, int nh) {
  constexpr int kCols = BF16 ? 8 : 4;
  const int t = blockIdx.y;
  const char *__restrict__ src = a.src[t];
  char *__restrict__ dst = a.dst[t];
  const int slot0 = blockIdx.x * G;
  const int slots = min(G, n_pad - slot0);
  const bool pool = pooled != nullptr && t < 2;
  int pos[NP];
  int64_t dofs[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    pos[k] = threadIdx.x + k * kPermThreads;
    const int h = pos[k] / cpr, c = pos[k] - (pos[k] / cpr) * cpr;
    dofs[k] = h * head_stride_bytes + static_cast<int64_t>(c) * 16;
  }
  float acc[NP][kCols];
#pragma unroll
  for (int k = 0; k < NP; ++k)
#pragma unroll
    for (int j = 0; j < kCols; ++j) acc[k][j] = 0.f;
  int real = 0;
  for (int j0 = 0; j0 < slots; j0 += 4) {
    uint4 v[4][NP];
    int tok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      tok[u] = (j0 + u < slots) ? perm[slot0 + j0 + u] : -1;
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        v[u][k] = make_uint4(0, 0, 0, 0);
        if (tok[u] >= 0 && pos[k] < P)
          v[u][k] = load_stream16(src + tok[u] * tok_stride_bytes + static_cast<int64_t>(pos[k]) * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u;
      if (j < slots) {
        const int64_t row = static_cast<int64_t>(slot0 + j) * cpr * 16;
        if (dst != nullptr) {  // null: the tensor is only pooled
#pragma unroll
          for (int k = 0; k < NP; ++k)
            if (pos[k] < P) *reinterpret_cast<uint4 *>(dst + dofs[k] + row) = v[u][k];
        }
        if (pool) {
          real += tok[u] >= 0;
#pragma unroll
          for (int k = 0; k < NP; ++k) add_chunk(acc[k], v[u][k], BF16);
          if ((j + 1) % s == 0) {  // sub-block complete: write its means
            const int U = n_pad / s;
            const int u_idx = (slot0 + j) / s;
            const float inv = real > 0 ? 1.f / static_cast<float>(real) : 0.f;
#pragma unroll
            for (int k = 0; k < NP; ++k) {
              if (pos[k] < P) {
                const int h = pos[k] / cpr, c = pos[k] - (pos[k] / cpr) * cpr;
                float *out = pooled + ((static_cast<int64_t>(t) * nh + h) * U + u_idx) * D + c * kCols;
#pragma unroll
                for (int q = 0; q < kCols; q += 4)
                  *reinterpret_cast<float4 *>(out + q) =
                      make_float4(acc[k][q] * inv, acc[k][q + 1] * inv, acc[k][q + 2] * inv,
                                  acc[k][q + 3] * inv);
              }
#pragma unroll
              for (int q = 0; q < kCols; ++q) acc[k][q] = 0.f;
            }
            real = 0;
          }
        }
      }
    }
  }
}

// op [nh][n_pad][D] -> o [token][nh][D] for real slots. All 256 threads
// stride over (slot, chunk) pairs of a 16-slot group, so every lane has work
// whatever nh*D is; reads are whole head rows, writes whole token rows.
constexpr int kScatterSlots = 16;

__global__ void __launch_bounds__(kPermThreads)
perm_scatter_kernel(const char *__restrict__ src, char *__restrict__ dst,
                    const int32_t *__restrict__ perm, int n_pad, int P, int cpr, int row_shift,
                    int64_t tok_stride_bytes, int64_t head_stride_bytes) {
  const int slot0 = blockIdx.x * kScatterSlots;
  const int total = kScatterSlots * P;
  for (int v = threadIdx.x; v < total; v += kPermThreads) {
    const int sl = v / P;
    const int rem = v - sl * P;
    const int slot = slot0 + sl;
    if (slot >= n_pad) break;
    const int tok = perm[slot];
    if (tok < 0) continue;
    const int h = rem >> row_shift;
    const int c = rem & (cpr - 1);
    const uint4 val = load_stream16(src + h * head_stride_bytes + (static_cast<int64_t>(slot) * cpr + c) * 16);
    *reinterpret_cast<uint4 *>(dst + tok * tok_stride_bytes + static_cast<int64_t>(rem) * 16) = val;
  }
}

}  // namespace hsa

namespace hsa_host {

static int positions_per_thread(int P) { return (P + hsa::kPermThreads - 1) / hsa::kPermThreads; }

hsa_status_t launch_perm(int n, const void *const *xs, void *const *xps, const int32_t *perm,
                         int n_pad, int nh, int D, int64_t tok_stride, int esize, int pool_s,
                         float *pooled, hipStream_t stream) {
  hsa::PermArgs a{};
  for (int i = 0; i < n; ++i) {
    a.src[i] = static_cast<const char *>(xs[i]);
    a.dst[i] = static_cast<char *>(xps[i]);
  }
  const int cpr = D * esize / 16;
  const int P = nh * cpr;
  // A group holds whole sub-blocks when pooling; 32 slots otherwise.
  const int G = pooled ? (pool_s >= 32 ? pool_s : 32) : 32;
  const int s = pooled ? pool_s : 1;
  const dim3 grid((n_pad + G - 1) / G, n);
  const int np = positions_per_thread(P);
  const int64_t ts = tok_stride * esize, hs = static_cast<int64_t>(n_pad) * D * esize;
#define HSA_PERM_LAUNCH(BF, NPV)                                                                  \
  hipLaunchKernelGGL((hsa::perm_gather_kernel<BF, NPV>), grid, dim3(hsa::kPermThreads), 0, stream, \
                     a, perm, n_pad, G, P, cpr, D, ts, hs, s, pooled, nh)
  if (esize == 2) {
    if (np <= 1) HSA_PERM_LAUNCH(true, 1);
    else if (np <= 2) HSA_PERM_LAUNCH(true, 2);
    else HSA_PERM_LAUNCH(true, 4);
  } else {
    if (np <= 1) HSA_PERM_LAUNCH(false, 1);
    else if (np <= 2) HSA_PERM_LAUNCH(false, 2);
    else HSA_PERM_LAUNCH(false, 4);
  }
#undef HSA_PERM_LAUNCH
  return check_launch("hsa_perm");
}

hsa_status_t launch_unperm(const void *op, void *o, const int32_t *perm, int n_pad, int nh, int D,
                           int64_t tok_stride, int esize, hipStream_t stream) {
  const int cpr = D * esize / 16;  // a power of two
  int shift = 0;
  while ((1 << shift) < cpr) ++shift;
  const int P = nh * cpr;
  const dim3 grid((n_pad + hsa::kScatterSlots - 1) / hsa::kScatterSlots);
  hipLaunchKernelGGL(hsa::perm_scatter_kernel, grid, dim3(hsa::kPermThreads), 0, stream,
                     static_cast<const char *>(op), static_cast<char *>(o), perm, n_pad, P, cpr,
                     shift, tok_stride * esize, static_cast<int64_t>(n_pad) * D * esize);
  return check_launch("hsa_unperm");
}

}  // namespace hsa_host

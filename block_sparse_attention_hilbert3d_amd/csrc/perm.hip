// Gather into / scatter out of the reordered head-major layout.
//
// DFSAttn (Methodology, design 1): tokens are reordered before attention so
// that blocks are spatiotemporal neighbourhoods; the inverse reorder follows
// attention. Both directions are pure HBM streams: every token row of every
// head moves once. A workgroup owns a run of consecutive slots; each 16-byte
// chunk is one lane's load and store. On the token-major side a slot's heads
// are contiguous (nh*D elements), on the reordered side each head row is a
// contiguous D-element run, so both sides move whole cache lines.
#include "common.h"

namespace hsa {

constexpr int kPermThreads = 256;
constexpr int kPermSlots = 16;  // slots per workgroup

struct PermArgs {
  const char *src[3];
  char *dst[3];
};

// x [token][nh][D] -> xp [nh][n_pad][D]; chunk = 16 bytes.
__global__ void __launch_bounds__(kPermThreads)
perm_gather_kernel(PermArgs a, const int32_t *__restrict__ perm, int n_pad, int nh,
                   int chunks_per_row /* D*e/16, power of two */, int row_shift,
                   int64_t tok_stride_bytes, int64_t head_stride_bytes) {
  const int t = blockIdx.y;
  const char *__restrict__ src = a.src[t];
  char *__restrict__ dst = a.dst[t];
  const int per_slot = nh * chunks_per_row;
  const int slot0 = blockIdx.x * kPermSlots;
  const int total = kPermSlots * per_slot;
  for (int v = threadIdx.x; v < total; v += kPermThreads) {
    const int sl = v / per_slot;
    const int rem = v - sl * per_slot;
    const int slot = slot0 + sl;
    if (slot >= n_pad) break;
    const int h = rem >> row_shift;
    const int c = rem & (chunks_per_row - 1);
    const int tok = perm[slot];
    uint4 val = make_uint4(0, 0, 0, 0);
    if (tok >= 0) {
      val = *reinterpret_cast<const uint4 *>(src + tok * tok_stride_bytes +
                                             static_cast<int64_t>(rem) * 16);
    }
    *reinterpret_cast<uint4 *>(dst + h * head_stride_bytes +
                               (static_cast<int64_t>(slot) * chunks_per_row + c) * 16) = val;
  }
}

// op [nh][n_pad][D] -> o [token][nh][D] for real slots.
__global__ void __launch_bounds__(kPermThreads)
perm_scatter_kernel(const char *__restrict__ src, char *__restrict__ dst,
                    const int32_t *__restrict__ perm, int n_pad, int nh, int chunks_per_row,
                    int row_shift, int64_t tok_stride_bytes, int64_t head_stride_bytes) {
  const int per_slot = nh * chunks_per_row;
  const int slot0 = blockIdx.x * kPermSlots;
  const int total = kPermSlots * per_slot;
  for (int v = threadIdx.x; v < total; v += kPermThreads) {
    const int sl = v / per_slot;
    const int rem = v - sl * per_slot;
    const int slot = slot0 + sl;
    if (slot >= n_pad) break;
    const int tok = perm[slot];
    if (tok < 0) continue;
    const int h = rem >> row_shift;
    const int c = rem & (chunks_per_row - 1);
    const uint4 val = *reinterpret_cast<const uint4 *>(
        src + h * head_stride_bytes + (static_cast<int64_t>(slot) * chunks_per_row + c) * 16);
    *reinterpret_cast<uint4 *>(dst + tok * tok_stride_bytes + static_cast<int64_t>(rem) * 16) =
        val;
  }
}

}  // namespace hsa

namespace hsa_host {

static int ilog2(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

hsa_status_t launch_perm(int n, const void *const *xs, void *const *xps, const int32_t *perm,
                         int n_pad, int nh, int D, int64_t tok_stride, int esize,
                         hipStream_t stream) {
  hsa::PermArgs a{};
  for (int i = 0; i < n; ++i) {
    a.src[i] = static_cast<const char *>(xs[i]);
    a.dst[i] = static_cast<char *>(xps[i]);
  }
  const int cpr = D * esize / 16;
  const dim3 grid((n_pad + hsa::kPermSlots - 1) / hsa::kPermSlots, n);
  hipLaunchKernelGGL(hsa::perm_gather_kernel, grid, dim3(hsa::kPermThreads), 0, stream, a, perm,
                     n_pad, nh, cpr, ilog2(cpr), tok_stride * esize,
                     static_cast<int64_t>(n_pad) * D * esize);
  return check_launch("hsa_perm");
}

hsa_status_t launch_unperm(const void *op, void *o, const int32_t *perm, int n_pad, int nh, int D,
                           int64_t tok_stride, int esize, hipStream_t stream) {
  const int cpr = D * esize / 16;
  const dim3 grid((n_pad + hsa::kPermSlots - 1) / hsa::kPermSlots);
  hipLaunchKernelGGL(hsa::perm_scatter_kernel, grid, dim3(hsa::kPermThreads), 0, stream,
                     static_cast<const char *>(op), static_cast<char *>(o), perm, n_pad, nh, cpr,
                     ilog2(cpr), tok_stride * esize, static_cast<int64_t>(n_pad) * D * esize);
  return check_launch("hsa_unperm");
}

}  // namespace hsa_host

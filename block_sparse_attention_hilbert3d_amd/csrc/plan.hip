// Token-order plan kernels.
//
// DFSAttn (Methodology, design 1): reorder every token along one global 3D
// Hilbert curve before attention. This file walks the enclosing 2^b cube in
// curve order by DECODING each curve index to its cell (Skilling's transpose
// method, "Programming the Hilbert curve", 2004: Gray-decode the transposed
// index, then undo the curve's excess work level by level), keeps in-grid
// cells, and compacts them with a two-kernel scan. Pads go at the tail.
#include "common.h"

namespace hsa {

constexpr int kPlanThreads = 256;
constexpr int kPlanItems = 8;  // consecutive curve indices per thread
constexpr int kPlanCells = kPlanThreads * kPlanItems;

// Cell (x0, x1, x2) = (t, y, x) visited at curve index h on the 2^b cube.
__device__ __forceinline__ void hilbert_decode3(uint32_t h, int b, uint32_t &x0, uint32_t &x1,
                                                uint32_t &x2) {
  uint32_t a0 = 0, a1 = 0, a2 = 0;
  // Transposed form: bit (3j + 2 - i) of h is bit j of axis word i.
  for (int j = 0; j < b; ++j) {
    a0 |= ((h >> (3 * j + 2)) & 1u) << j;
    a1 |= ((h >> (3 * j + 1)) & 1u) << j;
    a2 |= ((h >> (3 * j)) & 1u) << j;
  }
  // Gray decode across the three words.
  const uint32_t g = a2 >> 1;
  a2 ^= a1;
  a1 ^= a0;
  a0 ^= g;
  // Undo excess work from the lowest level up; words are visited last to
  // first at each level (a bit of word i inverts word 0's lower bits,
  // otherwise word 0 and word i exchange their lower bits).
  const uint32_t end = 2u << (b - 1);
  for (uint32_t q = 2; q != end; q <<= 1) {
    const uint32_t low = q - 1;
    uint32_t sw;
    if (a2 & q) {
      a0 ^= low;
    } else {
      sw = (a0 ^ a2) & low;
      a0 ^= sw;
      a2 ^= sw;
    }
    if (a1 & q) {
      a0 ^= low;
    } else {
      sw = (a0 ^ a1) & low;
      a0 ^= sw;
      a1 ^= sw;
    }
    if (a0 & q) a0 ^= low;
  }
  x0 = a0;
  x1 = a1;
  x2 = a2;
}

// Cell (x0, x1) = (y, x) visited at curve index h on the 2^b square: the
// same inverse transform in two dimensions.
__device__ __forceinline__ void hilbert_decode2(uint32_t h, int b, uint32_t &x0, uint32_t &x1) {
  uint32_t a0 = 0, a1 = 0;
  for (int j = 0; j < b; ++j) {
    a0 |= ((h >> (2 * j + 1)) & 1u) << j;
    a1 |= ((h >> (2 * j)) & 1u) << j;
  }
  const uint32_t g = a1 >> 1;
  a1 ^= a0;
  a0 ^= g;
  const uint32_t end = 2u << (b - 1);
  for (uint32_t q = 2; q != end; q <<= 1) {
    const uint32_t low = q - 1;
    if (a1 & q) {
      a0 ^= low;
    } else {
      const uint32_t sw = (a0 ^ a1) & low;
      a0 ^= sw;
      a1 ^= sw;
    }
    if (a0 & q) a0 ^= low;
  }
  x0 = a0;
  x1 = a1;
}

// Curve index h -> token, if its cell lies in the grid. DIMS = 3: the
// T x H x W grid in the 2^b cube; DIMS = 2: one H x W frame in the square.
template <int DIMS>
__device__ __forceinline__ bool in_grid(uint32_t h, int b, int T, int H, int W, int32_t &tok) {
  uint32_t t = 0, y, x;
  if constexpr (DIMS == 3) hilbert_decode3(h, b, t, y, x);
  else hilbert_decode2(h, b, y, x);
  tok = static_cast<int32_t>((t * static_cast<uint32_t>(H) + y) * static_cast<uint32_t>(W) + x);
  return t < static_cast<uint32_t>(T) && y < static_cast<uint32_t>(H) &&
         x < static_cast<uint32_t>(W);
}

// Block-wide exclusive scan of one int per thread; returns the total.
__device__ int block_exclusive_scan(int v, int &excl, int *sh /* kPlanThreads/64 + 1 */) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh[wid] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    if (w < wid) base += sh[w];
    total += sh[w];
  }
  excl = base + incl - v;
  __syncthreads();
  return total;
}

template <int DIMS>
__global__ void __launch_bounds__(kPlanThreads)
hilbert_count_kernel(int b, uint32_t cube, int T, int H, int W, int32_t *counts) {
  __shared__ int sh[kPlanThreads / 64 + 1];
  const uint32_t base = blockIdx.x * kPlanCells + threadIdx.x * kPlanItems;
  int c = 0;
  for (int j = 0; j < kPlanItems; ++j) {
    const uint32_t h = base + j;
    int32_t tok;
    if (h < cube && in_grid<DIMS>(h, b, T, H, W, tok)) ++c;
  }
  int excl;
  const int total = block_exclusive_scan(c, excl, sh);
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

template <int DIMS>
__global__ void __launch_bounds__(kPlanThreads)
hilbert_write_kernel(int b, uint32_t cube, int T, int H, int W, const int32_t *counts,
                     int32_t *perm) {
  __shared__ int sh[kPlanThreads / 64 + 1];
  __shared__ int sh_off;
  // Offset of this workgroup: sum of the counts of all earlier workgroups.
  int part = 0;
  for (int i = threadIdx.x; i < static_cast<int>(blockIdx.x); i += kPlanThreads) part += counts[i];
  int excl0;
  const int before = block_exclusive_scan(part, excl0, sh);
  if (threadIdx.x == 0) sh_off = before;
  __syncthreads();
  const int offset = sh_off;

  const uint32_t base = blockIdx.x * kPlanCells + threadIdx.x * kPlanItems;
  int c = 0;
  for (int j = 0; j < kPlanItems; ++j) {
    const uint32_t h = base + j;
    int32_t tok;
    if (h < cube && in_grid<DIMS>(h, b, T, H, W, tok)) ++c;
  }
  int excl;
  block_exclusive_scan(c, excl, sh);
  // Decode again rather than holding the cells in a dynamically indexed array.
  int k = offset + excl;
  for (int j = 0; j < kPlanItems; ++j) {
    const uint32_t h = base + j;
    int32_t tok;
    if (h < cube && in_grid<DIMS>(h, b, T, H, W, tok)) perm[k++] = tok;
  }
}

// Tiled partitions: block k is tile k (row-major over tile coordinates,
// tiles tT x tH x tW clipped to the grid); slot r of the block holds the
// r-th cell of the tile in row-major order, or a pad past its volume.
struct Tiling {
  int tT, tH, tW, nT, nH, nW;
};
__device__ __forceinline__ Tiling tiling_of(int order, int T, int H, int W, int B) {
  Tiling g;
  const bool two = order == HSA_ORDER_TILE2D;
  g.tT = two ? 1 : B / 64;
  g.tH = 8;
  g.tW = two ? B / 8 : 8;
  g.nT = (T + g.tT - 1) / g.tT;
  g.nH = (H + g.tH - 1) / g.tH;
  g.nW = (W + g.tW - 1) / g.tW;
  return g;
}
// volume of tile k; its origin and clipped extents through the references
__device__ __forceinline__ int tile_box(const Tiling &g, int k, int T, int H, int W, int &t0, int &y0,
                                        int &x0, int &eH, int &eW) {
  const int a = k / (g.nH * g.nW), rem = k - a * g.nH * g.nW;
  const int b = rem / g.nW, c = rem - b * g.nW;
  t0 = a * g.tT;
  y0 = b * g.tH;
  x0 = c * g.tW;
  const int eT = min(g.tT, T - t0);
  eH = min(g.tH, H - y0);
  eW = min(g.tW, W - x0);
  return eT * eH * eW;
}

// ROW / FRAME / TILE2D / CUBE3D plans are closed-form; HILBERT only needs
// tail pads here. Also fills blk_len for every order.
__global__ void plan_fill_kernel(int order, int T, int H, int W, int B, int n_pad, int nb,
                                 int32_t *perm, int32_t *blk_len) {
  const int N = T * H * W;
  const int P = H * W;
  const int tiles = (P + B - 1) / B;
  const int per = tiles * B;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_pad; i += gridDim.x * blockDim.x) {
    if (order == HSA_ORDER_FRAME) {
      const int f = i / per, r = i - f * per;
      perm[i] = (r < P) ? f * P + r : -1;
    } else if (order == HSA_ORDER_ROW) {
      perm[i] = (i < N) ? i : -1;
    } else if (order == HSA_ORDER_HILBERT2D) {
      // frame 0 was written in curve order; later frames repeat it
      if (i >= N) perm[i] = -1;
      else if (i >= P) perm[i] = (i / P) * P + perm[i % P];
    } else if (order == HSA_ORDER_TILE2D || order == HSA_ORDER_CUBE3D) {
      const Tiling g = tiling_of(order, T, H, W, B);
      const int k = i / B, r = i - k * B;
      int t0, y0, x0, eH, eW;
      const int vol = tile_box(g, k, T, H, W, t0, y0, x0, eH, eW);
      if (r < vol) {
        const int dt = r / (eH * eW), rr = r - dt * eH * eW, dy = rr / eW, dx = rr - dy * eW;
        perm[i] = ((t0 + dt) * H + (y0 + dy)) * W + (x0 + dx);
      } else {
        perm[i] = -1;
      }
    } else if (i >= N) {
      perm[i] = -1;
    }
    if (i < nb) {
      int len;
      if (order == HSA_ORDER_FRAME) {
        const int j = i % tiles;
        len = min(B, P - j * B);
      } else if (order == HSA_ORDER_TILE2D || order == HSA_ORDER_CUBE3D) {
        int t0, y0, x0, eH, eW;
        len = tile_box(tiling_of(order, T, H, W, B), i, T, H, W, t0, y0, x0, eH, eW);
      } else {
        len = min(B, N - i * B);
      }
      blk_len[i] = max(len, 0);
    }
  }
}

}  // namespace hsa

namespace hsa_host {

size_t plan_hilbert_groups(int T, int H, int W, int &bits, uint32_t &cube, int dims) {
  const int m = dims == 3 ? max(T, max(H, W)) : max(H, W);
  int b = 1;
  while ((1 << b) < m) ++b;
  bits = b;
  cube = 1u << (dims * b);
  return (cube + hsa::kPlanCells - 1) / hsa::kPlanCells;
}

hsa_status_t launch_plan(int T, int H, int W, int order, int B, int n_pad, int nb, int32_t *perm,
                         int32_t *blk_len, void *ws, hipStream_t stream) {
  if (order == HSA_ORDER_HILBERT3D) {
    int b;
    uint32_t cube;
    const size_t groups = plan_hilbert_groups(T, H, W, b, cube, 3);
    int32_t *counts = static_cast<int32_t *>(ws);
    hipLaunchKernelGGL(hsa::hilbert_count_kernel<3>, dim3(groups), dim3(hsa::kPlanThreads), 0,
                       stream, b, cube, T, H, W, counts);
    hipLaunchKernelGGL(hsa::hilbert_write_kernel<3>, dim3(groups), dim3(hsa::kPlanThreads), 0,
                       stream, b, cube, T, H, W, counts, perm);
  } else if (order == HSA_ORDER_HILBERT2D) {
    // frame 0's cells in curve order; plan_fill_kernel repeats them per frame
    int b;
    uint32_t sq;
    const size_t groups = plan_hilbert_groups(T, H, W, b, sq, 2);
    int32_t *counts = static_cast<int32_t *>(ws);
    hipLaunchKernelGGL(hsa::hilbert_count_kernel<2>, dim3(groups), dim3(hsa::kPlanThreads), 0,
                       stream, b, sq, 1, H, W, counts);
    hipLaunchKernelGGL(hsa::hilbert_write_kernel<2>, dim3(groups), dim3(hsa::kPlanThreads), 0,
                       stream, b, sq, 1, H, W, counts, perm);
  }
  const int blocks = min((n_pad + 255) / 256, 4096);
  hipLaunchKernelGGL(hsa::plan_fill_kernel, dim3(blocks), dim3(256), 0, stream, order, T, H, W,
                     B, n_pad, nb, perm, blk_len);
  return check_launch("hsa_plan");
}

}  // namespace hsa_host

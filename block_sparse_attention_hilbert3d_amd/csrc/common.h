// Shared device helpers for the gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hsa.h"

namespace hsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Lanes below this one, as a 64-bit mask.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return (l == 0) ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 takes the key of +0, since the two compare equal (and so tie).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// XCD-aware remap of a linear workgroup id: hardware hands consecutive ids to
// the 8 XCDs round-robin; this makes each XCD see a contiguous logical range
// (so neighbouring tiles share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int per = total / 8;
  const int full = per * 8;
  if (b >= full) return b;
  return (b % 8) * per + b / 8;
}

// Ordered launches: give each XCD runs of kRun consecutive order positions
// (rows next to each other in the order share key blocks in that XCD's L2)
// while the runs still go to the XCDs in turn, so the longest rows, which
// come first, stay spread over all of them.
__device__ __forceinline__ int xcd_runs(int b, int total) {
  constexpr int kRun = 4;
  const int full = total / (8 * kRun) * (8 * kRun);
  if (b >= full) return b;
  const int x = b & 7, q = b >> 3;
  return ((q / kRun) * 8 + x) * kRun + q % kRun;
}

// (head, list row) of workgroup b for kernels with one workgroup per (head,
// block). Without an order, neighbouring blocks of one head go to one XCD
// (shared L2). With one, the b-th workgroup takes row order[xcd_runs(b)]
// (longest lists first); shared lists order blocks, and the nh heads of a
// block are consecutive workgroups.
__device__ __forceinline__ void block_of(int b, const int32_t *order, int kv_shared, int nh, int nb,
                                         int &h, int &I) {
  if (order == nullptr) {
    const int bid = xcd_remap(b, nh * nb);
    h = bid / nb;
    I = bid - h * nb;
  } else if (kv_shared) {
    h = b % nh;
    I = min(max(order[b / nh], 0), nb - 1);
  } else {
    const int e = min(max(order[xcd_runs(b, nh * nb)], 0), nh * nb - 1);
    h = e / nb;
    I = e - h * nb;
  }
}

// One 16-byte-per-lane direct global->LDS load: lane l's 16 bytes come from
// sbase + voff (sbase wave-uniform) and land at lds_base + 16*l. Issued from
// asm so the compiler does not add blanket vmcnt(0) waits in front of
// unrelated LDS reads; the caller waits with wait_vmcnt() and a barrier
// before the data is read. No register is written.
__device__ __forceinline__ void load_lds16(const void *sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) (gfx9 encoding), leaving the other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) char lds_char_t;

// Generic pointer to a __shared__ object -> LDS pointer / LDS byte address.
__device__ __forceinline__ lds_char_t *to_lds(const void *p) { return (lds_char_t *)(p); }
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>((uintptr_t)to_lds(p));
}

// Tile layouts in LDS: BK rows (keys) of CPR 16-byte chunks (D bf16 each).
// K: chunk c of row r sits at slot c ^ (r mod CPR) so the 32 lanes reading a
//    fragment (32 rows, one chunk) hit distinct banks.
// V: chunk c of row r sits at slot c ^ ((4 (r mod 4)) mod CPR) so the
//    transposed reads (4 rows x 4 chunks per half-wave) hit distinct banks.
template <int CPR>
__device__ __forceinline__ int k_slot(int r, int c) { return r * CPR + (c ^ (r & (CPR - 1))); }
template <int CPR>
__device__ __forceinline__ int v_slot(int r, int c) { return r * CPR + (c ^ (((r & 3) << 2) & (CPR - 1))); }

// Per-lane byte offsets (within a 1 KB slice) of the direct tile loads.
// A wave's i-th load fills LDS slots P = (w*NI + i)*64 + lane, i.e. rows
// r = (w*NI + i)*(64/CPR) + lane/CPR, physical chunk lane%CPR; it reads the
// logical chunk that the swizzle stores there. The swizzle key depends on
// r mod CPR (K) or r mod 4 (V), which repeats every 4 loads (K) or never
// changes (V), so 4 offsets cover every load.
template <int D, bool IS_V>
__device__ __forceinline__ uint32_t tile_lane_offset(int i, int lane) {
  constexpr int CPR = D / 8;
  const int r = i * (64 / CPR) + lane / CPR;   // row within the slice group, mod 16 exact
  const int cs = lane & (CPR - 1);
  const int c = IS_V ? (cs ^ (((r & 3) << 2) & (CPR - 1))) : (cs ^ (r & (CPR - 1)));
  return static_cast<uint32_t>((lane / CPR) * D * 2 + c * 16);
}

// The logical chunk's byte offset within its row for load i of this lane
// (the chunk part of tile_lane_offset), for tiles gathered row by row.
template <int D, bool IS_V>
__device__ __forceinline__ uint32_t tile_lane_chunk(int i, int lane) {
  constexpr int CPR = D / 8;
  const int r = i * (64 / CPR) + lane / CPR;
  const int cs = lane & (CPR - 1);
  const int c = IS_V ? (cs ^ (((r & 3) << 2) & (CPR - 1))) : (cs ^ (r & (CPR - 1)));
  return static_cast<uint32_t>(c * 16);
}

// Loads per wave of one BKxD bf16 tile and the tile row that load i of a lane
// covers: row (w*NI + i)*(64/CPR) + lane/CPR.
template <int D, int BK, int NW>
struct TileLoads {
  static constexpr int CPR = D / 8;
  static constexpr int NI = BK * CPR / (64 * NW);
  static constexpr int RPL = 64 / CPR;  // rows per load instruction
  __device__ static __forceinline__ int row(int w, int i, int lane) { return (w * NI + i) * RPL + lane / CPR; }
};

// Issue the direct loads of one BKxD bf16 tile whose rows are gathered:
// this lane's load i reads gbase + off[i] (32-bit byte offsets) into the
// slot the swizzled layout assigns it.
template <int D, int BK, int NW>
__device__ __forceinline__ void issue_tile_offs(const uint16_t *gbase, uint32_t lds_tile, int w,
                                                const uint32_t (&off)[TileLoads<D, BK, NW>::NI]) {
  constexpr int NI = TileLoads<D, BK, NW>::NI;
  static_assert(D / 8 == 8 || NI % 4 == 0, "the swizzle key must not depend on the wave");
  const uint32_t lbase = lds_tile + w * NI * 1024;
#pragma unroll
  for (int i = 0; i < NI; ++i) load_lds16(gbase, off[i], lbase + i * 1024);
}

// Issue wave w's NI consecutive 1 KB slices of a row-major tile (slices
// w*NI .. w*NI + NI - 1) with one lane offset per load, for tiles whose
// swizzle key changes from wave to wave (off[i] from tile_lane_offset of
// slice w*NI + i).
template <int NI>
__device__ __forceinline__ void issue_tile_slices(const uint16_t *gtile, uint32_t lds_tile, int w,
                                                  const uint32_t (&off)[NI]) {
  const char *gb = reinterpret_cast<const char *>(gtile) + w * NI * 1024;
  const uint32_t lb = lds_tile + w * NI * 1024;
#pragma unroll
  for (int i = 0; i < NI; ++i) load_lds16(gb + i * 1024, off[i], lb + i * 1024);
}

// Issue the direct loads of one BKxD bf16 tile (row-major in HBM) into a
// swizzled LDS tile; each wave moves NI consecutive 1 KB slices.
template <int D, int BK, int NW>
__device__ __forceinline__ void issue_tile(const uint16_t *gtile, uint32_t lds_tile, int w,
                                           const uint32_t (&loff)[4]) {
  constexpr int CPR = D / 8;
  constexpr int NI = BK * CPR / (64 * NW);
  static_assert(CPR == 8 || NI % 4 == 0, "the swizzle key must not depend on the wave");
  const char *gbase = reinterpret_cast<const char *>(gtile) + w * NI * 1024;
  const uint32_t lbase = lds_tile + w * NI * 1024;
#pragma unroll
  for (int i = 0; i < NI; ++i)
    load_lds16(gbase + i * 1024, loff[i & 3], lbase + i * 1024);
}

}  // namespace hsa

// Host-side error plumbing (abi.hip).
namespace hsa_host {
hsa_status_t fail(hsa_status_t code, const char *fmt, ...);
hsa_status_t check_launch(const char *what);
}  // namespace hsa_host

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

// Order-preserving map of a float to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
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

}  // namespace hsa

// Host-side error plumbing (abi.hip).
namespace hsa_host {
hsa_status_t fail(hsa_status_t code, const char *fmt, ...);
hsa_status_t check_launch(const char *what);
}  // namespace hsa_host

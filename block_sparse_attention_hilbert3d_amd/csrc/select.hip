// Block selection: per-query-block ascending lists of key blocks.
//
// Ranking key of an entry: its score mapped to an order-preserving uint32,
// ties broken toward the lower index. One wave owns one row; its lanes hold
// the row strided (lane l, register r -> column l + 64 r), so "lower lane,
// then lower register" is ascending column order and every rank, prefix and
// compaction is a ballot plus a popcount on the scalar unit.
//
//  TOPK          DFSAttn (Methodology, design 3): the k best key blocks.
//                MSB-first bitwise search for the k-th largest key.
//  THRESH_GLOBAL VMoBA abstract: threshold selection by cumulative
//                similarity, then global selection over the head, under a
//                budget that shrinks across steps (DFSAttn design 3).
//                Per row: the count and exact 2^-62 fixed-point mass of
//                each 12-bit key bin in a window below the row's largest
//                key (one packed LDS atomic per column), a scan to the bin
//                where the mass reaches tau, and a register sort of that
//                bin's columns give the boundary key of the shortest prefix
//                reaching tau; rows whose boundary bin is crowded or below
//                the window take an MSB-first radix search (digits of up to
//                8 bits) in a pass of their own. Per head: an MSB-first
//                radix select of the remaining budget among the pairs
//                outside the row prefixes over 52-bit pair keys (score
//                order key, then the lower linear index): digit 0 counted
//                while the row prefixes are found, digit 1 in a second pass
//                over the scores (whose workgroups first pick digit 0), the
//                last 28 bits resolved among the few pairs left in the
//                boundary digits, which the emitting pass collects (its
//                workgroups first pick digit 1; a head's last one resolves
//                the rest). Lists are written in the emitting pass (rows
//                holding boundary pairs by a small pass after the resolve).
//  Every mode writes kv_cnt and the first kv_cnt entries of each list;
//  entries past the count are not written.
//  LVSA          LVSA section 2, A(t) = G_s u W(t): rotating anchors plus the
//                nearest non-anchor frames; tile lists shared by all heads.
#include <algorithm>

#include "common.h"

namespace hsa {

constexpr int kSelThreads = 256;  // four rows per workgroup

template <int KPL>
__device__ __forceinline__ void load_row_keys(const float *row, int nb, uint32_t (&key)[KPL]) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane + 64 * r;
    key[r] = (j < nb) ? float_order_key(row[j]) : 0u;
  }
}

// k-th largest key among the row (keys of absent columns are 0 and real keys
// are >= 1, so they never count when k <= number of real columns).
template <int KPL>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&key)[KPL], int k) {
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) cnt += popc64(__ballot(key[r] >= cand));
    if (cnt >= k) thr = cand;
  }
  return thr;
}


// Writes the columns with sel[r] set, ascending; returns the count. Entries
// past the count are not written.
template <int KPL>
__device__ __forceinline__ int emit_sel(const bool (&sel)[KPL], int32_t *out) {
  const int lane = lane_id();
  int before = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const uint64_t b = __ballot(sel[r]);
    if (sel[r]) out[before + popc64(b & lanemask_lt())] = lane + 64 * r;
    before += popc64(b);
  }
  return before;
}

template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
topk_kernel(const float *__restrict__ S, int rows, int nb, int k, int32_t *__restrict__ kv_idx,
            int32_t *__restrict__ kv_cnt, int max_kv) {
  const int row = blockIdx.x * (kSelThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = lane_id();
  uint32_t key[KPL];
  load_row_keys<KPL>(S + static_cast<int64_t>(row) * nb, nb, key);
  const uint32_t thr = kth_largest<KPL>(key, k);
  int gt = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) gt += popc64(__ballot(key[r] > thr));
  const int need = k - gt;  // ties at thr to take, lowest columns first
  bool sel[KPL];
  int ties = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const bool tie = key[r] == thr && (lane + 64 * r) < nb;
    const uint64_t b = __ballot(tie);
    const int rank = ties + popc64(b & lanemask_lt());
    sel[r] = key[r] > thr || (tie && rank < need);
    ties += popc64(b);
  }
  const int cnt = emit_sel<KPL>(sel, kv_idx + static_cast<int64_t>(row) * max_kv);
  if (lane == 0) kv_cnt[row] = cnt;
}

// floor(p * 2^62) exactly, for 0 <= p < 4 (p's bits, or its order key; the
// sign bit is ignored): the
// significand with its leading one, m, times 2^(e - 88), taken as
// (m * 2^40) >> (128 - e); exponents e <= 64 (p < 2^-62) give 0.
__device__ __forceinline__ uint64_t fixed62(uint32_t bits) {
  const uint32_t e = (bits >> 23) & 0xFFu;
  const uint64_t m = static_cast<uint64_t>((bits & 0x7FFFFFu) | 0x800000u) << 40;
  return e >= 65u ? (m >> ((128u - e) & 63u)) : 0ull;
}

// float bits of an order key (inverse of float_order_key)
__device__ __forceinline__ uint32_t order_key_bits(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}

// Wave-wide scans and reductions on DPP lane moves (row shifts, then row
// broadcasts 15 and 31): no LDS round trips. Lanes without a source take
// `ident`.
template <int CTRL, int RM = 0xf>
__device__ __forceinline__ uint32_t dpp_or(uint32_t x, uint32_t ident) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(ident), static_cast<int>(x), CTRL, RM, 0xf, false));
}
template <int CTRL, int RM = 0xf>
__device__ __forceinline__ uint64_t dpp_or0_u64(uint64_t x) {
  return (static_cast<uint64_t>(dpp_or<CTRL, RM>(static_cast<uint32_t>(x >> 32), 0u)) << 32) |
         dpp_or<CTRL, RM>(static_cast<uint32_t>(x), 0u);
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t x) {
  x += dpp_or0_u64<0x111>(x);
  x += dpp_or0_u64<0x112>(x);
  x += dpp_or0_u64<0x114>(x);
  x += dpp_or0_u64<0x118>(x);
  x += dpp_or0_u64<0x142, 0xa>(x);
  x += dpp_or0_u64<0x143, 0xc>(x);
  return x;
}
__device__ __forceinline__ uint64_t lane63_u64(uint64_t x) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), 63));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_total_u64(uint64_t x) { return lane63_u64(wave_scan_u64(x)); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_or<0x111>(x, 0u));
  x = max(x, dpp_or<0x112>(x, 0u));
  x = max(x, dpp_or<0x114>(x, 0u));
  x = max(x, dpp_or<0x118>(x, 0u));
  x = max(x, dpp_or<0x142, 0xa>(x, 0u));
  x = max(x, dpp_or<0x143, 0xc>(x, 0u));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_or<0x111>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<0x112>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<0x114>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<0x118>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<0x142, 0xa>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<0x143, 0xc>(x, 0xFFFFFFFFu));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// 64-bit ranking key of column j with order key ok: larger = better.
__device__ __forceinline__ uint64_t key64(uint32_t ok, uint32_t j) {
  return (static_cast<uint64_t>(ok) << 32) | (0xFFFFFFFFu - j);
}

// Global key of pair (I, J) of a head: order key of the score, then the
// lower linear index I*nb+J first (lin < 2^20 since nb <= 1024): 52 bits.
__device__ __forceinline__ uint64_t gkey(uint32_t ok, uint32_t lin) {
  return (static_cast<uint64_t>(ok) << 20) | (0xFFFFFu - lin);
}

// Threshold selection keeps, per row, the prefix T_I = {key64 >= K_I}, and
// per head the pairs outside the prefixes whose global key is at least the
// head's fill threshold. The fill threshold is found by an MSB-first radix
// select over the global keys of the pairs outside the prefixes: digit 0 is
// key bits 51..40 (the score's top 12 order-key bits), counted while the
// row prefixes are found; digit 1 bits 39..28, counted in a second pass;
// the pairs left in the boundary digit pair (b0, b1) are collected by the
// emitting pass and resolved exactly on their remaining 28 bits.
//
// Within one row the global key orders pairs exactly as key64 does (score,
// then the lower column), so the pairs of row I with global key >= t are the
// columns with key64 >= row_fill_key(t, I), and the row's whole list is the
// columns with key64 >= min(K_I, row_fill_key(t, I)): one 64-bit compare per
// column when the lists are written.
//
// Scores are non-negative here, so their order key is their bits with the
// top bit set (both zeros share one key, as they compare equal), and digit 0
// of a real key is at least 2048.
constexpr int kHBits = 12;
constexpr int kHBins = 1 << kHBits;
constexpr int kCandCap = 2048;  // collected boundary pairs per head
constexpr int kWin = 256;       // digit-0 bins of a row's histogram window (from its largest key down)
constexpr int kSortMax = 64;    // boundary-bin columns sorted in registers, one per lane

enum : int32_t {
  kFillNone = 0,    // the row prefixes alone exceed the budget
  kFillThr = 1,     // fill threshold known: thr
  kFillDigit0 = 2,  // boundary digit b0 known, rem of its pairs to take
  kFillDigit1 = 3   // boundary digits (b0, b1) known, rem of their pairs to take
};

struct ThreshState {
  uint64_t thr;    // kFillThr: pairs with gkey >= thr are filled
  int64_t rem;     // pairs still to take inside the boundary digit(s)
  int32_t mode;
  int32_t b0, b1;
  int32_t pad;
};

// Per-head counters, cleared by thresh_init_kernel.
struct ThreshCounters {
  unsigned long long prefix_total;  // sum of |T_I| over the head's rows
  int32_t done_emit, pad;          // finished workgroups of the emitting pass (which ends in a pick)
  int32_t cand;                     // collected boundary pairs
  int32_t nfix;                     // rows listed for thresh_fix_kernel
};

// order key of a non-negative score from its bits
__device__ __forceinline__ uint32_t mass_key(uint32_t bits) { return (bits & 0x7FFFFFFFu) | 0x80000000u; }

// Cross-workgroup hand-off without cache maintenance: what one workgroup
// leaves for the head's last one is written with atomics (histograms,
// counters) or agent-scope stores (collected pairs), each wave waits until
// its memory operations are acknowledged, the workgroup synchronises, and
// only then is the arrival counted; the last arrival reads with agent-scope
// loads. (A device fence here would write back and invalidate the whole L2
// of the XCD in every workgroup.)
__device__ __forceinline__ void last_arrival_wait() {
  wait_vmcnt<0>();
  __syncthreads();
}

// loads that bypass the non-coherent caches (data other workgroups wrote)
__device__ __forceinline__ uint32_t coherent_load_u32(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t coherent_load_u64(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// inclusive prefix sum over the 64 lanes (32-bit)
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
  x += dpp_or<0x111>(x, 0u);
  x += dpp_or<0x112>(x, 0u);
  x += dpp_or<0x114>(x, 0u);
  x += dpp_or<0x118>(x, 0u);
  x += dpp_or<0x142, 0xa>(x, 0u);
  x += dpp_or<0x143, 0xc>(x, 0u);
  return x;
}

// Lane moves for the register sort: quad permutations, row mirrors and row
// rotations (every lane has a source).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xf, 0xf, false));
}
// value of lane l ^ 4: rotations of the 16-lane row by 4 and by 12
__device__ __forceinline__ uint32_t lane_xor4(uint32_t v, int l) {
  const uint32_t a = dpp_mov<0x124>(v), b = dpp_mov<0x12C>(v);
  return (l & 4) ? a : b;
}
// compare-exchange with the partner's value: the lower lane of the pair keeps
// the larger one
__device__ __forceinline__ uint32_t cex(uint32_t v, uint32_t o, bool lower) {
  return lower ? max(v, o) : min(v, o);
}
// Sorts the values of lanes [0, n) into descending order (n <= 64; lanes at
// and above n hold 0, below every real value). Bitonic merges whose first
// step pairs mirrored lanes (lane i with lane i ^ (2m - 1) in merges of 2m
// lanes) and then halves, so every comparator keeps the larger value in the
// lower lane; merges wider than n are skipped (16-lane rows are each sorted,
// and all real values sit in the first one).
__device__ __forceinline__ uint32_t sort_desc(uint32_t v, int n) {
  const int l = lane_id();
  v = cex(v, dpp_mov<0xB1>(v), !(l & 1));   // quad_perm [1,0,3,2]: lane ^ 1
  v = cex(v, dpp_mov<0x1B>(v), !(l & 2));   // quad_perm [3,2,1,0]: lane ^ 3
  v = cex(v, dpp_mov<0xB1>(v), !(l & 1));
  v = cex(v, dpp_mov<0x141>(v), !(l & 4));  // row half mirror: lane ^ 7
  v = cex(v, dpp_mov<0x4E>(v), !(l & 2));   // quad_perm [2,3,0,1]: lane ^ 2
  v = cex(v, dpp_mov<0xB1>(v), !(l & 1));
  v = cex(v, dpp_mov<0x140>(v), !(l & 8));  // row mirror: lane ^ 15
  v = cex(v, lane_xor4(v, l), !(l & 4));
  v = cex(v, dpp_mov<0x4E>(v), !(l & 2));
  v = cex(v, dpp_mov<0xB1>(v), !(l & 1));
  if (n > 16) {
    v = cex(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 31, 64)), !(l & 16));
    v = cex(v, dpp_mov<0x128>(v), !(l & 8));  // row rotation by 8: lane ^ 8
    v = cex(v, lane_xor4(v, l), !(l & 4));
    v = cex(v, dpp_mov<0x4E>(v), !(l & 2));
    v = cex(v, dpp_mov<0xB1>(v), !(l & 1));
    if (n > 32) {
      v = cex(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 63, 64)), !(l & 32));
      v = cex(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 16, 64)), !(l & 16));
      v = cex(v, dpp_mov<0x128>(v), !(l & 8));
      v = cex(v, lane_xor4(v, l), !(l & 4));
      v = cex(v, dpp_mov<0x4E>(v), !(l & 2));
      v = cex(v, dpp_mov<0xB1>(v), !(l & 1));
    }
  }
  return v;
}

// Smallest key64 of row I whose pair has global key >= t (t < 2^52): the
// columns j with key64 >= it are exactly those with gkey(ok_j, I*nb + j) >= t.
__device__ __forceinline__ uint64_t row_fill_key(uint64_t t, int I, int nb) {
  const uint64_t th = t >> 20;
  const int64_t jm = 0xFFFFF - static_cast<int64_t>(I) * nb - static_cast<int64_t>(t & 0xFFFFFu);
  if (jm >= 0) return (th << 32) | (0xFFFFFFFFull - static_cast<uint64_t>(jm));
  return th >= 0xFFFFFFFFull ? ~0ull : ((th + 1) << 32);  // no column of score th qualifies
}

// Whole-workgroup (kSelThreads) pick over a count histogram of NB bins (NB a
// multiple of kSelThreads), digits scanned from the top: the digit whose
// cumulative count (from the top) first reaches `want` (>= 1). Returns the
// digit, the count above it and its own count (all threads). If the
// histogram holds fewer than `want` keys, digit = -1. wg_load_desc reads the
// bins (thread t holds bins NB - 1 - t PER - j), wg_pick_vals picks from
// them.
template <int NB, bool COHERENT>
__device__ __forceinline__ void wg_load_desc(const uint32_t *hist, uint32_t (&v)[NB / kSelThreads]) {
  constexpr int PER = NB / kSelThreads;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = NB - 1 - (static_cast<int>(threadIdx.x) * PER + j);
    v[j] = COHERENT ? coherent_load_u32(&hist[d]) : hist[d];
  }
}
template <int NB>
__device__ void wg_pick_vals(const uint32_t (&v)[NB / kSelThreads], int64_t want, int &digit, int64_t &above,
                             int64_t &count, int64_t (&part)[kSelThreads / 64], int64_t (&res)[3]) {
  constexpr int PER = NB / kSelThreads;
  const int t = threadIdx.x, lane = lane_id(), w = t >> 6;
  uint64_t loc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) loc += v[j];
  const uint64_t incl = wave_scan_u64(loc);
  if (lane == 63) part[w] = static_cast<int64_t>(incl);
  if (t == 0) res[0] = -1;
  __syncthreads();
  int64_t base = 0;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i)
    if (i < w) base += part[i];
  int64_t cum = base + static_cast<int64_t>(incl - loc);  // keys in higher digits
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (cum < want && cum + static_cast<int64_t>(v[j]) >= want) {
      res[0] = NB - 1 - (t * PER + j);
      res[1] = cum;
      res[2] = v[j];
    }
    cum += v[j];
  }
  __syncthreads();
  digit = static_cast<int>(res[0]);
  above = res[1];
  count = res[2];
  __syncthreads();  // part and res may be reused at once
}
template <int NB, bool COHERENT>
__device__ void wg_pick(const uint32_t *hist, int64_t want, int &digit, int64_t &above, int64_t &count,
                        int64_t (&part)[kSelThreads / 64], int64_t (&res)[3]) {
  uint32_t v[NB / kSelThreads];
  wg_load_desc<NB, COHERENT>(hist, v);
  wg_pick_vals<NB>(v, want, digit, above, count, part, res);
}

// The head's fill after digit 0, from its prefix total and its complete
// digit-0 histogram (bins as wg_load_desc reads them); the same in every
// thread, so every workgroup that needs it forms it.
__device__ ThreshState fill_state0(const uint32_t (&v0)[kHBins / kSelThreads], int64_t pref, int64_t budget,
                                   int64_t (&part)[kSelThreads / 64], int64_t (&res)[3]) {
  ThreshState ns{};
  const int64_t need = budget - pref;
  if (need <= 0) {
    ns.mode = kFillNone;
    return ns;
  }
  int d;
  int64_t above, count;
  wg_pick_vals<kHBins>(v0, need, d, above, count, part, res);
  if (d < 0) {  // fewer pairs outside the prefixes than the budget asks: all of them
    ns.mode = kFillThr;
    ns.thr = 0;
  } else {
    ns.b0 = d;
    ns.rem = need - above;
    if (count == ns.rem) {
      ns.mode = kFillThr;
      ns.thr = static_cast<uint64_t>(d) << 40;
    } else {
      ns.mode = kFillDigit0;
    }
  }
  return ns;
}

// A state formed in every thread, moved to scalar registers (the compiler
// cannot tell that values read back from LDS are the same in every lane).
__device__ __forceinline__ ThreshState uniform_state(const ThreshState &s) {
  ThreshState u;
  u.thr = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(s.thr >> 32))))
           << 32) |
          static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(s.thr))));
  u.rem = static_cast<int64_t>(
      (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint64_t>(s.rem) >> 32))))
       << 32) |
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(s.rem)))));
  u.mode = __builtin_amdgcn_readfirstlane(s.mode);
  u.b0 = __builtin_amdgcn_readfirstlane(s.b0);
  u.b1 = __builtin_amdgcn_readfirstlane(s.b1);
  u.pad = 0;
  return u;
}

// ... and after digit 1 (heads whose digit 0 is open), from the digit-1
// histogram of the pairs in b0 outside the prefixes.
__device__ ThreshState fill_state1(const ThreshState &s, const uint32_t (&v1)[kHBins / kSelThreads],
                                   int64_t (&part)[kSelThreads / 64], int64_t (&res)[3]) {
  if (s.mode != kFillDigit0) return s;
  int d;
  int64_t above, count;
  wg_pick_vals<kHBins>(v1, s.rem, d, above, count, part, res);
  ThreshState ns = s;
  ns.b1 = d;  // the rem pairs lie in digit 0's histogram, so d >= 0
  ns.rem = s.rem - above;
  if (count == ns.rem) {
    ns.mode = kFillThr;
    ns.thr = (static_cast<uint64_t>(s.b0) << 40) | (static_cast<uint64_t>(d) << 28);
  } else {
    ns.mode = kFillDigit1;
  }
  return ns;
}

// Per-head counters and histograms to zero before a selection; workgroup 0
// also clears the count of deferred rows.
__global__ void __launch_bounds__(256)
thresh_init_kernel(uint32_t *__restrict__ hist, ThreshCounters *__restrict__ ctr, int32_t *__restrict__ n_def) {
  const int h = blockIdx.x;
  uint32_t *hh = hist + static_cast<int64_t>(h) * 2 * kHBins;
  for (int i = threadIdx.x; i < 2 * kHBins; i += 256) hh[i] = 0;
  if (threadIdx.x == 0) {
    ctr[h].prefix_total = 0;
    ctr[h].done_emit = 0;
    ctr[h].cand = 0;
    ctr[h].nfix = 0;
    if (h == 0) *n_def = 0;
  }
}

// The lane index as a value the compiler cannot prove loop-invariant: taken
// once per row inside row loops, so per-register column numbers and masks are
// recomputed there rather than held in registers (or spilled) across them.
__device__ __forceinline__ int lane_opaque() {
  int l = lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

// Column lane + 64 r of a row held in registers exists. The dispatch picks
// KPL with 64 * KPL / 2 < nb, so only the upper half of the registers can
// reach past the row's end.
template <int KPL>
__device__ __forceinline__ bool col_live(int r, int lane, int nb) {
  return r < KPL / 2 || lane + 64 * r < nb;
}

// The scores of a row as raw float bits, column lane + 64 r in register r,
// through a buffer resource spanning exactly the row: the hardware's range
// check returns 0 (+0.0, masked with col_live) past the row's end, so every
// load is issued unconditionally and a wave's loads of a row are all in
// flight together.
// `row` is the same for the whole wave (taken from its first lane, so that
// the resource lives in scalar registers).
template <int KPL>
__device__ __forceinline__ void load_row_bits(const float *__restrict__ row, int nb, uint32_t (&raw)[KPL],
                                              int lane) {
  const uint64_t a = reinterpret_cast<uint64_t>(row);
  const uint64_t au = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32))) << 32) |
                      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void *>(au), 0, __builtin_amdgcn_readfirstlane(nb * static_cast<int>(sizeof(float))), 0x00020000);
#pragma unroll
  for (int r = 0; r < KPL; ++r)
    raw[r] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, (lane + 64 * r) * 4, 0, 0));
}

// One wave's LDS for the row search: mass and count of each digit-0 bin of
// the row's window, slot s holding the bin s below the row's top bin; slot
// kWin gathers every lower bin (mass and count in arrays of their own: the per-column atomics of one
// instruction then spread over the most banks); then the boundary bin's
// columns for the register sort.
struct RowWin {
  unsigned long long pk[kWin + 1];
  uint32_t cand[kSortMax];
};

// Every key of a digit-0 bin shares its exponent e and the top 3 significand
// bits m3, so the bin's exact 2^-62 mass is fixed by its count and the sum
// of its keys' low 20 significand bits: for e >= 88 (p >= 2^-39, where the
// fixed-point value p 2^62 is an integer) it is the significand sum
// (count (8 + m3) 2^20 + low-bit sum) times 2^(e - 88). A window slot packs
// both sums in one 64-bit LDS word, count above bit 32 (a row's low-bit sum
// stays below 2^30), so one atomic per column builds it.
constexpr uint32_t kBinE88 = (1u << 11) | (88u << 3);  // digit 0 of the smallest key with e = 88
__device__ __forceinline__ uint64_t bin_mass(uint64_t pk, uint32_t bin) {
  const uint32_t cnt = static_cast<uint32_t>(pk >> 32);
  const uint64_t sig = static_cast<uint64_t>(cnt) * ((8u + (bin & 7u)) << 20) + static_cast<uint32_t>(pk);
  return sig << (((bin >> 3) & 0xFFu) - 88u);
}

// Exact boundary key of the shortest prefix by an MSB-first radix search
// (digits of up to 8 bits, 2^-62 fixed-point mass histograms in `mh`), for
// rows whose boundary bin holds more columns than the register sort takes or
// lies below the window; ends once one key is left under the fixed digits.
// The search starts below key bit top0 with the bits above it fixed to those
// of thr0 and A0 the mass of the keys above that prefix (thr0 = 0, top0 =
// 31, A0 = 0: from the top). Returns the boundary key value.
template <int KPL>
__device__ uint32_t radix_boundary(const uint32_t (&key)[KPL], int nb, int lane, uint64_t target,
                                   uint64_t *mh, uint32_t thr0, int top0, uint64_t A0) {
  uint32_t thr = thr0;
  uint64_t A = A0;
  int top = top0;
#pragma unroll 1
  while (top >= 0) {
    const int width = min(8, top + 1);
    const int lo = top - width + 1;
    const uint32_t pmask = top >= 31 ? 0u : ~((2u << top) - 1u);
#pragma unroll
    for (int j = 0; j < 4; ++j) mh[lane * 4 + j] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (col_live<KPL>(r, lane, nb) && (key[r] & pmask) == thr)
        atomicAdd(reinterpret_cast<unsigned long long *>(&mh[(key[r] >> lo) & ((1u << width) - 1u)]),
                  static_cast<unsigned long long>(fixed62(key[r])));
    __builtin_amdgcn_wave_barrier();
    // lane l holds digits 255 - 4l - j (j = 0..3): lanes run from the top
    uint64_t v[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = mh[255 - 4 * lane - j];
      loc += v[j];
    }
    const uint64_t c = A + wave_scan_u64(loc) - loc;  // mass of the digits above this lane's
    int jhit = 4;
    uint64_t above_d = 0, run = c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // highest digit of the lane that reaches the target
      if (jhit == 4 && run + v[j] >= target) {
        jhit = j;
        above_d = run;
      }
      run += v[j];
    }
    const uint64_t hit = __ballot(jhit < 4);
    const int srcl = hit ? __builtin_ctzll(hit) : 63;  // the crossing lies in the first lane that reaches it
    const int jsel = hit ? __builtin_amdgcn_readlane(jhit, srcl) : 3;
    const uint32_t d = 255u - 4u * static_cast<uint32_t>(srcl) - static_cast<uint32_t>(jsel);
    thr |= d << lo;
    A = readlane_u64(above_d, srcl);
    top = lo - 1;
    __builtin_amdgcn_wave_barrier();
    if (top >= 0) {
      // keys left under the new prefix; the boundary key is one of them
      const uint32_t qmask = ~((2u << top) - 1u);
      int left = 0;
      uint32_t only = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        const bool m = col_live<KPL>(r, lane, nb) && (key[r] & qmask) == thr;
        const uint64_t b = __ballot(m);
        if (b != 0 && left == 0)
          only = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key[r]), __builtin_ctzll(b)));
        left += popc64(b);
      }
      if (left == 1) {
        thr = only;
        top = -1;
      }
    }
  }
  return thr;
}

// Row prefixes. One wave per row at a time, each wave walking `rpw`
// consecutive rows of one head (few registers, so that many waves hide the
// loads of each other's rows): the threshold key K_I such that T_I is exactly the
// columns with key64 >= K_I. One pass of LDS atomics (one per column)
// builds, over a window of up to kWin digit-0 bins below the row's largest
// key (bins of keys p >= 2^-39), the count and the exact 2^-62 fixed-point
// mass of each bin (see bin_mass); the scan from the top finds the bin where
// the cumulative mass reaches tau, whose columns (at most kSortMax) are then
// sorted in registers by key64 and scanned, which fixes the boundary column.
// The bins' counts (the boundary bin's part outside the prefix) feed global
// digit 0 of the columns outside the prefixes. Rows whose boundary bin holds
// more columns, or lies below the window, are listed for thresh_fix_kernel.
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_row_kernel(const float *__restrict__ S, int nb, int rpw, uint64_t target,
                  uint64_t *__restrict__ row_thr, uint32_t *__restrict__ hist,
                  ThreshCounters *__restrict__ ctr, int32_t *__restrict__ fix_rows) {
  __shared__ RowWin win[kSelThreads / 64];
  __shared__ uint32_t h0[kHBins / 2];  // digit-0 bins 2048.. (real keys)
  __shared__ int s_cnt[kSelThreads / 64];
  const int h = blockIdx.y;
  const int w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kHBins / 2; i += kSelThreads) h0[i] = 0;
  __syncthreads();
  RowWin &R = win[w];
  const int I0 = (blockIdx.x * (kSelThreads / 64) + w) * rpw;
  const int I1 = min(I0 + rpw, nb);
  const int64_t hrow = static_cast<int64_t>(h) * nb;
  int cnt_w = 0;
  for (int I = I0; I < I1; ++I) {
    const int lane = lane_opaque();
    uint32_t key[KPL];
    load_row_bits<KPL>(S + (hrow + I) * nb, nb, key, lane);
    uint32_t kmax = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      key[r] = mass_key(key[r]);  // columns past the end read +0.0: never above a real key
      kmax = max(kmax, key[r]);
    }
    kmax = wave_max_u32(kmax);
    const uint32_t ktop = kmax | 0xFFFFFu;  // (ktop - key) >> 20: bins below the top bin
    const int bmax = static_cast<int>(kmax >> 20);
#pragma unroll
    for (int q = 0; q < 4; ++q) R.pk[4 * lane + q] = 0;
    if (lane == 0) R.pk[kWin] = 0;
    // window slots 0 .. qlim - 1 (bins of keys with e >= 88); every lower
    // key goes to slot kWin
    const int qlim = min(max(bmax - static_cast<int>(kBinE88) + 1, 0), kWin);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (col_live<KPL>(r, lane, nb)) {  // (columns past the end would all hit one address)
        const uint32_t raw = (ktop - key[r]) >> 20;
        const uint32_t q = raw < static_cast<uint32_t>(qlim) ? raw : static_cast<uint32_t>(kWin);
        atomicAdd(&R.pk[q], (1ull << 32) | (key[r] & 0xFFFFFu));
      }
    __builtin_amdgcn_wave_barrier();
    // lane l holds window slots 4l + q (q = 0..3): lanes run from the top
    uint64_t mv[4], mloc = 0;
    uint32_t cv[4], cloc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sl = 4 * lane + q;
      const uint64_t pk = R.pk[sl];
      cv[q] = static_cast<uint32_t>(pk >> 32);
      mv[q] = sl < qlim ? bin_mass(pk, static_cast<uint32_t>(bmax - sl)) : 0ull;
      mloc += mv[q];
      cloc += cv[q];
    }
    const uint32_t under_cnt = static_cast<uint32_t>(R.pk[kWin] >> 32);
    const uint64_t mincl = wave_scan_u64(mloc);
    const uint64_t wtotal = readlane_u64(mincl, 63);  // (the mass below the window is not formed)
    uint64_t K = 0;
    int cnt = 0;
    int sc = kWin + 1;  // window slot holding the prefix boundary (kWin + 1: none)
    int sub = 0;        // that slot's columns inside the prefix
    bool fix = false;
    int fix_bin = -1;   // a crowded boundary bin handed to the fix pass
    if (target == 0) {
      // An empty prefix already reaches the threshold; keep the best block
      // (the lowest column among equal best scores).
      uint32_t jmin = 0xFFFFFFFFu;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        const uint64_t b = __ballot(key[r] == kmax && col_live<KPL>(r, lane, nb));
        if (b != 0 && jmin == 0xFFFFFFFFu) jmin = static_cast<uint32_t>(__builtin_ctzll(b) + 64 * r);
      }
      K = key64(kmax, jmin);
      cnt = 1;
      sc = 0;
      sub = 1;
    } else if (wtotal < target) {
      if (under_cnt == 0) {
        K = 0;  // the whole row
        cnt = nb;
      } else {
        fix = true;  // the boundary (or the row's end) lies below the window
      }
    } else {
      // first window slot (from the top) where the cumulative mass reaches the target
      const uint32_t cincl = wave_scan_u32(cloc);
      uint64_t run = mincl - mloc, above = 0;
      uint32_t crun = cincl - cloc, cabove = 0, cd = 0;
      int qhit = 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (qhit == 4 && run + mv[q] >= target) {
          qhit = q;
          above = run;
          cabove = crun;
          cd = cv[q];
        }
        run += mv[q];
        crun += cv[q];
      }
      const uint64_t hitm = __ballot(qhit < 4);
      const int srcl = hitm ? __builtin_ctzll(hitm) : 0;
      const int c_d = __builtin_amdgcn_readlane(static_cast<int>(cd), srcl);
      if (hitm == 0 || c_d > kSortMax) {
        fix = true;  // below the window, or a crowded boundary bin (whose digit 0 the fix pass takes as known)
        if (hitm != 0) fix_bin = bmax - (4 * srcl + __builtin_amdgcn_readlane(qhit, srcl));
      } else {
        sc = 4 * srcl + __builtin_amdgcn_readlane(qhit, srcl);
        const uint32_t d = static_cast<uint32_t>(bmax - sc);
        const uint64_t A = readlane_u64(above, srcl);
        // the bin's columns, one per lane, as (key bits 19..0, 1023 - column):
        // descending order is key64 order
        int n = 0;
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          const bool m = col_live<KPL>(r, lane, nb) && (key[r] >> 20) == d;
          const uint64_t b = __ballot(m);
          if (m) R.cand[n + popc64(b & lanemask_lt())] = ((key[r] & 0xFFFFFu) << 10) | static_cast<uint32_t>(1023 - lane - 64 * r);
          n += popc64(b);
        }
        __builtin_amdgcn_wave_barrier();
        uint32_t v = lane < c_d ? R.cand[lane] : 0u;
        v = sort_desc(v, c_d);
        const uint64_t f = lane < c_d ? fixed62((d << 20) | (v >> 10)) : 0ull;
        const uint64_t reach = A + wave_scan_u64(f);
        const uint64_t hb = __ballot(lane < c_d && reach >= target);
        const int hit = hb ? __builtin_ctzll(hb) : c_d - 1;  // always found for valid scores
        const uint32_t vh = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), hit));
        K = key64((d << 20) | (vh >> 10), 1023u - (vh & 1023u));
        cnt = __builtin_amdgcn_readlane(static_cast<int>(cabove), srcl) + hit + 1;
        sub = hit + 1;
      }
    }
    if (fix) {
      // (row, crowded boundary bin + 1 or 0) packed as I | bin' << 11 (I < 1024)
      if (lane == 0) fix_rows[hrow + atomicAdd(&ctr[h].nfix, 1)] = I | ((fix_bin + 1) << 11);
    } else {
      // global digit 0 of the columns outside the prefix: whole window bins
      // below the boundary bin, the boundary bin's columns after the
      // boundary, and, unless the whole row is the prefix, every column
      // below the window
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int sl = 4 * lane + q;
        const uint32_t o = sl > sc ? cv[q] : (sl == sc ? cv[q] - static_cast<uint32_t>(sub) : 0u);
        if (o != 0) atomicAdd(&h0[(bmax - sl) & (kHBins / 2 - 1)], o);
      }
      if (under_cnt != 0 && K != 0) {
        const uint32_t wlo = static_cast<uint32_t>(bmax - qlim + 1) << 20;  // lowest key of the window
#pragma unroll
        for (int r = 0; r < KPL; ++r)
          if (col_live<KPL>(r, lane, nb) && key[r] < wlo) atomicAdd(&h0[(key[r] >> 20) & (kHBins / 2 - 1)], 1u);
      }
      if (lane == 0) row_thr[hrow + I] = K;
      cnt_w += cnt;
    }
    __builtin_amdgcn_wave_barrier();  // the window is cleared for the next row only after every read
  }
  if (lane_id() == 0) s_cnt[w] = cnt_w;
  __syncthreads();
  uint32_t *gh = hist + static_cast<int64_t>(h) * 2 * kHBins + kHBins / 2;
  for (int i = threadIdx.x; i < kHBins / 2; i += kSelThreads) {
    const uint32_t c = h0[i];
    if (c) atomicAdd(&gh[i], c);
  }
  if (threadIdx.x == 0) {
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) sum += s_cnt[i];
    if (sum) atomicAdd(&ctr[h].prefix_total, static_cast<unsigned long long>(sum));
  }
}

// Rows the row pass listed (boundary below the window or in a crowded bin,
// or a row whose mass inside the window falls short of tau with columns
// below it): the whole row when its total mass falls short, else the
// full-key radix search; then digit 0 of their columns outside the prefix.
// (The passes after it pick the fill's boundary digits themselves.)
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_fix_kernel(const float *__restrict__ S, int nb, uint64_t target, uint64_t *__restrict__ row_thr,
                  uint32_t *__restrict__ hist, ThreshCounters *__restrict__ ctr,
                  const int32_t *__restrict__ fix_rows) {
  __shared__ uint64_t mh[kSelThreads / 64][256];
  __shared__ uint32_t h0[kHBins / 2];
  __shared__ int s_cnt[kSelThreads / 64];
  const int h = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int64_t hrow = static_cast<int64_t>(h) * nb;
  const int n_fix = ctr[h].nfix;
  uint32_t *gh = hist + static_cast<int64_t>(h) * 2 * kHBins;
  if (n_fix > 0) {
    for (int i = threadIdx.x; i < kHBins / 2; i += kSelThreads) h0[i] = 0;
    __syncthreads();
    int cnt_w = 0;
    for (int i = blockIdx.x * (kSelThreads / 64) + w; i < n_fix; i += gridDim.x * (kSelThreads / 64)) {
      const int e = fix_rows[hrow + i];
      const int I = e & 2047, fb = (e >> 11) - 1;  // fb: the crowded boundary bin, or -1
      uint32_t key[KPL];
      load_row_bits<KPL>(S + (hrow + I) * nb, nb, key, lane);
      uint64_t tot = 0;  // all of the row (fb < 0), or the mass above bin fb
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        key[r] = mass_key(key[r]);
        tot += (col_live<KPL>(r, lane, nb) && static_cast<int>(key[r] >> 20) > fb) ? fixed62(key[r]) : 0ull;
      }
      tot = wave_total_u64(tot);
      if (fb < 0 && tot < target) {  // the whole row is its prefix
        if (lane == 0) row_thr[hrow + I] = 0;
        cnt_w += nb;
        continue;
      }
      const uint32_t thr = radix_boundary<KPL>(key, nb, lane, target, mh[w], fb < 0 ? 0u : static_cast<uint32_t>(fb) << 20,
                                               fb < 0 ? 31 : 19, fb < 0 ? 0ull : tot);
      uint64_t above = 0;
      int n_above = 0, n_tie = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        const bool live = col_live<KPL>(r, lane, nb);
        above += (live && key[r] > thr) ? fixed62(key[r]) : 0ull;
        n_above += popc64(__ballot(live && key[r] > thr));
        n_tie += popc64(__ballot(live && key[r] == thr));
      }
      above = readlane_u64(wave_scan_u64(above), 63);
      // every tie has the same score, hence the same fixed-point value
      const uint64_t f_tie = fixed62(thr);
      const uint64_t need = target - above;  // > 0 and <= n_tie * f_tie
      const uint64_t n_take = (n_tie == 1 || need <= f_tie) ? 1ull : (need + f_tie - 1) / f_tie;
      // the n_take-th tie in column order (lowest columns first)
      uint32_t jcut = 0;
      int seen = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        uint64_t b = __ballot(col_live<KPL>(r, lane, nb) && key[r] == thr);
        const int pcn = popc64(b);
        if (seen < static_cast<int>(n_take) && seen + pcn >= static_cast<int>(n_take)) {
          for (int k = static_cast<int>(n_take) - seen - 1; k > 0; --k) b &= b - 1;  // drop lower ties
          jcut = static_cast<uint32_t>(__builtin_ctzll(b) + 64 * r);
        }
        seen += pcn;
      }
      const uint64_t K = key64(thr, jcut);
#pragma unroll
      for (int r = 0; r < KPL; ++r)
        if (col_live<KPL>(r, lane, nb) && key64(key[r], lane + 64 * r) < K)
          atomicAdd(&h0[(key[r] >> 20) & (kHBins / 2 - 1)], 1u);
      if (lane == 0) row_thr[hrow + I] = K;
      cnt_w += n_above + static_cast<int>(n_take);
    }
    if (lane == 0) s_cnt[w] = cnt_w;
    __syncthreads();
    for (int i = threadIdx.x; i < kHBins / 2; i += kSelThreads) {
      const uint32_t c = h0[i];
      if (c) atomicAdd(&gh[kHBins / 2 + i], c);
    }
    if (threadIdx.x == 0) {
      int sum = 0;
#pragma unroll
      for (int i = 0; i < kSelThreads / 64; ++i) sum += s_cnt[i];
      if (sum) atomicAdd(&ctr[h].prefix_total, static_cast<unsigned long long>(sum));
    }
  }
}

// Rows of a wave's walk in pairs: both rows' scores are loaded into fresh
// registers before either is worked on, so every wave keeps two rows of
// loads in flight (a buffer carried from one iteration to the next would be
// copied, and waited for, at the loop's back edge). `next()` yields the rows
// in order (-1 at the end); `work(key, I)` takes a row's order keys.
template <int KPL, class Next, class Work>
__device__ __forceinline__ void walk_row_pairs(const float *__restrict__ Sh, int nb, Next next, Work work) {
  for (int ra = next(); ra >= 0; ra = next()) {
    const int rb = next();
    const int lane = lane_opaque();
    uint32_t A[KPL], B[KPL];
    load_row_bits<KPL>(Sh + static_cast<int64_t>(ra) * nb, nb, A, lane);
    load_row_bits<KPL>(Sh + static_cast<int64_t>(rb >= 0 ? rb : ra) * nb, nb, B, lane);
#pragma unroll
    for (int r = 0; r < KPL; ++r) A[r] = mass_key(A[r]);
    work(A, ra);
    if (rb < 0) break;
#pragma unroll
    for (int r = 0; r < KPL; ++r) B[r] = mass_key(B[r]);
    work(B, rb);
  }
}

// Second pass: each workgroup picks the fill's digit 0 from the complete
// digit-0 histogram (the head's first one stores it for the emitting pass);
// heads whose boundary digit 0 is open then count digit 1
// of the pairs outside the prefixes in the boundary digit 0. Rows whose
// prefix boundary lies in a lower digit 0 than b0 hold every pair of b0
// inside their prefix and are not read.
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_hist1_kernel(const float *__restrict__ S, int nb, int rpw, int64_t budget,
                    const uint64_t *__restrict__ row_thr, uint32_t *__restrict__ hist,
                    const ThreshCounters *__restrict__ ctr, ThreshState *__restrict__ st) {
  __shared__ uint32_t h1[kHBins];
  __shared__ int64_t s_part[kSelThreads / 64], s_res[3];
  const int h = blockIdx.y;
  ThreshState s;
  {
    uint32_t v0[kHBins / kSelThreads];
    wg_load_desc<kHBins, false>(hist + static_cast<int64_t>(h) * 2 * kHBins, v0);
    s = uniform_state(fill_state0(v0, static_cast<int64_t>(ctr[h].prefix_total), budget, s_part, s_res));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) st[h] = s;  // for the emitting pass
  if (s.mode != kFillDigit0) return;
  const int w = threadIdx.x >> 6, lane = lane_id();
  for (int i = threadIdx.x; i < kHBins; i += kSelThreads) h1[i] = 0;
  __syncthreads();
  const int I0 = (blockIdx.x * (kSelThreads / 64) + w) * rpw;
  const int n = max(min(rpw, nb - I0), 0);
  const int64_t hrow = static_cast<int64_t>(h) * nb;
  const uint64_t Kl = lane < n ? row_thr[hrow + I0 + lane] : 0ull;  // the wave's row thresholds
  uint64_t rest = __ballot(lane < n && static_cast<int>(Kl >> 52) >= s.b0);
  const uint32_t b0 = static_cast<uint32_t>(s.b0);
  walk_row_pairs<KPL>(
      S + (hrow + I0) * nb, nb,
      [&]() {
        if (!rest) return -1;
        const int r = __builtin_ctzll(rest);
        rest &= rest - 1;
        return r;
      },
      [&](const uint32_t(&key)[KPL], int i) {
        const int ln = lane_opaque();
        const uint64_t K = readlane_u64(Kl, i);
        if (static_cast<uint32_t>(K >> 52) == b0) {  // the prefix boundary is in b0: compare with it
#pragma unroll
          for (int r = 0; r < KPL; ++r)
            if (col_live<KPL>(r, ln, nb) && (key[r] >> 20) == b0 && key64(key[r], ln + 64 * r) < K)
              atomicAdd(&h1[(key[r] >> 8) & (kHBins - 1)], 1u);
        } else {  // every column of b0 lies outside the prefix
#pragma unroll
          for (int r = 0; r < KPL; ++r)
            if (col_live<KPL>(r, ln, nb) && (key[r] >> 20) == b0) atomicAdd(&h1[(key[r] >> 8) & (kHBins - 1)], 1u);
        }
      });
  __syncthreads();
  uint32_t *gh = hist + (static_cast<int64_t>(h) * 2 + 1) * kHBins;
  for (int i = threadIdx.x; i < kHBins; i += kSelThreads) {
    const uint32_t c = h1[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Writes the row's list: the columns with key64 >= E, ascending; returns the
// count. Entries past the count are not written.
template <int KPL>
__device__ __forceinline__ int emit_row(const uint32_t (&key)[KPL], int nb, uint64_t E, int32_t *out, int lane) {
  int before = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const uint32_t j = static_cast<uint32_t>(lane + 64 * r);
    const bool sel = col_live<KPL>(r, lane, nb) && key64(key[r], j) >= E;
    const uint64_t b = __ballot(sel);
    if (sel) out[before + popc64(b & lanemask_lt())] = static_cast<int32_t>(j);
    before += popc64(b);
  }
  return before;
}

// Emitting pass: rows whose selection is settled are written now; rows
// holding pairs of the open boundary digits (b0, b1) outside their prefix
// are deferred (listed in def_rows) and those pairs collected; the head's
// last workgroup then resolves the exact fill threshold among the collected
// pairs (or, if more than kCandCap were found, among all of the head's pairs
// in that digit pair).
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_emit_kernel(const float *__restrict__ S, int nb, int rpw, const uint64_t *__restrict__ row_thr,
                   const uint32_t *__restrict__ hist,
                   ThreshState *__restrict__ st, ThreshCounters *__restrict__ ctr,
                   uint64_t *__restrict__ cand, int32_t *__restrict__ def_rows, int32_t *__restrict__ n_def,
                   int32_t *__restrict__ kv_idx, int32_t *__restrict__ kv_cnt, int max_kv) {
  __shared__ uint32_t rh[1024];
  __shared__ int s_last;
  __shared__ int64_t s_part[kSelThreads / 64], s_res[3];
  const int h = blockIdx.y;
  // the fill's state after digit 0 (from the digit-1 pass), then digit 1
  ThreshState s = st[h];
  if (s.mode == kFillDigit0) {
    uint32_t v1[kHBins / kSelThreads];
    wg_load_desc<kHBins, false>(hist + (static_cast<int64_t>(h) * 2 + 1) * kHBins, v1);
    s = uniform_state(fill_state1(s, v1, s_part, s_res));
  }
  const int w = threadIdx.x >> 6;
  const uint64_t hi01 = (static_cast<uint64_t>(s.b0) << 12) | static_cast<uint64_t>(s.b1);  // gkey >> 28 of the open digits
  const int I0 = (blockIdx.x * (kSelThreads / 64) + w) * rpw;
  const int n = max(min(rpw, nb - I0), 0);
  const int64_t hrow = static_cast<int64_t>(h) * nb;
  const uint64_t Kl = lane_id() < n ? row_thr[hrow + I0 + lane_id()] : 0ull;  // the wave's row thresholds
  int nxt = 0;
  walk_row_pairs<KPL>(
      S + (hrow + I0) * nb, nb, [&]() { return nxt < n ? nxt++ : -1; },
      [&](const uint32_t(&key)[KPL], int i) {
        const int lane = lane_opaque();
        const int I = I0 + i;
        const int64_t row = hrow + I;
        const uint64_t K = readlane_u64(Kl, i);
        uint64_t E = K;
        if (s.mode == kFillThr) {
          E = min(K, row_fill_key(s.thr, I, nb));
        } else if (s.mode == kFillDigit1) {
          // Pairs of the open digits are the columns with key bits 31..8
          // equal to hi01; those outside the prefix (key64 < K) make the row
          // wait for the exact fill threshold. Everything above the open
          // digits is filled.
          E = min(K, row_fill_key((hi01 + 1) << 28, I, nb));
          if ((K >> 40) >= hi01) {  // otherwise the open digits lie inside the prefix
            bool any = false;
#pragma unroll
            for (int r = 0; r < KPL; ++r)
              any |= col_live<KPL>(r, lane, nb) && (key[r] >> 8) == static_cast<uint32_t>(hi01);
            if (__any(any)) {
              int n = 0;
#pragma unroll
              for (int r = 0; r < KPL; ++r)
                n += popc64(__ballot(col_live<KPL>(r, lane, nb) && (key[r] >> 8) == static_cast<uint32_t>(hi01) &&
                                     key64(key[r], lane + 64 * r) < K));
              if (n != 0) {
                // defer the row and collect its boundary pairs (a few per head, typically)
                int base = 0;
                if (lane == 0) {
                  base = atomicAdd(&ctr[h].cand, n);
                  def_rows[atomicAdd(n_def, 1)] = static_cast<int32_t>(row);
                }
                base = __builtin_amdgcn_readlane(base, 0);
                uint64_t *dst = cand + static_cast<int64_t>(h) * kCandCap;
#pragma unroll
                for (int r = 0; r < KPL; ++r) {
                  const uint32_t j = static_cast<uint32_t>(lane + 64 * r);
                  const bool c = col_live<KPL>(r, lane, nb) && (key[r] >> 8) == static_cast<uint32_t>(hi01) &&
                                 key64(key[r], j) < K;
                  const uint64_t b = __ballot(c);
                  const int pos = base + popc64(b & lanemask_lt());
                  if (c && pos < kCandCap)
                    __hip_atomic_store(&dst[pos], gkey(key[r], static_cast<uint32_t>(I * nb) + j), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                  base += popc64(b);
                }
                return;
              }
            }
          }
        }
        const int c = emit_row<KPL>(key, nb, E, kv_idx + row * max_kv, lane);
        if (lane == 0) kv_cnt[row] = c;
      });
  if (s.mode != kFillDigit1) return;
  last_arrival_wait();
  if (threadIdx.x == 0) s_last = atomicAdd(&ctr[h].done_emit, 1) == static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!s_last) return;
  // Resolve the rem-th largest global key among the open digits' pairs:
  // radix over its remaining 28 bits (10, 10 and 8), from the collected
  // pairs, or from all the head's pairs when too many were collected.
  const int n_cand = __hip_atomic_load(&ctr[h].cand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool from_list = n_cand <= kCandCap;
  const uint64_t *lst = cand + static_cast<int64_t>(h) * kCandCap;
  const int64_t n_items = from_list ? n_cand : static_cast<int64_t>(nb) * nb;
  uint64_t pref = hi01 << 28;  // fixed bits so far
  uint64_t pmask = ~((1ull << 28) - 1);
  int64_t rem = s.rem;
#pragma unroll 1
  for (int round = 0; round < 3; ++round) {
    const int lo = round == 0 ? 18 : (round == 1 ? 8 : 0);
    const uint32_t dmask = round == 2 ? 0xFFu : 0x3FFu;
    for (int i = threadIdx.x; i < 1024; i += kSelThreads) rh[i] = 0;
    __syncthreads();
    for (int64_t it = threadIdx.x; it < n_items; it += kSelThreads) {
      uint64_t g;
      if (from_list) {
        g = coherent_load_u64(&lst[it]);
      } else {
        const int Ir = static_cast<int>(it / nb), j = static_cast<int>(it - static_cast<int64_t>(Ir) * nb);
        const uint32_t ok = mass_key(__float_as_uint(S[(hrow + Ir) * nb + j]));
        g = gkey(ok, static_cast<uint32_t>(it));
        const bool in_p = key64(ok, static_cast<uint32_t>(j)) >= row_thr[hrow + Ir];
        if (in_p || (g >> 28) != hi01) continue;
      }
      if ((g & pmask) == pref) atomicAdd(&rh[static_cast<uint32_t>(g >> lo) & dmask], 1u);
    }
    __syncthreads();
    int d;
    int64_t above, count;
    wg_pick<1024, false>(rh, rem, d, above, count, s_part, s_res);
    pref |= static_cast<uint64_t>(d) << lo;
    pmask |= static_cast<uint64_t>(dmask) << lo;
    rem -= above;
    if (count == rem) break;  // the whole digit is taken: lower bits zero
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    ThreshState ns = s;
    ns.mode = kFillThr;
    ns.thr = pref;
    st[h] = ns;
  }
}

// Rows deferred by the emitting pass, now that the fill threshold is exact:
// the waves of a small grid walk the deferred-row list.
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_emit_deferred_kernel(const float *__restrict__ S, int nb, const uint64_t *__restrict__ row_thr,
                            const ThreshState *__restrict__ st, const int32_t *__restrict__ def_rows,
                            const int32_t *__restrict__ n_def, int32_t *__restrict__ kv_idx,
                            int32_t *__restrict__ kv_cnt, int max_kv) {
  const int n = *n_def;
  const int waves = gridDim.x * (kSelThreads / 64);
  for (int i = blockIdx.x * (kSelThreads / 64) + (threadIdx.x >> 6); i < n; i += waves) {
    const int lane = lane_opaque();
    const int row = def_rows[i];
    const int h = row / nb, I = row - h * nb;
    const uint64_t E = min(row_thr[row], row_fill_key(st[h].thr, I, nb));
    uint32_t key[KPL];
    load_row_bits<KPL>(S + static_cast<int64_t>(row) * nb, nb, key, lane);
#pragma unroll
    for (int r = 0; r < KPL; ++r) key[r] = mass_key(key[r]);
    const int c = emit_row<KPL>(key, nb, E, kv_idx + static_cast<int64_t>(row) * max_kv, lane);
    if (lane == 0) kv_cnt[row] = c;
  }
}

// LVSA lists: one wave per query tile, frames strided over the lanes.
template <int FPL>
__global__ void __launch_bounds__(64)
lvsa_kernel(int T, int tiles, int C, int T_per, int step, int32_t *__restrict__ kv_idx,
            int32_t *__restrict__ kv_cnt, int max_kv) {
  const int I = blockIdx.x;
  const int t = I / tiles;
  const int lane = lane_id();
  const int rot = step % T_per;
  int n_anchor = 0;
  bool anchor[FPL];
  uint32_t near[FPL];  // larger = nearer: ~(|f - t| * 2^16 + f), 0 = not a candidate
#pragma unroll
  for (int r = 0; r < FPL; ++r) {
    const int f = lane + 64 * r;
    anchor[r] = f < T && (f % T_per) == rot;
    n_anchor += popc64(__ballot(anchor[r]));
    near[r] = (f < T && !anchor[r]) ? ~static_cast<uint32_t>((abs(f - t) << 16) | f) : 0u;
  }
  const int n_other = T - n_anchor;
  const int nw = min(max(C - n_anchor, 1), n_other);
  const uint32_t thr = nw > 0 ? kth_largest<FPL>(near, nw) : 0xFFFFFFFFu;
  bool sel[FPL];
#pragma unroll
  for (int r = 0; r < FPL; ++r) sel[r] = anchor[r] || (nw > 0 && near[r] != 0u && near[r] >= thr);
  // frames ascending -> their tiles ascending
  int32_t *out = kv_idx + static_cast<int64_t>(I) * max_kv;
  int before = 0;
#pragma unroll
  for (int r = 0; r < FPL; ++r) {
    const uint64_t b = __ballot(sel[r]);
    if (sel[r]) {
      const int pos = (before + popc64(b & lanemask_lt())) * tiles;
      const int f = lane + 64 * r;
      for (int j = 0; j < tiles; ++j) out[pos + j] = f * tiles + j;
    }
    before += popc64(b);
  }
  if (lane == 0) kv_cnt[I] = before * tiles;
}

// DynamicRad radial window (static-ratio mode): width w(d) of the window in
// a key frame at temporal distance d, and its first tile for query tile j.
__device__ __forceinline__ int radial_width_dev(int d, int P, int lam_tiles) {
  const int k = 31 - __clz(d + 1);  // floor(log2(d + 1))
  const int w = (P + (1 << k) - 1) >> k;
  return min(P, max(max(w, lam_tiles), 1));
}
__device__ __forceinline__ int radial_lo(int j, int w, int P) { return min(max(j - w / 2, 0), P - w); }

// Static radial lists: one wave per query tile, key frames over the lanes;
// a frame's window lands after the windows of all earlier frames.
__global__ void __launch_bounds__(64)
radial_kernel(int T, int P, int lam_tiles, int32_t *__restrict__ kv_idx, int32_t *__restrict__ kv_cnt,
              int max_kv) {
  const int I = blockIdx.x;
  const int t = I / P, j = I - t * P;
  const int lane = lane_id();
  int32_t *out = kv_idx + static_cast<int64_t>(I) * max_kv;
  int before = 0;
  for (int f0 = 0; f0 < T; f0 += 64) {
    const int f = f0 + lane;
    const int w = f < T ? radial_width_dev(abs(t - f), P, lam_tiles) : 0;
    // inclusive scan of w over the lanes
    int incl = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (f < T) {
      const int lo = radial_lo(j, w, P);
      const int pos = before + incl - w;
      for (int q = 0; q < w; ++q) out[pos + q] = f * P + lo + q;
    }
    before += __shfl(incl, 63, 64);
  }
  if (lane == 0) kv_cnt[I] = before;
}

// Dynamic radial lists: one wave per (head, query tile): the row's best
// logit, the float threshold best - delta, then every block inside the
// radial window or at/above the threshold, ascending.
__global__ void __launch_bounds__(256)
radial_dyn_kernel(const float *__restrict__ S, int rows, int nb, int T, int P, int lam_tiles,
                  float delta, int32_t *__restrict__ kv_idx, int32_t *__restrict__ kv_cnt, int max_kv) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = lane_id();
  const int I = row % nb;
  const int t = I / P, j = I - t * P;
  const float *srow = S + static_cast<int64_t>(row) * nb;
  float m = -INFINITY;
  for (int J = lane; J < nb; J += 64) m = fmaxf(m, srow[J]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float thr = m - delta;
  int32_t *out = kv_idx + static_cast<int64_t>(row) * max_kv;
  int before = 0;
  for (int J0 = 0; J0 < nb; J0 += 64) {
    const int J = J0 + lane;
    bool keep = false;
    if (J < nb) {
      const int f = J / P, jj = J - f * P;
      const int w = radial_width_dev(abs(t - f), P, lam_tiles);
      const int lo = radial_lo(j, w, P);
      keep = (jj >= lo && jj < lo + w) || srow[J] >= thr;
    }
    const uint64_t b = __ballot(keep);
    if (keep) out[before + popc64(b & lanemask_lt())] = J;
    before += popc64(b);
  }
  if (lane == 0) kv_cnt[row] = before;
}

}  // namespace hsa

namespace hsa_host {

static int keys_per_lane(int n) { return (n + 63) / 64; }

// THRESH_GLOBAL workspace: row thresholds, one row list (per head the rows
// for the full-key search, then, once that pass is done, the deferred rows)
// and the deferred-row count, the two digit histograms, per-head state and
// counters, collected boundary pairs.
struct ThreshWs {
  size_t row_thr, rows_list, n_def, hist, state, ctr, cand, total;
};
static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }
static ThreshWs thresh_ws(int nh, int nb) {
  const size_t rows = static_cast<size_t>(nh) * nb;
  ThreshWs w;
  w.row_thr = 0;
  w.rows_list = align256(w.row_thr + rows * sizeof(uint64_t));
  w.n_def = align256(w.rows_list + rows * sizeof(int32_t));
  w.hist = align256(w.n_def + sizeof(int32_t));
  w.state = align256(w.hist + static_cast<size_t>(nh) * 2 * hsa::kHBins * sizeof(uint32_t));
  w.ctr = align256(w.state + static_cast<size_t>(nh) * sizeof(hsa::ThreshState));
  w.cand = align256(w.ctr + static_cast<size_t>(nh) * sizeof(hsa::ThreshCounters));
  w.total = align256(w.cand + static_cast<size_t>(nh) * hsa::kCandCap * sizeof(uint64_t));
  return w;
}

size_t select_ws_bytes(int nh, int nb, int mode) {
  if (mode != HSA_SELECT_THRESH_GLOBAL) return 0;
  return thresh_ws(nh, nb).total;
}

#define HSA_KPL_DISPATCH(n, KERNEL, GRID, BLOCK, ...)                                           \
  do {                                                                                         \
    const int kpl_ = keys_per_lane(n);                                                         \
    if (kpl_ <= 1) hipLaunchKernelGGL((KERNEL<1>), GRID, BLOCK, 0, stream, __VA_ARGS__);       \
    else if (kpl_ <= 2) hipLaunchKernelGGL((KERNEL<2>), GRID, BLOCK, 0, stream, __VA_ARGS__);  \
    else if (kpl_ <= 4) hipLaunchKernelGGL((KERNEL<4>), GRID, BLOCK, 0, stream, __VA_ARGS__);  \
    else if (kpl_ <= 8) hipLaunchKernelGGL((KERNEL<8>), GRID, BLOCK, 0, stream, __VA_ARGS__);  \
    else hipLaunchKernelGGL((KERNEL<16>), GRID, BLOCK, 0, stream, __VA_ARGS__);                \
  } while (0)

hsa_status_t launch_select(const float *S, int nh, int nb, const hsa_select_params_t *p,
                           int32_t *kv_idx, int32_t *kv_cnt, int max_kv, void *ws,
                           hipStream_t stream) {
  const int rows_per_wg = hsa::kSelThreads / 64;
  if (p->mode == HSA_SELECT_TOPK) {
    const int rows = nh * nb;
    const dim3 grid((rows + rows_per_wg - 1) / rows_per_wg);
    HSA_KPL_DISPATCH(nb, hsa::topk_kernel, grid, dim3(hsa::kSelThreads), S, rows, nb, p->k,
                     kv_idx, kv_cnt, max_kv);
  } else if (p->mode == HSA_SELECT_THRESH_GLOBAL) {
    const int rows = nh * nb;
    char *base = static_cast<char *>(ws);
    const ThreshWs lay = thresh_ws(nh, nb);
    uint64_t *row_thr = reinterpret_cast<uint64_t *>(base + lay.row_thr);
    int32_t *fix_rows = reinterpret_cast<int32_t *>(base + lay.rows_list);  // row and fix passes
    int32_t *def_rows = fix_rows;                                                // emitting passes
    int32_t *n_def = reinterpret_cast<int32_t *>(base + lay.n_def);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base + lay.hist);
    hsa::ThreshState *st = reinterpret_cast<hsa::ThreshState *>(base + lay.state);
    hsa::ThreshCounters *ctr = reinterpret_cast<hsa::ThreshCounters *>(base + lay.ctr);
    uint64_t *cand = reinterpret_cast<uint64_t *>(base + lay.cand);
    const double one = 4611686018427387904.0;  // 2^62
    const uint64_t target = static_cast<uint64_t>(floor(p->tau * one));
    const int64_t budget = static_cast<int64_t>(floor(p->budget_ratio * (static_cast<double>(nb) * nb) + 0.5));
    // Rows per wave. The row pass and the emitting pass compute enough per
    // row to want every wave the chip holds (about 20 per CU at their
    // register use, in one round of workgroups); the digit-1 count is bound
    // by its per-workgroup histogram flush (device atomics), so it runs
    // fewer, longer-lived workgroups (about 8 waves per CU), which measured
    // faster at the 720p shape.
    auto grid_of = [&](int waves_per_cu, int &rpw) {
      rpw = std::min(64, std::max(1, (rows + 256 * waves_per_cu - 1) / (256 * waves_per_cu)));
      return dim3((nb + rows_per_wg * rpw - 1) / (rows_per_wg * rpw), nh);
    };
    int rpw_row, rpw_h1, rpw_emit;
    const dim3 rgrid = grid_of(20, rpw_row), hgrid = grid_of(8, rpw_h1), egrid = grid_of(20, rpw_emit);
    hipLaunchKernelGGL(hsa::thresh_init_kernel, dim3(nh), dim3(256), 0, stream, hist, ctr, n_def);
    HSA_KPL_DISPATCH(nb, hsa::thresh_row_kernel, rgrid, dim3(hsa::kSelThreads), S, nb, rpw_row, target,
                     row_thr, hist, ctr, fix_rows);
    HSA_KPL_DISPATCH(nb, hsa::thresh_fix_kernel, dim3(std::min(8, (nb + rows_per_wg - 1) / rows_per_wg), nh),
                     dim3(hsa::kSelThreads), S, nb, target, row_thr, hist, ctr, fix_rows);
    HSA_KPL_DISPATCH(nb, hsa::thresh_hist1_kernel, hgrid, dim3(hsa::kSelThreads), S, nb, rpw_h1, budget, row_thr,
                     hist, ctr, st);
    HSA_KPL_DISPATCH(nb, hsa::thresh_emit_kernel, egrid, dim3(hsa::kSelThreads), S, nb, rpw_emit, row_thr, hist, st,
                     ctr, cand, def_rows, n_def, kv_idx, kv_cnt, max_kv);
    const dim3 dgrid(std::min(256, (rows + rows_per_wg - 1) / rows_per_wg));
    HSA_KPL_DISPATCH(nb, hsa::thresh_emit_deferred_kernel, dgrid, dim3(hsa::kSelThreads), S, nb, row_thr, st,
                     def_rows, n_def, kv_idx, kv_cnt, max_kv);
  } else if (p->mode == HSA_SELECT_LVSA) {
    HSA_KPL_DISPATCH(p->frames, hsa::lvsa_kernel, dim3(nb), dim3(64), p->frames,
                     p->tiles_per_frame, p->C, p->T_per, p->step, kv_idx, kv_cnt, max_kv);
  } else {
    const int lam_tiles = static_cast<int>(ceil(p->lam * p->tiles_per_frame));
    if (p->mode == HSA_SELECT_RADIAL) {
      hipLaunchKernelGGL(hsa::radial_kernel, dim3(nb), dim3(64), 0, stream, p->frames,
                         p->tiles_per_frame, lam_tiles, kv_idx, kv_cnt, max_kv);
    } else {
      const int rows = nh * nb;
      hipLaunchKernelGGL(hsa::radial_dyn_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, S, rows,
                         nb, p->frames, p->tiles_per_frame, lam_tiles, static_cast<float>(p->delta),
                         kv_idx, kv_cnt, max_kv);
    }
  }
  return check_launch("hsa_select");
}

}  // namespace hsa_host

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
//                Per row: MSB-first radix search (digits of up to 8 bits
//                below the row's common key prefix, exact 2^-62 fixed-point
//                mass histograms in LDS) for the boundary key of the
//                shortest prefix reaching tau. Per head: an MSB-first radix
//                select of the remaining budget among the pairs outside the
//                row prefixes over 52-bit pair keys (score order key, then
//                the lower linear index): digit 0 counted while the row
//                prefixes are found, digit 1 in a second pass over the
//                scores, the last 28 bits resolved among the few pairs left
//                in the boundary digits, which the emitting pass collects;
//                each pass's last workgroup of a head picks that head's
//                digit, so there is no pass per digit and no pick launch.
//                Lists are written in the emitting pass (rows holding
//                boundary pairs right after the resolve).
//  Every mode writes kv_cnt and the first kv_cnt entries of each list;
//  entries past the count are not written.
//  LVSA          LVSA section 2, A(t) = G_s u W(t): rotating anchors plus the
//                nearest non-anchor frames; tile lists shared by all heads.
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

// floor(p * 2^62) exactly, for 0 <= p < 2 (p's bits, non-negative).
__device__ __forceinline__ uint64_t fixed62(uint32_t bits) {
  if (bits & 0x80000000u) return 0;  // negative scores are invalid input
  const int e = static_cast<int>(bits >> 23);
  if (e == 0) return 0;              // subnormals are below 2^-126
  const uint64_t m = (bits & 0x7FFFFFu) | 0x800000u;
  const int sh = e - 88;             // p * 2^62 = m * 2^(e - 150 + 62)
  if (sh >= 0) return sh >= 40 ? (1ull << 63) : (m << sh);
  return (-sh >= 24) ? 0 : (m >> (-sh));
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
constexpr int kHBits = 12;
constexpr int kHBins = 1 << kHBits;
constexpr int kCandCap = 2048;  // collected boundary pairs per head
constexpr int kRowsPerWave = 8;  // rows each wave of the threshold passes walks (histograms and
                                 // the arrival count are paid once per workgroup of 32 rows)

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
  int32_t done_row, done_hist1, done_emit;  // finished workgroups per pass
  int32_t cand;                             // collected boundary pairs
};

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

// Whole-workgroup (kSelThreads) pick over a count histogram of NB bins (NB a
// multiple of kSelThreads), digits scanned from the top: the digit whose
// cumulative count (from the top) first reaches `want` (>= 1). Returns the
// digit, the count above it and its own count (all threads). If the
// histogram holds fewer than `want` keys, digit = -1.
template <int NB, bool COHERENT>
__device__ void wg_pick(const uint32_t *hist, int64_t want, int &digit, int64_t &above, int64_t &count,
                        int64_t (&part)[kSelThreads / 64], int64_t (&res)[3]) {
  constexpr int PER = NB / kSelThreads;
  const int t = threadIdx.x, lane = lane_id(), w = t >> 6;
  uint32_t v[PER];
  uint64_t loc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = NB - 1 - (t * PER + j);
    v[j] = COHERENT ? coherent_load_u32(&hist[d]) : hist[d];
    loc += v[j];
  }
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
}

// Per-head counters and histograms to zero before a selection.
__global__ void __launch_bounds__(256)
thresh_init_kernel(uint32_t *__restrict__ hist, ThreshCounters *__restrict__ ctr) {
  const int h = blockIdx.x;
  uint32_t *hh = hist + static_cast<int64_t>(h) * 2 * kHBins;
  for (int i = threadIdx.x; i < 2 * kHBins; i += 256) hh[i] = 0;
  if (threadIdx.x == 0) {
    ctr[h].prefix_total = 0;
    ctr[h].done_row = ctr[h].done_hist1 = ctr[h].done_emit = 0;
    ctr[h].cand = 0;
  }
}

// Row prefixes. One wave per row at a time (each wave walks kRowsPerWave
// rows of one head; a workgroup holds four such waves): the
// threshold key K_I such that T_I is exactly the columns with key64 >= K_I,
// found by an MSB-first radix search over the order keys with exact 2^-62
// fixed-point mass histograms in LDS (digits of up to 8 bits starting at the
// highest bit in which the row's keys differ, one histogram per half-wave,
// ending once one key is left under the fixed digits). The columns outside
// the prefix are counted by global digit 0; the head's last workgroup then
// picks the boundary digit of the fill.
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_row_kernel(const float *__restrict__ S, int nb, uint64_t target, int64_t budget,
                  uint64_t *__restrict__ row_thr, uint32_t *__restrict__ hist,
                  ThreshCounters *__restrict__ ctr, ThreshState *__restrict__ st) {
  __shared__ uint64_t row_hist[kSelThreads / 64][2][256];
  __shared__ uint32_t h0[kHBins];
  __shared__ int s_cnt[kSelThreads / 64];
  __shared__ int s_last;
  __shared__ int64_t s_part[kSelThreads / 64], s_res[3];
  const int h = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = lane_id();
  for (int i = threadIdx.x; i < kHBins; i += kSelThreads) h0[i] = 0;
  __syncthreads();
  int cnt_w = 0;
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int I = (blockIdx.x * (kSelThreads / 64) + w) * kRowsPerWave + rr;
    if (I >= nb) break;
    int cnt = 0;
    const int64_t row = static_cast<int64_t>(h) * nb + I;
    const float *src = S + row * nb;
    uint32_t key[KPL];
    uint64_t fx[KPL];
    uint64_t total = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int j = lane + 64 * r;
      const uint32_t bits = (j < nb) ? __float_as_uint(src[j]) : 0u;
      key[r] = (j < nb) ? float_order_key(__uint_as_float(bits)) : 0u;
      fx[r] = (j < nb) ? fixed62(bits) : 0ull;
      total += fx[r];
    }
    total = wave_total_u64(total);
    uint64_t K;
    if (target == 0) {
      // An empty prefix already reaches the threshold; keep the best block
      // (the lowest column among equal best scores).
      uint32_t kmax = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) kmax = max(kmax, key[r]);
      kmax = wave_max_u32(kmax);
      uint32_t jmin = 0xFFFFFFFFu;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        const uint64_t b = __ballot(key[r] == kmax && lane + 64 * r < nb);
        if (b != 0 && jmin == 0xFFFFFFFFu) jmin = static_cast<uint32_t>(__builtin_ctzll(b) + 64 * r);
      }
      K = key64(kmax, jmin);
      cnt = 1;
    } else if (total < target) {
      K = 0;  // the whole row
      cnt = nb;
    } else {
      // Largest order key thr whose tail sum F(thr) = sum_{key >= thr} fx
      // still reaches the target: the boundary value of the shortest prefix.
      // With the higher bits fixed to P and A = mass of the keys above P,
      // the next digit is the highest d with A + (mass of digits >= d under
      // P) >= target.
      uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
      for (int r = 0; r < KPL; ++r)
        if (lane + 64 * r < nb) {
          kmax = max(kmax, key[r]);
          kmin = min(kmin, key[r]);
        }
      kmax = wave_max_u32(kmax);
      kmin = wave_min_u32(kmin);
      uint64_t(*mh)[256] = row_hist[w];
      uint64_t *mine = mh[lane >> 5];
      int top = 31 - static_cast<int>(__builtin_clz((kmax ^ kmin) | 1u));  // highest differing bit
      if (kmax == kmin) top = -1;                                        // one distinct key
      uint32_t thr = top >= 31 ? 0u : (kmax & ~((2u << top) - 1u));       // the common bits
      if (top < 0) thr = kmax;
      uint64_t A = 0;
#pragma unroll 1
      while (top >= 0) {
        const int width = min(8, top + 1);
        const int lo = top - width + 1;
        const uint32_t pmask = top >= 31 ? 0u : ~((2u << top) - 1u);
#pragma unroll
        for (int j = 0; j < 4; ++j) mh[0][lane * 4 + j] = mh[1][lane * 4 + j] = 0;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < KPL; ++r)
          if (lane + 64 * r < nb && (key[r] & pmask) == thr)
            atomicAdd(reinterpret_cast<unsigned long long *>(&mine[(key[r] >> lo) & ((1u << width) - 1u)]),
                      static_cast<unsigned long long>(fx[r]));
        __builtin_amdgcn_wave_barrier();
        // lane l holds digits 255 - 4l - j (j = 0..3): lanes run from the top
        uint64_t v[4], loc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = mh[0][255 - 4 * lane - j] + mh[1][255 - 4 * lane - j];
          loc += v[j];
        }
        const uint64_t c = A + wave_scan_u64(loc) - loc;  // mass of the digits above this lane's
        int jhit = 4;
#pragma unroll
        for (int j = 3; j >= 0; --j)  // highest digit of the lane that reaches the target
          if (c + v[0] + (j >= 1 ? v[1] : 0) + (j >= 2 ? v[2] : 0) + (j >= 3 ? v[3] : 0) >= target) jhit = j;
        const uint64_t hit = __ballot(jhit < 4);
        const int srcl = __builtin_ctzll(hit);  // the crossing lies in the first lane that reaches it
        const int jsel = __builtin_amdgcn_readlane(jhit, srcl);
        uint64_t above_d = c;                   // mass of the digits above the chosen one
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < jhit) above_d += v[j];
        const uint32_t ad_lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(above_d)), srcl));
        const uint32_t ad_hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(above_d >> 32)), srcl));
        const uint32_t d = 255u - 4u * static_cast<uint32_t>(srcl) - static_cast<uint32_t>(jsel);
        thr |= d << lo;
        A = (static_cast<uint64_t>(ad_hi) << 32) | ad_lo;
        top = lo - 1;
        __builtin_amdgcn_wave_barrier();
        if (top >= 0) {
          // keys left under the new prefix; the boundary key is one of them
          const uint32_t qmask = ~((2u << top) - 1u);
          int left = 0, lr = 0;
          uint64_t lb = 0;
#pragma unroll
          for (int r = 0; r < KPL; ++r) {
            const uint64_t b = __ballot(lane + 64 * r < nb && (key[r] & qmask) == thr);
            if (b != 0 && left == 0) {
              lb = b;
              lr = r;
            }
            left += popc64(b);
          }
          if (left == 1) {
#pragma unroll
            for (int r = 0; r < KPL; ++r)
              if (r == lr) thr = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key[r]), __builtin_ctzll(lb)));
            top = -1;
          }
        }
      }
      uint64_t above = 0;
      int n_above = 0, n_tie = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        above += (key[r] > thr) ? fx[r] : 0ull;
        n_above += popc64(__ballot(key[r] > thr));
        n_tie += popc64(__ballot(key[r] == thr && lane + 64 * r < nb));
      }
      above = wave_total_u64(above);
      // every tie has the same score, hence the same fixed-point value
      const uint64_t f_tie = fixed62(order_key_bits(thr));
      const uint64_t need = target - above;  // > 0 and <= n_tie * f_tie
      const uint64_t n_take = (n_tie == 1 || need <= f_tie) ? 1ull : (need + f_tie - 1) / f_tie;
      // the n_take-th tie in column order (lowest columns first)
      uint32_t jcut = 0;
      int seen = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        uint64_t b = __ballot(key[r] == thr && lane + 64 * r < nb);
        const int pc = popc64(b);
        if (seen < static_cast<int>(n_take) && seen + pc >= static_cast<int>(n_take)) {
          for (int k = static_cast<int>(n_take) - seen - 1; k > 0; --k) b &= b - 1;  // drop lower ties
          jcut = static_cast<uint32_t>(__builtin_ctzll(b) + 64 * r);
        }
        seen += pc;
      }
      K = key64(thr, jcut);
      cnt = n_above + static_cast<int>(n_take);
    }
    // global digit 0 of the columns outside the prefix
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const uint32_t j = static_cast<uint32_t>(lane + 64 * r);
      if (j < static_cast<uint32_t>(nb) && key64(key[r], j) < K) atomicAdd(&h0[key[r] >> 20], 1u);
    }
    if (lane == 0) row_thr[row] = K;
    cnt_w += cnt;
  }
  if (lane == 0) s_cnt[w] = cnt_w;
  __syncthreads();
  uint32_t *gh = hist + static_cast<int64_t>(h) * 2 * kHBins;
  for (int i = threadIdx.x; i < kHBins; i += kSelThreads) {
    const uint32_t c = h0[i];
    if (c) atomicAdd(&gh[i], c);
  }
  if (threadIdx.x == 0) {
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) sum += s_cnt[i];
    atomicAdd(&ctr[h].prefix_total, static_cast<unsigned long long>(sum));
  }
  // the head's last workgroup picks the boundary digit of the fill
  last_arrival_wait();
  if (threadIdx.x == 0) s_last = atomicAdd(&ctr[h].done_row, 1) == static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!s_last) return;
  const int64_t pref = static_cast<int64_t>(__hip_atomic_load(&ctr[h].prefix_total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const int64_t need = budget - pref;
  ThreshState ns{};
  if (need <= 0) {
    ns.mode = kFillNone;
  } else {
    int d;
    int64_t above, count;
    wg_pick<kHBins, true>(gh, need, d, above, count, s_part, s_res);
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
  }
  if (threadIdx.x == 0) st[h] = ns;
}

// Second pass (heads whose boundary digit 0 is open): count digit 1 of the
// pairs outside the prefixes in the boundary digit 0; the head's last
// workgroup picks the boundary digit 1.
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_hist1_kernel(const float *__restrict__ S, int nb, const uint64_t *__restrict__ row_thr,
                    uint32_t *__restrict__ hist, ThreshCounters *__restrict__ ctr,
                    ThreshState *__restrict__ st) {
  __shared__ uint32_t h1[kHBins];
  __shared__ int s_last;
  __shared__ int64_t s_part[kSelThreads / 64], s_res[3];
  const int h = blockIdx.y;
  const ThreshState s = st[h];
  if (s.mode != kFillDigit0) return;  // uniform across the head's workgroups
  const int w = threadIdx.x >> 6, lane = lane_id();
  for (int i = threadIdx.x; i < kHBins; i += kSelThreads) h1[i] = 0;
  __syncthreads();
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int I = (blockIdx.x * (kSelThreads / 64) + w) * kRowsPerWave + rr;
    if (I >= nb) break;
    const int64_t row = static_cast<int64_t>(h) * nb + I;
    const uint64_t K = row_thr[row];
    const float *src = S + row * nb;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const uint32_t j = static_cast<uint32_t>(lane + 64 * r);
      if (j < static_cast<uint32_t>(nb)) {
        const uint32_t ok = float_order_key(src[j]);
        if (key64(ok, j) < K && static_cast<int>(ok >> 20) == s.b0) atomicAdd(&h1[(ok >> 8) & (kHBins - 1)], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t *gh = hist + (static_cast<int64_t>(h) * 2 + 1) * kHBins;
  for (int i = threadIdx.x; i < kHBins; i += kSelThreads) {
    const uint32_t c = h1[i];
    if (c) atomicAdd(&gh[i], c);
  }
  last_arrival_wait();
  if (threadIdx.x == 0) s_last = atomicAdd(&ctr[h].done_hist1, 1) == static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!s_last) return;
  int d;
  int64_t above, count;
  wg_pick<kHBins, true>(gh, s.rem, d, above, count, s_part, s_res);
  ThreshState ns = s;
  ns.b1 = d;  // the rem pairs lie in digit 0's histogram, so d >= 0
  ns.rem = s.rem - above;
  if (count == ns.rem) {
    ns.mode = kFillThr;
    ns.thr = (static_cast<uint64_t>(s.b0) << 40) | (static_cast<uint64_t>(d) << 28);
  } else {
    ns.mode = kFillDigit1;
  }
  if (threadIdx.x == 0) st[h] = ns;
}

// Emitting pass: rows whose selection is settled are written now; rows
// holding pairs of the open boundary digits (b0, b1) are deferred and their
// boundary pairs collected; the head's last workgroup then resolves the
// exact fill threshold among the collected pairs (or, if more than
// kCandCap were found, among all of the head's pairs in that digit pair).
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_emit_kernel(const float *__restrict__ S, int nb, const uint64_t *__restrict__ row_thr,
                   ThreshState *__restrict__ st, ThreshCounters *__restrict__ ctr,
                   uint64_t *__restrict__ cand, int32_t *__restrict__ deferred,
                   int32_t *__restrict__ kv_idx, int32_t *__restrict__ kv_cnt, int max_kv) {
  __shared__ uint32_t rh[1024];
  __shared__ int s_last;
  __shared__ int64_t s_part[kSelThreads / 64], s_res[3];
  const int h = blockIdx.y;
  const ThreshState s = st[h];
  const int w = threadIdx.x >> 6, lane = lane_id();
  const uint64_t hi01 = (static_cast<uint64_t>(s.b0) << 12) | static_cast<uint64_t>(s.b1);  // gkey >> 28 of the open digits
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int I = (blockIdx.x * (kSelThreads / 64) + w) * kRowsPerWave + rr;
    if (I >= nb) break;
    const int64_t row = static_cast<int64_t>(h) * nb + I;
    const uint64_t K = row_thr[row];
    const float *src = S + row * nb;
    bool sel[KPL], cnd[KPL];
    uint64_t gk[KPL];
    bool any = false;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const uint32_t j = static_cast<uint32_t>(lane + 64 * r);
      sel[r] = cnd[r] = false;
      gk[r] = 0;
      if (j < static_cast<uint32_t>(nb)) {
        const uint32_t ok = float_order_key(src[j]);
        const bool in_p = key64(ok, j) >= K;
        gk[r] = gkey(ok, static_cast<uint32_t>(I * nb) + j);
        if (s.mode == kFillThr) {
          sel[r] = in_p || gk[r] >= s.thr;
        } else if (s.mode == kFillDigit1) {
          sel[r] = in_p || (gk[r] >> 28) > hi01;
          cnd[r] = !in_p && (gk[r] >> 28) == hi01;
        } else {
          sel[r] = in_p;
        }
      }
      any |= cnd[r];
    }
    const bool deferred_row = __any(any);
    if (lane == 0) deferred[row] = deferred_row ? 1 : 0;
    if (deferred_row) {
      // collect this row's boundary pairs (a few per head, typically)
      int n = 0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) n += popc64(__ballot(cnd[r]));
      int base = 0;
      if (lane == 0) base = atomicAdd(&ctr[h].cand, n);
      base = __builtin_amdgcn_readlane(base, 0);
      uint64_t *dst = cand + static_cast<int64_t>(h) * kCandCap;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        const uint64_t b = __ballot(cnd[r]);
        const int pos = base + popc64(b & lanemask_lt());
        if (cnd[r] && pos < kCandCap) __hip_atomic_store(&dst[pos], gk[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        base += popc64(b);
      }
    } else {
      const int c = emit_sel<KPL>(sel, kv_idx + row * max_kv);
      if (lane == 0) kv_cnt[row] = c;
    }
  }
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
  const int los[3] = {18, 8, 0}, wid[3] = {10, 10, 8};
  for (int round = 0; round < 3; ++round) {
    const int lo = los[round];
    const uint32_t dmask = (1u << wid[round]) - 1u;
    for (int i = threadIdx.x; i < 1024; i += kSelThreads) rh[i] = 0;
    __syncthreads();
    for (int64_t it = threadIdx.x; it < n_items; it += kSelThreads) {
      uint64_t g;
      if (from_list) {
        g = coherent_load_u64(&lst[it]);
      } else {
        const int Ir = static_cast<int>(it / nb), j = static_cast<int>(it - static_cast<int64_t>(Ir) * nb);
        const uint32_t ok = float_order_key(S[(static_cast<int64_t>(h) * nb + Ir) * nb + j]);
        g = gkey(ok, static_cast<uint32_t>(it));
        const bool in_p = key64(ok, static_cast<uint32_t>(j)) >= row_thr[static_cast<int64_t>(h) * nb + Ir];
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

// Rows deferred by the emitting pass, now that the fill threshold is exact.
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_emit_deferred_kernel(const float *__restrict__ S, int nh, int nb,
                            const uint64_t *__restrict__ row_thr, const ThreshState *__restrict__ st,
                            const int32_t *__restrict__ deferred, int32_t *__restrict__ kv_idx,
                            int32_t *__restrict__ kv_cnt, int max_kv) {
  const int row = blockIdx.x * (kSelThreads / 64) + (threadIdx.x >> 6);
  if (row >= nh * nb || !deferred[row]) return;
  const int h = row / nb, I = row - h * nb;
  const int lane = lane_id();
  const uint64_t K = row_thr[row];
  const uint64_t thr = st[h].thr;
  const float *src = S + static_cast<int64_t>(row) * nb;
  bool sel[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const uint32_t j = static_cast<uint32_t>(lane + 64 * r);
    sel[r] = false;
    if (j < static_cast<uint32_t>(nb)) {
      const uint32_t ok = float_order_key(src[j]);
      sel[r] = key64(ok, j) >= K || gkey(ok, static_cast<uint32_t>(I * nb) + j) >= thr;
    }
  }
  const int c = emit_sel<KPL>(sel, kv_idx + static_cast<int64_t>(row) * max_kv);
  if (lane == 0) kv_cnt[row] = c;
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

// THRESH_GLOBAL workspace: row thresholds, deferred-row flags, the two
// digit histograms, per-head state and counters, collected boundary pairs.
struct ThreshWs {
  size_t row_thr, deferred, hist, state, ctr, cand, total;
};
static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }
static ThreshWs thresh_ws(int nh, int nb) {
  const size_t rows = static_cast<size_t>(nh) * nb;
  ThreshWs w;
  w.row_thr = 0;
  w.deferred = align256(w.row_thr + rows * sizeof(uint64_t));
  w.hist = align256(w.deferred + rows * sizeof(int32_t));
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
    int32_t *deferred = reinterpret_cast<int32_t *>(base + lay.deferred);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base + lay.hist);
    hsa::ThreshState *st = reinterpret_cast<hsa::ThreshState *>(base + lay.state);
    hsa::ThreshCounters *ctr = reinterpret_cast<hsa::ThreshCounters *>(base + lay.ctr);
    uint64_t *cand = reinterpret_cast<uint64_t *>(base + lay.cand);
    const double one = 4611686018427387904.0;  // 2^62
    const uint64_t target = static_cast<uint64_t>(floor(p->tau * one));
    const int64_t budget = static_cast<int64_t>(floor(p->budget_ratio * (static_cast<double>(nb) * nb) + 0.5));
    const int rows_per_tg = rows_per_wg * hsa::kRowsPerWave;
    const dim3 hgrid((nb + rows_per_tg - 1) / rows_per_tg, nh);
    hipLaunchKernelGGL(hsa::thresh_init_kernel, dim3(nh), dim3(256), 0, stream, hist, ctr);
    HSA_KPL_DISPATCH(nb, hsa::thresh_row_kernel, hgrid, dim3(hsa::kSelThreads), S, nb, target, budget,
                     row_thr, hist, ctr, st);
    HSA_KPL_DISPATCH(nb, hsa::thresh_hist1_kernel, hgrid, dim3(hsa::kSelThreads), S, nb, row_thr, hist,
                     ctr, st);
    HSA_KPL_DISPATCH(nb, hsa::thresh_emit_kernel, hgrid, dim3(hsa::kSelThreads), S, nb, row_thr, st, ctr,
                     cand, deferred, kv_idx, kv_cnt, max_kv);
    const dim3 grid((rows + rows_per_wg - 1) / rows_per_wg);
    HSA_KPL_DISPATCH(nb, hsa::thresh_emit_deferred_kernel, grid, dim3(hsa::kSelThreads), S, nh, nb,
                     row_thr, st, deferred, kv_idx, kv_cnt, max_kv);
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

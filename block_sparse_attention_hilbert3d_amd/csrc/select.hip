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
//                shortest prefix reaching tau. Per head: an MSB-first
//                radix select (11-bit digits, count histograms) of the
//                remaining budget among pairs outside the row prefixes, a
//                small pick kernel choosing each digit; the search stops as
//                soon as the boundary digit's pairs are all taken (three
//                passes unless scores tie exactly). Then a compaction pass.
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

// Writes the columns with sel[r] set, ascending, -1 after; returns the count.
template <int KPL>
__device__ __forceinline__ int emit_row(const bool (&sel)[KPL], int32_t *out, int max_kv) {
  const int lane = lane_id();
  int before = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const uint64_t b = __ballot(sel[r]);
    if (sel[r]) out[before + popc64(b & lanemask_lt())] = lane + 64 * r;
    before += popc64(b);
  }
  for (int p = before + lane; p < max_kv; p += 64) out[p] = -1;
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
  const int cnt = emit_row<KPL>(sel, kv_idx + static_cast<int64_t>(row) * max_kv, max_kv);
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

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 64-bit ranking key of column j with order key ok: larger = better.
__device__ __forceinline__ uint64_t key64(uint32_t ok, uint32_t j) {
  return (static_cast<uint64_t>(ok) << 32) | (0xFFFFFFFFu - j);
}

// Per row: the threshold key K_I such that the row prefix T_I is exactly the
// columns with key64 >= K_I; and |T_I|.
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_row_kernel(const float *__restrict__ S, int rows, int nb, uint64_t target,
                  uint64_t *__restrict__ row_thr, int32_t *__restrict__ row_cnt) {
  __shared__ uint64_t row_hist[kSelThreads / 64][2][256];
  const int row = blockIdx.x * (kSelThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = lane_id();
  const float *src = S + static_cast<int64_t>(row) * nb;
  uint32_t key[KPL];
  uint64_t fx[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane + 64 * r;
    const uint32_t bits = (j < nb) ? __float_as_uint(src[j]) : 0u;
    key[r] = (j < nb) ? float_order_key(__uint_as_float(bits)) : 0u;
    fx[r] = (j < nb) ? fixed62(bits) : 0ull;
  }
  uint64_t K;
  int cnt;
  uint64_t total = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) total += fx[r];
  total = wave_sum_u64(total);
  if (target == 0) {
    // An empty prefix already reaches the threshold; keep the best block.
    const uint32_t thr = kth_largest<KPL>(key, 1);
    uint32_t jmin = 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (key[r] == thr && lane + 64 * r < nb) jmin = min(jmin, static_cast<uint32_t>(lane + 64 * r));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) jmin = min(jmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(jmin), off, 64)));
    K = key64(thr, jmin);
    cnt = 1;
  } else if (total < target) {
    K = 0;  // the whole row
    cnt = nb;
  } else {
    // Largest order key thr whose tail sum F(thr) = sum_{key >= thr} fx
    // still reaches the target: the boundary value of the shortest prefix.
    // Radix search from the highest bit in which the row's keys differ (the
    // bits above it are common to every key), in digits of up to 8 bits:
    // with the higher bits fixed to P and A = mass of the keys above P, the
    // next digit is the highest d with A + (mass of digits >= d under P) >=
    // target. Each half-wave has its own histogram (half the atomic
    // contention); the search ends early once one key is left under P.
    uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (lane + 64 * r < nb) {
        kmax = max(kmax, key[r]);
        kmin = min(kmin, key[r]);
      }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), off, 64)));
      kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), off, 64)));
    }
    uint64_t(*mh)[256] = row_hist[threadIdx.x >> 6];
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
      uint64_t incl = loc;  // inclusive prefix over lanes (higher digits first)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint64_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      uint64_t c = A + incl - loc;  // mass of the digits above this lane's
      int jhit = 4;
#pragma unroll
      for (int j = 3; j >= 0; --j) {  // highest digit of the lane that reaches the target
        if (c + v[0] + (j >= 1 ? v[1] : 0) + (j >= 2 ? v[2] : 0) + (j >= 3 ? v[3] : 0) >= target) jhit = j;
      }
      const uint64_t hit = __ballot(jhit < 4);
      const int src = __builtin_ctzll(hit);  // the crossing lies in the first lane that reaches it
      const int jsel = __shfl(jhit, src, 64);
      uint64_t above_d = c;                  // mass of the digits above the chosen one
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < jhit) above_d += v[j];
      above_d = __shfl(above_d, src, 64);
      const uint32_t d = 255u - 4u * static_cast<uint32_t>(src) - static_cast<uint32_t>(jsel);
      thr |= d << lo;
      A = above_d;
      top = lo - 1;
      __builtin_amdgcn_wave_barrier();
      if (top >= 0) {
        // keys left under the new prefix; the boundary key is one of them
        const uint32_t qmask = ~((2u << top) - 1u);
        int left = 0;
        uint32_t only = 0;
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          const bool in = lane + 64 * r < nb && (key[r] & qmask) == thr;
          left += popc64(__ballot(in));
          if (in) only = key[r];
        }
        if (left == 1) {
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) only = max(only, static_cast<uint32_t>(__shfl_xor(static_cast<int>(only), off, 64)));
          thr = only;
          top = -1;
        }
      }
    }
    uint64_t above = 0;
    int n_above = 0;
    uint64_t f_tie = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      above += (key[r] > thr) ? fx[r] : 0ull;
      n_above += popc64(__ballot(key[r] > thr));
      if (key[r] == thr && lane + 64 * r < nb) f_tie = fx[r];
    }
    above = wave_sum_u64(above);
    // every tie has the same score, hence the same fixed-point value
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t o = __shfl_xor(f_tie, off, 64);
      f_tie = o > f_tie ? o : f_tie;
    }
    const uint64_t need = target - above;                  // > 0 and <= ties * f_tie
    const uint64_t n_ties = (need + f_tie - 1) / f_tie;    // ties taken, lowest columns first
    uint32_t jcut = 0xFFFFFFFFu;
    uint64_t seen = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const bool tie = key[r] == thr && lane + 64 * r < nb;
      const uint64_t b = __ballot(tie);
      const uint64_t rank = seen + popc64(b & lanemask_lt());
      if (tie && rank + 1 == n_ties) jcut = lane + 64 * r;
      seen += popc64(b);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) jcut = min(jcut, static_cast<uint32_t>(__shfl_xor(static_cast<int>(jcut), off, 64)));
    K = key64(thr, jcut);
    cnt = n_above + static_cast<int>(n_ties);
  }
  if (lane == 0) {
    row_thr[row] = K;
    row_cnt[row] = cnt;
  }
}

// Global fill: MSB-first radix select over 52-bit pair keys (score order key,
// then lower linear index first; nb <= 1024 so I*nb+J < 2^20) in 11-bit
// digits: three passes fix the score bits, two more break exact ties.
constexpr int kGDigit = 11;
constexpr int kGBins = 1 << kGDigit;
constexpr int kGKeyBits = 52;
constexpr int kGPasses = 5;  // 5 x 11 bits cover the 52-bit key

__host__ __device__ constexpr int gfill_hi(int pass) { return kGKeyBits - 1 - kGDigit * pass; }
__host__ __device__ constexpr int gfill_lo(int pass) { return gfill_hi(pass) - kGDigit + 1 > 0 ? gfill_hi(pass) - kGDigit + 1 : 0; }

struct GlobalState {
  uint64_t prefix;    // digits fixed so far; once done: the smallest selected key
  int64_t remaining;  // rank still to find among the keys matching prefix
  int32_t fill;       // 1 if the head adds pairs beyond its row prefixes
  int32_t active;     // 1 while digits remain to be searched
};

// Per head: budget minus the row prefixes' size; clears the pass histograms.
__global__ void __launch_bounds__(256)
gfill_init_kernel(const int32_t *__restrict__ row_cnt, int nb, int64_t budget,
                  GlobalState *__restrict__ st, uint32_t *__restrict__ hist) {
  __shared__ int64_t part[4];
  const int h = blockIdx.x;
  int64_t c = 0;
  for (int i = threadIdx.x; i < nb; i += 256) c += row_cnt[static_cast<int64_t>(h) * nb + i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  uint32_t *hh = hist + static_cast<int64_t>(h) * kGPasses * kGBins;
  for (int i = threadIdx.x; i < kGPasses * kGBins; i += 256) hh[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t t = part[0] + part[1] + part[2] + part[3];
    const int64_t rem = budget - t;
    st[h].prefix = 0;
    st[h].remaining = rem > 0 ? rem : 0;
    st[h].fill = rem > 0 ? 1 : 0;
    st[h].active = rem > 0 ? 1 : 0;
  }
}

// Global key of pair (I, J): order key of the score, then lower I*nb+J first
// (lin < 2^20).
__device__ __forceinline__ uint64_t gkey(uint32_t ok, uint32_t lin) {
  return (static_cast<uint64_t>(ok) << 20) | (0xFFFFFu - lin);
}

// One digit of the global radix select: every workgroup counts the digits
// of the matching keys outside the row prefixes (LDS histogram, then global
// atomics into this pass's histogram).
template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
gfill_hist_kernel(const float *__restrict__ S, int nb, int pass,
                  const uint64_t *__restrict__ row_thr, const GlobalState *__restrict__ st,
                  uint32_t *__restrict__ hist) {
  __shared__ uint32_t lh[kGBins];
  const int h = blockIdx.y;
  if (!st[h].active) return;  // uniform across the workgroup
  for (int i = threadIdx.x; i < kGBins; i += kSelThreads) lh[i] = 0;
  __syncthreads();
  const int hi = gfill_hi(pass), lo = gfill_lo(pass);
  const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
  const uint64_t prefix = st[h].prefix;
  const uint64_t himask = (pass == 0) ? 0ull : (~0ull << (hi + 1));
  const int I = blockIdx.x * (kSelThreads / 64) + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (I < nb) {
    const int64_t row = static_cast<int64_t>(h) * nb + I;
    const uint64_t K = row_thr[row];
    const float *src = S + row * nb;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int j = lane + 64 * r;
      if (j < nb) {
        const uint32_t ok = float_order_key(src[j]);
        if (key64(ok, j) < K) {  // not already in the row prefix
          const uint64_t g = gkey(ok, static_cast<uint32_t>(I * nb + j));
          if ((g & himask) == (prefix & himask)) atomicAdd(&lh[static_cast<uint32_t>(g >> lo) & dmask], 1u);
        }
      }
    }
  }
  __syncthreads();
  uint32_t *gh = hist + (static_cast<int64_t>(h) * kGPasses + pass) * kGBins;
  for (int i = threadIdx.x; i < kGBins; i += kSelThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Pick the digit that holds the remaining-th largest matching key (one
// workgroup per head, a scan from the top digit) and advance the state. The
// search is over once the picked digit's keys are all taken (count <=
// remaining) or the last digit is fixed.
__global__ void __launch_bounds__(kSelThreads)
gfill_pick_kernel(int pass, GlobalState *__restrict__ st, const uint32_t *__restrict__ hist) {
  __shared__ uint32_t part[kSelThreads];
  const int h = blockIdx.x;
  if (!st[h].active) return;
  const int hi = gfill_hi(pass), lo = gfill_lo(pass);
  const int nd = 1 << (hi - lo + 1);
  const uint64_t himask = (pass == 0) ? 0ull : (~0ull << (hi + 1));
  const uint64_t prefix = st[h].prefix;
  const int64_t rem = st[h].remaining;
  const uint32_t *gh = hist + (static_cast<int64_t>(h) * kGPasses + pass) * kGBins;
  // thread t owns digits nd-1-8t .. nd-8-8t (top digits first)
  constexpr int kPer = kGBins / kSelThreads;
  uint32_t v[kPer];
  uint32_t loc = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int d = nd - 1 - (threadIdx.x * kPer + j);
    v[j] = d >= 0 ? gh[d] : 0u;
    loc += v[j];
  }
  part[threadIdx.x] = loc;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {  // inclusive scan
    const uint32_t o = threadIdx.x >= off ? part[threadIdx.x - off] : 0u;
    __syncthreads();
    part[threadIdx.x] += o;
    __syncthreads();
  }
  const int64_t total = part[kSelThreads - 1];
  int64_t cum = static_cast<int64_t>(part[threadIdx.x]) - loc;  // keys in higher digits
  __syncthreads();  // every thread has read st[h] before it is rewritten
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int d = nd - 1 - (threadIdx.x * kPer + j);
    // the digit whose cumulative count first reaches rem; with fewer matching
    // keys than rem (all taken) the lowest digit
    const bool hit = (cum < rem && cum + v[j] >= rem) || (total < rem && d == 0);
    if (d >= 0 && hit) {
      const int64_t r = rem - cum;  // rank within digit d
      GlobalState ns;
      ns.prefix = (prefix & himask) | (static_cast<uint64_t>(d) << lo);
      ns.remaining = r;
      ns.fill = 1;
      // done: the smallest selected key is prefix with the lower bits zero
      ns.active = (static_cast<int64_t>(v[j]) <= r || lo == 0) ? 0 : 1;
      st[h] = ns;
    }
    cum += v[j];
  }
}

template <int KPL>
__global__ void __launch_bounds__(kSelThreads)
thresh_emit_kernel(const float *__restrict__ S, int nh, int nb,
                   const uint64_t *__restrict__ row_thr, const GlobalState *__restrict__ st,
                   int32_t *__restrict__ kv_idx, int32_t *__restrict__ kv_cnt, int max_kv) {
  const int row = blockIdx.x * (kSelThreads / 64) + (threadIdx.x >> 6);
  if (row >= nh * nb) return;
  const int h = row / nb, I = row - h * nb;
  const int lane = lane_id();
  const uint64_t K = row_thr[row];
  const bool fill = st[h].fill != 0;
  const uint64_t lam = st[h].prefix;  // the smallest outside key selected
  const float *src = S + static_cast<int64_t>(row) * nb;
  bool sel[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int j = lane + 64 * r;
    sel[r] = false;
    if (j < nb) {
      const uint32_t ok = float_order_key(src[j]);
      sel[r] = key64(ok, j) >= K || (fill && gkey(ok, static_cast<uint32_t>(I * nb + j)) >= lam);
    }
  }
  const int cnt = emit_row<KPL>(sel, kv_idx + static_cast<int64_t>(row) * max_kv, max_kv);
  if (lane == 0) kv_cnt[row] = cnt;
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
  for (int p = before * tiles + lane; p < max_kv; p += 64) out[p] = -1;
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
  for (int p = before + lane; p < max_kv; p += 64) out[p] = -1;
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
  for (int p = before + lane; p < max_kv; p += 64) out[p] = -1;
  if (lane == 0) kv_cnt[row] = before;
}

}  // namespace hsa

namespace hsa_host {

static int keys_per_lane(int n) { return (n + 63) / 64; }

size_t select_ws_bytes(int nh, int nb, int mode) {
  if (mode != HSA_SELECT_THRESH_GLOBAL) return 0;
  size_t b = 0;
  b += static_cast<size_t>(nh) * nb * sizeof(uint64_t);   // row thresholds
  b += static_cast<size_t>(nh) * nb * sizeof(int32_t);    // row counts
  b = (b + 255) & ~static_cast<size_t>(255);
  b += static_cast<size_t>(nh) * sizeof(hsa::GlobalState);
  b = (b + 255) & ~static_cast<size_t>(255);
  b += static_cast<size_t>(nh) * hsa::kGPasses * hsa::kGBins * sizeof(uint32_t);  // histograms
  return b;
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
    uint64_t *row_thr = reinterpret_cast<uint64_t *>(base);
    int32_t *row_cnt = reinterpret_cast<int32_t *>(base + static_cast<size_t>(rows) * 8);
    size_t off = static_cast<size_t>(rows) * 12;
    off = (off + 255) & ~static_cast<size_t>(255);
    hsa::GlobalState *st = reinterpret_cast<hsa::GlobalState *>(base + off);
    off += static_cast<size_t>(nh) * sizeof(hsa::GlobalState);
    off = (off + 255) & ~static_cast<size_t>(255);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base + off);
    const double one = 4611686018427387904.0;  // 2^62
    const uint64_t target = static_cast<uint64_t>(floor(p->tau * one));
    const int64_t budget = static_cast<int64_t>(floor(p->budget_ratio * (static_cast<double>(nb) * nb) + 0.5));
    const dim3 grid((rows + rows_per_wg - 1) / rows_per_wg);
    HSA_KPL_DISPATCH(nb, hsa::thresh_row_kernel, grid, dim3(hsa::kSelThreads), S, rows, nb, target,
                     row_thr, row_cnt);
    hipLaunchKernelGGL(hsa::gfill_init_kernel, dim3(nh), dim3(256), 0, stream, row_cnt, nb, budget,
                       st, hist);
    const dim3 hgrid((nb + rows_per_wg - 1) / rows_per_wg, nh);
    for (int pass = 0; pass < hsa::kGPasses; ++pass) {  // passes after the search ends return at once
      HSA_KPL_DISPATCH(nb, hsa::gfill_hist_kernel, hgrid, dim3(hsa::kSelThreads), S, nb, pass,
                       row_thr, st, hist);
      hipLaunchKernelGGL(hsa::gfill_pick_kernel, dim3(nh), dim3(hsa::kSelThreads), 0, stream, pass, st,
                         hist);
    }
    HSA_KPL_DISPATCH(nb, hsa::thresh_emit_kernel, grid, dim3(hsa::kSelThreads), S, nh, nb, row_thr,
                     st, kv_idx, kv_cnt, max_kv);
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

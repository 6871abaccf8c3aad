// Exact top-k of one row of block scores by a group of 64 to 256 threads
// (MemLong 2.3.2: the top-k of the similarity scores, found by an exact
// search, 2.4.2).
//
// Order: score descending, then block index ascending; NaN below every
// number; -0 equal to +0.  Each thread holds up to KPT scores in registers,
// loaded coalesced (element i of thread t is column lo + tpr i + t).  Steps:
//   1. map each score to a 32-bit key whose unsigned order is the score
//      order (NaN -> 0, +-0 -> 0x80000000);
//   2. radix-select the k-th largest key, 8 bits per pass, with a 256-bin
//      histogram per row in LDS;
//   3. if more keys equal that threshold than there are places left, pick
//      the lowest indices among them by a second radix select on ~index;
//   4. gather the k kept entries (any order) and rank them by counting on the
//      64-bit key (score key, ~index), which is the output order.
// Returned scores are the row's own bits, kept beside the keys (a key does
// not hold the sign of zero or a NaN payload).
#ifndef BRS_WAVE_TOPK_H_
#define BRS_WAVE_TOPK_H_

#include "brs_internal.h"

namespace brs {

__device__ __forceinline__ uint32_t topk_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if (s == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inverse of topk_key for keys other than 0 (NaN) and 0x80000000 (zero)
__device__ __forceinline__ float topk_key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// makes this wave's LDS writes visible to its own later LDS reads
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Minimum and maximum over the wave: DPP moves within 16-lane rows, then the
// gfx950 row swaps (every lane gets the result; no LDS round trip).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ void wave_minmax_u32(uint32_t& mn, uint32_t& mx) {
  mn = min(mn, dpp_u32<0xb1>(mn));  // quad_perm [1,0,3,2]
  mx = max(mx, dpp_u32<0xb1>(mx));
  mn = min(mn, dpp_u32<0x4e>(mn));  // quad_perm [2,3,0,1]
  mx = max(mx, dpp_u32<0x4e>(mx));
  mn = min(mn, dpp_u32<0x141>(mn));  // row_half_mirror
  mx = max(mx, dpp_u32<0x141>(mx));
  mn = min(mn, dpp_u32<0x140>(mn));  // row_mirror
  mx = max(mx, dpp_u32<0x140>(mx));
  auto a = __builtin_amdgcn_permlane16_swap(mn, mn, false, false);
  auto b = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
  mn = min(a[0], a[1]);
  mx = max(b[0], b[1]);
  a = __builtin_amdgcn_permlane32_swap(mn, mn, false, false);
  b = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
  mn = min(a[0], a[1]);
  mx = max(b[0], b[1]);
}

// Inclusive prefix sum over the wave with DPP moves: shifts within each
// 16-lane row, then the row totals broadcast to the following rows.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Barrier of the threads that share one row: the workgroup, or (WAVE) the
// one wave that holds the row.
template <bool WAVE>
__device__ __forceinline__ void row_sync() {
  if constexpr (WAVE)
    wave_lds_sync();
  else
    __syncthreads();
}

// LDS state of one row's selection.
struct TopkRowShared {
  uint32_t hist[256];
  int wtot[4];
  int digit, above, neq, cnt;
};

// One radix pass over the keys still matching `prefix` under `mask`:
// finds the digit (bits shift..shift+7) that holds the kk-th largest key.
// Every thread of the row group must call it (three barriers).  hist is
// zero on entry and on exit.  A wave whose matching keys in one slot share
// a digit adds them with one atomic instead of one per lane.
template <int KPT, bool WAVE>
__device__ __forceinline__ void topk_radix_pass(const uint32_t (&keys)[KPT], uint32_t vmask, uint32_t prefix,
                                                uint32_t mask, int shift, int& kk, int tpr, TopkRowShared& sh,
                                                uint32_t& digit_out) {
  const int t = threadIdx.x % tpr, lane = threadIdx.x & 63, wv = t >> 6;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool match = ((vmask >> i) & 1u) && (keys[i] & mask) == prefix;
    const uint32_t dg = (keys[i] >> shift) & 255u;
    const uint64_t m = __ballot(match);
    if (m) {
      const int src = (int)__ffsll((long long)m) - 1;
      const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)dg, src);
      const bool same = __ballot(match && dg == d0) == m;
      if (same) {
        if (lane == src) atomicAdd(&sh.hist[d0], (uint32_t)__popcll(m));
      } else if (match) {
        atomicAdd(&sh.hist[dg], 1u);
      }
    }
  }
  row_sync<WAVE>();
  // bins in descending digit order, 256 / tpr per thread (tpr <= 256)
  const int bpt = 256 / tpr;
  int h[4] = {0, 0, 0, 0}, run = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < bpt) {
      const int bin = 255 - (bpt * t + j);
      h[j] = (int)sh.hist[bin];
      sh.hist[bin] = 0u;
      run += h[j];
    }
  const int incl = wave_scan_incl(run);
  if (lane == 63) sh.wtot[wv] = incl;
  row_sync<WAVE>();
  int before = incl - run;
  for (int w = 0; w < wv; ++w) before += sh.wtot[w];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j < bpt) {
      if (before < kk && before + h[j] >= kk) {
        sh.digit = 255 - (bpt * t + j);
        sh.above = before;
        sh.neq = h[j];
      }
      before += h[j];
    }
  row_sync<WAVE>();
  digit_out = (uint32_t)sh.digit;
  kk -= sh.above;
}

// Radix select of the kk-th largest key among the valid ones (4 passes).
// Returns the threshold key; kk becomes the number of keys equal to it to
// take, and sh.neq holds how many there are.
template <int KPT, bool WAVE>
__device__ __forceinline__ uint32_t topk_radix_select(const uint32_t (&keys)[KPT], uint32_t vmask, int& kk, int tpr,
                                                      TopkRowShared& sh) {
  uint32_t prefix = 0u, mask = 0u;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t dg;
    topk_radix_pass<KPT, WAVE>(keys, vmask, prefix, mask, shift, kk, tpr, sh, dg);
    prefix |= dg << shift;
    mask |= 0xffu << shift;
  }
  return prefix;
}

// The scores of one row as raw bits, thread t holding columns lo + tpr i + t
// (lanes past the end re-read column lo: the loads are unconditional, so
// they all stay in flight together).
template <int KPT>
__device__ __forceinline__ void topk_load_raw(const float* __restrict__ srow, int lo, int hi, int tpr,
                                              uint32_t (&raw)[KPT]) {
  const int t = threadIdx.x % tpr;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int e = lo + tpr * i + t;
    raw[i] = hi > lo ? __float_as_uint(srow[e < hi ? e : lo]) : 0u;
  }
}

// Top-k of srow[lo, hi) by the tpr threads of one row group (tpr a power of
// two in 64..256, hi - lo <= tpr * KPT, 1 <= k): the whole workgroup, or
// (WAVE, tpr = 64) a single wave.  raw: the row from topk_load_raw.  Every
// thread of the group must call it, with the same lo, hi and k (barriers).
// sh: zeroed hist and cnt; sel, selv: k 64-bit and k 32-bit words of LDS.
// Results in rank order go to gidx / gvals (global) and lidx / lvals (LDS),
// each of which may be null; slots past min(k, hi - lo) get -1 and -inf.
// The returned scores are the row's own bits (kept beside the keys, which
// do not hold the sign of zero or a NaN payload).
template <int KPT, bool WAVE = false>
__device__ void group_topk_raw(const uint32_t (&raw)[KPT], int lo, int hi, int k, int tpr, TopkRowShared& sh,
                               int* wg_flag, uint64_t* sel, uint32_t* selv, int32_t* gidx, float* gvals,
                               int32_t* lidx, float* lvals) {
  const int t = threadIdx.x % tpr;
  const int n = hi - lo;
  uint32_t keys[KPT];
  uint32_t vmask = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool v = lo + tpr * i + t < hi;
    keys[i] = n > 0 ? topk_key(__uint_as_float(raw[i])) : 0u;
    vmask |= v ? (1u << i) : 0u;
  }
  const bool all = n <= k;  // the same for every thread of the group
  uint32_t thresh = 0u, thresh2 = 0u;
  bool ties = false;
  if (!all) {
    int kk = k;
    thresh = topk_radix_select<KPT, WAVE>(keys, vmask, kk, tpr, sh);
    // more keys equal to the threshold than places: the lowest indices win,
    // i.e. the largest ~index, found by a second select among those keys
    ties = sh.neq > kk;
    if (t == 0 && ties) *wg_flag = 1;
    row_sync<WAVE>();
    if (*wg_flag) {
      uint32_t keys2[KPT];
      uint32_t vmask2 = 0u;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        keys2[i] = 0xffffffffu - (uint32_t)(lo + tpr * i + t);
        vmask2 |= (((vmask >> i) & 1u) && keys[i] == thresh) ? (1u << i) : 0u;
      }
      int kk2 = kk > 0 ? kk : 1;
      thresh2 = topk_radix_select<KPT, WAVE>(keys2, vmask2, kk2, tpr, sh);
      if (kk <= 0) thresh2 = 0xffffffffu;  // nothing equal to the threshold is taken
    }
  }
  // the kept keys, in any order, then ranked by (score key, ~index)
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool v = (vmask >> i) & 1u;
    const uint32_t inv_idx = 0xffffffffu - (uint32_t)(lo + tpr * i + t);
    const bool take = v && (all || keys[i] > thresh || (keys[i] == thresh && (!ties || inv_idx >= thresh2)));
    if (take) {
      const int p = atomicAdd(&sh.cnt, 1);
      if (p < k) {
        sel[p] = ((uint64_t)keys[i] << 32) | (uint64_t)inv_idx;
        selv[p] = raw[i];
      }
    }
  }
  row_sync<WAVE>();
  const int cnt = sh.cnt < k ? sh.cnt : k;
  for (int r = t; r < cnt; r += tpr) {
    const uint64_t me = sel[r];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < cnt; ++j) rank += sel[j] > me;
    const int b = (int)(0xffffffffu - (uint32_t)(me & 0xffffffffu));
    const float val = __uint_as_float(selv[r]);
    if (gidx) gidx[rank] = b;
    if (gvals) gvals[rank] = val;
    if (lidx) lidx[rank] = b;
    if (lvals) lvals[rank] = val;
  }
  for (int r = cnt + t; r < k; r += tpr) {
    if (gidx) gidx[r] = -1;
    if (gvals) gvals[r] = -INFINITY;
    if (lidx) lidx[r] = -1;
    if (lvals) lvals[r] = -INFINITY;
  }
}

// Exact top-k of one row by one wave, fast path (raw, lo, hi, k as in
// group_topk_raw; k <= 64).  A lower bound on the k-th largest key is the
// k-th largest of the 64 lane maxima (found bit by bit with ballots); the
// keys at or above it -- a few more than k on ordinary data -- are gathered
// in LDS and ranked by counting on (score key, ~index).  Returns false, with
// nothing written, when more than cap keys pass the bound (many equal
// scores); the radix select then does the work.  sel / selv: cap words.
constexpr int kBisect = 10;  // halvings of the lane-maximum range in wave_topk_filter

// sel / selv hold cap + 1 entries: entry cap is scratch.
template <int KPT>
__device__ bool wave_topk_filter(const uint32_t (&raw)[KPT], int lo, int hi, int k, int cap, uint64_t* sel,
                                 uint32_t* selv, int32_t* gidx, float* gvals, int32_t* lidx) {
  const int lane = threadIdx.x & 63;
  const int n = hi - lo;
  uint32_t keys[KPT];
  uint32_t vmask = 0u, mx = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool v = lo + 64 * i + lane < hi;
    keys[i] = n > 0 ? topk_key(__uint_as_float(raw[i])) : 0u;
    vmask |= v ? (1u << i) : 0u;
    mx = v ? max(mx, keys[i]) : mx;
  }
  uint32_t tau = 0u;
  if (n > k) {
    if (k > 64) return false;
    // bisection between the smallest and largest lane maximum, keeping
    // "at least k maxima >= tau" true; stopped after kBisect halvings (a
    // lower bound is all that is needed: a few more keys pass it)
    uint32_t lo_t = mx, hi_t = mx;
    wave_minmax_u32(lo_t, hi_t);
    lo_t = __builtin_amdgcn_readfirstlane(lo_t);
    hi_t = __builtin_amdgcn_readfirstlane(hi_t);
#pragma unroll
    for (int it = 0; it < kBisect; ++it) {
      const uint32_t mid = lo_t + ((hi_t - lo_t + 1u) >> 1);
      if (__popcll(__ballot(mx >= mid)) >= (uint64_t)k)
        lo_t = mid;
      else
        hi_t = mid - 1u;
    }
    tau = lo_t;
  }
  // the keys at or above tau, gathered in LDS (in order of i, then lane);
  // lanes with nothing to store write slot cap, a scratch slot (no branch)
  int total = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool take = ((vmask >> i) & 1u) && keys[i] >= tau;
    const uint64_t m = __ballot(take);
    const int p = total + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const int dst = (take && p < cap) ? p : cap;
    sel[dst] = ((uint64_t)keys[i] << 32) | (uint64_t)(0xffffffffu - (uint32_t)(lo + 64 * i + lane));
    selv[dst] = raw[i];
    total += (int)__popcll(m);
  }
  if (total > cap) return false;
  wave_lds_sync();
  for (int r = lane; r < total; r += 64) {
    const uint64_t me = sel[r];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < total; ++j) rank += sel[j] > me;
    if (rank < k) {
      const int b = (int)(0xffffffffu - (uint32_t)(me & 0xffffffffu));
      if (gidx) gidx[rank] = b;
      if (gvals) gvals[rank] = __uint_as_float(selv[r]);
      if (lidx) lidx[rank] = b;
    }
  }
  for (int r = total + lane; r < k; r += 64) {
    if (gidx) gidx[r] = -1;
    if (gvals) gvals[r] = -INFINITY;
    if (lidx) lidx[r] = -1;
  }
  return true;
}

// Load and select in one call (see group_topk_raw).
template <int KPT, bool WAVE = false>
__device__ void group_topk(const float* __restrict__ srow, int lo, int hi, int k, int tpr, TopkRowShared& sh,
                           int* wg_flag, uint64_t* sel, uint32_t* selv, int32_t* gidx, float* gvals,
                           int32_t* lidx) {
  uint32_t raw[KPT];
  topk_load_raw<KPT>(srow, lo, hi, tpr, raw);
  group_topk_raw<KPT, WAVE>(raw, lo, hi, k, tpr, sh, wg_flag, sel, selv, gidx, gvals, lidx, nullptr);
}

}  // namespace brs

#endif  // BRS_WAVE_TOPK_H_

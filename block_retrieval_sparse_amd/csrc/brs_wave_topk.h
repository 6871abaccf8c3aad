// Exact top-k of one row of block scores by a single wave (MemLong 2.3.2:
// the top-k of the similarity scores, found by an exact search, 2.4.2).
//
// Order: score descending, then block index ascending; NaN below every
// number; -0 equal to +0.  The wave holds up to 64 * KPL scores in
// registers, loaded coalesced (element i of lane l is column lo + 64 i + l,
// so index order is i-major, lane-minor).  Steps:
//   1. map each score to a 32-bit key whose unsigned order is the score
//      order (NaN -> 0, +-0 -> 0x80000000);
//   2. radix-select the k-th largest key, 8 bits per pass, with a 256-bin
//      histogram in the wave's own LDS (no workgroup barrier); a pass whose
//      remaining candidates all share one digit needs no histogram;
//   3. keep every key above it and, of the keys equal to it, those with the
//      lowest indices (ballot prefix counts in index order), compacted by
//      ballot into LDS;
//   4. rank the kept entries by counting on the 64-bit key (score key, ~index).
// Returned scores are the row's own values (re-read for the zero and NaN
// keys, whose sign or payload the key does not keep).
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

// wave-wide min / max of unsigned values (DPP within rows, then lane swaps)
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xb1, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4e, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = min(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return min(b[0], b[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xb1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4e, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(b[0], b[1]);
}

// makes this wave's LDS writes visible to its own later LDS reads
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// Top-k of srow[lo, hi) (hi - lo <= 64 * KPL, 1 <= k).  hist: 256 words
// of LDS, sel: k + 64 64-bit words of LDS (the last 64 absorb the writes of
// lanes that keep nothing), both private to the wave.  Results in rank
// order go to gidx / gvals (global; gvals may be null) and lidx (LDS; may be
// null); slots past min(k, hi - lo) get -1 and -inf.
template <int KPL>
__device__ void wave_topk(const float* __restrict__ srow, int lo, int hi, int k, uint32_t* hist, uint64_t* sel,
                          int32_t* gidx, float* gvals, int32_t* lidx) {
  const int lane = threadIdx.x & 63;
  const int n = hi - lo;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint32_t keys[KPL];
  uint32_t vmask = 0u;
  if (n > 0) {
    // unconditional loads (lanes past the end re-read column lo) keep them all in flight
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int e = lo + 64 * i + lane;
      const bool v = e < hi;
      keys[i] = topk_key(srow[v ? e : lo]);
      vmask |= v ? (1u << i) : 0u;
    }
  }
  const bool all = n <= k;
  uint32_t thresh = 0u;
  int take_eq = 0;
  if (!all) {
    uint32_t prefix = 0u, mask = 0u;
    int kk = k;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      // common case: every candidate still in play has the same digit
      {
        uint32_t dmin = 0xffffffffu, dmax = 0u;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
          if (((vmask >> i) & 1u) && (keys[i] & mask) == prefix) {
            const uint32_t dg = (keys[i] >> shift) & 255u;
            dmin = dg < dmin ? dg : dmin;
            dmax = dg > dmax ? dg : dmax;
          }
        dmin = (uint32_t)wave_min_u32(dmin);
        dmax = (uint32_t)wave_max_u32(dmax);
        if (dmin == dmax) {
          prefix |= dmin << shift;
          mask |= 0xffu << shift;
          continue;
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) hist[4 * lane + t] = 0u;
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (((vmask >> i) & 1u) && (keys[i] & mask) == prefix) atomicAdd(&hist[(keys[i] >> shift) & 255u], 1u);
      wave_lds_sync();
      // lane l holds the bins of digits 255 - 4l .. 252 - 4l (descending)
      int h[4], run = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        h[t] = (int)hist[255 - (4 * lane + t)];
        run += h[t];
      }
      int before = wave_scan_incl(run) - run;
      int found = -1, above = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (before < kk && before + h[t] >= kk) {
          found = 255 - (4 * lane + t);
          above = before;
        }
        before += h[t];
      }
      const uint64_t who = __ballot(found >= 0);
      const int src = who ? (int)__ffsll((long long)who) - 1 : 0;
      found = __shfl(found, src);
      above = __shfl(above, src);
      kk -= above;
      prefix |= (uint32_t)(found < 0 ? 0 : found) << shift;
      mask |= 0xffu << shift;
      wave_lds_sync();
    }
    thresh = prefix;
    take_eq = kk;
  }
  // keep, in index order: keys above the threshold, then the first take_eq equal to it
  int eq_base = 0, base = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const bool v = (vmask >> i) & 1u;
    const bool gt = v && (all || keys[i] > thresh);
    const bool eq = v && !all && keys[i] == thresh;
    const uint64_t em = __ballot(eq);
    const int er = eq_base + __popcll(em & lt);
    eq_base += __popcll(em);
    const bool take = gt || (eq && er < take_eq);
    const uint64_t tm = __ballot(take);
    const int p = base + __popcll(tm & lt);
    sel[(take && p < k) ? p : k + lane] =
        ((uint64_t)keys[i] << 32) | (uint64_t)(0xffffffffu - (uint32_t)(lo + 64 * i + lane));
    base += __popcll(tm);
  }
  const int cnt = base < k ? base : k;
  wave_lds_sync();
  for (int r = lane; r < cnt; r += 64) {
    const uint64_t me = sel[r];
    int rank = 0;
    for (int j = 0; j < cnt; ++j) rank += sel[j] > me;
    const int b = (int)(0xffffffffu - (uint32_t)(me & 0xffffffffu));
    const uint32_t key = (uint32_t)(me >> 32);
    const float val = (key == 0u || key == 0x80000000u) ? srow[b] : topk_key_value(key);
    gidx[rank] = b;
    if (gvals) gvals[rank] = val;
    if (lidx) lidx[rank] = b;
  }
  for (int r = cnt + lane; r < k; r += 64) {
    gidx[r] = -1;
    if (gvals) gvals[r] = -INFINITY;
    if (lidx) lidx[r] = -1;
  }
}

}  // namespace brs

#endif  // BRS_WAVE_TOPK_H_

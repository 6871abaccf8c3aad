// Exact top-k block selection per score head (MemLong 2.3.2: the top-k
// indices of the similarity scores, found with an exact search, 2.4.2).
//
// Order: score descending, then block index ascending; NaN below every
// number; -0 equal to +0.  Each score maps to a 32-bit key whose unsigned
// order is that score order (NaN -> 0).
//   k <= 64, up to 2048 candidates: one wave per row; a lower bound on the
//     k-th key from the lane maxima, then the keys above it ranked by
//     counting (a one-wave radix select when too many keys reach the bound);
//   k <= 512, up to 2048 candidates: one 256-thread workgroup per row, radix
//     select of the k-th key with a 256-bin histogram in LDS, ties at it to
//     the lowest indices, rank sort of the winners;
//   otherwise: the same with 1024 threads, keys in registers or re-read,
//     histograms per wave (atomics never contend across waves); once the
//     keys at or above the digits found so far number at most 2k, they are
//     gathered and ranked directly instead of running the remaining passes.
#include "brs_wave_topk.h"

namespace brs {
namespace {

constexpr int kGather = 2048;  // keys gathered for the final ranking (k <= kGather)

template <int NT, int KPT>  // KPT = 0: keys re-read from global memory each pass
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores, int64_t stride, int64_t lo,
                                                  int64_t hi, int k, int32_t* __restrict__ idx,
                                                  float* __restrict__ vals) {
  constexpr int NW = NT / 64;
  // per wave (no atomics across waves), four histograms by lane mod 4 in the
  // first pass, whose digit (sign and top exponent bits) many keys share;
  // one in the later passes
  constexpr int NSUB = 4;
  __shared__ uint32_t whist[NW][NSUB][256];
  __shared__ uint32_t hist[256];
  __shared__ int wave_tot[16];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_above, sh_neq;
  __shared__ int srank[kGather];
  __shared__ int sel_count;
  __shared__ __align__(16) uint64_t sel_key[kGather];

  const int64_t row = blockIdx.x;
  const float* s = scores + row * stride;
  const int64_t n = hi - lo;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t c = (n + NT - 1) / NT;  // candidates per thread, contiguous
  const int64_t my0 = lo + tid * c;
  const int64_t my1 = (my0 + c < hi) ? my0 + c : hi;

  uint32_t keys[KPT > 0 ? KPT : 1];
  if constexpr (KPT > 0) {
    // a thread's run as 16-byte loads when the row and the runs are 16-byte
    // aligned and whole (a wave's loads then touch each cache line in one
    // instruction instead of one per element)
    const bool vec = KPT % 4 == 0 && c == KPT && ((uintptr_t)(s + lo) & 15) == 0 && my1 - my0 == KPT;
    if (vec) {
#pragma unroll
      for (int i = 0; i < KPT; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(s + my0 + i);
        keys[i] = topk_key(v.x);
        keys[i + 1] = topk_key(v.y);
        keys[i + 2] = topk_key(v.z);
        keys[i + 3] = topk_key(v.w);
      }
    } else if (n > 0) {
      // unconditional loads (past the run: column lo again, never used), so
      // they are all in flight together
#pragma unroll
      for (int i = 0; i < KPT; ++i) keys[i] = topk_key(s[my0 + i < my1 ? my0 + i : lo]);
    }
  }
  const int64_t mine = my1 > my0 ? my1 - my0 : 0;
  // f(i, key) for this thread's keys in index order (register keys: the
  // loop is unrolled, so no register array is indexed at run time)
  auto for_keys = [&](auto&& f) {
    if constexpr (KPT > 0) {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (i < mine) f((int64_t)i, keys[i]);
    } else {
      for (int64_t i = 0; i < mine; ++i) f(i, topk_key(s[my0 + i]));
    }
  };

  if (tid == 0) sel_count = 0;
  // Radix select, 8 bits per pass.  After each pass, when the keys at or
  // above the lowest key with the digits found so far number at most 2k (and
  // kGather), they are gathered and ranked directly (the usual case: few keys
  // share the top digits); otherwise the select runs on to the exact k-th key
  // and the keys equal to it are taken in index order.
  uint32_t thresh = 0, lb = 0;
  int take_eq = 0;
  bool direct = false;
  const bool all = n <= k;
  if (!all) {
    uint32_t prefix = 0, mask = 0;
    int kk = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      uint32_t* wflat = &whist[0][0][0];
      if (pass == 0) {
        for (int i = tid; i < NW * NSUB * 256; i += NT) wflat[i] = 0u;
      } else {
        for (int i = tid; i < NW * 256; i += NT) wflat[(i >> 8) * (NSUB * 256) + (i & 255)] = 0u;
      }
      __syncthreads();
      const int wv = tid >> 6, sub = pass == 0 ? (lane & (NSUB - 1)) : 0;
      if constexpr (KPT > 0) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const bool match = i < mine && (keys[i] & mask) == prefix;
          const uint32_t dg = (keys[i] >> shift) & 255u;
          if (match) atomicAdd(&whist[wv][sub][dg], 1u);
        }
      } else {
        for_keys([&](int64_t, uint32_t x) {
          if ((x & mask) == prefix) atomicAdd(&whist[wv][sub][(x >> shift) & 255u], 1u);
        });
      }
      __syncthreads();
      for (int i = tid; i < 256; i += NT) {
        uint32_t t = 0u;
        if (pass == 0) {
#pragma unroll
          for (int w = 0; w < NW; ++w)
#pragma unroll
            for (int u = 0; u < NSUB; ++u) t += whist[w][u][i];
        } else {
#pragma unroll
          for (int w = 0; w < NW; ++w) t += whist[w][0][i];
        }
        hist[i] = t;
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds reversed positions p = 4l..4l+3, i.e. digits 255-p
        int h[4], run = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = (int)hist[255 - (4 * tid + i)];
          run += h[i];
        }
        int incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(incl, off);
          if (tid >= off) incl += o;
        }
        int before = incl - run;  // keys with a larger digit than my first position
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (before < kk && before + h[i] >= kk) {
            sh_digit = 255u - (uint32_t)(4 * tid + i);
            sh_above = before;
            sh_neq = h[i];
          }
          before += h[i];
        }
      }
      __syncthreads();
      kk -= sh_above;
      prefix |= sh_digit << shift;
      mask |= 0xffu << shift;
      const int neq = sh_neq;
      __syncthreads();
      // keys >= prefix: the k - kk above it and the neq sharing its digits
      // (ranked by counting: at most 2k of them)
      if (k - kk + neq <= min(kGather, 2 * k)) {
        lb = prefix;
        direct = true;
        break;
      }
    }
    if (!direct) {
      thresh = prefix;
      take_eq = kk;
    }
  }

  // gather: every key >= lb (direct), or the k winners with the keys equal
  // to the threshold taken in index order; one slot reservation per wave
  int rank_eq = 0;
  if (!all && !direct) {
    int eq = 0;
    for_keys([&](int64_t, uint32_t x) { eq += x == thresh; });
    rank_eq = block_inclusive_scan(eq, wave_tot) - eq;
  }
  for (int i = tid; i < kGather; i += NT) srank[i] = 0;
  const int cap = direct ? kGather : k;
  auto taken = [&](uint32_t x) {
    if (all) return true;
    if (direct) return x >= lb;
    bool t = x > thresh;
    if (x == thresh) {
      t = rank_eq < take_eq;
      ++rank_eq;
    }
    return t;
  };
  if constexpr (KPT > 0) {
    uint32_t tk = 0u;  // bit i: key i taken
    int total = 0;     // the wave's taken keys
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool take = i < mine && taken(keys[i]);
      tk |= take ? (1u << i) : 0u;
      total += (int)__popcll(__ballot(take));
    }
    if (total > 0) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&sel_count, total);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool take = (tk >> i) & 1u;
        const uint64_t m = __ballot(take);
        const int p = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint32_t b = (uint32_t)(my0 + i);
        if (take && p < cap) sel_key[p] = ((uint64_t)keys[i] << 32) | (uint64_t)(0xffffffffu - b);
        base += (int)__popcll(m);
      }
    }
  } else {
    for_keys([&](int64_t i, uint32_t x) {
      if (taken(x)) {
        const int p = atomicAdd(&sel_count, 1);
        const uint32_t b = (uint32_t)(my0 + i);
        if (p < cap) sel_key[p] = ((uint64_t)x << 32) | (uint64_t)(0xffffffffu - b);
      }
    });
  }
  __syncthreads();
  const int cnt = min(sel_count, cap);
  int32_t* orow = idx + row * k;
  float* vrow = vals ? vals + row * k : nullptr;
  // ranks by counting on (key, ~index); each count is split over P threads
  // whose partial counts are summed in LDS, so that every thread takes part
  const int P = cnt > 0 ? max(1, NT / cnt) : 1;
  for (int u = tid; u < P * cnt; u += NT) {
    const int i = u % cnt, part = u / cnt;
    const int j0 = part * cnt / P, j1 = (part + 1) * cnt / P;
    const uint64_t me = sel_key[i];
    int c = 0;
    int j = j0;
    if ((j & 1) && j < j1) c += sel_key[j++] > me;
    // two keys per 16-byte read
#pragma unroll 4
    for (; j + 1 < j1; j += 2) {
      const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(&sel_key[j]);
      c += (v.x > me) + (v.y > me);
    }
    if (j < j1) c += sel_key[j] > me;
    atomicAdd(&srank[i], c);
  }
  __syncthreads();
  for (int i = tid; i < cnt; i += NT) {
    const int rank = srank[i];
    if (rank < k) {
      const int64_t b = (int64_t)(0xffffffffu - (uint32_t)(sel_key[i] & 0xffffffffu));
      orow[rank] = (int32_t)b;
      if (vrow) vrow[rank] = s[b];
    }
  }
  const int filled = min(cnt, k);
  for (int i = filled + tid; i < k; i += NT) {
    orow[i] = -1;
    if (vrow) vrow[i] = -INFINITY;
  }
}

// One 256-thread workgroup per row for up to 256 * KPT candidates and
// k <= kGroupK (the selection of brs_wave_topk.h).
constexpr int kGroupK = 512;

template <int KPT>
__global__ __launch_bounds__(256) void topk_group_kernel(const float* __restrict__ scores, int64_t stride, int64_t lo,
                                                         int64_t hi, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ vals) {
  __shared__ TopkRowShared sh;
  __shared__ uint64_t sel[kGroupK];
  __shared__ uint32_t selv[kGroupK];
  __shared__ int flag;
  const int64_t row = blockIdx.x;
  for (int i = threadIdx.x; i < 256; i += 256) sh.hist[i] = 0u;
  if (threadIdx.x == 0) {
    sh.cnt = 0;
    flag = 0;
  }
  __syncthreads();
  group_topk<KPT>(scores + row * stride, (int)lo, (int)hi, k, 256, sh, &flag, sel, selv, idx + row * k,
                  vals ? vals + row * k : nullptr, nullptr);
}

// One wave per row (four rows per 256-thread workgroup) for k <= 64 and up
// to 64 * KPT candidates: the bound-and-rank selection of brs_wave_topk.h,
// with the one-wave radix select for rows with too many keys at the bound.
constexpr int kWaveCand = 256;

template <int KPT>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ scores, int64_t stride, int64_t lo,
                                                        int64_t hi, int k, int64_t rows, int32_t* __restrict__ idx,
                                                        float* __restrict__ vals) {
  __shared__ TopkRowShared sh[4];
  __shared__ uint64_t sel[4][kWaveCand];
  __shared__ uint32_t selv[4][kWaveCand];
  __shared__ int flag[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;  // whole waves only: the code below syncs within the wave
  uint32_t raw[KPT];
  topk_load_raw<KPT>(scores + row * stride, (int)lo, (int)hi, 64, raw);
  int32_t* gi = idx + row * k;
  float* gv = vals ? vals + row * k : nullptr;
  if (wave_topk_filter<KPT>(raw, (int)lo, (int)hi, k, kWaveCand - 1, sel[wave], selv[wave], gi, gv, nullptr)) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) sh[wave].hist[lane + 64 * j] = 0u;
  if (lane == 0) {
    sh[wave].cnt = 0;
    flag[wave] = 0;
  }
  wave_lds_sync();
  group_topk_raw<KPT, true>(raw, (int)lo, (int)hi, k, 64, sh[wave], &flag[wave], sel[wave], selv[wave], gi, gv,
                            nullptr, nullptr);
}

}  // namespace

hipError_t launch_select_topk(const float* scores, int batch, int heads, int64_t stride, int64_t lo, int64_t hi,
                              int k, int32_t* idx, float* vals, hipStream_t s) {
  const int64_t rows = (int64_t)batch * heads;
  const int64_t n = hi - lo;
  if (k <= 64 && n <= 64 * 32) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (n <= 64 * 4)
      hipLaunchKernelGGL((topk_wave_kernel<4>), grid, block, 0, s, scores, stride, lo, hi, k, rows, idx, vals);
    else if (n <= 64 * 8)
      hipLaunchKernelGGL((topk_wave_kernel<8>), grid, block, 0, s, scores, stride, lo, hi, k, rows, idx, vals);
    else if (n <= 64 * 16)
      hipLaunchKernelGGL((topk_wave_kernel<16>), grid, block, 0, s, scores, stride, lo, hi, k, rows, idx, vals);
    else
      hipLaunchKernelGGL((topk_wave_kernel<32>), grid, block, 0, s, scores, stride, lo, hi, k, rows, idx, vals);
    return hipGetLastError();
  }
  if (k <= kGroupK && n <= 256 * 8) {
    const dim3 grid((unsigned)rows), block(256);
    if (n <= 256)
      hipLaunchKernelGGL((topk_group_kernel<1>), grid, block, 0, s, scores, stride, lo, hi, k, idx, vals);
    else if (n <= 512)
      hipLaunchKernelGGL((topk_group_kernel<2>), grid, block, 0, s, scores, stride, lo, hi, k, idx, vals);
    else if (n <= 1024)
      hipLaunchKernelGGL((topk_group_kernel<4>), grid, block, 0, s, scores, stride, lo, hi, k, idx, vals);
    else
      hipLaunchKernelGGL((topk_group_kernel<8>), grid, block, 0, s, scores, stride, lo, hi, k, idx, vals);
    return hipGetLastError();
  }
  if (n <= 256 * 4)
    hipLaunchKernelGGL((topk_kernel<256, 4>), dim3((unsigned)rows), dim3(256), 0, s, scores, stride, lo, hi, k, idx,
                       vals);
  else if (n <= 1024 * 16)
    hipLaunchKernelGGL((topk_kernel<1024, 16>), dim3((unsigned)rows), dim3(1024), 0, s, scores, stride, lo, hi, k,
                       idx, vals);
  else
    hipLaunchKernelGGL((topk_kernel<1024, 0>), dim3((unsigned)rows), dim3(1024), 0, s, scores, stride, lo, hi, k,
                       idx, vals);
  return hipGetLastError();
}

}  // namespace brs

// Block scoring (Landmark Attention "proposed method": query-landmark
// similarity; InfLLM "method": block-level relevance instead of token-level;
// MemLong 2.3.2: cosine similarity of chunk embeddings).
//
// Scores are exact: every product of two stored values is exact in float64
// and the sums are float64, rounded once to float32 at the end, so the
// result does not depend on how lanes split the sum.
//
// Dot-max layout: one workgroup streams a range of blocks of one
// (batch, kv head); each block's R representatives are contiguous rows, read
// once and dotted with all G query heads of the group (grouped-query sharing:
// the representative bytes are read once per kv head, not once per query
// head).  L lanes share one row (16-byte loads, coalesced); each lane holds
// its slice of the G queries in float64 registers.  With `grouped` set the
// kernels write one score per kv head instead of one per query head: the
// maximum over the group's heads (for a selection the group shares).
#include <hip/hip_ext.h>

#include "brs_internal.h"

namespace brs {

namespace {
thread_local hipEvent_t g_score_stop = nullptr;  // stamped when the next score kernel completes

hipEvent_t take_score_stop() {
  hipEvent_t e = g_score_stop;
  g_score_stop = nullptr;
  return e;
}
}  // namespace

void set_score_stop_event(hipEvent_t e) { g_score_stop = e; }

// a score launch, with the pending stop event attached when there is one
#define BRS_SCORE_LAUNCH(K, GRID, BLOCK, S, ...)                                      \
  do {                                                                                \
    hipEvent_t ev_ = take_score_stop();                                               \
    if (ev_)                                                                          \
      hipExtLaunchKernelGGL(K, GRID, BLOCK, 0, S, nullptr, ev_, 0, __VA_ARGS__);      \
    else                                                                              \
      hipLaunchKernelGGL(K, GRID, BLOCK, 0, S, __VA_ARGS__);                          \
  } while (0)

namespace {

template <typename T>
struct Vec;  // 16-byte unit of T
template <>
struct Vec<uint16_t> {
  static constexpr int n = 8;
  __device__ static void to_f64(const uint4& u, double* out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = (double)bf16_lo(w[i]);
      out[2 * i + 1] = (double)bf16_hi(w[i]);
    }
  }
};
template <>
struct Vec<float> {
  static constexpr int n = 4;
  __device__ static void to_f64(const uint4& u, double* out) {
    out[0] = (double)__uint_as_float(u.x);
    out[1] = (double)__uint_as_float(u.y);
    out[2] = (double)__uint_as_float(u.z);
    out[3] = (double)__uint_as_float(u.w);
  }
};

__device__ __forceinline__ double nan_max(double a, double b) {
  // max that keeps NaN (a NaN representative dot makes the block score NaN)
  return (b > a || b != b) ? b : a;
}

// p0, p1 = this lane's value and its partner's, in either order: the partner
// is lane ^ OFF for OFF = 1, 2, 16, 32, and for OFF = 4, 8 the half-row /
// row mirror (lane 2*OFF-1-i of its group of 2*OFF: the same value as
// lane ^ OFF once each group of OFF lanes holds one value).  DPP moves and
// gfx950 row swaps on the two 32-bit halves: VALU work, no LDS permutes.
template <int OFF>
__device__ __forceinline__ void lane_pair(double v, double& p0, double& p1) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  auto join = [](uint32_t l, uint32_t h) { return __builtin_bit_cast(double, ((uint64_t)h << 32) | l); };
  if constexpr (OFF <= 8) {
    constexpr int ctrl = OFF == 1 ? 0xb1 : OFF == 2 ? 0x4e : OFF == 4 ? 0x141 : 0x140;
    p0 = v;
    // every lane is written by these permutations: no old value to keep
    p1 = join((uint32_t)__builtin_amdgcn_mov_dpp((int)lo, ctrl, 0xf, 0xf, true),
              (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, ctrl, 0xf, 0xf, true));
  } else if constexpr (OFF == 16) {
    // a swap returns {own, partner} or {partner, own} by row; both halves
    // are swapped alike, so element e of the two halves is one value
    const auto x = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto y = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    p0 = join(x[0], y[0]);
    p1 = join(x[1], y[1]);
  } else {
    static_assert(OFF == 32, "offset");
    const auto x = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto y = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    p0 = join(x[0], y[0]);
    p1 = join(x[1], y[1]);
  }
}
template <int OFF>
__device__ __forceinline__ double pair_sum(double v) {
  double p0, p1;
  lane_pair<OFF>(v, p0, p1);
  return p0 + p1;
}
template <int OFF>
__device__ __forceinline__ double pair_max(double v) {
  double p0, p1;
  lane_pair<OFF>(v, p0, p1);
  return nan_max(p0, p1);
}

// Sum over aligned groups of L lanes (every lane gets its group's total).
template <int L>
__device__ __forceinline__ double group_sum_f64(double v) {
  if constexpr (L >= 2) v = pair_sum<1>(v);
  if constexpr (L >= 4) v = pair_sum<2>(v);
  if constexpr (L >= 8) v = pair_sum<4>(v);
  if constexpr (L >= 16) v = pair_sum<8>(v);
  if constexpr (L >= 32) v = pair_sum<16>(v);
  if constexpr (L >= 64) v = pair_sum<32>(v);
  return v;
}

// NaN-keeping max over aligned groups of n = L * R lanes whose groups of L
// lanes each hold one value (n a power of two up to 64).
template <int L>
__device__ __forceinline__ double group_max_f64(double v, int n) {
  if constexpr (L <= 1) if (n > 1) v = pair_max<1>(v);
  if constexpr (L <= 2) if (n > 2) v = pair_max<2>(v);
  if constexpr (L <= 4) if (n > 4) v = pair_max<4>(v);
  if constexpr (L <= 8) if (n > 8) v = pair_max<8>(v);
  if constexpr (L <= 16) if (n > 16) v = pair_max<16>(v);
  if constexpr (L <= 32) if (n > 32) v = pair_max<32>(v);
  return v;
}

template <typename T>
__device__ __forceinline__ double elem_f64(const T* p, int64_t i);
template <>
__device__ __forceinline__ double elem_f64<float>(const float* p, int64_t i) { return (double)p[i]; }
template <>
__device__ __forceinline__ double elem_f64<uint16_t>(const uint16_t* p, int64_t i) {
  return (double)bf16_to_f32(p[i]);
}

// EPL: elements per lane (EPL * sizeof(T) is a multiple of 16 bytes).
// L = d / EPL lanes per row.  G: query heads per kv head.
template <typename T, int EPL, int G>
__global__ __launch_bounds__(256) void score_dot_kernel(const T* __restrict__ q, const T* __restrict__ reps,
                                                        float* __restrict__ scores, int d, int R, int hkv,
                                                        int64_t capB, int64_t lo, int64_t hi, int bps,
                                                        int grouped) {
  constexpr int UPL = EPL / Vec<T>::n;  // 16-byte units per lane
  const int L = d / EPL;
  const int lane = threadIdx.x & 63;
  const int slot_in_wave = lane / L, sub = lane - slot_in_wave * L;
  const int slots_per_wave = 64 / L;
  const int slot = (threadIdx.x >> 6) * slots_per_wave + slot_in_wave;
  const int slots = (blockDim.x >> 6) * slots_per_wave;
  const int bg = blockIdx.y;
  const int b = bg / hkv, g = bg - b * hkv;
  const int hq = hkv * G;

  double qd[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const T* qrow = q + ((int64_t)b * hq + g * G + j) * d + sub * EPL;
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + u * Vec<T>::n);
      Vec<T>::to_f64(raw, &qd[j][u * Vec<T>::n]);
    }
  }

  const T* rbase = reps + ((int64_t)bg * capB) * R * d + sub * EPL;
  float* sbase = scores + ((int64_t)b * hq + g * G) * capB;
  const int64_t tile0 = lo + (int64_t)blockIdx.x * slots * bps;
  for (int i = 0; i < bps; ++i) {
    const int64_t blk = tile0 + (int64_t)i * slots + slot;
    const bool valid = blk < hi;
    double best[G];
#pragma unroll
    for (int j = 0; j < G; ++j) best[j] = -INFINITY;
    for (int r = 0; r < R; ++r) {
      uint4 raw[UPL];
#pragma unroll
      for (int u = 0; u < UPL; ++u)
        raw[u] = valid ? *reinterpret_cast<const uint4*>(rbase + (blk * R + r) * d + u * Vec<T>::n)
                       : make_uint4(0, 0, 0, 0);
      double x[EPL];
#pragma unroll
      for (int u = 0; u < UPL; ++u) Vec<T>::to_f64(raw[u], &x[u * Vec<T>::n]);
      double acc[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        double a = 0.0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fma(qd[j][e], x[e], a);
        acc[j] = a;
      }
      for (int off = 1; off < L; off <<= 1) {
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j] += __shfl_xor(acc[j], off);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) best[j] = nan_max(best[j], acc[j]);
    }
    if (valid) {
      if (grouped) {
        double gb = best[0];
#pragma unroll
        for (int j = 1; j < G; ++j) gb = nan_max(gb, best[j]);
        if (sub == 0) scores[(int64_t)bg * capB + blk] = (float)gb;
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j)
          if (sub == (j % L)) sbase[(int64_t)j * capB + blk] = (float)best[j];
      }
    }
  }
}

// Row-granular variant, used when R divides the slots of a wave: each slot
// (L lanes) takes one representative row, RPS rows in flight per slot, and a
// block's R rows sit in R adjacent slots, so the max over representatives is
// a shuffle.  Rows of one (batch, kv head) are contiguous in memory.
template <typename T, int EPL, int G, int L, int RPS>
__global__ __launch_bounds__(256) void score_dot_rows_kernel(const T* __restrict__ q, const T* __restrict__ reps,
                                                             float* __restrict__ scores, int d, int R, int hkv,
                                                             int64_t capB, int64_t lo, int64_t hi, int grouped) {
  constexpr int UPL = EPL / Vec<T>::n;
  constexpr int SPW = 64 / L;
  const int lane = threadIdx.x & 63;
  const int sw = lane / L, sub = lane % L;
  const int slot = (threadIdx.x >> 6) * SPW + sw;
  const int slots = (blockDim.x >> 6) * SPW;
  const int bg = blockIdx.y;
  const int b = bg / hkv, g = bg - b * hkv;
  const int hq = hkv * G;

  double qd[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const T* qrow = q + ((int64_t)b * hq + g * G + j) * d + sub * EPL;
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + u * Vec<T>::n);
      Vec<T>::to_f64(raw, &qd[j][u * Vec<T>::n]);
    }
  }
  const int64_t row_lo = lo * R, row_hi = hi * R;
  const int64_t row0 = row_lo + (int64_t)blockIdx.x * slots * RPS;
  const T* rbase = reps + (int64_t)bg * capB * R * d + sub * EPL;
  float* sbase = scores + ((int64_t)b * hq + g * G) * capB;

  uint4 raw[RPS][UPL];
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    const int64_t row = row0 + (int64_t)i * slots + slot;
#pragma unroll
    for (int u = 0; u < UPL; ++u)
      raw[i][u] = row < row_hi ? *reinterpret_cast<const uint4*>(rbase + row * d + u * Vec<T>::n)
                               : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < RPS; ++i) {
    const int64_t row = row0 + (int64_t)i * slots + slot;
    double x[EPL];
#pragma unroll
    for (int u = 0; u < UPL; ++u) Vec<T>::to_f64(raw[i][u], &x[u * Vec<T>::n]);
    double acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = fma(qd[j][e], x[e], a);
      acc[j] = a;
    }
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = group_max_f64<L>(group_sum_f64<L>(acc[j]), L * R);
    if (row < row_hi && (row % R) == 0) {
      const int64_t blk = row / R;
      if (grouped) {
        double gb = acc[0];
#pragma unroll
        for (int j = 1; j < G; ++j) gb = nan_max(gb, acc[j]);
        if (sub == 0) scores[(int64_t)bg * capB + blk] = (float)gb;
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j)
          if (sub == (j % L)) sbase[(int64_t)j * capB + blk] = (float)acc[j];
      }
    }
  }
}

// Any shape: one wave per block, lanes stride over the elements, up to 32
// query heads per kv head.
template <typename T>
__global__ __launch_bounds__(256) void score_dot_generic_kernel(const T* __restrict__ q, const T* __restrict__ reps,
                                                                float* __restrict__ scores, int d, int R, int hkv,
                                                                int G, int64_t capB, int64_t lo, int64_t hi,
                                                                int grouped) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = lo + (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (blk >= hi) return;
  const int bg = blockIdx.y;
  const int b = bg / hkv, g = bg - b * hkv;
  const int hq = hkv * G;
  const T* rrow = reps + ((int64_t)bg * capB + blk) * R * d;
  double gb = -INFINITY;
  for (int j = 0; j < G; ++j) {
    const T* qrow = q + ((int64_t)b * hq + g * G + j) * d;
    double best = -INFINITY;
    for (int r = 0; r < R; ++r) {
      double a = 0.0;
      for (int e = lane; e < d; e += 64) a = fma(elem_f64(qrow, e), elem_f64(rrow + (int64_t)r * d, e), a);
      for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off);
      best = nan_max(best, a);
    }
    gb = j == 0 ? best : nan_max(gb, best);
    if (lane == 0 && !grouped) scores[((int64_t)b * hq + g * G + j) * capB + blk] = (float)best;
  }
  if (lane == 0 && grouped) scores[(int64_t)bg * capB + blk] = (float)gb;
}

// Cosine (one score head per sequence): s = q.e / (sqrt(q.q) sqrt(e.e)),
// float64 throughout, 0 if either norm is 0.
template <typename T>
__global__ __launch_bounds__(256) void score_cosine_kernel(const T* __restrict__ rq, const T* __restrict__ emb,
                                                           float* __restrict__ scores, int D, int64_t capB,
                                                           int64_t lo, int64_t hi) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = lo + (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (blk >= hi) return;
  const int b = blockIdx.y;
  const T* qv = rq + (int64_t)b * D;
  const T* ev = emb + ((int64_t)b * capB + blk) * D;
  double dot = 0.0, qq = 0.0, ee = 0.0;
  for (int e = lane; e < D; e += 64) {
    const double x = elem_f64(qv, e), y = elem_f64(ev, e);
    dot = fma(x, y, dot);
    qq = fma(x, x, qq);
    ee = fma(y, y, ee);
  }
  for (int off = 32; off > 0; off >>= 1) {
    dot += __shfl_xor(dot, off);
    qq += __shfl_xor(qq, off);
    ee += __shfl_xor(ee, off);
  }
  if (lane == 0) {
    const double den = sqrt(qq) * sqrt(ee);
    scores[(int64_t)b * capB + blk] = den != 0.0 ? (float)(dot / den) : 0.0f;
  }
}

// Cosine with 16 lanes per embedding row (16-byte loads, lane l takes
// units l, l + 16, ...; UPL units per lane), 4 rows per wave, the three sums
// reduced over the 16 lanes with DPP moves.  Same products, float64 sums and
// final rounding as score_cosine_kernel.
constexpr int kCosLanes = 16;

template <typename T, int UPL>
__global__ __launch_bounds__(256) void score_cosine_rows_kernel(const T* __restrict__ rq, const T* __restrict__ emb,
                                                                float* __restrict__ scores, int D, int64_t capB,
                                                                int64_t lo, int64_t hi) {
  constexpr int VN = Vec<T>::n;
  const int lane = threadIdx.x & 63;
  const int sub = lane & (kCosLanes - 1);
  const int64_t blk = lo + (int64_t)blockIdx.x * (blockDim.x / kCosLanes) + (threadIdx.x / kCosLanes);
  const int b = blockIdx.y;
  const int units = D / VN;
  const int64_t row = blk < hi ? blk : lo;  // rows past the range repeat row lo (nothing is stored)
  const T* qrow = rq + (int64_t)b * D;
  const T* erow = emb + ((int64_t)b * capB + row) * D;
  uint4 qr[UPL], er[UPL];
#pragma unroll
  for (int u = 0; u < UPL; ++u) {
    const int un = min(sub + kCosLanes * u, units - 1);
    qr[u] = *reinterpret_cast<const uint4*>(qrow + (int64_t)un * VN);
    er[u] = *reinterpret_cast<const uint4*>(erow + (int64_t)un * VN);
  }
  double dot = 0.0, qq = 0.0, ee = 0.0;
#pragma unroll
  for (int u = 0; u < UPL; ++u) {
    if (sub + kCosLanes * u >= units) continue;  // a unit another lane already holds
    double x[VN], y[VN];
    Vec<T>::to_f64(qr[u], x);
    Vec<T>::to_f64(er[u], y);
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      dot = fma(x[e], y[e], dot);
      qq = fma(x[e], x[e], qq);
      ee = fma(y[e], y[e], ee);
    }
  }
  dot = group_sum_f64<kCosLanes>(dot);
  qq = group_sum_f64<kCosLanes>(qq);
  ee = group_sum_f64<kCosLanes>(ee);
  if (sub == 0 && blk < hi) {
    const double den = sqrt(qq) * sqrt(ee);
    scores[(int64_t)b * capB + blk] = den != 0.0 ? (float)(dot / den) : 0.0f;
  }
}

template <typename T, int EPL, int G>
hipError_t run_dot(const brs_memory& m, const void* q, int64_t lo, int64_t hi, float* scores, int grouped,
                   hipStream_t s) {
  const int L = m.head_dim / EPL;
  const int slots = 4 * (64 / L);
  const int64_t nblk = hi - lo;
  const int64_t bg = (int64_t)m.batch * m.n_kv_heads;
  // blocks per slot: enough workgroups to fill the chip, a few rows per lane
  int bps = (int)((nblk * bg) / (slots * 2048));
  bps = bps < 1 ? 1 : (bps > 8 ? 8 : bps);
  const int64_t gx = (nblk + (int64_t)slots * bps - 1) / ((int64_t)slots * bps);
  BRS_SCORE_LAUNCH((score_dot_kernel<T, EPL, G>), dim3((unsigned)gx, (unsigned)bg), dim3(256), s,
                     (const T*)q, (const T*)m.reps, scores, m.head_dim, m.reps_per_block, m.n_kv_heads,
                     m.capacity / m.block_size, lo, hi, bps, grouped);
  return hipGetLastError();
}

template <typename T, int EPL, int G, int L>
hipError_t run_rows(const brs_memory& m, const void* q, int64_t lo, int64_t hi, float* scores, int grouped,
                    hipStream_t s) {
  constexpr int slots = 4 * (64 / L);
  const int64_t rows = (hi - lo) * m.reps_per_block;
  const int64_t bg = (int64_t)m.batch * m.n_kv_heads;
  const int64_t want = rows * bg / (slots * 2048);
  const dim3 block(256);
  const int64_t capB = m.capacity / m.block_size;
  if (want >= 4) {
    const int64_t gx = (rows + slots * 4 - 1) / (slots * 4);
    BRS_SCORE_LAUNCH((score_dot_rows_kernel<T, EPL, G, L, 4>), dim3((unsigned)gx, (unsigned)bg), block, s,
                       (const T*)q, (const T*)m.reps, scores, m.head_dim, m.reps_per_block, m.n_kv_heads, capB, lo,
                       hi, grouped);
  } else if (want >= 2) {
    const int64_t gx = (rows + slots * 2 - 1) / (slots * 2);
    BRS_SCORE_LAUNCH((score_dot_rows_kernel<T, EPL, G, L, 2>), dim3((unsigned)gx, (unsigned)bg), block, s,
                       (const T*)q, (const T*)m.reps, scores, m.head_dim, m.reps_per_block, m.n_kv_heads, capB, lo,
                       hi, grouped);
  } else {
    const int64_t gx = (rows + slots - 1) / slots;
    BRS_SCORE_LAUNCH((score_dot_rows_kernel<T, EPL, G, L, 1>), dim3((unsigned)gx, (unsigned)bg), block, s,
                       (const T*)q, (const T*)m.reps, scores, m.head_dim, m.reps_per_block, m.n_kv_heads, capB, lo,
                       hi, grouped);
  }
  return hipGetLastError();
}

template <typename T, int EPL, int G>
hipError_t run_dot_any(const brs_memory& m, const void* q, int64_t lo, int64_t hi, float* scores, int grouped,
                       hipStream_t s) {
  // the row kernel needs R to divide the slots of a wave (64 / L of them)
  const int L = m.head_dim / EPL;
  const int R = m.reps_per_block;
  const bool rows_ok = (R & (R - 1)) == 0 && R <= 64 / L;
  if (rows_ok) {
    if (L == 4) return run_rows<T, EPL, G, 4>(m, q, lo, hi, scores, grouped, s);
    if (L == 8) return run_rows<T, EPL, G, 8>(m, q, lo, hi, scores, grouped, s);
    if (L == 16) return run_rows<T, EPL, G, 16>(m, q, lo, hi, scores, grouped, s);
  }
  return run_dot<T, EPL, G>(m, q, lo, hi, scores, grouped, s);
}

template <typename T>
hipError_t dispatch_dot(const brs_memory& m, const void* q, int G, int64_t lo, int64_t hi, float* scores,
                        int grouped, hipStream_t s) {
  constexpr int E16 = 16 / sizeof(T);  // elements per 16 bytes
  const int d = m.head_dim;
  auto fits = [&](int epl) {
    if (d % epl) return false;
    const int L = d / epl;
    return L >= 1 && L <= 64 && (L & (L - 1)) == 0;
  };
  auto qal = ((uintptr_t)q % 16) == 0;
  if (qal && (d * (int)sizeof(T)) % 16 == 0) {
    if (G <= 4 && fits(2 * E16)) {
      if (G == 1) return run_dot_any<T, 2 * E16, 1>(m, q, lo, hi, scores, grouped, s);
      if (G == 2) return run_dot_any<T, 2 * E16, 2>(m, q, lo, hi, scores, grouped, s);
      if (G == 4) return run_dot_any<T, 2 * E16, 4>(m, q, lo, hi, scores, grouped, s);
    }
    if (G == 8 && fits(E16)) return run_dot_any<T, E16, 8>(m, q, lo, hi, scores, grouped, s);
  }
  const int64_t bg = (int64_t)m.batch * m.n_kv_heads;
  const int64_t gx = (hi - lo + 3) / 4;
  BRS_SCORE_LAUNCH(score_dot_generic_kernel<T>, dim3((unsigned)gx, (unsigned)bg), dim3(256), s, (const T*)q,
                     (const T*)m.reps, scores, d, m.reps_per_block, m.n_kv_heads, G, m.capacity / m.block_size,
                     lo, hi, grouped);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_dot(const brs_memory& m, const void* q, int hq, int64_t lo, int64_t hi, float* scores,
                            bool grouped, hipStream_t s) {
  const int G = hq / m.n_kv_heads;
  const int gr = grouped ? 1 : 0;
  if (m.dtype == BRS_F32) return dispatch_dot<float>(m, q, G, lo, hi, scores, gr, s);
  return dispatch_dot<uint16_t>(m, q, G, lo, hi, scores, gr, s);
}

hipError_t launch_score_cosine(const brs_memory& m, const void* rq, int64_t lo, int64_t hi, float* scores,
                               hipStream_t s) {
  // whole 16-byte units, at most 8 per lane: the 16-lane rows
  const int vn = m.rep_dtype == BRS_F32 ? 4 : 8;
  const int upl = (m.rep_dim / vn + kCosLanes - 1) / kCosLanes;
  if (m.rep_dim % vn == 0 && upl <= 8) {
    const dim3 grid((unsigned)((hi - lo + 15) / 16), (unsigned)m.batch), block(256);
    const int64_t capB = m.capacity / m.block_size;
#define BRS_COS_ROWS(T, U)                                                                                 \
  BRS_SCORE_LAUNCH((score_cosine_rows_kernel<T, U>), grid, block, s, (const T*)rq, (const T*)m.reps, scores, \
                   m.rep_dim, capB, lo, hi)
    if (m.rep_dtype == BRS_F32) {
      if (upl <= 2) BRS_COS_ROWS(float, 2);
      else if (upl <= 4) BRS_COS_ROWS(float, 4);
      else BRS_COS_ROWS(float, 8);
    } else {
      if (upl <= 2) BRS_COS_ROWS(uint16_t, 2);
      else if (upl <= 4) BRS_COS_ROWS(uint16_t, 4);
      else if (upl <= 6) BRS_COS_ROWS(uint16_t, 6);
      else BRS_COS_ROWS(uint16_t, 8);
    }
#undef BRS_COS_ROWS
    return hipGetLastError();
  }
  const int64_t gx = (hi - lo + 3) / 4;
  if (m.rep_dtype == BRS_F32)
    BRS_SCORE_LAUNCH(score_cosine_kernel<float>, dim3((unsigned)gx, (unsigned)m.batch), dim3(256), s,
                       (const float*)rq, (const float*)m.reps, scores, m.rep_dim, m.capacity / m.block_size, lo,
                       hi);
  else
    BRS_SCORE_LAUNCH(score_cosine_kernel<uint16_t>, dim3((unsigned)gx, (unsigned)m.batch), dim3(256), s,
                       (const uint16_t*)rq, (const uint16_t*)m.reps, scores, m.rep_dim,
                       m.capacity / m.block_size, lo, hi);
  return hipGetLastError();
}

}  // namespace brs

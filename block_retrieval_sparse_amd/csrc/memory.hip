// Memory write path: copy new K/V rows into the block-contiguous memory and
// build the representatives of every block an append completes (MemLong
// 2.3.2 memorisation: K-V pairs stored with their index-aligned
// representation; InfLLM "method": a few tokens stand for each memory unit;
// Landmark Attention "proposed method": one landmark key per block).
#include "brs_internal.h"

namespace brs {
namespace {

// ---------------------------------------------------------------------------
// K/V append: rows of head_dim elements into rows of row_stride elements,
// padding columns set to zero.  U is the copy unit (16, 4 or 2 bytes).

template <typename U>
__global__ __launch_bounds__(256) void kv_append_kernel(const U* __restrict__ ksrc, const U* __restrict__ vsrc,
                                                        U* __restrict__ kdst, U* __restrict__ vdst,
                                                        int64_t rows, int hkv, int64_t n_new, int64_t cap,
                                                        int64_t len, int src_units, int dst_units) {
  const int64_t total = rows * dst_units;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / dst_units;
    const int u = (int)(i - r * dst_units);
    const int64_t t = r % n_new;
    const int64_t bg = r / n_new;  // batch * hkv + head
    const int64_t dst = ((bg * cap) + len + t) * dst_units + u;
    U kv{}, vv{};
    if (u < src_units) {
      kv = ksrc[r * src_units + u];
      vv = vsrc[r * src_units + u];
    }
    kdst[dst] = kv;
    vdst[dst] = vv;
  }
  (void)hkv;
}

// ---------------------------------------------------------------------------
// MEAN: rep = RNE_dtype( (sum of the block's keys in float64) / B ).

template <typename T>
__device__ __forceinline__ double load_as_f64(const T* p);
template <>
__device__ __forceinline__ double load_as_f64<float>(const float* p) { return (double)*p; }
template <>
__device__ __forceinline__ double load_as_f64<uint16_t>(const uint16_t* p) { return (double)bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_rounded(T* p, double x);
template <>
__device__ __forceinline__ void store_rounded<float>(float* p, double x) { *p = (float)x; }
template <>
__device__ __forceinline__ void store_rounded<uint16_t>(uint16_t* p, double x) { *p = f64_to_bf16_rne(x); }

template <typename T>
__global__ __launch_bounds__(256) void rep_mean_kernel(const T* __restrict__ K, T* __restrict__ reps, int64_t b0,
                                                       int B, int d, int rs, int64_t cap, int64_t capB) {
  const int64_t blk = b0 + blockIdx.x;
  const int64_t bg = blockIdx.y;
  const T* base = K + (bg * cap + blk * B) * (int64_t)rs;
  T* dst = reps + (bg * capB + blk) * (int64_t)d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    double s = 0.0;
    for (int t = 0; t < B; ++t) s += load_as_f64(base + (int64_t)t * rs + c);
    store_rounded(dst + c, s / (double)B);
  }
}

// ---------------------------------------------------------------------------
// TOPNORM: the R keys with the largest squared norm (float64 sums), ties to
// the lower token, copied unchanged in that order.

// Ranks the block's B keys in `key` (largest first, ties to the lower token)
// and copies the rows of the first R into dst, in rank order.  `chosen`
// starts as 0..R-1 so every slot names a valid token even for NaN keys.
template <typename T>
__device__ void rank_and_copy(const double* key, int* chosen, const T* base, T* dst, int B, int R, int d,
                              int rs) {
  for (int t = threadIdx.x; t < B; t += blockDim.x) {
    const double mine = key[t];
    int rank = 0;
    for (int u = 0; u < B; ++u) {
      const double o = key[u];
      rank += (o > mine) || (o == mine && u < t);
    }
    if (rank < R) chosen[rank] = t;  // ranks are distinct for finite keys
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * d; i += blockDim.x) {
    const int r = i / d, c = i - r * d;
    dst[i] = base[(int64_t)chosen[r] * rs + c];
  }
}

// Row-parallel forms of MEAN and TOPNORM, for rows whose head dims are whole
// 16-byte units (U per row, U <= L): L lanes share a row, lane `sub` holding
// unit `sub`, 256 / L rows per pass, `passes` passes (at most kRowPasses);
// every load of the block is issued before any is used.  Same arithmetic
// as the per-column / per-row forms: float64 sums, one rounding.
constexpr int kRowPasses = 16;

template <typename T>
struct Unit;  // the elements of a 16-byte unit as float64
template <>
struct Unit<uint16_t> {
  static constexpr int n = 8;
  __device__ static double at(const uint4& u, int e) {
    const int k = e >> 1;  // the 32-bit word; element 2k in its low half, 2k + 1 in its high half
    const uint32_t w = k == 0 ? u.x : (k == 1 ? u.y : (k == 2 ? u.z : u.w));
    return (double)((e & 1) ? bf16_hi(w) : bf16_lo(w));
  }
};
template <>
struct Unit<float> {
  static constexpr int n = 4;
  __device__ static double at(const uint4& u, int e) {
    return (double)__uint_as_float(e == 0 ? u.x : (e == 1 ? u.y : (e == 2 ? u.z : u.w)));
  }
};

template <typename T, int L>
__device__ __forceinline__ void load_block_rows(const T* base, int B, int rs, int U, int passes, uint4 (&raw)[kRowPasses]) {
  constexpr int RPP = 256 / L;
  const int sub = threadIdx.x % L, rw = threadIdx.x / L;
  const int uu = sub < U ? sub : 0;
#pragma unroll
  for (int p = 0; p < kRowPasses; ++p) {
    if (p < passes) {
      const int t = p * RPP + rw;
      const int tt = t < B ? t : 0;  // rows past the block re-read row 0 (no branch around the loads)
      raw[p] = *reinterpret_cast<const uint4*>(base + (int64_t)tt * rs + uu * Unit<T>::n);
    }
  }
}

template <typename T, int L>
__global__ __launch_bounds__(256) void rep_mean_rows_kernel(const T* __restrict__ K, T* __restrict__ reps,
                                                            int64_t b0, int B, int d, int rs, int64_t cap,
                                                            int64_t capB, int passes) {
  constexpr int RPP = 256 / L, VN = Unit<T>::n;
  __shared__ double part[RPP][L * VN];
  const int64_t blk = b0 + blockIdx.x;
  const int64_t bg = blockIdx.y;
  const T* base = K + (bg * cap + blk * B) * (int64_t)rs;
  const int U = d / VN;
  const int sub = threadIdx.x % L, rw = threadIdx.x / L;
  uint4 raw[kRowPasses];
  load_block_rows<T, L>(base, B, rs, U, passes, raw);
  double acc[VN];
#pragma unroll
  for (int e = 0; e < VN; ++e) acc[e] = 0.0;
#pragma unroll
  for (int p = 0; p < kRowPasses; ++p)
    if (p < passes && p * RPP + rw < B) {
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] += Unit<T>::at(raw[p], e);
    }
#pragma unroll
  for (int e = 0; e < VN; ++e) part[rw][sub * VN + e] = acc[e];
  __syncthreads();
  T* dst = reps + (bg * capB + blk) * (int64_t)d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    double s = 0.0;
    for (int r = 0; r < RPP; ++r) s += part[r][c];
    store_rounded(dst + c, s / (double)B);
  }
}

template <typename T, int L>
__global__ __launch_bounds__(256) void rep_topnorm_rows_kernel(const T* __restrict__ K, T* __restrict__ reps,
                                                               int64_t b0, int B, int R, int d, int rs, int64_t cap,
                                                               int64_t capB, int passes) {
  constexpr int RPP = 256 / L, VN = Unit<T>::n;
  __shared__ double n2[kRowPasses * RPP];
  __shared__ int chosen[64];
  const int64_t blk = b0 + blockIdx.x;
  const int64_t bg = blockIdx.y;
  const T* base = K + (bg * cap + blk * B) * (int64_t)rs;
  const int U = d / VN;
  const int sub = threadIdx.x % L, rw = threadIdx.x / L;
  if (threadIdx.x < R) chosen[threadIdx.x] = threadIdx.x;
  uint4 raw[kRowPasses];
  load_block_rows<T, L>(base, B, rs, U, passes, raw);
#pragma unroll
  for (int p = 0; p < kRowPasses; ++p) {
    if (p < passes) {
      double s = 0.0;
      if (sub < U) {
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          const double x = Unit<T>::at(raw[p], e);
          s = fma(x, x, s);
        }
      }
      for (int off = 1; off < L; off <<= 1) s += __shfl_xor(s, off);
      const int t = p * RPP + rw;
      if (sub == 0 && t < B) n2[t] = s;
    }
  }
  __syncthreads();
  rank_and_copy(n2, chosen, base, reps + (bg * capB + blk) * (int64_t)R * d, B, R, d, rs);
}

template <typename T>
__global__ __launch_bounds__(256) void rep_topnorm_kernel(const T* __restrict__ K, T* __restrict__ reps,
                                                          int64_t b0, int B, int R, int d, int rs, int64_t cap,
                                                          int64_t capB) {
  __shared__ double n2[1024];
  __shared__ int chosen[64];
  const int64_t blk = b0 + blockIdx.x;
  const int64_t bg = blockIdx.y;
  const T* base = K + (bg * cap + blk * B) * (int64_t)rs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  if (threadIdx.x < R) chosen[threadIdx.x] = threadIdx.x;
  for (int t = wave; t < B; t += nwaves) {
    double s = 0.0;
    for (int c = lane; c < d; c += 64) {
      const double x = load_as_f64(base + (int64_t)t * rs + c);
      s = fma(x, x, s);
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) n2[t] = s;
  }
  __syncthreads();
  rank_and_copy(n2, chosen, base, reps + (bg * capB + blk) * (int64_t)R * d, B, R, d, rs);
}

// ---------------------------------------------------------------------------
// ATTNSCORE: the R keys with the largest accumulated attention mass (InfLLM
// "method"), ties to the lower token, copied unchanged in that order.

template <typename T>
__global__ __launch_bounds__(256) void rep_mass_kernel(const T* __restrict__ K, T* __restrict__ reps,
                                                       const float* __restrict__ mass, int64_t b0, int B, int R,
                                                       int d, int rs, int64_t cap, int64_t capB) {
  __shared__ double key[1024];
  __shared__ int chosen[64];
  const int64_t blk = b0 + blockIdx.x;
  const int64_t bg = blockIdx.y;
  const T* base = K + (bg * cap + blk * B) * (int64_t)rs;
  if (threadIdx.x < R) chosen[threadIdx.x] = threadIdx.x;
  for (int t = threadIdx.x; t < B; t += blockDim.x) key[t] = (double)mass[bg * cap + blk * B + t];
  __syncthreads();
  rank_and_copy(key, chosen, base, reps + (bg * capB + blk) * (int64_t)R * d, B, R, d, rs);
}

// ---------------------------------------------------------------------------
// GIVEN / EMBED: copy the caller's vectors into the block slots.

template <typename T>
__global__ __launch_bounds__(256) void rep_copy_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t per_head,
                                                       int64_t heads, int64_t head_stride, int64_t dst_off) {
  const int64_t total = per_head * heads;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t h = i / per_head, e = i - h * per_head;
    dst[h * head_stride + dst_off + e] = src[i];
  }
}

int grid_for(int64_t work) {
  int64_t g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_kv_append(const brs_memory& m, const void* k_new, const void* v_new, int64_t n_new,
                            hipStream_t s) {
  const int es = elem_bytes(m.dtype);
  const int64_t rows = (int64_t)m.batch * m.n_kv_heads * n_new;
  const int src_bytes = m.head_dim * es, dst_bytes = m.row_stride * es;
  auto al = [](const void* p, int a) { return ((uintptr_t)p % a) == 0; };
  if (src_bytes % 16 == 0 && dst_bytes % 16 == 0 && al(k_new, 16) && al(v_new, 16)) {
    hipLaunchKernelGGL(kv_append_kernel<uint4>, dim3(grid_for(rows * (dst_bytes / 16))), dim3(256), 0, s,
                       (const uint4*)k_new, (const uint4*)v_new, (uint4*)m.k, (uint4*)m.v, rows, m.n_kv_heads,
                       n_new, m.capacity, m.length, src_bytes / 16, dst_bytes / 16);
  } else if (src_bytes % 4 == 0 && al(k_new, 4) && al(v_new, 4)) {
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, dim3(grid_for(rows * (dst_bytes / 4))), dim3(256), 0, s,
                       (const uint32_t*)k_new, (const uint32_t*)v_new, (uint32_t*)m.k, (uint32_t*)m.v, rows,
                       m.n_kv_heads, n_new, m.capacity, m.length, src_bytes / 4, dst_bytes / 4);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(grid_for(rows * (dst_bytes / 2))), dim3(256), 0, s,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)m.k, (uint16_t*)m.v, rows,
                       m.n_kv_heads, n_new, m.capacity, m.length, src_bytes / 2, dst_bytes / 2);
  }
  return hipGetLastError();
}

hipError_t launch_reps_from_mass(const brs_memory& m, const float* mass, int64_t b0, int64_t b1, hipStream_t s) {
  const int64_t capB = m.capacity / m.block_size;
  const int64_t heads = (int64_t)m.batch * m.n_kv_heads;
  for (int64_t done = 0; done < b1 - b0; done += 65535) {
    const int64_t n = b1 - b0 - done < 65535 ? b1 - b0 - done : 65535;
    const dim3 grid((unsigned)n, (unsigned)heads);
    if (m.dtype == BRS_F32)
      hipLaunchKernelGGL(rep_mass_kernel<float>, grid, dim3(256), 0, s, (const float*)m.k, (float*)m.reps, mass,
                         b0 + done, m.block_size, m.reps_per_block, m.head_dim, m.row_stride, m.capacity, capB);
    else
      hipLaunchKernelGGL(rep_mass_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)m.k,
                         (uint16_t*)m.reps, mass, b0 + done, m.block_size, m.reps_per_block, m.head_dim,
                         m.row_stride, m.capacity, capB);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_rep_build(const brs_memory& m, int64_t b0, int64_t b1, const void* reps_new, hipStream_t s) {
  const int64_t nblk = b1 - b0;
  const int64_t capB = m.capacity / m.block_size;
  const int64_t heads = (int64_t)m.batch * m.rep_heads;
  if (m.rep_mode == BRS_REP_GIVEN || m.rep_mode == BRS_REP_EMBED) {
    const int64_t per_block = (int64_t)m.reps_per_block * m.rep_dim;
    const int64_t per_head = nblk * per_block;
    if (m.rep_dtype == BRS_F32)
      hipLaunchKernelGGL(rep_copy_kernel<float>, dim3(grid_for(per_head * heads)), dim3(256), 0, s,
                         (const float*)reps_new, (float*)m.reps, per_head, heads, capB * per_block,
                         b0 * per_block);
    else
      hipLaunchKernelGGL(rep_copy_kernel<uint16_t>, dim3(grid_for(per_head * heads)), dim3(256), 0, s,
                         (const uint16_t*)reps_new, (uint16_t*)m.reps, per_head, heads, capB * per_block,
                         b0 * per_block);
    return hipGetLastError();
  }
  // the row-parallel forms when a row's head dims are whole 16-byte units
  // (at most 32 per row) and the block fits in kRowPasses passes
  const int es = elem_bytes(m.dtype);
  const int U = (m.head_dim * es) % 16 == 0 ? m.head_dim * es / 16 : 0;
  const int L = U <= 0 ? 0 : (U <= 4 ? 4 : (U <= 8 ? 8 : (U <= 16 ? 16 : (U <= 32 ? 32 : 0))));
  const int passes = L ? (m.block_size + 256 / L - 1) / (256 / L) : 0;
  const bool rows = L > 0 && passes <= kRowPasses && (m.row_stride * es) % 16 == 0 &&
                    ((uintptr_t)m.k % 16) == 0;
  // the grid's y dimension covers (batch, kv head); x covers the new blocks
  for (int64_t done = 0; done < nblk; done += 65535) {
    const int64_t n = nblk - done < 65535 ? nblk - done : 65535;
    const dim3 grid((unsigned)n, (unsigned)heads);
    if (rows && (m.rep_mode == BRS_REP_MEAN || m.rep_mode == BRS_REP_TOPNORM)) {
      const bool mean = m.rep_mode == BRS_REP_MEAN;
#define BRS_ROWS_LAUNCH(T, LL)                                                                                   \
  if (L == LL) {                                                                                                 \
    if (mean)                                                                                                    \
      hipLaunchKernelGGL((rep_mean_rows_kernel<T, LL>), grid, dim3(256), 0, s, (const T*)m.k, (T*)m.reps,       \
                         b0 + done, m.block_size, m.head_dim, m.row_stride, m.capacity, capB, passes);          \
    else                                                                                                         \
      hipLaunchKernelGGL((rep_topnorm_rows_kernel<T, LL>), grid, dim3(256), 0, s, (const T*)m.k, (T*)m.reps,    \
                         b0 + done, m.block_size, m.reps_per_block, m.head_dim, m.row_stride, m.capacity, capB, \
                         passes);                                                                                \
  }
      if (m.dtype == BRS_F32) {
        BRS_ROWS_LAUNCH(float, 4)
        BRS_ROWS_LAUNCH(float, 8)
        BRS_ROWS_LAUNCH(float, 16)
        BRS_ROWS_LAUNCH(float, 32)
      } else {
        BRS_ROWS_LAUNCH(uint16_t, 4)
        BRS_ROWS_LAUNCH(uint16_t, 8)
        BRS_ROWS_LAUNCH(uint16_t, 16)
        BRS_ROWS_LAUNCH(uint16_t, 32)
      }
#undef BRS_ROWS_LAUNCH
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      continue;
    }
    if (m.rep_mode == BRS_REP_MEAN) {
      if (m.dtype == BRS_F32)
        hipLaunchKernelGGL(rep_mean_kernel<float>, grid, dim3(128), 0, s, (const float*)m.k, (float*)m.reps,
                           b0 + done, m.block_size, m.head_dim, m.row_stride, m.capacity, capB);
      else
        hipLaunchKernelGGL(rep_mean_kernel<uint16_t>, grid, dim3(128), 0, s, (const uint16_t*)m.k,
                           (uint16_t*)m.reps, b0 + done, m.block_size, m.head_dim, m.row_stride, m.capacity,
                           capB);
    } else {
      if (m.dtype == BRS_F32)
        hipLaunchKernelGGL(rep_topnorm_kernel<float>, grid, dim3(256), 0, s, (const float*)m.k, (float*)m.reps,
                           b0 + done, m.block_size, m.reps_per_block, m.head_dim, m.row_stride, m.capacity,
                           capB);
      else
        hipLaunchKernelGGL(rep_topnorm_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)m.k,
                           (uint16_t*)m.reps, b0 + done, m.block_size, m.reps_per_block, m.head_dim,
                           m.row_stride, m.capacity, capB);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace brs

// Attention mass of the local window (InfLLM "method": the representative
// tokens of a memory unit are the ones that received the highest attention
// scores in earlier attention computations).
//
// After an attention call that reported each query's log-sum-exp, every
// token t of the window gains the softmax weight it received,
//     exp(scale * q.k_t - lse),
// summed over the query heads of its kv head and the queries that see it.
//
// Layout: one workgroup per (batch, kv head, 64 window tokens).  The group's
// query rows (G heads x n_q queries) are taken 64 at a time; the K tile and
// the query tile move through LDS as float32 in 64-column chunks, and each
// thread forms a 4 x 4 block of (token, row) dot products.  A token's sum is
// added to its mass entry by the one thread that owns it, after a reduction
// in a fixed order, so the result is deterministic.
#include <hip/hip_ext.h>

#include "brs_internal.h"

namespace brs {
namespace {

constexpr int kMassTok = 64;   // window tokens per workgroup
constexpr int kMassRows = 64;  // query rows per pass
constexpr int kMassCols = 64;  // head-dim columns per LDS chunk
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ float elem_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float elem_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float elem_f32<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

struct MassArgs {
  const void* k;
  const void* q;
  const float* lse;
  float* mass;
  int64_t cap;   // token rows per (batch, kv head)
  int rs;        // row stride (elements)
  int d, hq, hkv, G, n_q, N;
  int w0;        // first window token
  float scale2;  // scale * log2(e)
};

template <typename T>
__global__ __launch_bounds__(256) void window_mass_kernel(MassArgs a) {
  __shared__ float sk[kMassTok][kMassCols + 1];
  __shared__ float sq[kMassRows][kMassCols + 1];
  __shared__ float s_lse[kMassRows];
  __shared__ int s_pos[kMassRows];
  __shared__ float s_part[16][kMassTok];

  const int tid = threadIdx.x;
  const int tt = tid & 15, rr = tid >> 4;  // tokens tt + 16 i, rows rr + 16 j
  const int bg = blockIdx.y;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int t0 = a.w0 + blockIdx.x * kMassTok;
  const T* K = reinterpret_cast<const T*>(a.k) + ((int64_t)bg * a.cap) * a.rs;
  const T* Q = reinterpret_cast<const T*>(a.q);
  const int n_rows = a.G * a.n_q;

  float tsum[4] = {0.f, 0.f, 0.f, 0.f};
  int tpos[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tpos[i] = t0 + tt + 16 * i;

  for (int r0 = 0; r0 < n_rows; r0 += kMassRows) {
    __syncthreads();  // the previous pass's readers of s_lse / s_pos are done
    if (tid < kMassRows) {
      const int r = r0 + tid;
      if (r < n_rows) {
        const int h = g * a.G + r / a.n_q, j = r % a.n_q;
        s_lse[tid] = a.lse[((int64_t)b * a.hq + h) * a.n_q + j] * kLog2e;
        s_pos[tid] = a.N - a.n_q + j;
      } else {
        s_lse[tid] = INFINITY;  // weight exp2(x - inf) = 0
        s_pos[tid] = -1;
      }
    }
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int c0 = 0; c0 < a.d; c0 += kMassCols) {
      __syncthreads();
      // K rows t0.., query rows r0.., columns c0.. (zeros past the ends)
      const int c = c0 + (tid & 63);
      for (int u = tid >> 6; u < kMassTok; u += 4) {
        const int t = t0 + u;
        sk[u][tid & 63] = (t < a.N && c < a.d) ? elem_f32<T>(K, (int64_t)t * a.rs + c) : 0.f;
        const int r = r0 + u;
        float qv = 0.f;
        if (r < n_rows && c < a.d) {
          const int h = g * a.G + r / a.n_q, j = r % a.n_q;
          qv = elem_f32<T>(Q, (((int64_t)b * a.hq + h) * a.n_q + j) * a.d + c);
        }
        sq[u][tid & 63] = qv;
      }
      __syncthreads();
#pragma unroll 4
      for (int cc = 0; cc < kMassCols; ++cc) {
        float kv[4], qv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kv[i] = sk[tt + 16 * i][cc];
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[j] = sq[rr + 16 * j][cc];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(kv[i], qv[j], acc[i][j]);
      }
    }
    // softmax weights of this pass's rows, summed per token
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rl = rr + 16 * j;
        const bool vis = tpos[i] < a.N && tpos[i] <= s_pos[rl];
        tsum[i] += vis ? exp2f(fmaf(acc[i][j], a.scale2, -s_lse[rl])) : 0.f;
      }
  }
  // reduce over the 16 row groups in a fixed order; one thread per token adds
#pragma unroll
  for (int i = 0; i < 4; ++i) s_part[rr][tt + 16 * i] = tsum[i];
  __syncthreads();
  if (tid < kMassTok) {
    const int t = t0 + tid;
    if (t < a.N) {
      float s = 0.f;
      for (int k = 0; k < 16; ++k) s += s_part[k][tid];
      float* m = a.mass + (int64_t)bg * a.cap + t;
      *m += s;
    }
  }
}

// Few query rows (decode: G heads x n_q <= 16): a token row is read with one
// 16-byte load per lane, L lanes per token, and every lane keeps its slice of
// all the rows' queries in registers; the dot products are summed across the
// L lanes with DPP moves.  Each wave issues the loads of IT token steps at
// once.  Requires d = L * (16 / sizeof(T)) and 16-byte aligned rows.
template <int L>
__device__ __forceinline__ float lanes_sum(float v) {
  if constexpr (L >= 2) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
  if constexpr (L >= 4) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
  if constexpr (L >= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));
  if constexpr (L >= 16) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false));
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  return v;
}

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& u, float* x);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& u, float* x) {
  x[0] = __uint_as_float(u.x);
  x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z);
  x[3] = __uint_as_float(u.w);
}

constexpr int kMassIt = 4;  // token steps per wave

template <typename T, int L, int NR>
__global__ __launch_bounds__(256) void window_mass_rows_kernel(MassArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int TPW = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % L, slot = lane / L;
  const int bg = blockIdx.y;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int n_rows = a.G * a.n_q;
  const T* Q = reinterpret_cast<const T*>(a.q);
  float qv[NR][EPL], lse2[NR];
  int pos[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r < n_rows) {
      const int h = g * a.G + r / a.n_q, j = r % a.n_q;
      const int64_t row = ((int64_t)b * a.hq + h) * a.n_q + j;
      unpack16<T>(*reinterpret_cast<const uint4*>(Q + row * a.d + sub * EPL), qv[r]);
      lse2[r] = a.lse[row] * kLog2e;
      pos[r] = a.N - a.n_q + j;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[r][e] = 0.f;
      lse2[r] = 0.f;
      pos[r] = -1;  // sees nothing
    }
  }
  const T* K = reinterpret_cast<const T*>(a.k) + ((int64_t)bg * a.cap) * a.rs + sub * EPL;
  const int tw = a.w0 + (blockIdx.x * 4 + wave) * (kMassIt * TPW) + slot;
  uint4 raw[kMassIt];
#pragma unroll
  for (int it = 0; it < kMassIt; ++it) {
    const int t = tw + it * TPW;
    raw[it] = t < a.N ? *reinterpret_cast<const uint4*>(K + (int64_t)t * a.rs) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < kMassIt; ++it) {
    const int t = tw + it * TPW;
    float x[EPL];
    unpack16<T>(raw[it], x);
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(x[e], qv[r][e], dot);
      dot = lanes_sum<L>(dot);
      acc += (t <= pos[r]) ? exp2f(fmaf(dot, a.scale2, -lse2[r])) : 0.f;
    }
    if (sub == 0 && t < a.N) a.mass[(int64_t)bg * a.cap + t] += acc;
  }
}

// launch, with the caller's timing events attached when given
template <typename K>
void launch(K kernel, dim3 grid, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const MassArgs& a) {
  if (ev0)
    hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, s, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, a);
}

template <typename T, int L>
bool launch_rows(const MassArgs& a, int n_rows, int64_t n_tok, int heads, hipStream_t s, hipEvent_t ev0,
                 hipEvent_t ev1) {
  constexpr int per_wg = 4 * kMassIt * (64 / L);
  const dim3 grid((unsigned)((n_tok + per_wg - 1) / per_wg), (unsigned)heads);
  if (n_rows <= 4)
    launch(window_mass_rows_kernel<T, L, 4>, grid, s, ev0, ev1, a);
  else if (n_rows <= 8)
    launch(window_mass_rows_kernel<T, L, 8>, grid, s, ev0, ev1, a);
  else if (n_rows <= 16)
    launch(window_mass_rows_kernel<T, L, 16>, grid, s, ev0, ev1, a);
  else
    return false;
  return true;
}

template <typename T>
bool try_rows(const MassArgs& a, const brs_memory& m, int n_rows, int64_t n_tok, hipStream_t s, hipEvent_t ev0,
              hipEvent_t ev1) {
  const int es = (int)sizeof(T), epl = 16 / es;
  if (m.head_dim % epl || (m.row_stride * es) % 16 || ((uintptr_t)a.q % 16)) return false;
  const int L = m.head_dim / epl;
  const int heads = m.batch * m.n_kv_heads;
  if (L == 8) return launch_rows<T, 8>(a, n_rows, n_tok, heads, s, ev0, ev1);
  if (L == 16) return launch_rows<T, 16>(a, n_rows, n_tok, heads, s, ev0, ev1);
  if (L == 32) return launch_rows<T, 32>(a, n_rows, n_tok, heads, s, ev0, ev1);
  return false;
}

}  // namespace

hipError_t launch_window_mass(const brs_memory& m, const void* q, int hq, int n_q, const float* lse, int64_t w0,
                              float scale, float* mass, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  MassArgs a;
  a.k = m.k;
  a.q = q;
  a.lse = lse;
  a.mass = mass;
  a.cap = m.capacity;
  a.rs = m.row_stride;
  a.d = m.head_dim;
  a.hq = hq;
  a.hkv = m.n_kv_heads;
  a.G = hq / m.n_kv_heads;
  a.n_q = n_q;
  a.N = (int)m.length;
  a.w0 = (int)w0;
  a.scale2 = scale * kLog2e;
  const int64_t tiles = (m.length - w0 + kMassTok - 1) / kMassTok;
  if (tiles <= 0) return hipSuccess;
  const int n_rows = a.G * n_q;
  const bool rows = m.dtype == BRS_F32 ? try_rows<float>(a, m, n_rows, m.length - w0, s, ev0, ev1)
                                       : try_rows<uint16_t>(a, m, n_rows, m.length - w0, s, ev0, ev1);
  if (rows) return hipGetLastError();
  const dim3 grid((unsigned)tiles, (unsigned)(m.batch * m.n_kv_heads));
  if (m.dtype == BRS_F32)
    launch(window_mass_kernel<float>, grid, s, ev0, ev1, a);
  else
    launch(window_mass_kernel<uint16_t>, grid, s, ev0, ev1, a);
  return hipGetLastError();
}

}  // namespace brs

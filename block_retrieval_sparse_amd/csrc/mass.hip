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

}  // namespace

hipError_t launch_window_mass(const brs_memory& m, const void* q, int hq, int n_q, const float* lse, int64_t w0,
                              float scale, float* mass, hipStream_t s) {
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
  const dim3 grid((unsigned)tiles, (unsigned)(m.batch * m.n_kv_heads));
  if (m.dtype == BRS_F32)
    hipLaunchKernelGGL(window_mass_kernel<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(window_mass_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace brs

// Retrieval attention, split-K over the attended set (InfLLM "method":
// local tokens plus a few memory units; Landmark Attention "proposed method":
// a block's tokens are read only when the block is selected;
// RetrievalAttention "proposed method": attention restricted to the tokens
// that matter, exact over them).
//
//   plan   one workgroup per (batch, kv head): marks the blocks any query
//          head of the group selected (a head bitmask per block, in LDS),
//          clips them against sinks and window so every token appears once,
//          and writes work items (first row, length <= 128, head mask):
//          sinks, window, then the selected blocks in index order.
//   split  one workgroup per (batch, kv head, run of items): streams each
//          item's K and V rows once for all query rows of the group, with an
//          online softmax in float32 (log2 domain), and writes a partial
//          (max, sum, weighted V) per query row.
//   merge  one wave per query row: combines the partials by log-sum-exp in
//          a fixed order (deterministic).
#include <hip/hip_ext.h>
#include <math.h>

#include "brs_internal.h"

namespace brs {
namespace {

constexpr float kNegInf = -INFINITY;

struct PlanArgs {
  const int32_t* idx;
  int4* plan;
  int64_t max_items;
  int hq, hkv, G, k, idx_heads;
  int N, B, nb, sink_end, win_start;
};

// ---------------------------------------------------------------------------
// plan

__global__ __launch_bounds__(1024) void attn_plan_kernel(PlanArgs a) {
  __shared__ uint32_t marks[kMarkBlocks];
  __shared__ int wave_tot[16];
  __shared__ int sh_total;
  const int bg = blockIdx.x;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  int4* plan = a.plan + (int64_t)bg * (1 + a.max_items);
  const int tid = threadIdx.x, nt = blockDim.x;
  const uint32_t full = a.G >= 32 ? 0xffffffffu : ((1u << a.G) - 1u);

  // shared part: sinks [0, S') and window [ws, N), in pieces of <= kItemTokens
  const int n_sink_items = (a.sink_end + kItemTokens - 1) / kItemTokens;
  const int n_win_items = (a.N - a.win_start + kItemTokens - 1) / kItemTokens;
  for (int i = tid; i < n_sink_items + n_win_items; i += nt) {
    int p0, end;
    if (i < n_sink_items) {
      p0 = i * kItemTokens;
      end = a.sink_end;
    } else {
      p0 = a.win_start + (i - n_sink_items) * kItemTokens;
      end = a.N;
    }
    plan[1 + i] = make_int4(p0, min(kItemTokens, end - p0), (int)full, 0);
  }

  const int E = a.idx_heads == 1 ? a.k : a.G * a.k;
  int written = n_sink_items + n_win_items;
  for (int base = 0; base < a.nb; base += kMarkBlocks) {
    for (int i = tid; i < kMarkBlocks; i += nt) marks[i] = 0u;
    __syncthreads();
    const int top = min(a.nb, base + kMarkBlocks);
    for (int e = tid; e < E; e += nt) {
      int blk;
      uint32_t bit;
      if (a.idx_heads == 1) {
        blk = a.idx[(int64_t)b * a.k + e];
        bit = full;
      } else {
        const int j = e / a.k;
        blk = a.idx[((int64_t)b * a.hq + g * a.G + j) * a.k + (e - j * a.k)];
        bit = 1u << j;
      }
      if (blk >= base && blk < top) {
        const int lo_t = max(blk * a.B, a.sink_end);
        const int hi_t = min((blk + 1) * a.B, a.win_start);
        if (lo_t < hi_t) atomicOr(&marks[blk - base], bit);
      }
    }
    __syncthreads();
    // each thread owns a contiguous run of blocks
    const int per = (kMarkBlocks + nt - 1) / nt;
    const int r0 = base + tid * per, r1 = min(top, r0 + per);
    int cnt = 0;
    for (int blk = r0; blk < r1; ++blk) {
      if (marks[blk - base]) {
        const int len = min((blk + 1) * a.B, a.win_start) - max(blk * a.B, a.sink_end);
        cnt += (len + kItemTokens - 1) / kItemTokens;
      }
    }
    const int incl = block_inclusive_scan(cnt, wave_tot);
    int off = written + incl - cnt;
    for (int blk = r0; blk < r1; ++blk) {
      const uint32_t mk = marks[blk - base];
      if (!mk) continue;
      const int lo_t = max(blk * a.B, a.sink_end);
      const int hi_t = min((blk + 1) * a.B, a.win_start);
      for (int p = lo_t; p < hi_t; p += kItemTokens) plan[1 + off++] = make_int4(p, min(kItemTokens, hi_t - p), (int)mk, 0);
    }
    if (tid == nt - 1) sh_total = incl;
    __syncthreads();
    written += sh_total;
    __syncthreads();
  }
  if (tid == 0) plan[0] = make_int4(written, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// split

struct SplitArgs {
  const void* k;
  const void* v;
  const void* q;
  const int4* plan;
  float2* ml;
  float* o;
  int64_t max_items;
  int64_t head_stride;
  int row_stride;
  int hq, hkv, G, n_q, N, d;
  float qscale;
  int ipw, nw, max_chunks;
  int rows, rows_per_group;
};

template <typename T>
struct Elt;
template <>
struct Elt<uint16_t> {  // bfloat16 storage
  static constexpr int per16 = 8;
  __device__ static void unpack(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  __device__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
};
template <>
struct Elt<float> {
  static constexpr int per16 = 4;
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ static float load(const float* p) { return *p; }
};

// Writes the workgroup's combined partial for each active row.  o_lane holds
// this lane's DPL dims [sub*DPL, sub*DPL+DPL) for each row; rows beyond
// `rows` are ignored.
template <int D, int DPL, int ROWS>
__device__ void write_partials(const SplitArgs& a, int bg, int c, int rg, int rows_here, float (&m)[ROWS],
                               float (&l)[ROWS], float (&o)[ROWS][DPL], int slot, int sub, int wave, int nw) {
  __shared__ float s_o[4][ROWS][D];
  __shared__ float s_m[4][ROWS];
  __shared__ float s_l[4][ROWS];
  if (slot == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) s_o[wave][r][sub * DPL + e] = o[r][e];
      if (sub == 0) {
        s_m[wave][r] = m[r];
        s_l[wave][r] = l[r];
      }
    }
  }
  __syncthreads();
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  for (int t = threadIdx.x; t < rows_here * D; t += blockDim.x) {
    const int r = t / D, e = t - r * D;
    float M = kNegInf;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, s_m[w][r]);
    float Ls = 0.f, Os = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float mw = s_m[w][r];
      const float f = (mw == kNegInf) ? 0.f : exp2f(mw - M);
      Ls += s_l[w][r] * f;
      Os += s_o[w][r][e] * f;
    }
    const int gr = rg * a.rows_per_group + r;
    const int j = gr / a.n_q, i = gr - j * a.n_q;
    const int64_t row = ((int64_t)b * a.hq + g * a.G + j) * a.n_q + i;
    const int64_t pidx = row * a.max_chunks + c;
    a.o[pidx * D + e] = Os;
    if (e == 0) a.ml[pidx] = make_float2(M, Ls);
  }
}

// Fast path: D = head_dim, rows 16-byte aligned.  L = D / DPL lanes share a
// token (each loads DPL contiguous elements of the K row and of the V row),
// TPS = 64 / L tokens per wave step, U steps in flight.
template <typename T, int D, int DPL, int ROWS>
__global__ __launch_bounds__(256) void attn_split_kernel(SplitArgs a) {
  constexpr int L = D / DPL;
  constexpr int TPS = 64 / L;
  constexpr int NU = DPL / Elt<T>::per16;  // 16-byte units per lane per row
  constexpr int U = 2;
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lanes per token");
  static_assert(NU >= 1 && NU * Elt<T>::per16 == DPL, "16-byte units");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / L, sub = lane % L;
  const int c = blockIdx.x, bg = blockIdx.y, rg = blockIdx.z;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int4* plan = a.plan + (int64_t)bg * (1 + a.max_items);
  const int n_items = min((int64_t)plan[0].x, a.max_items);
  const int it0 = c * a.ipw;
  if (it0 >= n_items) return;
  const int it1 = min(it0 + a.ipw, n_items);
  const int rows_here = min(a.rows_per_group, a.rows - rg * a.rows_per_group);

  // query rows of this group, pre-multiplied by scale * log2(e)
  float qf[ROWS][DPL];
  uint32_t rowbit[ROWS];
  int plim[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int gr = rg * a.rows_per_group + r;
    const bool act = r < rows_here;
    const int j = act ? gr / a.n_q : 0, i = act ? gr - j * a.n_q : 0;
    rowbit[r] = act ? (1u << j) : 0u;
    plim[r] = a.N - a.n_q + i;
    const T* qrow = (const T*)a.q + (((int64_t)b * a.hq + g * a.G + j) * a.n_q + i) * D + sub * DPL;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      uint4 raw = act ? *reinterpret_cast<const uint4*>(qrow + u * Elt<T>::per16) : make_uint4(0, 0, 0, 0);
      Elt<T>::unpack(raw, &qf[r][u * Elt<T>::per16]);
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) qf[r][e] *= a.qscale;
  }

  float m[ROWS], l[ROWS], o[ROWS][DPL];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[r][e] = 0.f;
  }

  const T* kb = (const T*)a.k + (int64_t)bg * a.head_stride + sub * DPL;
  const T* vb = (const T*)a.v + (int64_t)bg * a.head_stride + sub * DPL;

  for (int it = it0 + wave; it < it1; it += a.nw) {
    const int4 item = plan[1 + it];
    const int pos0 = item.x, len = item.y;
    const uint32_t mask = (uint32_t)item.z;
    for (int t0 = 0; t0 < len; t0 += TPS * U) {
      uint4 kr[U][NU], vr[U][NU];
      int pos[U];
      bool val[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * TPS + slot;
        val[u] = t < len;
        pos[u] = pos0 + t;
        const int64_t off = (int64_t)(val[u] ? pos[u] : pos0) * a.row_stride;
#pragma unroll
        for (int w = 0; w < NU; ++w) {
          kr[u][w] = *reinterpret_cast<const uint4*>(kb + off + w * Elt<T>::per16);
          vr[u][w] = *reinterpret_cast<const uint4*>(vb + off + w * Elt<T>::per16);
        }
      }
      float s[U][ROWS];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kf[DPL];
#pragma unroll
        for (int w = 0; w < NU; ++w) Elt<T>::unpack(kr[u][w], &kf[w * Elt<T>::per16]);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc = fmaf(qf[r][e], kf[e], acc);
#pragma unroll
          for (int off = 1; off < L; off <<= 1) acc += __shfl_xor(acc, off);
          const bool pass = val[u] && (mask & rowbit[r]) && pos[u] <= plim[r];
          s[u][r] = pass ? acc : kNegInf;
        }
      }
      bool grow = false;
      float mt[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        mt[r] = m[r];
#pragma unroll
        for (int u = 0; u < U; ++u) mt[r] = fmaxf(mt[r], s[u][r]);
        grow |= mt[r] > m[r];
      }
      if (__ballot(grow)) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const float al = (mt[r] == m[r]) ? 1.f : exp2f(m[r] - mt[r]);
          l[r] *= al;
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[r][e] *= al;
          m[r] = mt[r];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[DPL];
#pragma unroll
        for (int w = 0; w < NU; ++w) Elt<T>::unpack(vr[u][w], &vf[w * Elt<T>::per16]);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const float p = (s[u][r] == kNegInf) ? 0.f : exp2f(s[u][r] - m[r]);
          l[r] += p;
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
        }
      }
    }
  }

  // combine the TPS token slots of the wave (lanes with equal `sub`)
#pragma unroll
  for (int off = L; off < 64; off <<= 1) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float mo = __shfl_xor(m[r], off);
      const float lo = __shfl_xor(l[r], off);
      const float M = fmaxf(m[r], mo);
      const float f1 = (m[r] == kNegInf) ? 0.f : exp2f(m[r] - M);
      const float f2 = (mo == kNegInf) ? 0.f : exp2f(mo - M);
      l[r] = l[r] * f1 + lo * f2;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float oo = __shfl_xor(o[r][e], off);
        o[r][e] = o[r][e] * f1 + oo * f2;
      }
      m[r] = M;
    }
  }
  write_partials<D, DPL, ROWS>(a, bg, c, rg, rows_here, m, l, o, slot, sub, wave, a.nw);
}

// Any head_dim <= 512 and any row stride: one token at a time per wave,
// lanes across the dims.  One wave per workgroup.
template <typename T>
__global__ __launch_bounds__(64) void attn_split_generic_kernel(SplitArgs a) {
  constexpr int NE = 8;  // dims per lane, head_dim <= 512
  const int lane = threadIdx.x;
  const int c = blockIdx.x, bg = blockIdx.y, rg = blockIdx.z;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int4* plan = a.plan + (int64_t)bg * (1 + a.max_items);
  const int n_items = min((int64_t)plan[0].x, a.max_items);
  const int it0 = c * a.ipw;
  if (it0 >= n_items) return;
  const int it1 = min(it0 + a.ipw, n_items);
  const int rows_here = min(a.rows_per_group, a.rows - rg * a.rows_per_group);
  const int D = a.d;

  float qf[kRowsMax][NE], m[kRowsMax], l[kRowsMax], o[kRowsMax][NE];
  uint32_t rowbit[kRowsMax];
  int plim[kRowsMax];
#pragma unroll
  for (int r = 0; r < kRowsMax; ++r) {
    const int gr = rg * a.rows_per_group + r;
    const bool act = r < rows_here;
    const int j = act ? gr / a.n_q : 0, i = act ? gr - j * a.n_q : 0;
    rowbit[r] = act ? (1u << j) : 0u;
    plim[r] = a.N - a.n_q + i;
    const T* qrow = (const T*)a.q + (((int64_t)b * a.hq + g * a.G + j) * a.n_q + i) * D;
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = lane + 64 * u;
      qf[r][u] = (act && e < D) ? Elt<T>::load(qrow + e) * a.qscale : 0.f;
      o[r][u] = 0.f;
    }
    m[r] = kNegInf;
    l[r] = 0.f;
  }
  const T* kb = (const T*)a.k + (int64_t)bg * a.head_stride;
  const T* vb = (const T*)a.v + (int64_t)bg * a.head_stride;
  for (int it = it0; it < it1; ++it) {
    const int4 item = plan[1 + it];
    const uint32_t mask = (uint32_t)item.z;
    for (int t = 0; t < item.y; ++t) {
      const int pos = item.x + t;
      float kf[NE], vf[NE];
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int e = lane + 64 * u;
        kf[u] = e < D ? Elt<T>::load(kb + (int64_t)pos * a.row_stride + e) : 0.f;
        vf[u] = e < D ? Elt<T>::load(vb + (int64_t)pos * a.row_stride + e) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < kRowsMax; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < NE; ++u) acc = fmaf(qf[r][u], kf[u], acc);
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        const float sc = ((mask & rowbit[r]) && pos <= plim[r]) ? acc : kNegInf;
        const float mn = fmaxf(m[r], sc);
        const float al = (mn == m[r]) ? 1.f : exp2f(m[r] - mn);
        const float p = (sc == kNegInf) ? 0.f : exp2f(sc - mn);
        l[r] = l[r] * al + p;
#pragma unroll
        for (int u = 0; u < NE; ++u) o[r][u] = o[r][u] * al + p * vf[u];
        m[r] = mn;
      }
    }
  }
  for (int r = 0; r < rows_here; ++r) {
    const int gr = rg * a.rows_per_group + r;
    const int j = gr / a.n_q, i = gr - j * a.n_q;
    const int64_t row = ((int64_t)b * a.hq + g * a.G + j) * a.n_q + i;
    const int64_t pidx = row * a.max_chunks + c;
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = lane + 64 * u;
      if (e < D) a.o[pidx * D + e] = o[r][u];
    }
    if (lane == 0) a.ml[pidx] = make_float2(m[r], l[r]);
  }
}

// ---------------------------------------------------------------------------
// merge: out = sum_c o_c 2^(m_c - M) / sum_c l_c 2^(m_c - M)

__global__ __launch_bounds__(64) void attn_merge_kernel(const int4* __restrict__ plan, const float2* __restrict__ ml,
                                                        const float* __restrict__ o, float* __restrict__ out,
                                                        int64_t max_items, int hq, int hkv, int n_q, int d,
                                                        int ipw, int max_chunks) {
  const int64_t row = blockIdx.x;  // ((b * hq + h) * n_q + i)
  const int lane = threadIdx.x;
  const int64_t bh = row / n_q;
  const int b = (int)(bh / hq), h = (int)(bh - (int64_t)b * hq);
  const int G = hq / hkv;
  const int bg = b * hkv + h / G;
  const int n_items = (int)min((int64_t)plan[(int64_t)bg * (1 + max_items)].x, max_items);
  const int nch = (n_items + ipw - 1) / ipw;
  const float2* mlr = ml + row * max_chunks;
  float M = kNegInf;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, mlr[c].x);
  float Ls = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float2 v = mlr[c];
    if (v.x != kNegInf) Ls += v.y * exp2f(v.x - M);
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  for (int e = lane; e < d; e += 64) {
    float acc = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float mc = mlr[c].x;
      if (mc != kNegInf) acc += o[(row * max_chunks + c) * d + e] * exp2f(mc - M);
    }
    out[row * d + e] = acc * inv;
  }
}

// ---------------------------------------------------------------------------
// dispatch

template <typename T, int D, int ROWS>
constexpr int dpl_for() {
  return ROWS <= 4 ? 32 / (int)sizeof(T) : 16 / (int)sizeof(T);
}

template <typename T, int D>
bool launch_fast_d(const AttnGeom& g, dim3 grid, dim3 block, hipStream_t s, const SplitArgs& a, hipEvent_t ev0,
                   hipEvent_t ev1) {
  const int rows = g.rows_per_group;
#define BRS_LAUNCH_ROWS(R)                                                                                    \
  if (rows <= R) {                                                                                            \
    constexpr int DPL = dpl_for<T, D, R>();                                                                   \
    if (ev0)                                                                                                  \
      hipExtLaunchKernelGGL((attn_split_kernel<T, D, DPL, R>), grid, block, 0, s, ev0, ev1, 0, a);            \
    else                                                                                                      \
      hipLaunchKernelGGL((attn_split_kernel<T, D, DPL, R>), grid, block, 0, s, a);                            \
    return true;                                                                                              \
  }
  BRS_LAUNCH_ROWS(1)
  BRS_LAUNCH_ROWS(2)
  BRS_LAUNCH_ROWS(4)
  BRS_LAUNCH_ROWS(8)
#undef BRS_LAUNCH_ROWS
  return false;
}

bool fast_supported(const AttnGeom& g) {
  const int es = elem_bytes(g.dtype);
  if ((g.row_stride * es) % 16 != 0) return false;
  if (g.dtype == BRS_BF16) return g.d == 64 || g.d == 128 || g.d == 256;
  return g.d == 32 || g.d == 64 || g.d == 128;
}

}  // namespace

bool attn_geometry(AttnGeom& g) {
  if (g.d > 512) return false;
  const int64_t E = g.idx_heads == 1 ? (int64_t)g.k : (int64_t)g.group * g.k;
  const int64_t n_sh = (g.sink_end + kItemTokens - 1) / kItemTokens + (g.N - g.win_start + kItemTokens - 1) / kItemTokens;
  const int64_t per_block = (g.B + kItemTokens - 1) / kItemTokens;
  const int64_t uniq = E < g.nb ? E : g.nb;
  g.max_items = n_sh + uniq * per_block;
  const int rows = g.group * g.n_q;
  g.row_groups = (rows + kRowsMax - 1) / kRowsMax;
  g.rows_per_group = rows < kRowsMax ? rows : kRowsMax;
  const int64_t bg = (int64_t)g.batch * g.hkv;
  const int64_t work = g.max_items * bg * g.row_groups;  // items over all workgroups
  if (!fast_supported(g)) {
    g.nw = 1;
    g.ipw = 1;
  } else {
    int64_t per_wave = work / 2048;
    per_wave = per_wave < 1 ? 1 : (per_wave > 8 ? 8 : per_wave);
    g.nw = (work / per_wave >= 4096) ? 4 : 1;
    g.ipw = (int)(per_wave * g.nw);
  }
  g.max_chunks = (int)((g.max_items + g.ipw - 1) / g.ipw);
  if (g.max_chunks < 1) g.max_chunks = 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows_total = (size_t)g.batch * g.hq * g.n_q;
  g.plan_off = 0;
  g.ml_off = up((size_t)bg * (1 + g.max_items) * sizeof(int4));
  g.o_off = g.ml_off + up(rows_total * g.max_chunks * sizeof(float2));
  g.total = g.o_off + up(rows_total * g.max_chunks * (size_t)g.d * sizeof(float));
  return true;
}

hipError_t launch_attn_plan(const AttnGeom& g, const int32_t* idx, void* ws, hipStream_t s) {
  PlanArgs a;
  a.idx = idx;
  a.plan = (int4*)((char*)ws + g.plan_off);
  a.max_items = g.max_items;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.G = g.group;
  a.k = idx ? g.k : 0;
  a.idx_heads = g.idx_heads;
  a.N = g.N;
  a.B = g.B;
  a.nb = g.nb;
  a.sink_end = g.sink_end;
  a.win_start = g.win_start;
  hipLaunchKernelGGL(attn_plan_kernel, dim3((unsigned)(g.batch * g.hkv)), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_split(const AttnGeom& g, const void* k, const void* v, const void* q, void* ws,
                             hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  SplitArgs a;
  a.k = k;
  a.v = v;
  a.q = q;
  a.plan = (const int4*)((char*)ws + g.plan_off);
  a.ml = (float2*)((char*)ws + g.ml_off);
  a.o = (float*)((char*)ws + g.o_off);
  a.max_items = g.max_items;
  a.head_stride = g.head_stride;
  a.row_stride = g.row_stride;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.G = g.group;
  a.n_q = g.n_q;
  a.N = g.N;
  a.d = g.d;
  a.qscale = g.qscale;
  a.ipw = g.ipw;
  a.nw = g.nw;
  a.max_chunks = g.max_chunks;
  a.rows = g.group * g.n_q;
  a.rows_per_group = g.rows_per_group;
  const dim3 grid((unsigned)g.max_chunks, (unsigned)(g.batch * g.hkv), (unsigned)g.row_groups);
  if (fast_supported(g)) {
    const dim3 block(64 * g.nw);
    bool done = false;
    if (g.dtype == BRS_BF16) {
      if (g.d == 64) done = launch_fast_d<uint16_t, 64>(g, grid, block, s, a, ev0, ev1);
      if (g.d == 128) done = launch_fast_d<uint16_t, 128>(g, grid, block, s, a, ev0, ev1);
      if (g.d == 256) done = launch_fast_d<uint16_t, 256>(g, grid, block, s, a, ev0, ev1);
    } else {
      if (g.d == 32) done = launch_fast_d<float, 32>(g, grid, block, s, a, ev0, ev1);
      if (g.d == 64) done = launch_fast_d<float, 64>(g, grid, block, s, a, ev0, ev1);
      if (g.d == 128) done = launch_fast_d<float, 128>(g, grid, block, s, a, ev0, ev1);
    }
    if (!done) return hipErrorInvalidValue;
  } else if (g.dtype == BRS_BF16) {
    if (ev0)
      hipExtLaunchKernelGGL(attn_split_generic_kernel<uint16_t>, grid, dim3(64), 0, s, ev0, ev1, 0, a);
    else
      hipLaunchKernelGGL(attn_split_generic_kernel<uint16_t>, grid, dim3(64), 0, s, a);
  } else {
    if (ev0)
      hipExtLaunchKernelGGL(attn_split_generic_kernel<float>, grid, dim3(64), 0, s, ev0, ev1, 0, a);
    else
      hipLaunchKernelGGL(attn_split_generic_kernel<float>, grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnGeom& g, void* ws, float* out, hipStream_t s) {
  const int64_t rows = (int64_t)g.batch * g.hq * g.n_q;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)rows), dim3(64), 0, s,
                     (const int4*)((char*)ws + g.plan_off), (const float2*)((char*)ws + g.ml_off),
                     (const float*)((char*)ws + g.o_off), out, g.max_items, g.hq, g.hkv, g.n_q, g.d, g.ipw,
                     g.max_chunks);
  return hipGetLastError();
}

bool prefill_supported(const AttnGeom&) { return false; }

hipError_t launch_attn_prefill(const AttnGeom&, const void*, const void*, const void*, const int32_t*, float*,
                               hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorNotSupported;
}

}  // namespace brs

// Retrieval attention for a chunk of queries on the matrix cores (MemLong
// Figure 3 and 2.3.4: the queries of the current chunk attend, with one
// softmax, to the retrieved chunks in full and to the local context causally;
// InfLLM "method": the same over memory units during chunked prefill).
//
// Here queries x tokens is a dense contraction: every retrieved token meets
// every query of the chunk.  One workgroup of 8 waves takes 64 consecutive
// queries of one query head:
//   - waves 0-3 and 4-7 own query rows 16w..16w+15 (w = wave % 4) and split
//     the token stream between them (even / odd 32-token halves of each
//     64-token stage); the two partial softmaxes are merged at the end;
//   - the attended segments of the (batch, kv head) come from the plan
//     kernel; the workgroup keeps those that hold its head, clips them to
//     positions <= its last query (the causal limit), and flattens them;
//   - each 64-token stage of K and V is staged once in LDS for all 8 waves,
//     double buffered: the next stage's global loads are in flight while the
//     current one is multiplied;
//   - S^T = K Q^T and O += P V on v_mfma_f32_16x16x32_bf16 with the layouts
//     of the decode kernel (V read back transposed with ds_read_b64_tr_b16,
//     P split into bf16 high and low parts so weights keep ~16 bits);
//   - online softmax in the log2 domain with a lazy reference (moves only
//     when a tile's maximum exceeds it by more than 2^8).
// Workgroups are numbered so that all query tiles of one head land on the
// same XCD (dispatch goes round-robin over the 8 XCDs): the head's K/V are
// then fetched from HBM once into that XCD's L2 and shared by its tiles.
#include <hip/hip_ext.h>
#include <math.h>
#include <stdlib.h>

#include "brs_internal.h"

namespace brs {
namespace {

constexpr int kPrefItems = 256;  // segments of one (batch, kv head) held in LDS
constexpr int kPrefQ = 64;       // queries per workgroup
constexpr int kStage = 64;       // tokens per stage (two 32-token halves)
constexpr float kLazyP = 8.0f;
constexpr float kFarNegP = -1e30f;
constexpr int kXcds = 8;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_p;
typedef __attribute__((ext_vector_type(4))) float f32x4_p;
typedef __attribute__((ext_vector_type(4))) short i16x4_p;
typedef __attribute__((address_space(3))) i16x4_p lds_i16x4_p;

struct PrefillArgs {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;
  float* out;
  const int4* hdr;
  const int4* items;
  int64_t max_items;
  int64_t head_stride;
  int row_stride, hq, hkv, G, n_q, N, d, nvec, nj;
  float qscale;
  int n_tiles, n_units, per_xcd;
};

__device__ __forceinline__ bf16x8_p as_bf16x8_p(const uint4& u) { return __builtin_bit_cast(bf16x8_p, u); }

__device__ __forceinline__ uint32_t pack2_rne(float lo, float hi) {
  auto rne = [](float f) -> uint32_t {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  };
  return rne(lo) | (rne(hi) << 16);
}

int env_flag(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DP: head dim rounded up to a multiple of 32 (the k chunk of the S^T MFMA).
template <int DP>
__global__ __launch_bounds__(512) void attn_prefill_kernel(PrefillArgs a) {
  constexpr int KC = DP / 32;
  constexpr int NJ = DP / 16;
  constexpr int KP = DP + 16;  // LDS row pitch in halves (keeps transposed reads conflict-free)
  constexpr int VPT = (2 * kStage * (DP / 8) + 511) / 512;  // 16-byte vectors staged per thread
  __shared__ __align__(16) uint16_t s_k[2][kStage][KP];
  __shared__ __align__(16) uint16_t s_v[2][kStage][KP];
  __shared__ int2 s_meta[3][kStage];
  __shared__ int4 s_items[kPrefItems];
  __shared__ int wave_tot[16];
  __shared__ int sh_tot[2];
  __shared__ float s_ml[4][16][2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, n = lane & 15;
  const int qg = wave & 3, kh = wave >> 2;

  // workgroup -> (head, query tile), all tiles of a head on one XCD
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u = xcd * a.per_xcd + slot;
  if (u >= a.n_units) return;
  const int bh = u / a.n_tiles, tile = u - bh * a.n_tiles;
  const int b = bh / a.hq, h = bh - b * a.hq;
  const int g = h / a.G;
  const int bg = b * a.hkv + g;
  const uint32_t headbit = 1u << (h - g * a.G);
  const int q0 = tile * kPrefQ;
  const int qlast = min(q0 + kPrefQ, a.n_q) - 1;
  const int pmax = a.N - a.n_q + qlast;

  // segments of this head, clipped to positions <= pmax, flattened
  const int4 hd = a.hdr[bg];
  const int n_in = hd.x;
  int4 it = make_int4(0, 0, 0, 0);
  int keep = 0, len = 0;
  if (tid < n_in) {
    it = a.items[(int64_t)bg * a.max_items + tid];
    if ((uint32_t)it.z & headbit) {
      len = min(it.x + it.y, pmax + 1) - it.x;
      len = len < 0 ? 0 : len;
      keep = len > 0;
    }
  }
  const int inc_k = block_inclusive_scan(keep, wave_tot);
  const int inc_t = block_inclusive_scan(len, wave_tot);
  if (keep) s_items[inc_k - 1] = make_int4(it.x, len, 0, inc_t - len);
  if (tid == 511) {
    sh_tot[0] = inc_k;
    sh_tot[1] = inc_t;
  }
  // zero the pad columns of K and V once (never written by the staging)
  for (int i = tid; i < 2 * 2 * kStage; i += 512) {
    uint16_t* row = (i < 2 * kStage) ? &s_k[i >> 6][i & 63][0] : &s_v[(i >> 6) - 2][i & 63][0];
    for (int c = 8 * a.nvec; c < KP; ++c) row[c] = 0;
  }
  __syncthreads();
  const int ns = sh_tot[0], n_tok = sh_tot[1];
  const int n_stages = (n_tok + kStage - 1) / kStage;

  // stage metadata (position of each of the 64 rows, -1 = none), computed by wave 0 with a cursor
  int cur = 0;
  int4 ci = ns > 0 ? s_items[0] : make_int4(0, 0, 0, 0);
  auto meta = [&](int stage) {
    const int tau = stage * kStage + lane;
    int pos = -1;
    if (tau < n_tok) {
      while (tau >= ci.w + ci.y && cur + 1 < ns) ci = s_items[++cur];
      pos = ci.x + (tau - ci.w);
    }
    s_meta[stage % 3][lane] = make_int2(pos, 0);
  };

  // staging: thread t moves vectors e = t + 512 j of the stage (K rows first, then V)
  const int kvec = kStage * a.nvec;
  const uint16_t* kb = a.k + (int64_t)bg * a.head_stride;
  const uint16_t* vb = a.v + (int64_t)bg * a.head_stride;
  uint4 stg[VPT];
  auto stage_load = [&](int stage) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = tid + 512 * j;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (e < 2 * kvec) {
        const bool isv = e >= kvec;
        const int ee = isv ? e - kvec : e;
        const int r = ee / a.nvec, c = ee - r * a.nvec;
        const int pos = s_meta[stage % 3][r].x;
        if (pos >= 0) x = *reinterpret_cast<const uint4*>((isv ? vb : kb) + (int64_t)pos * a.row_stride + 8 * c);
      }
      stg[j] = x;
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = tid + 512 * j;
      if (e < 2 * kvec) {
        const bool isv = e >= kvec;
        const int ee = isv ? e - kvec : e;
        const int r = ee / a.nvec, c = ee - r * a.nvec;
        uint16_t* dst = isv ? &s_v[buf][r][8 * c] : &s_k[buf][r][8 * c];
        *reinterpret_cast<uint4*>(dst) = stg[j];
      }
    }
  };

  // query rows of this wave as the B operand of S^T = K Q^T
  const int qi = q0 + 16 * qg + n;
  const bool act = qi < a.n_q;
  const int plim = a.N - a.n_q + qi;
  uint4 qb[KC];
  {
    const uint16_t* qrow = a.q + ((int64_t)bh * a.n_q + (act ? qi : 0)) * a.d;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e0 = 32 * kk + 8 * g4 + 2 * p;
        const uint32_t lo = (act && e0 < a.d) ? qrow[e0] : 0u;
        const uint32_t hi = (act && e0 + 1 < a.d) ? qrow[e0 + 1] : 0u;
        w[p] = lo | (hi << 16);
      }
      qb[kk] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  const float qs = a.qscale;

  f32x4_p o[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) o[jj] = f32x4_p{0.f, 0.f, 0.f, 0.f};
  float mref = kFarNegP, lpart = 0.f;

  if (n_stages > 0) {
    if (wave == 0) {
      meta(0);
      if (n_stages > 1) meta(1);
    }
    __syncthreads();
    stage_load(0);
    stage_store(0);
    __syncthreads();
  }

  for (int s = 0; s < n_stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < n_stages) stage_load(s + 1);
    if (wave == 0 && s + 2 < n_stages) meta(s + 2);

    // this wave's 32 tokens: stage rows 32 kh .. 32 kh + 31
    const int r0 = 32 * kh;
    f32x4_p st[2];
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      st[sidx] = f32x4_p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&s_k[buf][r0 + 16 * sidx + n][32 * kk + 8 * g4]);
        st[sidx] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_p(ka), as_bf16x8_p(qb[kk]), st[sidx], 0, 0, 0);
      }
    }
    float sv[8];
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = s_meta[s % 3][r0 + 16 * sidx + 4 * g4 + i].x;
        const bool pass = act && pos >= 0 && pos <= plim;
        sv[4 * sidx + i] = pass ? st[sidx][i] * qs : -INFINITY;
      }
    float tm = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tm = fmaxf(tm, sv[i]);
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    if (__ballot(tm > mref + kLazyP)) {
      const float nm = fmaxf(mref, tm);
      const float al = exp2_fast(mref - nm);
      mref = nm;
      lpart *= al;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(al, 4 * g4 + i);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) o[jj][i] *= ai;
      }
    }
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = exp2_fast(sv[i] - mref);
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[i] = pack2_rne(pv[2 * i], pv[2 * i + 1]);
      const float h0 = __uint_as_float(ph[i] << 16), h1 = __uint_as_float(ph[i] & 0xffff0000u);
      pl[i] = pack2_rne(pv[2 * i] - h0, pv[2 * i + 1] - h1);
      lpart += pv[2 * i] + pv[2 * i + 1];
    }
    const bf16x8_p pa_hi = __builtin_bit_cast(bf16x8_p, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8_p pa_lo = __builtin_bit_cast(bf16x8_p, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      if (jj < a.nj) {
        const int col = 16 * jj + 4 * (n & 3);
        const i16x4_p v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)&s_v[buf][r0 + 4 * g4 + (n >> 2)][col]);
        const i16x4_p v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)&s_v[buf][r0 + 16 + 4 * g4 + (n >> 2)][col]);
        const bf16x8_p vbv = __builtin_bit_cast(bf16x8_p, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vbv, o[jj], 0, 0, 0);
        o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vbv, o[jj], 0, 0, 0);
      }
    }
    if (s + 1 < n_stages) stage_store(buf ^ 1);
    __syncthreads();
  }

  // row sums over the four lanes that share a query row
  lpart += __shfl_xor(lpart, 16);
  lpart += __shfl_xor(lpart, 32);

  // merge the two token halves: waves 4-7 hand (max, sum, O) to waves 0-3 through LDS
  float* s_o = reinterpret_cast<float*>(&s_k[0][0][0]);  // [4][16][DP] floats
  if (kh == 1) {
    if (lane < 16) {
      s_ml[qg][lane][0] = mref;
      s_ml[qg][lane][1] = lpart;
    }
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[(qg * 16 + 4 * g4 + i) * DP + 16 * jj + n] = o[jj][i];
  }
  __syncthreads();
  if (kh == 0) {
    const float m2 = s_ml[qg][n][0], l2 = s_ml[qg][n][1];
    const float M = fmaxf(mref, m2);
    const float f1 = exp2_fast(mref - M), f2 = exp2_fast(m2 - M);
    const float L = lpart * f1 + l2 * f2;
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const float c1 = f1 * inv, c2 = f2 * inv;
    float* orow = a.out + ((int64_t)bh * a.n_q + q0 + 16 * qg) * a.d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g4 + i;
      const float a1 = __shfl(c1, r), a2 = __shfl(c2, r);
      if (q0 + 16 * qg + r < a.n_q) {
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          const int col = 16 * jj + n;
          if (col < a.d) orow[(int64_t)r * a.d + col] = o[jj][i] * a1 + s_o[(qg * 16 + r) * DP + col] * a2;
        }
      }
    }
  }
}

}  // namespace

bool prefill_supported(const AttnGeom& g) {
  if (env_flag("BRS_PREFILL", 1) == 0) return false;
  return g.dtype == BRS_BF16 && g.n_q >= kPrefQ && g.d <= 128 && g.row_stride % 8 == 0 &&
         ((g.d + 7) / 8) * 8 <= g.row_stride && g.max_items <= kPrefItems && g.N <= INT32_MAX / 2;
}

hipError_t launch_attn_prefill(const AttnGeom& g, const void* k, const void* v, const void* q, void* ws, float* out,
                               hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  PrefillArgs a;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.q = (const uint16_t*)q;
  a.out = out;
  a.hdr = (const int4*)((char*)ws + g.hdr_off);
  a.items = (const int4*)((char*)ws + g.items_off);
  a.max_items = g.max_items;
  a.head_stride = g.head_stride;
  a.row_stride = g.row_stride;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.G = g.group;
  a.n_q = g.n_q;
  a.N = g.N;
  a.d = g.d;
  a.nvec = (g.d + 7) / 8;
  a.nj = (g.d + 15) / 16;
  a.qscale = g.qscale;
  a.n_tiles = (g.n_q + kPrefQ - 1) / kPrefQ;
  a.n_units = a.n_tiles * g.batch * g.hq;
  a.per_xcd = (a.n_units + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(a.per_xcd * kXcds)), block(512);
  if (g.d <= 64) {
    if (ev0)
      hipExtLaunchKernelGGL(attn_prefill_kernel<64>, grid, block, 0, s, ev0, ev1, 0, a);
    else
      hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, block, 0, s, a);
  } else {
    if (ev0)
      hipExtLaunchKernelGGL(attn_prefill_kernel<128>, grid, block, 0, s, ev0, ev1, 0, a);
    else
      hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace brs

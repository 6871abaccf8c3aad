// Retrieval attention, split-K over the attended set (InfLLM "method":
// local tokens plus a few memory units; Landmark Attention "proposed method":
// a block's tokens are read only when the block is selected;
// RetrievalAttention "proposed method": attention restricted to the tokens
// that matter, exact over them).
//
//   plan   one workgroup per (batch, kv head): marks the blocks any query
//          head of the group selected (a head bitmask per block, in LDS),
//          clips them against sinks and window so every token appears once,
//          and writes the segments of the attended set with their offsets in
//          the flattened token list, plus the segment that starts each chunk.
//   split  one workgroup per (batch, kv head, row group, chunk of
//          chunk_tokens flattened tokens); each wave takes an equal run of
//          the chunk, so work is balanced whatever the segment lengths.  K and
//          V rows are streamed once for all query rows of the group, with an
//          online softmax in float32 (log2 domain); the workgroup writes a
//          partial (max, sum, weighted V) per query row.
//   merge  one workgroup per query row combines the partials by log-sum-exp
//          in a fixed order (deterministic).  A kernel of its own: merging in
//          the last split workgroup would need an agent-scope release/acquire
//          per workgroup, which on this GPU writes back and invalidates the
//          whole L2 of the XCD each time.
#include <hip/hip_ext.h>
#include <math.h>
#include <stdlib.h>

#include "brs_internal.h"
#include "brs_wave_topk.h"

namespace brs {
namespace {

constexpr float kNegInf = -INFINITY;
constexpr int kItemsLds = 256;  // segments of one chunk staged in LDS
constexpr int kTargetWaves = 2048;  // waves the split decomposition aims for
constexpr int kSplitU = 2;          // vector split kernel: token steps per group
constexpr int kSlotWgs = 256;       // slot layout: workgroups aimed for (about one per CU)

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Sum over aligned groups of L lanes (L a power of two).  Within a 16-lane
// row the exchanges are DPP moves (quad permutes, then half-row and row
// mirrors: each pairs lanes so that every lane ends with the group total);
// wider groups fall back to cross-row shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp_mov<0xb1>(v);   // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v += dpp_mov<0x4e>(v);   // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (L >= 16) v += dpp_mov<0x140>(v); // row_mirror
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  if constexpr (L >= 64) v += __shfl_xor(v, 32);
  return v;
}

// 2^x with the hardware instruction (about 1 ulp; tiny results flush to 0,
// which only drops softmax weights below 2^-126).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct PlanArgs {
  const int32_t* idx;
  int4* hdr;          // [bg]: (segments, tokens)
  int4* items;        // [bg][max_items]: (first row, length, head mask, flattened offset)
  int* chunk_first;   // [bg][max_chunks]: segment holding the chunk's first token
  int4* chunks;       // [bg][max_chunks]: (first segment, end segment, end token, 0)
  float* out;
  int64_t max_items;
  int max_chunks;
  int hq, hkv, G, k, idx_heads, n_q, d, row_groups;
  int N, B, nb, sink_end, win_start, chunk_tokens;
};

// ---------------------------------------------------------------------------
// plan

__device__ __forceinline__ void mark_chunks(int* first, int item, int off, int len, int CH) {
  for (int c = (off + CH - 1) / CH; c * CH < off + len; ++c) first[c] = item;
}

__global__ __launch_bounds__(1024) void attn_plan_kernel(PlanArgs a) {
  __shared__ uint32_t marks[kMarkBlocks];
  __shared__ int wave_tot[16];
  __shared__ int sh_items, sh_tokens;
  const int bg = blockIdx.x;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  int4* items = a.items + (int64_t)bg * a.max_items;
  int* first = a.chunk_first + (int64_t)bg * a.max_chunks;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int CH = a.chunk_tokens;
  const uint32_t full = a.G >= 32 ? 0xffffffffu : ((1u << a.G) - 1u);

  // shared part: sinks [0, S') then window [ws, N)
  const int S = a.sink_end, Wn = a.N - a.win_start;
  if (tid == 0) {
    int i = 0;
    if (S > 0) {
      items[i] = make_int4(0, S, (int)full, 0);
      mark_chunks(first, i, 0, S, CH);
      ++i;
    }
    if (Wn > 0) {
      items[i] = make_int4(a.win_start, Wn, (int)full, S);
      mark_chunks(first, i, S, Wn, CH);
    }
  }
  int n_items = (S > 0) + (Wn > 0), n_tokens = S + Wn;

  const int nl = sel_lists(a.idx_heads, a.hkv);
  const int E = nl * a.k;
  for (int base = 0; base < a.nb; base += kMarkBlocks) {
    const int top = min(a.nb, base + kMarkBlocks);
    for (int i = tid; i < top - base; i += nt) marks[i] = 0u;
    __syncthreads();
    for (int e = tid; e < E; e += nt) {
      const int j = e / a.k;
      const int blk = a.idx[sel_row(a.idx_heads, a.hkv, b, g, j) * a.k + (e - j * a.k)];
      const uint32_t bit = nl == a.G ? 1u << j : full;
      if (blk >= base && blk < top) {
        const int lo_t = max(blk * a.B, S);
        const int hi_t = min((blk + 1) * a.B, a.win_start);
        if (lo_t < hi_t) atomicOr(&marks[blk - base], bit);
      }
    }
    __syncthreads();
    // each thread owns a contiguous run of blocks
    const int per = (kMarkBlocks + nt - 1) / nt;
    const int r0 = base + tid * per, r1 = min(top, r0 + per);
    int ci = 0, ct = 0;
    for (int blk = r0; blk < r1; ++blk) {
      if (marks[blk - base]) {
        ++ci;
        ct += min((blk + 1) * a.B, a.win_start) - max(blk * a.B, S);
      }
    }
    const int inc_i = block_inclusive_scan(ci, wave_tot);
    const int inc_t = block_inclusive_scan(ct, wave_tot);
    int oi = n_items + inc_i - ci, ot = n_tokens + inc_t - ct;
    for (int blk = r0; blk < r1; ++blk) {
      const uint32_t mk = marks[blk - base];
      if (!mk) continue;
      const int lo_t = max(blk * a.B, S);
      const int len = min((blk + 1) * a.B, a.win_start) - lo_t;
      items[oi] = make_int4(lo_t, len, (int)mk, ot);
      mark_chunks(first, oi, ot, len, CH);
      ++oi;
      ot += len;
    }
    if (tid == nt - 1) {
      sh_items = inc_i;
      sh_tokens = inc_t;
    }
    __syncthreads();
    n_items += sh_items;
    n_tokens += sh_tokens;
    __syncthreads();
  }
  if (tid == 0) a.hdr[bg] = make_int4(n_items, n_tokens, 0, 0);
  // chunk descriptors: every chunk c < max_chunks gets one (empty beyond the last)
  __syncthreads();
  const int n_chunks = (n_tokens + CH - 1) / CH;
  int4* chunks = a.chunks + (int64_t)bg * a.max_chunks;
  for (int c = tid; c < a.max_chunks; c += nt) {
    if (c < n_chunks)
      chunks[c] = make_int4(first[c], c + 1 < n_chunks ? first[c + 1] + 1 : n_items, min((c + 1) * CH, n_tokens), 0);
    else
      chunks[c] = make_int4(0, 0, 0, 0);
  }
  if (n_tokens == 0) {
    // nothing to attend for this (batch, kv head): its rows are zeros
    const int rows = a.G * a.n_q;
    float* o = a.out + (((int64_t)b * a.hq + g * a.G) * a.n_q) * a.d;
    for (int i = tid; i < rows * a.d; i += nt) o[i] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// split

struct SplitArgs {
  const void* k;
  const void* v;
  const void* q;
  const int4* hdr;
  const int4* items;
  const int4* chunks;
  float2* ml;
  float* o;
  int64_t max_items;
  int max_chunks;
  int64_t head_stride;
  int row_stride;
  int hq, hkv, G, n_q, N, d;
  float qscale;
  int chunk_tokens, wave_tokens, nw;
  int rows, rows_per_group, row_groups;
  // in-kernel plan (when `local`): the selections and the set's geometry
  int local;
  const int32_t* idx;
  int kk, idx_heads, B, nb, sink_end, win_start;  // kk: selections per row
  int4* hdr_out;  // (segments, tokens) per (batch, kv head), for the merge
  float* out;     // zero rows when nothing is attended
  // slot layout: padded sinks (tokens), slot stride, sink/window and slot
  // tokens, selection entries per kv slice
  int slot_ps, slot_bs, len_a, len_b, n_ent;
  int slice_bytes;  // bytes of one (batch, kv head) slice of k / v
  // in-kernel selection: the score rows and where the selection goes
  const float* scores;
  int64_t score_stride;
  int sel_lo, sel_hi;
  int32_t* idx_out;
  float* vals_out;
  int n_units;                   // one-dimensional grid of units
  // K/V read through a page table (a device cache of blocks; k and v then
  // point to the page pool): page of block x of slice bg at pages[bg *
  // pages_stride + x]
  const int32_t* pages;
  int pages_stride;
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

__device__ __forceinline__ int64_t row_index(const SplitArgs& a, int b, int g, int gr) {
  const int j = gr / a.n_q, i = gr - j * a.n_q;
  return ((int64_t)b * a.hq + g * a.G + j) * a.n_q + i;
}

// The segments of one chunk, staged in LDS (the chunk size is capped so that
// they always fit).  A cursor walks them as the flattened token index grows.
__device__ __forceinline__ int stage_items(const SplitArgs& a, int bg, const int4& desc, int4* lds) {
  const int4* g = a.items + (int64_t)bg * a.max_items;
  const int ns = min(desc.y - desc.x, kItemsLds);
  for (int j = threadIdx.x; j < ns; j += blockDim.x) lds[j] = g[desc.x + j];
  __syncthreads();
  return ns;
}

// The segments of chunk c computed in the workgroup itself from the
// selections (no plan kernel): per-head bitmaps of the selected blocks that
// hold a token outside sinks and window, a prefix count of the union over
// 32-block words, and the flattened offsets in closed form -- every
// selected block has B tokens in the set except the first eligible block
// (cut by the sinks) and the last (cut by the window), which are the first
// and last of the union when selected.  Same segments, in the same order,
// as the plan kernel: sinks, window, then blocks in block order.
// Returns the number of segments staged in `lds`, or -1 when the chunk lies
// past the end; *t_end is the chunk's last flattened token + 1.
constexpr int kPlanWords = 1024;  // bitmap words in LDS: heads x ceil(nb / 32)

struct ChunkPlanLds {
  uint32_t bits[kPlanWords];
  int misc[4];  // segments, chunk end token, (unused), (unused)
};

__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

__device__ int chunk_plan(const SplitArgs& a, int b, int g, int c, int rg, int4* lds, ChunkPlanLds& pl,
                          int* t_end) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  const int W = (a.nb + 31) >> 5;
  const int hb = sel_lists(a.idx_heads, a.hkv);  // bitmaps: one per head, or one shared
  const int S = a.sink_end, ws = a.win_start, B = a.B;
  for (int i = tid; i < hb * W; i += nt) pl.bits[i] = 0u;
  __syncthreads();
  const int E = hb * a.kk;
  for (int e = tid; e < E; e += nt) {
    const int j = e / a.kk;
    const int blk = a.idx[sel_row(a.idx_heads, a.hkv, b, g, j) * a.kk + (e - j * a.kk)];
    if (blk >= 0 && blk < a.nb && max(blk * B, S) < min((blk + 1) * B, ws))
      atomicOr(&pl.bits[j * W + (blk >> 5)], 1u << (blk & 31));
  }
  __syncthreads();
  if (tid < 64) {
    // wave 0: the union's popcounts by word, their prefix (DPP scan, 64 words
    // at a time), the set's size, then each lane expands its word's blocks
    // that fall in this chunk into segments
    auto word = [&](int w) -> uint32_t {
      uint32_t u = 0u;
      if (w < W)
        for (int j = 0; j < hb; ++j) u |= pl.bits[j * W + w];
      return u;
    };
    int n_sel = 0;
    for (int w0 = 0; w0 < W; w0 += 64) n_sel += __builtin_amdgcn_readlane(wave_incl_scan_dpp(__popc(word(w0 + lane))), 63);
    auto in_union = [&](int blk) -> bool {
      if (blk < 0 || blk >= a.nb) return false;
      return (word(blk >> 5) >> (blk & 31)) & 1u;
    };
    const int bs = S / B, bw = ws / B;
    const int cut_s = (S % B != 0 && in_union(bs)) ? S - bs * B : 0;
    const int cut_w = (ws % B != 0 && in_union(bw)) ? (bw + 1) * B - ws : 0;
    const int Wn = a.N - ws;
    const int n_tokens = S + Wn + n_sel * B - cut_s - cut_w;
    const int t0 = c * a.chunk_tokens;
    if (c == 0 && rg == 0 && lane == 0)
      a.hdr_out[(int64_t)b * a.hkv + g] = make_int4((S > 0) + (Wn > 0) + n_sel, n_tokens, 0, 0);
    int ns = -1, t1 = 0;
    if (n_tokens > 0 && t0 < n_tokens) {
      t1 = min(t0 + a.chunk_tokens, n_tokens);
      const uint32_t full = a.G >= 32 ? 0xffffffffu : ((1u << a.G) - 1u);
      int nhead = 0;
      if (S > 0 && t0 < S) nhead++;
      if (Wn > 0 && t0 < S + Wn && t1 > S) nhead++;
      if (lane == 0) {
        int i = 0;
        if (S > 0 && t0 < S) lds[i++] = make_int4(0, S, (int)full, 0);
        if (Wn > 0 && t0 < S + Wn && t1 > S) lds[i++] = make_int4(ws, Wn, (int)full, S);
      }
      // ranks [r0, r1) overlap the chunk: offset of rank r = base + r B - (r > 0 ? cut_s : 0)
      const int base = S + Wn;
      int r0 = 0;
      if (t0 > base) r0 = (t0 - base + cut_s) / B;
      int r1 = n_sel;
      if (t1 - base < n_sel * B) {
        const int num = t1 - base + cut_s + B - 1;
        r1 = num > 0 ? num / B : 0;
        r1 = min(r1, n_sel);
      }
      int before = 0;  // selected blocks in earlier word groups
      for (int w0 = 0; w0 < W; w0 += 64) {
        const int w = w0 + lane;
        uint32_t u = word(w);
        const int cnt = __popc(u);
        const int incl = wave_incl_scan_dpp(cnt);
        int r = before + incl - cnt;
        while (u) {
          const int bit = __builtin_ctz(u);
          u &= u - 1u;
          if (r >= r0 && r < r1) {
            const int blk = w * 32 + bit;
            uint32_t mk = full;
            if (hb > 1) {
              mk = 0u;
              for (int j = 0; j < hb; ++j) mk |= ((pl.bits[j * W + w] >> bit) & 1u) << j;
            }
            const int pos = max(blk * B, S);
            lds[nhead + (r - r0)] = make_int4(pos, min((blk + 1) * B, ws) - pos, (int)mk, base + r * B - (r > 0 ? cut_s : 0));
          }
          ++r;
        }
        before += __builtin_amdgcn_readlane(incl, 63);
      }
      ns = nhead + (r1 > r0 ? r1 - r0 : 0);
    } else if (n_tokens == 0 && c == 0 && rg == 0) {
      // nothing attended: this (batch, kv head)'s rows are zeros (written once)
      float* o = a.out + (((int64_t)b * a.hq + g * a.G) * a.n_q) * a.d;
      for (int i = lane; i < a.G * a.n_q * a.d; i += 64) o[i] = 0.f;
    }
    if (lane == 0) {
      pl.misc[0] = ns;
      pl.misc[1] = t1;
    }
  }
  __syncthreads();
  *t_end = pl.misc[1];
  return pl.misc[0];
}

// ---------------------------------------------------------------------------
// merge: one workgroup per query row.
//   out = sum_c o_c 2^(m_c - M) / sum_c l_c 2^(m_c - M),  M = max_c m_c.
// Chunks are split into `slices` interleaved runs; each thread issues the
// loads of eight chunks at once and keeps a running log-sum-exp; the runs
// are combined in increasing slice order (deterministic).

// lse (optional): the row's log-sum-exp of its scaled logits in natural
// units, ln(2^M * L) with M the log2-domain reference and L the sum.
__device__ __forceinline__ float row_lse(float M, float L) {
  return L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

__global__ __launch_bounds__(256) void attn_merge_kernel(const int4* __restrict__ hdr, const float2* __restrict__ ml,
                                                        const float* __restrict__ o, float* __restrict__ out,
                                                        float* __restrict__ lse, int hq, int hkv, int n_q, int d,
                                                        int chunk_tokens, int max_chunks, int used_chunks) {
  __shared__ float4 s_acc[256];
  __shared__ float2 s_ml[256];
  const int64_t row = blockIdx.x;  // ((b * hq + h) * n_q + i)
  const int64_t bh = row / n_q;
  const int b = (int)(bh / hq), h = (int)(bh - (int64_t)b * hq);
  const int bg = b * hkv + h / (hq / hkv);
  // chunk_tokens = 0: the first used_chunks chunks hold partials (slot
  // layout); else the plan's token count says how many do
  int n_chunks = used_chunks;
  if (chunk_tokens > 0) {
    const int n_tokens = hdr[bg].y;
    if (n_tokens == 0) {  // the plan kernel wrote zeros
      if (lse && threadIdx.x == 0) lse[row] = -INFINITY;
      return;
    }
    n_chunks = min((n_tokens + chunk_tokens - 1) / chunk_tokens, max_chunks);
  }
  const float2* mlr = ml + row * max_chunks;
  const float* ob = o + row * max_chunks * (int64_t)d;
  if ((d & 3) == 0 && d / 4 <= (int)blockDim.x) {
    // thread (slice sl, float4 column e4) takes chunks sl, sl + slices, ...:
    // all its loads are issued together, then a local log-sum-exp, then the
    // slices combine in slice order
    const int D4 = d >> 2;
    const int slices = blockDim.x / D4;
    const int e4 = threadIdx.x % D4, sl = threadIdx.x / D4;
    float m = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (sl < slices) {
      const float4* p = reinterpret_cast<const float4*>(ob) + e4;
      for (int c0 = sl; c0 < n_chunks; c0 += 8 * slices) {
        float2 v[8];
        float4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = c0 + u * slices;
          const bool ok = c < n_chunks;
          v[u] = ok ? mlr[c] : make_float2(-INFINITY, 0.f);
          x[u] = ok ? p[(int64_t)c * D4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float mn = m;
#pragma unroll
        for (int u = 0; u < 8; ++u) mn = fmaxf(mn, v[u].x);
        if (mn != -INFINITY) {
          const float al = exp2f(m - mn);  // m = -inf gives 0
          l *= al;
          acc.x *= al;
          acc.y *= al;
          acc.z *= al;
          acc.w *= al;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float w = v[u].x == -INFINITY ? 0.f : exp2f(v[u].x - mn);
            l = fmaf(v[u].y, w, l);
            acc.x = fmaf(x[u].x, w, acc.x);
            acc.y = fmaf(x[u].y, w, acc.y);
            acc.z = fmaf(x[u].z, w, acc.z);
            acc.w = fmaf(x[u].w, w, acc.w);
          }
          m = mn;
        }
      }
    }
    s_acc[threadIdx.x] = acc;
    s_ml[threadIdx.x] = make_float2(m, l);
    __syncthreads();
    if (threadIdx.x < D4) {
      float M = -INFINITY;
      for (int s2 = 0; s2 < slices; ++s2) M = fmaxf(M, s_ml[s2 * D4 + threadIdx.x].x);
      float L = 0.f;
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M != -INFINITY) {
        for (int s2 = 0; s2 < slices; ++s2) {
          const float2 q = s_ml[s2 * D4 + threadIdx.x];
          const float w = q.x == -INFINITY ? 0.f : exp2f(q.x - M);
          const float4 v = s_acc[s2 * D4 + threadIdx.x];
          L = fmaf(q.y, w, L);
          t.x = fmaf(v.x, w, t.x);
          t.y = fmaf(v.y, w, t.y);
          t.z = fmaf(v.z, w, t.z);
          t.w = fmaf(v.w, w, t.w);
        }
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
      reinterpret_cast<float4*>(out + row * d)[threadIdx.x] = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
      if (lse && threadIdx.x == 0) lse[row] = row_lse(M, L);
    }
    return;
  }
  // any head dim: one pass for the maximum, one for the sum and the output
  float M = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, mlr[c].x);
  float L = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    const float2 v = mlr[c];
    L += v.x == -INFINITY ? 0.f : v.y * exp2f(v.x - M);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    float acc = 0.f;
    for (int c = 0; c < n_chunks; ++c) {
      const float mc = mlr[c].x;
      acc = fmaf(ob[(int64_t)c * d + e], mc == -INFINITY ? 0.f : exp2f(mc - M) * inv, acc);
    }
    out[row * d + e] = acc;
  }
  if (lse && threadIdx.x == 0) lse[row] = row_lse(M, L);
}

// Fast path: D = head_dim, rows 16-byte aligned.  L = D / DPL lanes share a
// token; lane `sub` holds the 16-byte units sub, sub + L, ... of the row, so
// each load instruction reads whole cache lines of every token.  TPS = 64 / L
// tokens per wave step; steps are taken in groups of U and two groups are in
// flight (one computed while the next loads).  Query logits use bf16 pair
// dot products (exact products, float32 sums) for bfloat16 data.
template <typename T, int DPL, int U>
struct Group {
  static constexpr int NU = DPL / Elt<T>::per16;
  uint4 k[U][NU], v[U][NU];
  int pos[U];
  uint32_t msk[U];
};

template <typename T, int D, int DPL, int ROWS, int U, int NWMAX>
__global__ __launch_bounds__(64 * NWMAX) void attn_split_kernel(SplitArgs a) {
  constexpr int L = D / DPL;
  constexpr int TPS = 64 / L;
  constexpr int E16 = Elt<T>::per16;        // elements per 16-byte unit
  constexpr int NU = DPL / E16;             // units per lane per row
  constexpr bool BF = sizeof(T) == 2;
  constexpr int QW = BF ? DPL / 2 : DPL;    // query registers per row
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lanes per token");
  static_assert(NU >= 1 && NU * E16 == DPL, "16-byte units");
  __shared__ int4 s_items[kItemsLds];
  __shared__ ChunkPlanLds s_plan;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / L, sub = lane % L;
  const int c = blockIdx.x, bg = blockIdx.y, rg = blockIdx.z;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int rows_here = min(a.rows_per_group, a.rows - rg * a.rows_per_group);

  // query rows of this group (independent of the plan: issued first)
  uint32_t qw[ROWS][QW];
  uint32_t rowbit[ROWS];
  int plim[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int gr = rg * a.rows_per_group + r;
    const bool act = r < rows_here;
    const int j = act ? gr / a.n_q : 0, i = act ? gr - j * a.n_q : 0;
    rowbit[r] = act ? (1u << j) : 0u;
    plim[r] = a.N - a.n_q + i;
    const T* qrow = (const T*)a.q + (((int64_t)b * a.hq + g * a.G + j) * a.n_q + i) * D + sub * E16;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const uint4 raw = act ? *reinterpret_cast<const uint4*>(qrow + u * L * E16) : make_uint4(0, 0, 0, 0);
      qw[r][4 * u] = raw.x;
      qw[r][4 * u + 1] = raw.y;
      qw[r][4 * u + 2] = raw.z;
      qw[r][4 * u + 3] = raw.w;
    }
  }

  int ns, t_end;
  if (a.local) {
    ns = chunk_plan(a, b, g, c, rg, s_items, s_plan, &t_end);
    if (ns < 0) return;  // past the end of this (batch, kv head)'s tokens
  } else {
    const int4 desc = a.chunks[(int64_t)bg * a.max_chunks + c];
    if (desc.x >= desc.y) return;
    ns = stage_items(a, bg, desc, s_items);
    t_end = desc.z;
  }
  const int t0 = c * a.chunk_tokens;

  float m[ROWS], l[ROWS], o[ROWS][DPL];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[r][e] = 0.f;
  }

  const T* kb = (const T*)a.k + (int64_t)bg * a.head_stride + sub * E16;
  const T* vb = (const T*)a.v + (int64_t)bg * a.head_stride + sub * E16;
  const float qs = a.qscale;

  // this wave's run of the flattened token list
  const int w0 = t0 + wave * a.wave_tokens;
  const int w1 = min(w0 + a.wave_tokens, t_end);
  int cur = 0;
  int4 it = s_items[0];

  auto load = [&](Group<T, DPL, U>& gr, int tb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tau = tb + u * TPS + slot;
      bool val = tau < w1;
      if (val) {
        while (tau >= it.w + it.y && cur + 1 < ns) it = s_items[++cur];
        val = tau >= it.w && tau < it.w + it.y;
      }
      gr.pos[u] = it.x + (tau - it.w);
      gr.msk[u] = val ? (uint32_t)it.z : 0u;
      const int64_t off = (int64_t)(val ? gr.pos[u] : it.x) * a.row_stride;
#pragma unroll
      for (int w = 0; w < NU; ++w) gr.k[u][w] = *reinterpret_cast<const uint4*>(kb + off + w * L * E16);
#pragma unroll
      for (int w = 0; w < NU; ++w) gr.v[u][w] = *reinterpret_cast<const uint4*>(vb + off + w * L * E16);
    }
  };

  auto compute = [&](const Group<T, DPL, U>& gr) {
    float s[U][ROWS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t kw[4 * NU];
#pragma unroll
      for (int w = 0; w < NU; ++w) {
        kw[4 * w] = gr.k[u][w].x;
        kw[4 * w + 1] = gr.k[u][w].y;
        kw[4 * w + 2] = gr.k[u][w].z;
        kw[4 * w + 3] = gr.k[u][w].w;
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float acc = 0.f;
        if constexpr (BF) {
#pragma unroll
          for (int e = 0; e < QW; ++e)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[r][e]),
                                                  __builtin_bit_cast(bf16x2_t, kw[e]), acc, false);
        } else {
#pragma unroll
          for (int e = 0; e < QW; ++e) acc = fmaf(__uint_as_float(qw[r][e]), __uint_as_float(kw[e]), acc);
        }
        acc = group_sum<L>(acc);
        const bool pass = (gr.msk[u] & rowbit[r]) && gr.pos[u] <= plim[r];
        s[u][r] = pass ? acc * qs : kNegInf;
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
        const float al = (mt[r] == m[r]) ? 1.f : fast_exp2(m[r] - mt[r]);
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
      for (int w = 0; w < NU; ++w) Elt<T>::unpack(gr.v[u][w], &vf[w * E16]);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float p = (s[u][r] == kNegInf) ? 0.f : fast_exp2(s[u][r] - m[r]);
        l[r] += p;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
      }
    }
  };

  constexpr int GT = TPS * U;  // tokens per group
  Group<T, DPL, U> ga, gb;
  int tb = w0;
  if (tb < w1) load(ga, tb);
  if (tb + GT < w1) load(gb, tb + GT);
  while (tb < w1) {
    compute(ga);
    tb += GT;
    if (tb + GT < w1) load(ga, tb + GT);
    if (tb >= w1) break;
    compute(gb);
    tb += GT;
    if (tb + GT < w1) load(gb, tb + GT);
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

  // combine the waves of the workgroup in LDS and write this chunk's partials
  __shared__ float s_o[NWMAX][ROWS][D];
  __shared__ float s_m[NWMAX][ROWS];
  __shared__ float s_l[NWMAX][ROWS];
  if (slot == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
#pragma unroll
      for (int w = 0; w < NU; ++w)
#pragma unroll
        for (int e = 0; e < E16; ++e) s_o[wave][r][(w * L + sub) * E16 + e] = o[r][w * E16 + e];
      if (sub == 0) {
        s_m[wave][r] = m[r];
        s_l[wave][r] = l[r];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < rows_here * D; t += blockDim.x) {
    const int r = t / D, e = t - r * D;
    float M = kNegInf;
    for (int w = 0; w < a.nw; ++w) M = fmaxf(M, s_m[w][r]);
    float Ls = 0.f, Os = 0.f;
    for (int w = 0; w < a.nw; ++w) {
      const float mw = s_m[w][r];
      const float f = (mw == kNegInf) ? 0.f : exp2f(mw - M);
      Ls += s_l[w][r] * f;
      Os += s_o[w][r][e] * f;
    }
    const int64_t pidx = row_index(a, b, g, rg * a.rows_per_group + r) * a.max_chunks + c;
    a.o[pidx * D + e] = Os;
    if (e == 0) a.ml[pidx] = make_float2(M, Ls);
  }
}

// Matrix-core path (bfloat16, head_dim 64/128/256, up to 16 query rows per
// group).  Per wave, tiles of 32 tokens:
//   S^T = K Q^T  with v_mfma_f32_16x16x32_bf16: A = 16 token rows of K (each
//                lane loads 16 contiguous bytes of a row), B = the query rows
//                (zero beyond the group), accumulator lane l = tokens
//                4(l/16)+i of the 16, query row l%16;
//   O  += P V    with the same instruction: that accumulator layout is already
//                the A operand (query row l%16, 8 tokens), and V is read back
//                from LDS with the transposing ds_read_b64_tr_b16 into the B
//                operand.  P is split into bf16 high and low parts (two MFMAs),
//                so the weights keep about 16 significant bits.
// Softmax is online with a lazy reference: the row reference only moves when
// a tile's maximum exceeds it by more than 2^8, so rescaling is rare and
// weights stay below 256.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLazy = 8.0f;      // log2 headroom before the reference moves
constexpr float kFarNeg = -1e30f;  // initial reference (finite: keeps 2^(s - ref) NaN-free)

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even, two values into one register
  auto rne = [](float f) -> uint32_t {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  };
  return rne(lo) | (rne(hi) << 16);
}

template <int D, int NWMAX>
__global__ __launch_bounds__(64 * NWMAX) void attn_split_mfma_kernel(SplitArgs a) {
  constexpr int KC = D / 32;  // 32-wide k chunks of the head dim
  constexpr int NJ = D / 16;  // 16-wide output column tiles
  __shared__ int4 s_items[kItemsLds];
  __shared__ ChunkPlanLds s_plan;
  // V tiles, rows padded by 32 bytes: the four rows one transposed read
  // gathers then fall on disjoint banks.  Reused to combine the waves.
  constexpr int VS = D + 16;
  __shared__ __align__(16) uint16_t s_v[NWMAX][32][VS];
  __shared__ int2 s_meta[NWMAX][32];
  __shared__ float s_m[NWMAX][16], s_l[NWMAX][16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, n = lane & 15;
  const int c = blockIdx.x, bg = blockIdx.y, rg = blockIdx.z;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int rows_here = min(a.rows_per_group, a.rows - rg * a.rows_per_group);

  // query row n of this group as the B operand
  const bool act = n < rows_here;
  const int gr = rg * a.rows_per_group + n;
  const int jh = act ? gr / a.n_q : 0, qi = act ? gr - jh * a.n_q : 0;
  const uint32_t rowbit = act ? (1u << jh) : 0u;
  const int plim = a.N - a.n_q + qi;
  uint4 qb[KC];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((int64_t)b * a.hq + g * a.G + jh) * a.n_q + qi) * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
      qb[kk] = act ? *reinterpret_cast<const uint4*>(qrow + 32 * kk) : make_uint4(0, 0, 0, 0);
  }

  int ns, t_end;
  if (a.local) {
    ns = chunk_plan(a, b, g, c, rg, s_items, s_plan, &t_end);
    if (ns < 0) return;
  } else {
    const int4 desc = a.chunks[(int64_t)bg * a.max_chunks + c];
    if (desc.x >= desc.y) return;
    ns = stage_items(a, bg, desc, s_items);
    t_end = desc.z;
  }
  const int t0 = c * a.chunk_tokens;
  const int w0 = t0 + wave * a.wave_tokens;
  const int w1 = min(w0 + a.wave_tokens, t_end);

  const uint16_t* kb = (const uint16_t*)a.k + (int64_t)bg * a.head_stride + 8 * g4;
  const uint16_t* vb = (const uint16_t*)a.v + (int64_t)bg * a.head_stride + 8 * g4;
  const float qs = a.qscale;

  f32x4_t o[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) o[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = kFarNeg, lpart = 0.f;

  // cursor over the chunk's segments (each lane follows tokens tile + n and tile + 16 + n)
  int cur = 0;
  int4 it = s_items[0];
  auto locate = [&](int tau, int& pos, uint32_t& msk) {
    bool val = tau < w1;
    if (val) {
      while (tau >= it.w + it.y && cur + 1 < ns) it = s_items[++cur];
      val = tau >= it.w && tau < it.w + it.y;
    }
    pos = it.x + (tau - it.w);
    msk = val ? (uint32_t)it.z : 0u;
    return val;
  };

  struct Tile {
    uint4 k[2][KC], v[2][KC];
    int pos[2];
    uint32_t msk[2];
  };
  auto load = [&](Tile& tl, int tb) {
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      const bool val = locate(tb + 16 * sidx + n, tl.pos[sidx], tl.msk[sidx]);
      const int64_t off = (int64_t)(val ? tl.pos[sidx] : it.x) * a.row_stride;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) tl.k[sidx][kk] = *reinterpret_cast<const uint4*>(kb + off + 32 * kk);
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) tl.v[sidx][kk] = *reinterpret_cast<const uint4*>(vb + off + 32 * kk);
    }
  };

  // One tile of registers: its K feeds the S^T MFMAs and its V goes to LDS,
  // then the next tile's loads are issued into the same registers while the
  // softmax and the P V products of this tile run.
  Tile tl;
  if (w0 < w1) load(tl, w0);
  for (int tb = w0; tb < w1; tb += 32) {
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
        *reinterpret_cast<uint4*>(&s_v[wave][16 * sidx + n][32 * kk + 8 * g4]) = tl.v[sidx][kk];
    if (g4 == 0) {
      s_meta[wave][n] = make_int2(tl.pos[0], (int)tl.msk[0]);
      s_meta[wave][16 + n] = make_int2(tl.pos[1], (int)tl.msk[1]);
    }
    f32x4_t st[2];
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      st[sidx] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
        st[sidx] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tl.k[sidx][kk]), as_bf16x8(qb[kk]), st[sidx], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (tb + 32 < w1) load(tl, tb + 32);
    // logits of this lane: tokens 4*g4 + i (first half) and 16 + 4*g4 + i, query row n
    float sv[8];
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int2 md = s_meta[wave][16 * sidx + 4 * g4 + i];
        const bool pass = (((uint32_t)md.y & rowbit) != 0u) & (md.x <= plim);  // no branch around the read
        sv[4 * sidx + i] = pass ? st[sidx][i] * qs : kNegInf;
      }
    float tm = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tm = fmaxf(tm, sv[i]);
    tm = xmax16_32(tm);
    if (__ballot(tm > mref + kLazy)) {
      const float nm = fmaxf(mref, tm);
      const float al = fast_exp2(mref - nm);
      mref = nm;
      lpart *= al;
      // accumulator rows are 4*g4 + i: fetch their factors from lanes 4*g4 + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(al, 4 * g4 + i);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) o[jj][i] *= ai;
      }
    }
    // weights: high and low bf16 parts
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(sv[i] - mref);
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
      const float h0 = __uint_as_float(ph[i] << 16), h1 = __uint_as_float(ph[i] & 0xffff0000u);
      pl[i] = pack_bf16x2(pv[2 * i] - h0, pv[2 * i + 1] - h1);
      lpart += pv[2 * i] + pv[2 * i + 1];
    }
    const bf16x8_t pa_hi = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8_t pa_lo = __builtin_bit_cast(bf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
    // O += P V, V columns 16*jj..16*jj+15 read transposed from LDS
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int col = 16 * jj + 4 * (n & 3);
      const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&s_v[wave][4 * g4 + (n >> 2)][col]);
      const i16x4_t v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&s_v[wave][16 + 4 * g4 + (n >> 2)][col]);
      const bf16x8_t vbv = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vbv, o[jj], 0, 0, 0);
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vbv, o[jj], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // row sums over the four lanes that share a query row
  lpart += __shfl_xor(lpart, 16);
  lpart += __shfl_xor(lpart, 32);

  // combine the waves: O rows 4*g4 + i, columns 16*jj + n; V tiles' LDS reused
  __syncthreads();
  float* s_o = reinterpret_cast<float*>(&s_v[0][0][0]);  // [NWMAX][16][D] floats fit in [NWMAX][32][VS] halves
  if (lane < 16) {
    s_m[wave][lane] = mref;
    s_l[wave][lane] = lpart;
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[((int64_t)wave * 16 + 4 * g4 + i) * D + 16 * jj + n] = o[jj][i];
  __syncthreads();
  for (int t = threadIdx.x; t < rows_here * D; t += blockDim.x) {
    const int r = t / D, e = t - r * D;
    float M = kFarNeg;
    for (int w = 0; w < a.nw; ++w) M = fmaxf(M, s_m[w][r]);
    float Ls = 0.f, Os = 0.f;
    for (int w = 0; w < a.nw; ++w) {
      const float f = fast_exp2(s_m[w][r] - M);
      Ls += s_l[w][r] * f;
      Os += s_o[((int64_t)w * 16 + r) * D + e] * f;
    }
    const int64_t pidx = row_index(a, b, g, rg * a.rows_per_group + r) * a.max_chunks + c;
    a.o[pidx * D + e] = Os;
    if (e == 0) a.ml[pidx] = make_float2(M, Ls);
  }
}

// Slot layout (matrix cores, bfloat16): the token list of a kv slice is
// fixed before any selection is read -- the sinks, the window (each padded to
// whole 32-token tiles), then one slot of roundup(B, 32) tokens per
// selection entry (head-major, rank order).  A slot tile is resolved from
// the entries alone: the block it names is clipped against sinks and
// window, dropped when an earlier entry names the same block (the union:
// each token once per kv slice), and masked to every query head whose
// selection holds it.  No plan kernel and no LDS bitmap.
//
// A unit (kv slice, row group, chunk) is one workgroup of eight waves, about
// one per CU.  Waves 0-3 first obtain the selections -- read from idx, or
// selected in the kernel itself (attn_step_kernel: wave w takes the top-k of
// its kv slice's score row w) -- while waves 4-7 run the sink/window tiles,
// which need none (the slice's waves 4-7 take them in turn: tiles gw, gw + W,
// ...).  After one barrier every wave runs its equal share of slot tiles,
// dealt from the slice's last wave backwards.
// K and V come through buffer loads with one 32-bit offset per token;
// invalid tokens get an offset past the slice and read zeros without
// touching memory.
constexpr int kXcdCount = 8;           // XCDs; consecutive workgroups go to consecutive XCDs
constexpr int kSlotRegs = 8;           // selection entries per lane: at most 512 per kv slice
constexpr int kSlotRegsMax = 20;       // the wider instantiation (idx read by the split kernel): 1280
constexpr int kSlotOOR = 0x7ffff000;   // buffer offset past any slice
constexpr int kSlotFlags = 0x00020000; // raw buffer resource word 3 (32-bit data, no swizzle)
constexpr int kSlotWaves = 8;          // waves per slot workgroup
constexpr int kSelWaves = 4;           // waves 0..R-1 select (R <= 4 score rows); the others take the sink/window tiles
constexpr int kStepK = 128;            // largest k selected inside the attention kernel
constexpr int kStepCand = 256;         // candidates the fast selection ranks (else the radix select)
constexpr int kWaitVm0 = 0x0F70;       // s_waitcnt vmcnt(0), other counters unconstrained
constexpr int kKvStream = 2;            // cache policy of the whole-row K/V loads: non-temporal

// A pointer the compiler keeps in scalar registers (a buffer resource built
// from a vector register would need a loop over its distinct values).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

template <int D, int REGS = kSlotRegs>
struct SlotLds {
  __align__(16) uint16_t v[kSlotWaves][32][D + 16];  // V rows padded by 32 bytes (conflict-free transposed reads)
  float m[kSlotWaves][16], l[kSlotWaves][16];
  int ents[64 * REGS];  // the kv slice's selection entries, head-major
};

// In-kernel selection: one score row per selection wave.
struct StepLds {
  TopkRowShared tk[kSelWaves];
  uint64_t sel[kSelWaves][kStepCand];  // kStepCand >= kStepK: also the radix select's kept keys
  uint32_t selv[kSelWaves][kStepCand];
  int flag[kSelWaves];
};

template <int D, int KPTW, int REGS = kSlotRegs, bool PAGED = false>  // KPTW > 0: select in the kernel, KPTW
                                                                     // scores per lane; REGS selection entries
                                                                     // per lane; PAGED: K/V through a page table
__device__ __forceinline__ void slot_unit(const SplitArgs& a, int unit, SlotLds<D, REGS>& sm, StepLds* st) {
  constexpr bool STEP = KPTW > 0;
  constexpr int KC = D / 32;  // 32-wide k chunks of the head dim
  constexpr int NJ = D / 16;  // 16-wide output column tiles
  auto& s_v = sm.v;
  auto& s_m = sm.m;
  auto& s_l = sm.l;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, n = lane & 15;
  const int c = unit % a.max_chunks, rest = unit / a.max_chunks;
  const int rg = rest % a.row_groups, bg = rest / a.row_groups;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int rows_here = min(a.rows_per_group, a.rows - rg * a.rows_per_group);

  // Selection waves issue their score loads first: issued behind the query
  // loads (or behind other waves' tile loads in the same code), they would
  // wait for those before starting.
  const int R = sel_lists(a.idx_heads, a.hkv);  // selection rows of this kv slice
  uint32_t raw[STEP ? KPTW : 1];
  if constexpr (STEP) {
    if (wave < R) {
      const int64_t row = sel_row(a.idx_heads, a.hkv, b, g, wave);
      topk_load_raw<KPTW>(a.scores + row * a.score_stride, a.sel_lo, a.sel_hi, 64, raw);
    }
  }

  // query row n of this group as the B operand; lanes past the group's rows
  // load row 0 again: their logits are masked (rowbit 0) and their output
  // rows never written, so no zeroing (which would wait for the loads)
  const bool act = n < rows_here;
  const int gr = rg * a.rows_per_group + n;
  const int jh = act ? gr / a.n_q : 0, qi = act ? gr - jh * a.n_q : 0;
  const uint32_t rowbit = act ? (1u << jh) : 0u;
  const int plim = a.N - a.n_q + qi;
  uint4 qb[KC];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((int64_t)b * a.hq + g * a.G + jh) * a.n_q + qi) * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) qb[kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
  }

  // the wave's tiles: fa sink/window tiles, then its run of slot tiles.  The
  // sink/window tiles are strided over the waves past the selection waves
  // (waves nsel .. 7 of every chunk, nsel = the slice's score rows, at most
  // kSelWaves), with the same dealing when the selections come from idx, so
  // both kernels give the same partials.
  const int nsel = min(R, kSelWaves), nfix = kSlotWaves - nsel;
  const bool fixw = wave >= nsel;
  const int tA = a.len_a >> 5, tB = a.len_b >> 5;
  const int wf_all = a.max_chunks * nfix, gwf = c * nfix + (wave - nsel);
  const int fa = fixw && tA > gwf ? (tA - 1 - gwf) / wf_all + 1 : 0;
  // slot runs are dealt from the slice's last wave backwards: the fixed
  // tiles that do not divide evenly land on the first chunks, so a short slot
  // list (few selections) goes to chunks without an extra fixed tile
  const int wt_all = a.max_chunks * kSlotWaves, gw = wt_all - 1 - (c * kSlotWaves + wave);
  const int qB = (tB + wt_all - 1) / wt_all, b0 = gw * qB;
  const int n_tiles = fa + max(0, min(b0 + qB, tB) - b0);

  // selection entries of this (batch, kv head): entry e = lane + 64 r, head e / K
  const int E = a.n_ent, K = a.kk;
  const int nreg = (E + 63) >> 6;
  const uint32_t full = a.G >= 32 ? 0xffffffffu : ((1u << a.G) - 1u);
  int ent[REGS];
  if constexpr (!STEP) {
#pragma unroll
    for (int r = 0; r < REGS; ++r) {
      const int e = lane + 64 * r, ec = min(e, E - 1);
      const int j = ec / K;
      const int v = a.idx[sel_row(a.idx_heads, a.hkv, b, g, j) * K + (ec - j * K)];
      ent[r] = e < E ? v : -2;
    }
  }

  // the slot last resolved (wave-uniform): its block, head mask (0: skipped)
  // and, through a page table, the first physical row of its block
  int c_slot = -1, c_blk = 0, c_row = 0;
  uint32_t c_mk = 0u;
  const int32_t* ptab = PAGED ? a.pages + (int64_t)bg * a.pages_stride : nullptr;
  auto resolve = [&](int s) {
    c_slot = s;
    c_mk = 0u;
    c_blk = __builtin_amdgcn_readfirstlane(sm.ents[s]);
    const int X = c_blk;
    if (X < 0 || X >= a.nb || max(X * a.B, a.sink_end) >= min(X * a.B + a.B, a.win_start)) return;
    if constexpr (PAGED) c_row = __builtin_amdgcn_readfirstlane(ptab[X]) * a.B;
    // entries naming the same block: the first one attends it for all their heads
    int first = 1 << 30, tot = 0;
#pragma unroll
    for (int rr = 0; rr < REGS; ++rr) {
      if (rr < nreg) {
        const uint64_t m = __ballot(ent[rr] == X);
        tot += __popcll(m);
        if (m && first == 1 << 30) first = 64 * rr + __builtin_ctzll(m);
      }
    }
    if (first < s) return;
    if (R != a.G) {  // one list shared by every head of the slice
      c_mk = full;
    } else if (tot == 1) {
      c_mk = 1u << (s / K);
    } else {
#pragma unroll
      for (int rr = 0; rr < REGS; ++rr) {
        if (rr < nreg) {
          uint64_t m = __ballot(ent[rr] == X);
          while (m) {
            c_mk |= 1u << ((64 * rr + __builtin_ctzll(m)) / K);
            m &= m - 1ull;
          }
        }
      }
    }
  };
  // the wave's tile i (wave-uniform): first row, valid row range, head mask;
  // slots = false leaves slot tiles empty (before the selections are known)
  auto tile_info = [&](int i, int& pos0, int& vlo, int& vhi, uint32_t& mk, int& row0, bool slots) {
    pos0 = 0;
    row0 = -1;
    vlo = 0;
    vhi = 0;
    mk = 0u;
    if (i >= n_tiles) return;
    if (i < fa) {
      const int tb = (gwf + i * wf_all) << 5;
      if (tb < a.slot_ps) {
        pos0 = tb;
        vhi = a.sink_end;
      } else {
        pos0 = a.win_start + (tb - a.slot_ps);
        vlo = a.win_start;
        vhi = a.N;
      }
      mk = full;
    } else {
      if (!slots) return;
      const int tb = (b0 + i - fa) << 5;
      const int s = tb / a.slot_bs, off = tb - s * a.slot_bs;
      if (s != c_slot) resolve(s);
      if (c_mk == 0u) return;
      const int X = c_blk;
      vlo = max(X * a.B, a.sink_end);
      vhi = min(X * a.B + a.B, a.win_start);
      pos0 = X * a.B + off;
      row0 = PAGED ? c_row + off : pos0;
      mk = c_mk;
    }
  };

  const int rs2 = a.row_stride * 2;
  // whole-row V loads: VRPI tile rows per load instruction, lane (vr, vu)
  constexpr int VUPR = D / 8, VRPI = 64 / VUPR;
  static_assert(VRPI * 2 * KC == 32, "a tile's 32 V rows in 2 KC loads per lane");
  const int vr = lane / VUPR, vu = lane - vr * VUPR;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr((const uint16_t*)a.k + (int64_t)bg * a.head_stride), (short)0, a.slice_bytes, kSlotFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr((const uint16_t*)a.v + (int64_t)bg * a.head_stride), (short)0, a.slice_bytes, kSlotFlags);
  const float qs = a.qscale;

  f32x4_t o[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) o[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = kFarNeg, lpart = 0.f;

  struct Tile {
    uint4 k[2][KC], v[2][KC];
    int pos0, vlo, vhi;  // first position, valid positions [vlo, vhi)
    int row0;            // physical row of pos0 (a slot tile), or -1 (sinks/window through the page table)
    uint32_t mk;         // query heads that attend the tile
  };
  // loads are issued whatever the tile: invalid tokens read zeros
  auto load = [&](Tile& tl, int i, bool slots) {
    tile_info(i, tl.pos0, tl.vlo, tl.vhi, tl.mk, tl.row0, slots);
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      const int pos = tl.pos0 + 16 * sidx + n;
      const bool val = (tl.mk != 0u) & (pos >= tl.vlo) & (pos < tl.vhi);
      int row = pos;
      if constexpr (PAGED) {
        const int blk = val ? pos / a.B : 0;
        row = tl.row0 >= 0 ? tl.row0 + 16 * sidx + n : ptab[blk] * a.B + (pos - blk * a.B);
      }
      if constexpr (PAGED) {
        const int off = val ? row * rs2 + 16 * g4 : kSlotOOR;
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          tl.k[sidx][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 64 * kk, 0, 0));
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          tl.v[sidx][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off + 64 * kk, 0, 0));
      }
    }
    if constexpr (!PAGED) {
      // K and V pass through LDS, so their loads need not follow the operand
      // layout: load j of lane l takes 16-byte unit vu of tile row
      // VRPI j + vr, so an instruction reads whole rows (whole cache lines),
      // with the non-temporal policy (each row is read once)
#pragma unroll
      for (int j = 0; j < 2 * KC; ++j) {
        const int pos = tl.pos0 + VRPI * j + vr;
        const bool val = (tl.mk != 0u) & (pos >= tl.vlo) & (pos < tl.vhi);
        const int off = val ? pos * rs2 + 16 * vu : kSlotOOR;
        tl.k[j / KC][j % KC] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kKvStream));
        tl.v[j / KC][j % KC] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kKvStream));
      }
    }
  };

  // one tile: V to LDS, S^T on the matrix cores, the loads of tile tn into
  // the same registers, then softmax and O += P V
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto step = [&](Tile& tl, int tn, bool slots) {
    f32x4_t st2[2];
    const int p0 = tl.pos0, vlo = tl.vlo, vhi = tl.vhi;
    const bool rowok = (tl.mk & rowbit) != 0u;
    if constexpr (PAGED) {
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          *reinterpret_cast<uint4*>(&s_v[wave][16 * sidx + n][32 * kk + 8 * g4]) = tl.v[sidx][kk];
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) {
        st2[sidx] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          st2[sidx] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(tl.k[sidx][kk]), as_bf16x8(qb[kk]), st2[sidx], 0, 0, 0);
      }
    } else {
      // K rows through the wave's LDS tile into the operand layout (lane
      // (g4, n): 16 bytes of row 16 sidx + n per k chunk), then V into the
      // same tile
#pragma unroll
      for (int j = 0; j < 2 * KC; ++j)
        *reinterpret_cast<uint4*>(&s_v[wave][VRPI * j + vr][8 * vu]) = tl.k[j / KC][j % KC];
      wave_sync();
      uint4 kop[2][KC];
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          kop[sidx][kk] = *reinterpret_cast<const uint4*>(&s_v[wave][16 * sidx + n][32 * kk + 8 * g4]);
      wave_sync();
#pragma unroll
      for (int j = 0; j < 2 * KC; ++j)
        *reinterpret_cast<uint4*>(&s_v[wave][VRPI * j + vr][8 * vu]) = tl.v[j / KC][j % KC];
      load(tl, tn, slots);  // the tile's registers are free: the next loads go out now
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) {
        st2[sidx] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          st2[sidx] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[sidx][kk]), as_bf16x8(qb[kk]), st2[sidx], 0, 0, 0);
      }
    }
    wave_sync();
    if constexpr (PAGED) load(tl, tn, slots);
    // logits of this lane: tokens 4*g4 + i (first half) and 16 + 4*g4 + i, query row n
    float sv[8];
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = p0 + 16 * sidx + 4 * g4 + i;
        const bool pass = rowok & (pos >= vlo) & (pos < vhi) & (pos <= plim);
        sv[4 * sidx + i] = pass ? st2[sidx][i] * qs : kNegInf;
      }
    float tm = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tm = fmaxf(tm, sv[i]);
    tm = xmax16_32(tm);
    if (__ballot(tm > mref + kLazy)) {
      const float nm = fmaxf(mref, tm);
      const float al = fast_exp2(mref - nm);
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
    for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(sv[i] - mref);
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
      const float h0 = __uint_as_float(ph[i] << 16), h1 = __uint_as_float(ph[i] & 0xffff0000u);
      pl[i] = pack_bf16x2(pv[2 * i] - h0, pv[2 * i + 1] - h1);
      lpart += pv[2 * i] + pv[2 * i + 1];
    }
    const bf16x8_t pa_hi = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8_t pa_lo = __builtin_bit_cast(bf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int col = 16 * jj + 4 * (n & 3);
      const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&s_v[wave][4 * g4 + (n >> 2)][col]);
      const i16x4_t v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&s_v[wave][16 + 4 * g4 + (n >> 2)][col]);
      const bf16x8_t vbv = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vbv, o[jj], 0, 0, 0);
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vbv, o[jj], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Phase 1: waves 4-7 run their sink/window tiles (the prefetch past the
  // last one stays empty); waves 0-3 obtain the selections.  Phase 2, after
  // the barrier: every wave runs its slot tiles.
  Tile ta;
  if (fixw && fa > 0) {
    load(ta, 0, false);
    for (int it = 0; it < fa; ++it) step(ta, it + 1, false);
  }
  if constexpr (STEP) {
    // wave w selects score row w of the kv slice (loaded at the start)
    if (wave < R) {
      const int64_t row = sel_row(a.idx_heads, a.hkv, b, g, wave);
      const bool out = c == 0 && rg == 0;  // one workgroup per kv slice writes the selection
      int32_t* gi = out ? a.idx_out + row * K : nullptr;
      float* gv = out && a.vals_out ? a.vals_out + row * K : nullptr;
      if (!wave_topk_filter<KPTW>(raw, a.sel_lo, a.sel_hi, K, kStepCand - 1, st->sel[wave], st->selv[wave], gi, gv,
                                  sm.ents + wave * K)) {
        TopkRowShared& tk = st->tk[wave];
#pragma unroll
        for (int j = 0; j < 4; ++j) tk.hist[lane + 64 * j] = 0u;
        if (lane == 0) {
          tk.cnt = 0;
          st->flag[wave] = 0;
        }
        wave_lds_sync();
        group_topk_raw<KPTW, true>(raw, a.sel_lo, a.sel_hi, K, 64, tk, &st->flag[wave], st->sel[wave],
                                   st->selv[wave], gi, gv, sm.ents + wave * K, nullptr);
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < REGS; ++r) {
      const int e = lane + 64 * r;
      ent[r] = e < E ? sm.ents[min(e, E - 1)] : -2;
    }
  } else {
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < REGS; ++r)
        if (r < nreg) sm.ents[lane + 64 * r] = ent[r];
    }
    __syncthreads();
  }
  const int ns = n_tiles - fa;  // slot tiles of this wave
  load(ta, fa, true);
  for (int it = 0; it < ns; ++it) step(ta, fa + it + 1, true);

  // row sums over the four lanes that share a query row
  lpart += __shfl_xor(lpart, 16);
  lpart += __shfl_xor(lpart, 32);

  // combine the waves: O rows 4*g4 + i, columns 16*jj + n; V tiles' LDS reused
  __syncthreads();
  float* s_o = reinterpret_cast<float*>(&sm.v[0][0][0]);  // [8][16][D] floats fit in [8][32][D + 16] halves
  if (lane < 16) {
    s_m[wave][lane] = mref;
    s_l[wave][lane] = lpart;
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[((int64_t)wave * 16 + 4 * g4 + i) * D + 16 * jj + n] = o[jj][i];
  __syncthreads();
  for (int t = threadIdx.x; t < rows_here * D; t += blockDim.x) {
    const int r = t / D, e = t - r * D;
    float M = kFarNeg;
    for (int w = 0; w < kSlotWaves; ++w) M = fmaxf(M, s_m[w][r]);
    float Ls = 0.f, Os = 0.f;
    for (int w = 0; w < kSlotWaves; ++w) {
      const float f = fast_exp2(s_m[w][r] - M);
      Ls += s_l[w][r] * f;
      Os += s_o[((int64_t)w * 16 + r) * D + e] * f;
    }
    const int64_t pidx = row_index(a, b, g, rg * a.rows_per_group + r) * a.max_chunks + c;
    a.o[pidx * D + e] = Os;
    if (e == 0) a.ml[pidx] = make_float2(M, Ls);
  }
}

// Units go out in dispatch order, which deals them round-robin over the 8
// XCDs: every XCD gets an eighth of each kv slice's chunks, which balances
// the slices' unequal work (measured 0.4-0.9 us faster per step than one
// slice per XCD).

// Attention over the slot layout with the selections read from idx (PAGED:
// K/V through the page table of a block cache).
template <int D, int REGS, bool PAGED>
__global__ __launch_bounds__(64 * kSlotWaves) void attn_split_slot_kernel(SplitArgs a) {
  __shared__ SlotLds<D, REGS> sm;
  const int unit = blockIdx.x;
  if (unit >= a.n_units) return;
  slot_unit<D, 0, REGS, PAGED>(a, unit, sm, nullptr);
}

// The whole decode step after scoring: the selection of every score row of
// the kv slice (written out by the slice's first workgroup), then the same
// attention as attn_split_slot_kernel -- identical partials.
template <int D, int KPTW>
__global__ __launch_bounds__(64 * kSlotWaves) void attn_step_kernel(SplitArgs a) {
  __shared__ SlotLds<D> sm;
  __shared__ StepLds st;
  const int unit = blockIdx.x;
  if (unit >= a.n_units) return;
  slot_unit<D, KPTW>(a, unit, sm, &st);
}

// Any head_dim <= 512 and any row stride: one token at a time per wave,
// lanes across the dims.  One wave per workgroup.
template <typename T>
__global__ __launch_bounds__(64) void attn_split_generic_kernel(SplitArgs a) {
  constexpr int NE = 8;  // dims per lane, head_dim <= 512
  __shared__ int4 s_items[kItemsLds];
  __shared__ ChunkPlanLds s_plan;
  const int lane = threadIdx.x;
  const int c = blockIdx.x, bg = blockIdx.y, rg = blockIdx.z;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  int ns, t1;
  if (a.local) {
    ns = chunk_plan(a, b, g, c, rg, s_items, s_plan, &t1);
    if (ns < 0) return;  // past the end of this (batch, kv head)'s tokens
  } else {
    const int4 desc = a.chunks[(int64_t)bg * a.max_chunks + c];
    if (desc.x >= desc.y) return;
    ns = stage_items(a, bg, desc, s_items);
    t1 = desc.z;
  }
  const int t0 = c * a.chunk_tokens;
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
      qf[r][u] = (act && e < D) ? Elt<T>::load(qrow + e) : 0.f;
      o[r][u] = 0.f;
    }
    m[r] = kNegInf;
    l[r] = 0.f;
  }
  const T* kb = (const T*)a.k + (int64_t)bg * a.head_stride;
  const T* vb = (const T*)a.v + (int64_t)bg * a.head_stride;
  int cur = 0;
  int4 it = s_items[0];
  for (int tau = t0; tau < t1; ++tau) {
    while (tau >= it.w + it.y && cur + 1 < ns) it = s_items[++cur];
    const bool val = tau >= it.w && tau < it.w + it.y;
    const int pos = val ? it.x + (tau - it.w) : it.x;
    const uint32_t mask = val ? (uint32_t)it.z : 0u;
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
      const float sc = ((mask & rowbit[r]) && pos <= plim[r]) ? acc * a.qscale : kNegInf;
      const float mn = fmaxf(m[r], sc);
      const float al = (mn == m[r]) ? 1.f : exp2f(m[r] - mn);
      const float p = (sc == kNegInf) ? 0.f : exp2f(sc - mn);
      l[r] = l[r] * al + p;
#pragma unroll
      for (int u = 0; u < NE; ++u) o[r][u] = o[r][u] * al + p * vf[u];
      m[r] = mn;
    }
  }
  for (int r = 0; r < rows_here; ++r) {
    const int64_t pidx = row_index(a, b, g, rg * a.rows_per_group + r) * a.max_chunks + c;
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = lane + 64 * u;
      if (e < D) a.o[pidx * D + e] = o[r][u];
    }
    if (lane == 0) a.ml[pidx] = make_float2(m[r], l[r]);
  }
}

// ---------------------------------------------------------------------------
// dispatch

template <int D, int ROWS>
constexpr int nwmax_for() {
  return ROWS * D <= 1024 ? 8 : 4;
}

// Each lane holds 16 bytes of a row (16 lanes per 128-dim bf16 row: fewer
// registers and more waves than 32 bytes per lane, measured faster).
// Tokens of one group of the vector kernel: TPS * U.
int step_tokens(const AttnGeom& g) {
  const int es = elem_bytes(g.dtype);
  const int L = g.d / (16 / es);
  return (64 / L) * kSplitU;
}

int nw_max(const AttnGeom& g) {
  const int R = g.rows_per_group <= 1 ? 1 : g.rows_per_group <= 2 ? 2 : g.rows_per_group <= 4 ? 4 : 8;
  return R * g.d <= 1024 ? 8 : 4;
}

template <typename T, int D>
bool launch_fast_d(const AttnGeom& g, dim3 grid, dim3 block, hipStream_t s, const SplitArgs& a, hipEvent_t ev0,
                   hipEvent_t ev1) {
  const int rows = g.rows_per_group;
  constexpr int DPL = 16 / (int)sizeof(T);
#define BRS_LAUNCH_ROWS(R)                                                                                    \
  if (rows <= R) {                                                                                            \
    constexpr int NWM = nwmax_for<D, R>();                                                                    \
    if (ev0)                                                                                                  \
      hipExtLaunchKernelGGL((attn_split_kernel<T, D, DPL, R, kSplitU, NWM>), grid, block, 0, s, ev0, ev1, 0, a); \
    else                                                                                                      \
      hipLaunchKernelGGL((attn_split_kernel<T, D, DPL, R, kSplitU, NWM>), grid, block, 0, s, a);             \
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
  const int64_t E = (int64_t)sel_lists(g.idx_heads, g.hkv) * g.k;
  const int64_t uniq = E < g.nb ? E : g.nb;
  const int rows = g.group * g.n_q;
  g.fast = fast_supported(g);
  g.mfma = g.fast && g.dtype == BRS_BF16 && g.d <= 128;
  const int rmax = g.mfma ? 16 : kRowsMax;
  g.row_groups = (rows + rmax - 1) / rmax;
  g.rows_per_group = rows < rmax ? rows : rmax;
  const int64_t bg = (int64_t)g.batch * g.hkv;
  g.max_items = 2 + uniq;
  g.max_tokens = (int64_t)g.sink_end + (g.N - g.win_start) + uniq * g.B;
  // the prefill kernel needs only the plan; the split path also keeps partials
  g.prefill = prefill_supported(g);
  // slot layout: every selection entry gets its own padded slot
  g.slot = g.mfma && !g.prefill && E >= 1 && E <= 64 * kSlotRegsMax && E <= g.nb &&
           g.head_stride * 2 < (int64_t)kSlotOOR - 4096;
  g.slot_regs = E <= 64 * kSlotRegs ? kSlotRegs : kSlotRegsMax;
  if (g.slot) {
    auto pad32 = [](int64_t x) { return (x + 31) / 32 * 32; };
    g.slot_ps = (int)pad32(g.sink_end);
    g.slot_bs = (int)pad32(g.B);
    g.len_a = g.slot_ps + (int)pad32(g.N - g.win_start);
    g.len_b = (int)(E * g.slot_bs);
    g.max_tokens = (int64_t)g.len_a + g.len_b;
  }
  if (g.max_tokens > INT32_MAX) return false;
  // tokens per wave: about kTargetWaves waves over the whole problem, in whole steps
  const int64_t total = g.max_tokens * bg * g.row_groups;
  const int st = g.mfma ? 32 : (g.fast ? step_tokens(g) : 1);
  int64_t wt = (total + kTargetWaves - 1) / kTargetWaves;
  wt = ((wt + st - 1) / st) * st;
  const int64_t wmin = g.mfma ? 32 : (g.fast ? 2 * st : 16);
  wt = wt < wmin ? wmin : (wt > 4096 ? 4096 : wt);
  g.wave_tokens = (int)wt;
  const int64_t waves = (total + wt - 1) / wt;
  const int nwm = g.mfma ? (g.d <= 128 ? 8 : 4) : nw_max(g);
  g.nw = !g.fast ? 1 : (waves >= 2048 ? nwm : (waves >= 1024 ? 4 : 1));
  // a chunk meets at most chunk_tokens / B + 6 segments (sinks, window, the two
  // blocks cut by them, whole blocks, one more at each end): keep them in LDS
  if (!g.slot) {
    const int64_t cap = (int64_t)(kItemsLds - 8) * g.B;
    while ((int64_t)g.nw * g.wave_tokens > cap && g.wave_tokens > st) g.wave_tokens -= st;
    while ((int64_t)g.nw * g.wave_tokens > cap && g.nw > 1) g.nw >>= 1;
    if ((int64_t)g.nw * g.wave_tokens > cap) return false;
  }
  g.chunk_tokens = g.nw * g.wave_tokens;
  int64_t mc = (g.max_tokens + g.chunk_tokens - 1) / g.chunk_tokens;
  g.max_chunks = (int)(mc < 1 ? 1 : mc);
  if (g.slot) {
    // about one four-wave workgroup per CU, each wave with at least one tile
    const int units = g.batch * g.hkv * g.row_groups;
    const int tiles = (int)(g.max_tokens / 32);
    int nc = kSlotWgs / units;
    nc = nc > tiles / kSlotWaves ? tiles / kSlotWaves : nc;
    g.nw = kSlotWaves;
    g.max_chunks = nc < 1 ? 1 : nc;
  }
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows_total = (size_t)g.batch * g.hq * g.n_q;
  g.hdr_off = 0;
  g.items_off = up((size_t)bg * sizeof(int4));
  g.first_off = g.items_off + up((size_t)bg * g.max_items * sizeof(int4));
  g.chunks_off = g.first_off + up((size_t)bg * g.max_chunks * sizeof(int));
  g.ml_off = g.chunks_off + up((size_t)bg * g.max_chunks * sizeof(int4));
  {
    const int64_t W = ((int64_t)g.nb + 31) / 32;
    const int64_t hb = sel_lists(g.idx_heads, g.hkv);
    g.local_plan = !g.prefill && !g.slot && hb * W <= kPlanWords;
  }
  const size_t parts = g.prefill ? 0 : rows_total * g.max_chunks;
  g.o_off = g.ml_off + up(parts * sizeof(float2));
  g.total = g.o_off + up(parts * (size_t)g.d * sizeof(float));
  return true;
}

hipError_t launch_attn_plan(const AttnGeom& g, const int32_t* idx, void* ws, float* out, hipStream_t s) {
  PlanArgs a;
  a.idx = idx;
  a.hdr = (int4*)((char*)ws + g.hdr_off);
  a.items = (int4*)((char*)ws + g.items_off);
  a.chunk_first = (int*)((char*)ws + g.first_off);
  a.chunks = (int4*)((char*)ws + g.chunks_off);
  a.out = out;
  a.max_items = g.max_items;
  a.max_chunks = g.max_chunks;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.G = g.group;
  a.k = idx ? g.k : 0;
  a.idx_heads = g.idx_heads;
  a.n_q = g.n_q;
  a.d = g.d;
  a.row_groups = g.row_groups;
  a.N = g.N;
  a.B = g.B;
  a.nb = g.nb;
  a.sink_end = g.sink_end;
  a.win_start = g.win_start;
  a.chunk_tokens = g.chunk_tokens;
  hipLaunchKernelGGL(attn_plan_kernel, dim3((unsigned)(g.batch * g.hkv)), dim3(1024), 0, s, a);
  return hipGetLastError();
}

namespace {
void slot_args(const AttnGeom& g, SplitArgs& a) {
  a.slot_ps = g.slot_ps;
  a.slot_bs = g.slot_bs;
  a.len_a = g.len_a;
  a.len_b = g.len_b;
  a.n_ent = sel_lists(g.idx_heads, g.hkv) * g.k;
  a.slice_bytes = (int)(g.head_stride * 2);
}

SplitArgs split_args(const AttnGeom& g, const void* k, const void* v, const void* q, const int32_t* idx, void* ws,
                     float* out) {
  SplitArgs a;
  a.k = k;
  a.v = v;
  a.q = q;
  a.hdr = (const int4*)((char*)ws + g.hdr_off);
  a.items = (const int4*)((char*)ws + g.items_off);
  a.chunks = (const int4*)((char*)ws + g.chunks_off);
  a.ml = (float2*)((char*)ws + g.ml_off);
  a.o = (float*)((char*)ws + g.o_off);
  a.max_items = g.max_items;
  a.max_chunks = g.max_chunks;
  a.head_stride = g.head_stride;
  a.row_stride = g.row_stride;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.G = g.group;
  a.n_q = g.n_q;
  a.N = g.N;
  a.d = g.d;
  a.qscale = g.qscale;
  a.chunk_tokens = g.chunk_tokens;
  a.wave_tokens = g.wave_tokens;
  a.nw = g.nw;
  a.rows = g.group * g.n_q;
  a.rows_per_group = g.rows_per_group;
  a.row_groups = g.row_groups;
  a.local = g.local_plan ? 1 : 0;
  a.idx = idx;
  a.kk = idx ? g.k : 0;
  a.idx_heads = g.idx_heads;
  a.B = g.B;
  a.nb = g.nb;
  a.sink_end = g.sink_end;
  a.win_start = g.win_start;
  a.hdr_out = (int4*)((char*)ws + g.hdr_off);
  a.out = out;
  slot_args(g, a);
  a.n_units = g.max_chunks * g.batch * g.hkv * g.row_groups;
  a.pages = g.pages;
  a.pages_stride = g.pages_stride;
  return a;
}
unsigned slot_grid(const SplitArgs& a) { return (unsigned)a.n_units; }
}  // namespace

bool step_supported(const AttnGeom& g, int64_t lo, int64_t hi, int k) {
  const int R = sel_lists(g.idx_heads, g.hkv);
  return g.slot && g.slot_regs == kSlotRegs && R <= kSelWaves && k >= 1 && k <= kStepK && hi - lo <= 64 * 32 &&
         (g.d == 64 || g.d == 128);
}

hipError_t launch_attn_step(const AttnGeom& g, const void* k, const void* v, const void* q, const float* scores,
                            int64_t stride, int64_t lo, int64_t hi, int32_t* idx, float* vals, void* ws, float* out,
                            hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  SplitArgs a = split_args(g, k, v, q, idx, ws, out);
  a.scores = scores;
  a.score_stride = stride;
  a.sel_lo = (int)lo;
  a.sel_hi = (int)hi;
  a.idx_out = idx;
  a.vals_out = vals;
  const dim3 grid(slot_grid(a)), block(64 * kSlotWaves);
  const int64_t n = hi - lo;
#define BRS_LAUNCH_STEP(DD, KP)                                                                     \
  if (g.d == DD) {                                                                                  \
    if (ev0 || ev1)                                                                                 \
      hipExtLaunchKernelGGL((attn_step_kernel<DD, KP>), grid, block, 0, s, ev0, ev1, 0, a);         \
    else                                                                                            \
      hipLaunchKernelGGL((attn_step_kernel<DD, KP>), grid, block, 0, s, a);                         \
    return hipGetLastError();                                                                       \
  }
  if (n <= 256) {
    BRS_LAUNCH_STEP(64, 4)
    BRS_LAUNCH_STEP(128, 4)
  } else if (n <= 512) {
    BRS_LAUNCH_STEP(64, 8)
    BRS_LAUNCH_STEP(128, 8)
  } else if (n <= 1024) {
    BRS_LAUNCH_STEP(64, 16)
    BRS_LAUNCH_STEP(128, 16)
  } else {
    BRS_LAUNCH_STEP(64, 32)
    BRS_LAUNCH_STEP(128, 32)
  }
#undef BRS_LAUNCH_STEP
  return hipErrorInvalidValue;
}

hipError_t launch_attn_split(const AttnGeom& g, const void* k, const void* v, const void* q, const int32_t* idx,
                             void* ws, float* out, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  SplitArgs a = split_args(g, k, v, q, idx, ws, out);
  const dim3 grid((unsigned)g.max_chunks, (unsigned)(g.batch * g.hkv), (unsigned)g.row_groups);
  if (g.slot) {
    const dim3 grid1(slot_grid(a)), block(64 * kSlotWaves);
#define BRS_LAUNCH_SLOT(DD, RG, PG)                                                                      \
  if (g.d == DD && g.slot_regs == RG && (g.pages != nullptr) == PG) {                                    \
    if (ev0)                                                                                             \
      hipExtLaunchKernelGGL((attn_split_slot_kernel<DD, RG, PG>), grid1, block, 0, s, ev0, ev1, 0, a);   \
    else                                                                                                 \
      hipLaunchKernelGGL((attn_split_slot_kernel<DD, RG, PG>), grid1, block, 0, s, a);                   \
    return hipGetLastError();                                                                            \
  }
    BRS_LAUNCH_SLOT(64, kSlotRegs, false)
    BRS_LAUNCH_SLOT(128, kSlotRegs, false)
    BRS_LAUNCH_SLOT(64, kSlotRegsMax, false)
    BRS_LAUNCH_SLOT(128, kSlotRegsMax, false)
    BRS_LAUNCH_SLOT(64, kSlotRegs, true)
    BRS_LAUNCH_SLOT(128, kSlotRegs, true)
    BRS_LAUNCH_SLOT(64, kSlotRegsMax, true)
    BRS_LAUNCH_SLOT(128, kSlotRegsMax, true)
#undef BRS_LAUNCH_SLOT
    return hipErrorInvalidValue;
  }
  if (g.mfma) {
    const dim3 block(64 * g.nw);
  // LDS sized for the waves actually launched: a smaller footprint lets
  // several workgroups share a CU
#define BRS_LAUNCH_MFMA(DD, NWM)                                                                            \
  if (g.d == DD && g.nw <= NWM) {                                                                           \
    if (ev0)                                                                                                \
      hipExtLaunchKernelGGL((attn_split_mfma_kernel<DD, NWM>), grid, block, 0, s, ev0, ev1, 0, a);         \
    else                                                                                                    \
      hipLaunchKernelGGL((attn_split_mfma_kernel<DD, NWM>), grid, block, 0, s, a);                         \
    return hipGetLastError();                                                                               \
  }
    BRS_LAUNCH_MFMA(64, 2)
    BRS_LAUNCH_MFMA(64, 4)
    BRS_LAUNCH_MFMA(64, 8)
    BRS_LAUNCH_MFMA(128, 2)
    BRS_LAUNCH_MFMA(128, 4)
    BRS_LAUNCH_MFMA(128, 8)
#undef BRS_LAUNCH_MFMA
    return hipErrorInvalidValue;
  }
  if (g.fast) {
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

hipError_t launch_attn_merge(const AttnGeom& g, void* ws, float* out, float* lse, hipStream_t s) {
  const int64_t rows = (int64_t)g.batch * g.hq * g.n_q;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)rows), dim3(256), 0, s, (const int4*)((char*)ws + g.hdr_off),
                     (const float2*)((char*)ws + g.ml_off), (const float*)((char*)ws + g.o_off), out, lse, g.hq,
                     g.hkv, g.n_q, g.d, g.slot ? 0 : g.chunk_tokens, g.max_chunks, g.max_chunks);
  return hipGetLastError();
}


}  // namespace brs

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
//   - the workgroup builds its head's attended segments from the selection
//     row (sinks, the selected blocks in block order, window), clips them to
//     positions <= its last query (the causal limit), and flattens them into
//     a token stream with a position table in LDS;
//   - each 64-token stage of K and V is staged once in LDS for all 8 waves,
//     in three buffers fed by a ring of loads four stages ahead, so global
//     loads are in flight while earlier stages are multiplied;
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
constexpr int kAhead = 4;         // stages of K/V loads in flight per thread (register ring)
constexpr int kBufs = 3;          // stage buffers in LDS
constexpr int kTabTokens = 4096;  // token table ring (64 stages)
constexpr int kRefill = 32;       // stages refilled at a time (half the ring)
constexpr int kNoPos = 0x7fffffff;
constexpr int kOutOfRange = 0x7ffff000;  // buffer offset past any slice: loads return zeros
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource word 3 (32-bit data, no swizzle)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_p;
typedef __attribute__((ext_vector_type(4))) float f32x4_p;
typedef __attribute__((ext_vector_type(2))) float f32x2_p;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_p;
typedef __attribute__((ext_vector_type(4))) short i16x4_p;
typedef __attribute__((address_space(3))) i16x4_p lds_i16x4_p;

struct PrefillArgs {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;
  float* out;
  float* lse;  // per query row, ln of the softmax denominator (may be null)
  const int32_t* idx;  // selections, [batch][idx_heads][kk]
  int kk, idx_heads, B, nb, sink_end;
  int64_t head_stride;
  int row_stride, hq, hkv, G, n_q, N, d, nvec, nj;
  int slice_bytes;  // bytes of one (batch, kv head) slice of k / v (buffer range)
  int win_start;
  float qscale;
  int n_tiles, n_units, per_xcd;
};

__device__ __forceinline__ bf16x8_p as_bf16x8_p(const uint4& u) { return __builtin_bit_cast(bf16x8_p, u); }

int env_flag(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}


// DP: head dim rounded up to a multiple of 32 (the k chunk of the S^T MFMA).
// NJ: 16-column output tiles in use, ceil(d / 16) (compile-time, so the
// P V loop has no branches).
// ONES: V carries a column of ones in a spare padded column (head dims with
// d mod 16 in 1..8), so the P V products also yield the softmax row sums.
template <int DP, int NJ, bool ONES>
__global__ __launch_bounds__(512) void attn_prefill_kernel(PrefillArgs a) {
  constexpr int KC = DP / 32;
  static_assert(NJ >= 1 && NJ <= DP / 16, "output tiles");
  constexpr int KP = DP + 16;  // LDS row pitch in halves (keeps transposed reads conflict-free)
  constexpr int VPT = (kStage * (DP / 8) + 255) / 256;  // 16-byte vectors per thread and stage
  constexpr int BUF = kStage * KP;                      // halves per stage buffer
  // stage buffers: K in [0, 3 BUF), V in [3 BUF, 6 BUF)
  __shared__ __align__(16) uint16_t s_kv[2 * kBufs * BUF];
  __shared__ int2 s_tab[kTabTokens];  // (position, K/V row byte offset) of stream tokens, a ring
  __shared__ uint4 s_junk[256];
  __shared__ int4 s_items[kPrefItems];
  __shared__ int s_blk[kPrefItems];
  __shared__ int wave_tot[16];
  __shared__ int sh_tot[4];
  __shared__ float s_ml[4][16][2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int q0 = tile * kPrefQ;
  const int qlast = min(q0 + kPrefQ, a.n_q) - 1;
  const int pmax = a.N - a.n_q + qlast;

  // The segments of this head in position order, clipped to positions
  // <= pmax: the sinks [0, S'), the blocks its score head selected, in block
  // order, then the window [win_start, N).  A selected block contributes
  // [max(blk B, S'), min((blk + 1) B, win_start)); invalid entries, blocks
  // that lie inside the sinks or the window, and repeats are dropped.  The
  // selection row is requested before the query rows so that the two loads
  // overlap (the memory counter waits in issue order).
  int blk;
  {
    const int row = a.idx_heads == 1 ? b : b * a.hq + h;
    const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.idx + (int64_t)row * a.kk), (short)0, a.kk * 4, kBufferFlags);
    blk = (int)__builtin_amdgcn_raw_buffer_load_b32(irs, tid < a.kk ? tid * 4 : kOutOfRange, 0, 0);
  }

  // query rows of this wave as the B operand of S^T = K Q^T: lane (g4, n)
  // holds row q0 + 16 qg + n, columns 32 kk + 8 g4 .. + 7, as 32-bit pairs
  // (d is even).  Unconditional buffer loads: columns past d and rows past
  // n_q take an offset past the end of the rows and read zeros.
  const int qi = q0 + 16 * qg + n;
  const bool act = qi < a.n_q;
  uint4 qb[KC];
  {
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.q + (int64_t)bh * a.n_q * a.d), (short)0, a.n_q * a.d * 2, kBufferFlags);
    uint32_t w[KC][4];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e0 = 32 * kk + 8 * g4 + 2 * p;
        const int off = (act && e0 < a.d) ? (qi * a.d + e0) * 2 : kOutOfRange;
        w[kk][p] = __builtin_amdgcn_raw_buffer_load_b32(qrs, off, 0, 0);
      }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) qb[kk] = make_uint4(w[kk][0], w[kk][1], w[kk][2], w[kk][3]);
  }

  const int S = a.sink_end;
  if (tid < kPrefItems) {
    const bool valid = tid < a.kk && blk >= 0 && blk < a.nb &&
                       max(blk * a.B, S) < min((blk + 1) * a.B, a.win_start);
    s_blk[tid] = valid ? blk : -1;
  }
  __syncthreads();
  bool dup = false;  // an earlier entry holds the same block
  if (tid < a.kk && s_blk[tid] >= 0)
    for (int j = 0; j < tid; ++j) dup |= s_blk[j] == s_blk[tid];
  __syncthreads();
  if (dup) s_blk[tid] = -1;
  __syncthreads();
  const int mine = tid < a.kk ? s_blk[tid] : -1;
  int rank = 0;  // kept blocks below this one
  if (mine >= 0)
    for (int j = 0; j < a.kk; ++j) {
      const int o = s_blk[j];
      rank += o >= 0 && o < mine;
    }
  const int n_kept = __syncthreads_count(mine >= 0);
  const int hs = S > 0 ? 1 : 0;
  const int n_items = hs + n_kept + 1;
  if (mine >= 0) {
    const int lo_t = max(mine * a.B, S);
    const int hi_t = min(min((mine + 1) * a.B, a.win_start), pmax + 1);
    s_items[hs + rank] = make_int4(lo_t, max(hi_t - lo_t, 0), 0, 0);
  }
  if (tid == 0 && hs) s_items[0] = make_int4(0, min(S, pmax + 1), 0, 0);
  if (tid == 0) s_items[hs + n_kept] = make_int4(a.win_start, max(min(a.N, pmax + 1) - a.win_start, 0), 0, 0);
  __syncthreads();
  // stream offsets (segments past pmax have length 0; they come last)
  {
    const int len = tid < n_items ? s_items[tid].y : 0;
    const int inc = block_inclusive_scan(len, wave_tot);
    if (tid < n_items) s_items[tid].w = inc - len;
    if (tid == 511) sh_tot[0] = inc;
  }
  // pad columns of K and V (columns 8 nvec .. DP - 1, which the products
  // read): zero, except V's column of ones.  Rows and pads are whole
  // 16-byte units.
  {
    const int npad = DP / 8 - a.nvec;
    for (int e = tid; e < 2 * kBufs * kStage * npad; e += 512) {
      const int i = e / npad, c = e - i * npad;
      const bool ones = ONES && i >= kBufs * kStage && c == 0;
      *reinterpret_cast<uint4*>(s_kv + i * KP + 8 * (a.nvec + c)) = make_uint4(ones ? 0x3f80u : 0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  const int ns = n_items;
  const int n_tok = sh_tot[0];
  const int n_stages = (n_tok + kStage - 1) / kStage;

  // token table: stream offset tau -> (position, byte offset), kNoPos past the end
  const int row_bytes = a.row_stride * 2;
  // (count a multiple of 512: each thread fills a run of count / 512
  // consecutive entries, with one search for the run's first segment)
  auto fill = [&](int tau0, int count) {
    const int per = count / 512, t0 = tau0 + tid * per;
    int lo = 0, hi = ns - 1;  // last item with w <= t0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_items[mid].w <= t0) lo = mid; else hi = mid - 1;
    }
    int4 c = s_items[lo];
    for (int j = 0; j < per; ++j) {
      const int tau = t0 + j;
      int2 e = make_int2(kNoPos, kOutOfRange);
      if (tau < n_tok) {
        while (tau >= c.w + c.y) c = s_items[++lo];  // segments are contiguous in the stream
        const int pos = c.x + (tau - c.w);
        e = make_int2(pos, pos * row_bytes);
      }
      s_tab[tau & (kTabTokens - 1)] = e;
    }
  };
  fill(0, kTabTokens);

  // staging: waves 0-3 move K, waves 4-7 move V; thread t of the 256 moves
  // vectors e = t + 256 j of the stage.  Buffer loads with one 32-bit offset
  // per vector (rows past the end read zeros); kAhead stages of loads are in
  // flight in a ring of registers.
  const int kvec = kStage * a.nvec;
  const bool stage_v = wave >= 4;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((stage_v ? a.v : a.k) + (int64_t)bg * a.head_stride), (short)0, a.slice_bytes, kBufferFlags);
  const int t256 = tid & 255;
  // Per vector: its row's table entry within a stage (byte offset), its
  // column in bytes, and its LDS slot.  A lane without a vector gets column
  // kOutOfRange: row offset + kOutOfRange stays below 2^32 (a slice is under
  // kOutOfRange - 4096 bytes) and past the buffer's end, so it reads zeros.
  uint32_t stab[VPT], scol[VPT];
  int soff[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int e = t256 + 256 * j;
    const int r = e / a.nvec, c = e - r * a.nvec;
    stab[j] = (uint32_t)(r < kStage ? r : 0) * (uint32_t)sizeof(int2);
    scol[j] = e < kvec ? 16u * c : (uint32_t)kOutOfRange;
    soff[j] = e < kvec ? (stage_v ? kBufs * BUF : 0) + r * KP + 8 * c : -1;
  }
  uint4 stg[kAhead][VPT];
  auto stage_offsets = [&](int(&at)[VPT], int stage) {
    // a stage's 64 table entries never wrap around the ring
    const char* tab = reinterpret_cast<const char*>(s_tab) + ((stage * kStage) & (kTabTokens - 1)) * sizeof(int2);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const uint32_t off = (uint32_t)reinterpret_cast<const int2*>(tab + stab[j])->y;
      at[j] = (int)(off + scol[j]);
    }
  };
  auto stage_load = [&](uint4(&dst)[VPT], const int(&at)[VPT]) {
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      dst[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, at[j], 0, 0));
  };
  // lanes without a vector store into a junk slot: no branch around the stores
  auto stage_store = [&](const uint4(&src)[VPT], int stage) {
    const int base = (stage % kBufs) * BUF;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      uint4* dst = soff[j] >= 0 ? reinterpret_cast<uint4*>(s_kv + base + soff[j]) : &s_junk[t256];
      *dst = src[j];
    }
  };

  // Rows past the last query compute unused values (rows never mix in
  // either product).
  const int plim = a.N - a.n_q + qi;                // last visible position of this lane's row
  const int plim_min = a.N - a.n_q + q0 + 16 * qg;  // the wave's smallest one
  // a negative scale is taken as |scale| with the query negated (exact in
  // bf16), so the logits below are always scaled by a positive factor
  const float qs = fabsf(a.qscale);
  if (a.qscale < 0.f) {
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      qb[kk].x ^= 0x80008000u;
      qb[kk].y ^= 0x80008000u;
      qb[kk].z ^= 0x80008000u;
      qb[kk].w ^= 0x80008000u;
    }
  }

  f32x4_p o[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) o[jj] = f32x4_p{0.f, 0.f, 0.f, 0.f};
  float mref = kFarNegP, lpart = 0.f;
  const int r0 = 32 * kh;  // this wave's 32 rows of every stage

  // S^T for this wave's rows of stage s
  auto qk = [&](f32x4_p(&st)[2], int s) {
    const uint16_t* kbuf = s_kv + (s % kBufs) * BUF;
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      st[sidx] = f32x4_p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const uint4 ka = *reinterpret_cast<const uint4*>(kbuf + (r0 + 16 * sidx + n) * KP + 32 * kk + 8 * g4);
        st[sidx] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_p(ka), as_bf16x8_p(qb[kk]), st[sidx], 0, 0, 0);
      }
    }
  };

  // softmax of stage s from its S^T, then O += P V
  auto softmax_pv = [&](f32x4_p(&st)[2], int s) {  // st: masked in place
    const uint16_t* vbuf = s_kv + kBufs * BUF + (s % kBufs) * BUF;
    bf16x8_p vb[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      {
        const int col = 16 * jj + 4 * (n & 3);
        const i16x4_p v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(vbuf + (r0 + 4 * g4 + (n >> 2)) * KP + col));
        const i16x4_p v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_p*)(vbuf + (r0 + 16 + 4 * g4 + (n >> 2)) * KP + col));
        vb[jj] = __builtin_bit_cast(bf16x8_p, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    const int tbase = s * kStage + r0;
    // whole: the stream is in position order, so its last token bounds the half
    const bool whole = s_tab[(tbase + 31) & (kTabTokens - 1)].x <= plim_min;
    // logits of tokens past a row's causal limit become -inf, so their
    // weights come out as zero
    // (in place, so both branches leave the logits in the same registers)
    if (!whole) {
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = s_tab[(tbase + 16 * sidx + 4 * g4 + i) & (kTabTokens - 1)].x;
          st[sidx][i] = pos <= plim ? st[sidx][i] : -INFINITY;
        }
    }
    float x[8];
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * sidx + i] = st[sidx][i];
    // row maximum of the scaled logits (log2 units): the raw maximum times
    // the scale, so the scale itself goes into the exponent's fma
    float e = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) e = fmaxf(e, x[i]);
    const float tm = xmax16_32(e) * qs;
    if (__ballot(tm > mref + kLazyP)) {
      const float nm = fmaxf(mref, tm);
      const float al = exp2_fast(mref - nm);
      mref = nm;
      if (!ONES) lpart *= al;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(al, 4 * g4 + i);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) o[jj][i] *= ai;
      }
    }
    // weights 2^(scale s - ref) as bf16 high parts plus bf16 low parts
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2_p p2;
      p2.x = exp2_fast(fmaf(x[2 * i], qs, -mref));
      p2.y = exp2_fast(fmaf(x[2 * i + 1], qs, -mref));
      const bf16x2_p hi = __builtin_convertvector(p2, bf16x2_p);
      const f32x2_p back = __builtin_convertvector(hi, f32x2_p);
      ph[i] = __builtin_bit_cast(uint32_t, hi);
      pl[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p2 - back, bf16x2_p));
      if (!ONES) lpart += p2.x + p2.y;
    }
    const bf16x8_p pa_hi = __builtin_bit_cast(bf16x8_p, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8_p pa_lo = __builtin_bit_cast(bf16x8_p, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vb[jj], o[jj], 0, 0, 0);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb[jj], o[jj], 0, 0, 0);
  };

  // Pipeline over stages, three LDS buffers: in iteration s the wave
  // multiplies S^T of stage s+1 while it finishes the softmax and P V of
  // stage s; stage s+2 moves from registers to LDS and stage s+2+kAhead is
  // requested into the registers it frees (stages s+3 .. s+1+kAhead are in
  // flight).  Loads, stores and barriers run unconditionally (past the end
  // the loads read zeros) so the memory waits stay one ring slot deep.
  if (n_stages > 0) {
    __syncthreads();  // token table
    int at[VPT];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      stage_offsets(at, j);
      stage_load(stg[j], at);
    }
    stage_store(stg[0], 0);
    stage_offsets(at, kAhead);
    stage_load(stg[0], at);
    stage_store(stg[1], 1);
    stage_offsets(at, kAhead + 1);
    stage_load(stg[1], at);
    __syncthreads();
    // S^T tiles of even stages in st_a, odd ones in st_b (kAhead is even)
    static_assert(kAhead % 2 == 0, "stage parity");
    f32x4_p st_a[2], st_b[2];
    qk(st_a, 0);
    for (int s0 = 0; s0 < n_stages; s0 += kAhead) {
#pragma unroll
      for (int j = 0; j < kAhead; ++j) {
        const int s = s0 + j;
        f32x4_p(&st_cur)[2] = (j % 2 == 0) ? st_a : st_b;
        f32x4_p(&st_nxt)[2] = (j % 2 == 0) ? st_b : st_a;
        // refill the token table half a ring ahead (entries of finished stages)
        if (s % kRefill == 0 && s >= kRefill) fill((s + kRefill) * kStage, kRefill * kStage);
        stage_offsets(at, s + 2 + kAhead);
        if (s + 1 < n_stages) qk(st_nxt, s + 1);
        if (s < n_stages) softmax_pv(st_cur, s);
        stage_store(stg[(j + 2) % kAhead], s + 2);
        stage_load(stg[(j + 2) % kAhead], at);
        __syncthreads();
      }
    }
  }

  // row sums: from the ones column, or over the four lanes that share a row
  if (ONES) {
    // o[jj1][i] at lane (g4, n1) holds the sum of row 4 g4 + i; bring row n's to lane n
    const int c1 = 8 * a.nvec, jj1 = c1 >> 4, n1 = c1 & 15;
    float li = 0.f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      if (jj == jj1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = __shfl(o[jj][i], 16 * (n >> 2) + n1);
          li = (i == (n & 3)) ? v : li;
        }
      }
    lpart = li;
  } else {
    lpart = xsum16_32(lpart);
  }

  // merge the two token halves: waves 4-7 hand (max, sum, O) to waves 0-3 through LDS
  __syncthreads();
  float* s_o = reinterpret_cast<float*>(s_kv);  // [4][16][DP] floats
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
    if (a.lse && g4 == 0 && q0 + 16 * qg + n < a.n_q)
      a.lse[(int64_t)bh * a.n_q + q0 + 16 * qg + n] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
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
  return g.dtype == BRS_BF16 && g.n_q >= kPrefQ && g.d <= 128 && g.d % 2 == 0 && g.row_stride % 8 == 0 &&
         ((g.d + 7) / 8) * 8 <= g.row_stride && g.k + 2 <= kPrefItems &&
         g.head_stride * 2 < (int64_t)kOutOfRange - 4096 && (int64_t)g.n_q * g.d * 2 < (int64_t)kOutOfRange - 4096;
}

hipError_t launch_attn_prefill(const AttnGeom& g, const void* k, const void* v, const void* q, const int32_t* idx,
                               float* out, float* lse, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  PrefillArgs a;
  a.lse = lse;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.q = (const uint16_t*)q;
  a.out = out;
  a.idx = idx;
  a.kk = idx ? g.k : 0;
  a.idx_heads = g.idx_heads;
  a.B = g.B;
  a.nb = g.nb;
  a.sink_end = g.sink_end;
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
  a.slice_bytes = (int)(g.head_stride * 2);
  a.win_start = g.win_start;
  const dim3 grid((unsigned)(a.per_xcd * kXcds)), block(512);
  const bool ones = 8 * a.nvec < 16 * a.nj;  // a spare padded column exists
#define BRS_PREFILL_LAUNCH(DP, NJ, ONES)                                                      \
  if (a.nj == NJ && ones == ONES) {                                                          \
    if (ev0)                                                                                  \
      hipExtLaunchKernelGGL((attn_prefill_kernel<DP, NJ, ONES>), grid, block, 0, s, ev0, ev1, 0, a); \
    else                                                                                      \
      hipLaunchKernelGGL((attn_prefill_kernel<DP, NJ, ONES>), grid, block, 0, s, a);          \
    return hipGetLastError();                                                                 \
  }
  if (g.d <= 64) {
    BRS_PREFILL_LAUNCH(64, 1, true)
    BRS_PREFILL_LAUNCH(64, 1, false)
    BRS_PREFILL_LAUNCH(64, 2, true)
    BRS_PREFILL_LAUNCH(64, 2, false)
    BRS_PREFILL_LAUNCH(64, 3, true)
    BRS_PREFILL_LAUNCH(64, 3, false)
    BRS_PREFILL_LAUNCH(64, 4, true)
    BRS_PREFILL_LAUNCH(64, 4, false)
  } else {
    BRS_PREFILL_LAUNCH(128, 5, true)
    BRS_PREFILL_LAUNCH(128, 5, false)
    BRS_PREFILL_LAUNCH(128, 6, true)
    BRS_PREFILL_LAUNCH(128, 6, false)
    BRS_PREFILL_LAUNCH(128, 7, true)
    BRS_PREFILL_LAUNCH(128, 7, false)
    BRS_PREFILL_LAUNCH(128, 8, true)
    BRS_PREFILL_LAUNCH(128, 8, false)
  }
#undef BRS_PREFILL_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace brs

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
//     in two buffers each (K is stored two stages ahead of the softmax, V
//     one), fed by a ring of loads four stages ahead, so global loads are in
//     flight while earlier stages are multiplied;
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

#include "brs_internal.h"

namespace brs {
namespace {

constexpr int kPrefItems = 256;  // segments of one (batch, kv head) held in LDS
constexpr int kPrefQ = 64;       // queries per workgroup
constexpr float kLazyP = 8.0f;
constexpr float kFarNegP = -1e30f;
constexpr int kXcds = 8;
constexpr int kParts = 2;      // token parts: waves per query group
constexpr int kThreads = 256 * kParts;
constexpr int kStage = 32 * kParts;  // tokens per stage
constexpr int kAhead = 4;      // stages of K/V loads in flight per thread (register ring)
constexpr int kRefill = 32;    // token-table stages refilled at a time (half the ring)
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
  // K/V read through a page table (a device cache of blocks; k and v then
  // point to the page pool): page of block x of slice bg at pages[bg *
  // pages_stride + x]; null: the memory itself
  const int32_t* pages;
  int pages_stride;
};

__device__ __forceinline__ bf16x8_p as_bf16x8_p(const uint4& u) { return __builtin_bit_cast(bf16x8_p, u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}


// PAGED: K/V rows are read through the page table of a block cache.
// DP: head dim rounded up to a multiple of 32 (the k chunk of the S^T MFMA).
// NJ: 16-column output tiles in use, ceil(d / 16) (compile-time, so the
// P V loop has no branches).
// ONES: V carries a column of ones in a spare padded column (head dims with
// d mod 16 in 1..8), so the P V products also yield the softmax row sums.
template <bool PAGED, int DP, int NJ, bool ONES>
__global__ __launch_bounds__(kThreads) void attn_prefill_kernel(PrefillArgs a) {
  constexpr int NT = kThreads;
  constexpr int HT = NT / 2;  // threads that move K (the others move V)
  constexpr int STG = kStage;
  constexpr int KH = kParts;
  constexpr int AH = kAhead;
  constexpr int KC = DP / 32;
  static_assert(NJ >= 1 && NJ <= DP / 16, "output tiles");
  // LDS row pitch in halves, for K and V: V rows are read transposed, 8 rows
  // by 4 lanes of 8 bytes, and a pitch of an odd multiple of 8 dwords spreads
  // the 8 rows over all banks; the unit at column DP of a K row is never read
  // (lanes without a vector store there)
  constexpr int PK = DP + 16;
  constexpr int PV = DP + 16;
  constexpr int VOFF = 2 * STG * PK;  // V buffers after the two K buffers
  constexpr int VPT = (STG * (DP / 8) + HT - 1) / HT;  // 16-byte vectors per thread and stage
  constexpr int RF = kRefill;
  static_assert(RF >= AH + 3, "a refilled stage is first read after the barrier that follows the refill");
  constexpr int TABST = 2 * RF;     // stages in the token table ring
  constexpr int TAB = TABST * STG;  // token table ring entries
  constexpr int OC = 16 * NJ;                         // output columns in the merge
  // stage buffers: K in [0, VOFF), V in [VOFF, VOFF + 2 STG PV); after the
  // loop they hold the partial outputs of the merge
  __shared__ __align__(16) uint16_t s_kv[VOFF + 2 * STG * PV];
  static_assert(KH * 64 * OC * 4 <= (int)sizeof(s_kv), "merge area");
  __shared__ int2 s_tab[TAB];  // (position, K/V row byte offset) of stream tokens, a ring
  __shared__ int4 s_items[kPrefItems];
  __shared__ int s_blk[kPrefItems];   // valid selection entries (-1: none)
  __shared__ int s_keep[kPrefItems];  // the same without repeats
  __shared__ int sh_tot[2];           // stream tokens, items
  __shared__ float s_ml[KH][64][2];  // per part and row: (max, sum)
  __shared__ float s_f[KH][64];      // per part and row: merge factor over the sum

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
  // every wave also reads the whole row (contiguous layout), to find the
  // stream's first segment without waiting for the workgroup
  int erow[kPrefItems / 64];
  {
    // this head's list: its own, its kv head's, or its sequence's
    const int row = (int)sel_row(a.idx_heads, a.hkv, b, g, sel_lists(a.idx_heads, a.hkv) == a.G ? h - g * a.G : 0);
    const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.idx + (int64_t)row * a.kk), (short)0, a.kk * 4, kBufferFlags);
    blk = (int)__builtin_amdgcn_raw_buffer_load_b32(irs, tid < a.kk ? tid * 4 : kOutOfRange, 0, 0);
    if constexpr (!PAGED) {
#pragma unroll
      for (int j = 0; j < kPrefItems / 64; ++j) {
        const int e = lane + 64 * j;
        erow[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(irs, e < a.kk ? e * 4 : kOutOfRange, 0, 0);
      }
    }
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
  const int s_len = min(S, pmax + 1);  // the sinks, clipped to the causal limit
  const int row_bytes = a.row_stride * 2;
  auto seg_lo = [&](int x) { return max(x * a.B, S); };
  auto seg_len = [&](int x) { return max(min(min((x + 1) * a.B, a.win_start), pmax + 1) - seg_lo(x), 0); };
  // staging: threads [0, HT) move K, [HT, NT) move V; thread t of its half
  // moves vectors e = t + HT j of the stage.  Buffer loads with one 32-bit
  // offset per vector (rows past the end read zeros); AH stages of loads
  // are in flight in a ring of registers.  K is stored two stages ahead of
  // the one whose softmax runs, V one stage ahead, so two buffers of each
  // suffice.
  const int kvec = STG * a.nvec;
  const bool stage_v = wave >= 2 * KH;  // wave-uniform, so the buffer resource stays scalar
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((stage_v ? a.v : a.k) + (int64_t)bg * a.head_stride), (short)0, a.slice_bytes, kBufferFlags);
  const int th = stage_v ? tid - HT : tid;
  // Per vector: its row's table entry within a stage (byte offset), its
  // column in bytes, and its LDS slot in buffer 0 (-1: none).  A lane without
  // a vector gets column kOutOfRange: row offset + kOutOfRange stays below
  // 2^32 (a slice is under kOutOfRange - 4096 bytes) and past the buffer's
  // end, so it reads zeros, which it stores into the unread unit of a K row.
  uint32_t stab[VPT], scol[VPT];
  int soff[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int e = th + HT * j;
    const int r = e / a.nvec, c = e - r * a.nvec;
    stab[j] = (uint32_t)(r < STG ? r : 0) * (uint32_t)sizeof(int2);
    scol[j] = e < kvec ? 16u * c : (uint32_t)kOutOfRange;
    soff[j] = e < kvec ? (stage_v ? VOFF + r * PV : r * PK) + 8 * c : -1;
  }
  const int junk = (th % STG) * PK + DP;
  const int bstride = stage_v ? STG * PV : STG * PK;
  uint4 stg[AH][VPT];
  auto stage_offsets = [&](int(&at)[VPT], int stage) {
    // a stage's entries never wrap around the ring
    const char* tab = reinterpret_cast<const char*>(s_tab) + (stage % TABST) * STG * (int)sizeof(int2);
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
  auto stage_store = [&](const uint4(&src)[VPT], int stage) {
    const int base = (stage & 1) * bstride;
#pragma unroll
    for (int j = 0; j < VPT; ++j) *reinterpret_cast<uint4*>(s_kv + (soff[j] >= 0 ? base + soff[j] : junk)) = src[j];
  };

  // The stream's first segment (the sinks, else the lowest valid selected
  // block, else the window), from the selection row alone.  When it covers
  // the first AH stages (contiguous layout), their K/V loads are issued now,
  // so that they are in flight while the segments and the token table are
  // built; the prologue below then skips them.
  bool early = false;
  if constexpr (!PAGED) {
    int mn = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kPrefItems / 64; ++j) {
      const int x = erow[j];
      const bool v = lane + 64 * j < a.kk && x >= 0 && x < a.nb && max(x * a.B, S) < min((x + 1) * a.B, a.win_start);
      mn = v ? min(mn, x) : mn;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mn = min(mn, __shfl_xor(mn, o));
    int lo0, len0;
    if (s_len > 0) {
      lo0 = 0;
      len0 = s_len;
    } else if (mn != 0x7fffffff) {
      lo0 = seg_lo(mn);
      len0 = seg_len(mn);
    } else {
      lo0 = a.win_start;
      len0 = max(min(a.N, pmax + 1) - a.win_start, 0);
    }
    early = __builtin_amdgcn_readfirstlane(len0 >= AH * STG ? 1 : 0) != 0;
    if (early) {
      // stage t, vector j: token lo0 + STG t + (its row in the stage)
      auto direct = [&](int(&at)[VPT], int t) {
#pragma unroll
        for (int j = 0; j < VPT; ++j)
          at[j] = (int)((uint32_t)(lo0 + STG * t + (int)(stab[j] / (uint32_t)sizeof(int2))) * (uint32_t)row_bytes +
                        scol[j]);
      };
      // ring slot sl holds stage sl (K) or stage sl - 1 mod AH (V): the role
      // enters the address only, so no value is selected after its load
      int at0[VPT];
#pragma unroll
      for (int sl = 0; sl < AH; ++sl) {
        direct(at0, stage_v ? (sl + AH - 1) % AH : sl);
        stage_load(stg[sl], at0);
      }
    }
  }

  // Three barriers: the entries, the kept entries, the items.  Every kept
  // block finds its rank in block order, its stream offset and (thread 0)
  // the totals by one pass over the kept entries, with no block-wide scan.
  if (tid < kPrefItems) {
    const bool valid = tid < a.kk && blk >= 0 && blk < a.nb &&
                       max(blk * a.B, S) < min((blk + 1) * a.B, a.win_start);
    s_blk[tid] = valid ? blk : -1;
  }
  // pad columns that the products read (K: 8 nvec .. DP - 1, V: 8 nvec ..
  // 16 NJ - 1): zero, except V's column of ones.  Whole 16-byte units.
  {
    const int kpad = DP / 8 - a.nvec, vpad = 2 * NJ - a.nvec;
    for (int e = tid; e < 2 * STG * kpad; e += NT) {
      const int i = e / kpad, c = e - i * kpad;
      *reinterpret_cast<uint4*>(s_kv + i * PK + 8 * (a.nvec + c)) = make_uint4(0u, 0u, 0u, 0u);
    }
    for (int e = tid; e < 2 * STG * vpad; e += NT) {
      const int i = e / vpad, c = e - i * vpad;
      const bool ones = ONES && c == 0;
      *reinterpret_cast<uint4*>(s_kv + VOFF + i * PV + 8 * (a.nvec + c)) =
          make_uint4(ones ? 0x3f80u : 0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  // an entry is kept unless an earlier entry holds the same block
  if (tid < kPrefItems) {
    const int x = tid < a.kk ? s_blk[tid] : -1;
    bool dup = false;
    if (x >= 0)
      for (int j = 0; j < tid; ++j) dup |= s_blk[j] == x;
    s_keep[tid] = dup ? -1 : x;
  }
  __syncthreads();
  {
    const int mine = tid < a.kk ? s_keep[tid] : -1;
    if (mine >= 0 || tid == 0) {
      int rank = 0, before = 0, n_kept = 0, kept_tok = 0;  // kept blocks below mine and their tokens; totals
      for (int j = 0; j < a.kk; ++j) {
        const int o = s_keep[j];
        if (o >= 0) {
          const int len = seg_len(o);
          ++n_kept;
          kept_tok += len;
          if (o < mine) {
            ++rank;
            before += len;
          }
        }
      }
      const int hs = S > 0 ? 1 : 0;
      // segments past pmax have length 0; they come last among the blocks
      if (mine >= 0) s_items[hs + rank] = make_int4(seg_lo(mine), seg_len(mine), 0, s_len + before);
      if (tid == 0) {
        if (hs) s_items[0] = make_int4(0, s_len, 0, 0);
        const int win_len = max(min(a.N, pmax + 1) - a.win_start, 0);
        s_items[hs + n_kept] = make_int4(a.win_start, win_len, 0, s_len + kept_tok);
        sh_tot[0] = s_len + kept_tok + win_len;
        sh_tot[1] = hs + n_kept + 1;
      }
    }
  }
  __syncthreads();
  const int ns = sh_tot[1];  // items
  const int n_tok = sh_tot[0];
  const int n_stages = (n_tok + STG - 1) / STG;

  // token table: stream offset tau -> (position, byte offset of its K/V
  // row: position order in the memory, or through the page table), kNoPos
  // past the end; entry tau sits at tau mod TAB
  const int32_t* ptab = PAGED ? a.pages + (int64_t)bg * a.pages_stride : nullptr;
  // each thread fills a run of consecutive entries, with one search for the
  // run's first segment
  auto fill = [&](int tau0, int count) {
    const int per = (count + NT - 1) / NT;
    const int first = tid * per;
    if (first < count) {
      const int t0 = tau0 + first;
      int lo = 0, hi = ns - 1;  // last item with w <= t0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_items[mid].w <= t0) lo = mid; else hi = mid - 1;
      }
      int4 c = s_items[lo];
      const int cnt = min(per, count - first);
      for (int j = 0; j < cnt; ++j) {
        const int tau = t0 + j;
        int2 e = make_int2(kNoPos, kOutOfRange);
        if (tau < n_tok) {
          while (tau >= c.w + c.y) c = s_items[++lo];  // segments are contiguous in the stream
          const int pos = c.x + (tau - c.w);
          int row = pos;
          if (PAGED) {
            const int x = pos / a.B;
            row = ptab[x] * a.B + (pos - x * a.B);
          }
          e = make_int2(pos, row * row_bytes);
        }
        s_tab[tau % TAB] = e;
      }
    }
  };
  fill(0, RF * STG);  // the rest after the first loads are issued

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
    const uint16_t* kbuf = s_kv + (s & 1) * (STG * PK);
    st[0] = f32x4_p{0.f, 0.f, 0.f, 0.f};
    st[1] = f32x4_p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const uint4 qv = qb[kk];
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx) {
        const uint4 ka = *reinterpret_cast<const uint4*>(kbuf + (r0 + 16 * sidx + n) * PK + 32 * kk + 8 * g4);
        st[sidx] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_p(ka), as_bf16x8_p(qv), st[sidx], 0, 0, 0);
      }
    }
  };

  // softmax of stage s from its S^T, then O += P V
  auto softmax_pv = [&](f32x4_p(&st)[2], int s) {  // st: masked in place
    const uint16_t* vbuf = s_kv + VOFF + (s & 1) * (STG * PV);
    // V of tile jj as the B operand of P V: lane (g4, n) holds column
    // 16 jj + n of this wave's rows 4 g4 .. + 3 and 16 + 4 g4 .. + 3 (the
    // token order of the S^T accumulator)
    auto vtile = [&](int jj) {
      const int col = 16 * jj + 4 * (n & 3);
      const i16x4_p v0 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(vbuf + (r0 + 4 * g4 + (n >> 2)) * PV + col));
      const i16x4_p v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_p*)(vbuf + (r0 + 16 + 4 * g4 + (n >> 2)) * PV + col));
      return __builtin_bit_cast(bf16x8_p, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // all V tiles are requested before the softmax, whose VALU work hides
    // their latency
    bf16x8_p vb[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) vb[jj] = vtile(jj);
    const int2* tabs = s_tab + (s % TABST) * STG + r0;
    // whole: the stream is in position order, so its last token bounds the part
    const bool whole = tabs[31].x <= plim_min;
    // logits of tokens past a row's causal limit become -inf, so their
    // weights come out as zero
    // (in place, so both branches leave the logits in the same registers)
    if (!whole) {
#pragma unroll
      for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = tabs[16 * sidx + 4 * g4 + i].x;
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
    for (int jj = 0; jj < NJ; ++jj) {
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vb[jj], o[jj], 0, 0, 0);
      o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb[jj], o[jj], 0, 0, 0);
    }
  };

  // Pipeline over stages, two LDS buffers for K and two for V: in iteration
  // s the wave multiplies S^T of stage s+1 while it finishes the softmax and
  // P V of stage s; K of stage s+2 and V of stage s+1 move from registers to
  // LDS, and the loads of K s+2+AH and V s+1+AH go into the registers they
  // free.
  // Loads, stores and barriers run unconditionally (past the end the loads
  // read zeros) so the memory waits stay one ring slot deep.
  if (n_stages > 0) {
    __syncthreads();  // token table, pads
    int at[VPT];
    // Ring slot of stage t: (t + 2 - lag) mod AH, the same slot for the K and
    // the V stage that an iteration stores (no branch between the movers in
    // the loop).  Stages 0 .. AH-1 are requested together; K stages 0 and 1
    // (V stage 0) then go to LDS, each slot refilled with the stage AH later.
    static_assert(AH >= 2, "K stages 0 and 1 take two ring slots");
    const int lag = stage_v ? 1 : 2;
    if (stage_v) {
      if (!early) {
#pragma unroll
        for (int t = 0; t < AH; ++t) {
          stage_offsets(at, t);
          stage_load(stg[(t + 1) % AH], at);
        }
      }
      stage_store(stg[1 % AH], 0);
      stage_offsets(at, AH);
      stage_load(stg[1 % AH], at);
    } else {
      if (!early) {
#pragma unroll
        for (int t = 0; t < AH; ++t) {
          stage_offsets(at, t);
          stage_load(stg[t], at);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        stage_store(stg[t], t);
        stage_offsets(at, t + AH);
        stage_load(stg[t], at);
      }
    }
    // the table's second half, behind the loads in flight
    fill(RF * STG, RF * STG);
    __syncthreads();
    // S^T tiles of even stages in st_a, odd ones in st_b
    f32x4_p st_a[2], st_b[2];
    qk(st_a, 0);
    __syncthreads();  // K buffer 0 takes stage 2 in the first iteration
    // unrolled over U stages: the S^T pair and the ring slots repeat with it
    constexpr int U = AH > 2 ? AH : 2;
    for (int s0 = 0; s0 < n_stages; s0 += U) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int s = s0 + j;
        f32x4_p(&st_cur)[2] = (j % 2 == 0) ? st_a : st_b;
        f32x4_p(&st_nxt)[2] = (j % 2 == 0) ? st_b : st_a;
        // refill the table half a ring ahead (entries of finished stages)
        if (s % RF == 0 && s >= RF) fill((s + RF) * STG, RF * STG);
        if (s + 1 < n_stages) qk(st_nxt, s + 1);
        if (s < n_stages) softmax_pv(st_cur, s);
        // (s0 is a multiple of AH)
        stage_offsets(at, s + lag + AH);
        stage_store(stg[(j + 2) % AH], s + lag);
        stage_load(stg[(j + 2) % AH], at);
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

  // merge the KH token parts: every wave hands (max, sum) of its rows and its
  // O tile to LDS; one thread per row finds the row's factors; then all
  // threads combine the parts two columns at a time and write the output
  // rows in order (consecutive threads, consecutive columns)
  __syncthreads();
  float* s_o = reinterpret_cast<float*>(s_kv);  // [KH][64][OC] floats
  if (lane < 16) {
    s_ml[kh][16 * qg + lane][0] = mref;
    s_ml[kh][16 * qg + lane][1] = lpart;
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[(kh * 64 + 16 * qg + 4 * g4 + i) * OC + 16 * jj + n] = o[jj][i];
  __syncthreads();
  const int rows = min(kPrefQ, a.n_q - q0);
  if (tid < rows) {
    float M = s_ml[0][tid][0];
#pragma unroll
    for (int p = 1; p < KH; ++p) M = fmaxf(M, s_ml[p][tid][0]);
    float f[KH], L = 0.f;
#pragma unroll
    for (int p = 0; p < KH; ++p) {
      f[p] = exp2_fast(s_ml[p][tid][0] - M);
      L += s_ml[p][tid][1] * f[p];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    if (a.lse) a.lse[(int64_t)bh * a.n_q + q0 + tid] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
#pragma unroll
    for (int p = 0; p < KH; ++p) s_f[p][tid] = f[p] * inv;
  }
  __syncthreads();
  // element e = (row r, column pair c2) of the rows x d/2 float2 units (d is even)
  const int h2 = a.d >> 1;
  const int dr = NT / h2, dc = NT - dr * h2;
  int r = tid / h2, c2 = tid - r * h2;
  float* obase = a.out + ((int64_t)bh * a.n_q + q0) * a.d;
  for (int e = tid; e < rows * h2; e += NT) {
    float2 acc = make_float2(0.f, 0.f);
#pragma unroll
    for (int p = 0; p < KH; ++p) {
      const float f = s_f[p][r];
      const float2 v = *reinterpret_cast<const float2*>(s_o + (p * 64 + r) * OC + 2 * c2);
      acc.x += v.x * f;
      acc.y += v.y * f;
    }
    *reinterpret_cast<float2*>(obase + (int64_t)r * a.d + 2 * c2) = acc;
    c2 += dc;
    r += dr;
    if (c2 >= h2) {
      c2 -= h2;
      ++r;
    }
  }
}

}  // namespace

bool prefill_supported(const AttnGeom& g) {
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
  a.pages = g.pages;
  a.pages_stride = g.pages_stride;
  const dim3 grid((unsigned)(a.per_xcd * kXcds)), block(kThreads);
  const bool ones = 8 * a.nvec < 16 * a.nj;  // a spare padded column exists
  const bool paged = a.pages != nullptr;
#define BRS_PREFILL_LAUNCH(PAGED, DP, NJ, ONES)                                                 \
  if (paged == PAGED && a.nj == NJ && ones == ONES) {                                         \
    if (ev0)                                                                                  \
      hipExtLaunchKernelGGL((attn_prefill_kernel<PAGED, DP, NJ, ONES>), grid, block, 0, s, ev0, ev1, 0, a); \
    else                                                                                      \
      hipLaunchKernelGGL((attn_prefill_kernel<PAGED, DP, NJ, ONES>), grid, block, 0, s, a);   \
    return hipGetLastError();                                                                 \
  }
#define BRS_PREFILL_ALL(P)                                                                    \
  if (g.d <= 64) {                                                                            \
    BRS_PREFILL_LAUNCH(P, 64, 1, true) BRS_PREFILL_LAUNCH(P, 64, 1, false)                    \
    BRS_PREFILL_LAUNCH(P, 64, 2, true) BRS_PREFILL_LAUNCH(P, 64, 2, false)                    \
    BRS_PREFILL_LAUNCH(P, 64, 3, true) BRS_PREFILL_LAUNCH(P, 64, 3, false)                    \
    BRS_PREFILL_LAUNCH(P, 64, 4, true) BRS_PREFILL_LAUNCH(P, 64, 4, false)                    \
  } else {                                                                                    \
    BRS_PREFILL_LAUNCH(P, 128, 5, true) BRS_PREFILL_LAUNCH(P, 128, 5, false)                  \
    BRS_PREFILL_LAUNCH(P, 128, 6, true) BRS_PREFILL_LAUNCH(P, 128, 6, false)                  \
    BRS_PREFILL_LAUNCH(P, 128, 7, true) BRS_PREFILL_LAUNCH(P, 128, 7, false)                  \
    BRS_PREFILL_LAUNCH(P, 128, 8, true) BRS_PREFILL_LAUNCH(P, 128, 8, false)                  \
  }
  BRS_PREFILL_ALL(true)
  BRS_PREFILL_ALL(false)
#undef BRS_PREFILL_ALL
#undef BRS_PREFILL_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace brs

// Internal declarations shared by the HIP translation units of libbrs.
// Nothing here crosses the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "brs.h"

namespace brs {

// ---------------------------------------------------------------------------
// element helpers

__host__ __device__ inline int elem_bytes(int dtype) { return dtype == BRS_F32 ? 4 : 2; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round a float64 to the nearest bfloat16, ties to even, in one step (no
// intermediate float32 rounding).  Finite, normal-range inputs; values in
// the subnormal range use the fixed subnormal spacing.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  if (x == 0.0 || !isfinite(x)) {
    return (uint16_t)(__float_as_uint((float)x) >> 16);
  }
  int e;
  frexp(x, &e);                 // x = m 2^e, 0.5 <= |m| < 1
  int binade = e - 1;
  if (binade < -126) binade = -126;
  const int sp = binade - 7;    // spacing exponent for 8 significant bits
  double r = ldexp(rint(ldexp(x, -sp)), sp);   // exact, representable in bf16
  float f = (float)r;           // exact conversion (or overflow to inf)
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// Inclusive prefix sum of one int per thread over the whole workgroup
// (blockDim.x a multiple of 64, at most 1024).  Contains barriers: every
// thread of the workgroup must call it.
__device__ inline int block_inclusive_scan(int v, int* wave_tot /* [16] shared */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += wave_tot[w];
  __syncthreads();
  return v + add;
}

// Reductions over the four lanes l, l^16, l^32, l^48 (same column of the
// accumulator) with the gfx950 lane-swap moves (no LDS round trip).
__device__ __forceinline__ float xmax16_32(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xmin16_32(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xsum16_32(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------------------
// selection lists of a kv slice
//
// idx holds batch * idx_heads rows: idx_heads = 1 (one list per sequence,
// shared by every head), n_kv_heads (one per kv head, shared by its query
// heads) or n_q_heads (one per query head).  A kv slice (b, g) reads
// sel_lists rows; list j is row sel_row(.., j).  With one list per query
// head, list j belongs to query head j of the group; otherwise every head of
// the slice attends it.

__host__ __device__ inline int sel_lists(int idx_heads, int hkv) { return idx_heads >= hkv ? idx_heads / hkv : 1; }
__host__ __device__ inline int64_t sel_row(int idx_heads, int hkv, int b, int g, int j) {
  return (int64_t)b * idx_heads + (idx_heads >= hkv ? (int64_t)g * (idx_heads / hkv) : 0) + j;
}

// ---------------------------------------------------------------------------
// attention plan
//
// For every (batch, kv head) the plan kernel writes the attended token set as
// a list of disjoint segments (first row, length, head mask, offset in the
// flattened list): the sinks, the window, then every selected block clipped
// against both, in block order.  Each token appears once per (batch, kv
// head) however many query heads selected its block, so the K/V bytes of a
// block shared by several heads are read once.  The flattened list is cut
// into equal chunks of chunk_tokens; chunk_first[c] names the segment that
// holds the first token of chunk c.

constexpr int kMarkBlocks = 8192;  // blocks marked per pass of the plan kernel
constexpr int kRowsMax = 8;        // query rows one split workgroup handles

struct AttnGeom {
  int batch, hq, hkv, group, n_q, d, row_stride, dtype;
  int N, B, nb;
  int sink_end;           // S' = min(n_sink, N)
  int win_start;          // max(N - window, S')
  int idx_heads, k;
  int64_t head_stride;    // elements between consecutive (batch, kv head) slices of k / v
  float qscale;           // softmax scale * log2(e)
  // decomposition
  bool fast;              // head_dim and row layout served by the vector kernel
  bool mfma;              // bfloat16 served by the matrix-core kernel
  bool prefill;           // chunk of queries served by the matrix-core prefill kernel
  bool local_plan;        // split workgroups build their segments from idx (no plan kernel)
  bool slot;              // split workgroups read the selections directly (slot layout, no plan)
  int slot_ps, slot_bs;   // slot layout: padded sinks, slot stride (tokens)
  int slot_regs;          // slot layout: selection entries per lane (8, or 20 past 512 entries)
  int len_a, len_b;       // slot layout: sink/window tokens, slot tokens (padded)
  int64_t max_items;      // segments per (batch, kv head)
  int64_t max_tokens;     // bound on attended tokens per (batch, kv head)
  int nw;                 // waves per split workgroup
  int wave_tokens;        // tokens per wave
  int chunk_tokens;       // nw * wave_tokens
  int max_chunks;         // split workgroups per (batch, kv head, row group)
  int row_groups;         // ceil(group * n_q / kRowsMax)
  int rows_per_group;
  // a block cache: k / v are the page pool, block x of slice bg at page
  // pages[bg * pages_stride + x] (nullptr: the memory itself)
  const int32_t* pages;
  int pages_stride;
  // workspace offsets (bytes)
  size_t hdr_off, items_off, first_off, chunks_off, ml_off, o_off, total;
};

// Fills the decomposition and workspace layout; returns false if unsupported.
bool attn_geometry(AttnGeom& g);

hipError_t launch_attn_plan(const AttnGeom& g, const int32_t* idx, void* ws, float* out, hipStream_t s);

hipError_t launch_attn_split(const AttnGeom& g, const void* k, const void* v, const void* q, const int32_t* idx,
                             void* ws, float* out, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// lse (may be null): per query row, the natural log of the softmax denominator
hipError_t launch_attn_merge(const AttnGeom& g, void* ws, float* out, float* lse, hipStream_t s);
// Whole decode step after scoring in one attention launch, the selection
// made inside it (slot layout): same partials as launch_attn_split given
// that selection.
bool step_supported(const AttnGeom& g, int64_t lo, int64_t hi, int k);
hipError_t launch_attn_step(const AttnGeom& g, const void* k, const void* v, const void* q, const float* scores,
                            int64_t stride, int64_t lo, int64_t hi, int32_t* idx, float* vals, void* ws, float* out,
                            hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// Chunked prefill on the matrix cores; each workgroup builds its head's
// segments from idx itself (no plan kernel).
hipError_t launch_attn_prefill(const AttnGeom& g, const void* k, const void* v, const void* q, const int32_t* idx,
                               float* out, float* lse, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
bool prefill_supported(const AttnGeom& g);

// ---------------------------------------------------------------------------
// memory, scores, selection

hipError_t launch_kv_append(const brs_memory& m, const void* k_new, const void* v_new, int64_t n_new,
                            hipStream_t s);
hipError_t launch_reps_from_mass(const brs_memory& m, const float* mass, int64_t b0, int64_t b1, hipStream_t s);
hipError_t launch_window_mass(const brs_memory& m, const void* q, int hq, int n_q, const float* lse, int64_t w0,
                              float scale, float* mass, hipStream_t s, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr);
hipError_t launch_count_hits(const brs_memory& m, const int32_t* idx, int idx_heads, int k, int32_t* hits,
                             hipStream_t s);
int prune_max_middle();
int prune_max_blocks();
hipError_t launch_prune(const brs_memory& src, const brs_memory& dst, const int32_t* hits, int32_t* dst_hits,
                        int32_t* plan, int nb, int n10, int n_evict, int kept, int tail, hipStream_t s);
hipError_t launch_rep_build(const brs_memory& m, int64_t b0, int64_t b1, const void* reps_new,
                            hipStream_t s);
// the next score launch on this thread records e when its kernel completes
void set_score_stop_event(hipEvent_t e);
// grouped: one score per kv head, the maximum over its query heads
hipError_t launch_score_dot(const brs_memory& m, const void* q, int hq, int64_t lo, int64_t hi,
                            float* scores, bool grouped, hipStream_t s);
hipError_t launch_score_cosine(const brs_memory& m, const void* rq, int64_t lo, int64_t hi,
                               float* scores, hipStream_t s);
// block cache of an offloaded memory
int cache_max_pages();
int64_t cache_max_blocks();
hipError_t launch_cache_reset(const brs_memory& m, const brs_page_cache& c, hipStream_t s);
hipError_t launch_cache_fetch(const brs_memory& m, const brs_page_cache& c, const int32_t* idx, int idx_heads,
                              int k, int64_t sink_end, int64_t win_start, int step, int32_t* fetched,
                              hipStream_t s);
hipError_t launch_select_topk(const float* scores, int batch, int heads, int64_t stride, int64_t lo,
                              int64_t hi, int k, int32_t* idx, float* vals, hipStream_t s);

}  // namespace brs

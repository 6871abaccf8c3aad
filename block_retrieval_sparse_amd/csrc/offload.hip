// Offload of the key/value memory to host memory with a device cache of
// blocks (InfLLM "method": every memory unit is kept in CPU memory and the
// GPU keeps a cache of the units used most, loading the missing ones a step
// needs; RetrievalAttention "proposed method": the KV cache split between GPU
// and CPU memory).
//
// K and V of the memory live in pinned host memory that the device reads
// and writes directly.  A pool of pages in device memory, one block of rows
// each, caches blocks per (batch, kv head); page_of_block maps a block to its
// page.  Before an attention call, brs_cache_fetch makes every block that
// call reads resident: one workgroup per (batch, kv head) marks the blocks
// of the sinks, the window and the selection, keeps the pages already
// holding them (copying the rows a growing tail block gained since), and
// fills the others into pages that are free or were needed least recently
// (lowest last-use step, then lowest page), reading the rows from host
// memory.  The attention then reads K/V through the page table.
#include <hip/hip_runtime.h>

#include "brs_internal.h"

namespace brs {
namespace {

constexpr int kThreads = 256;
constexpr int kNeedWords = 8192;  // blocks per (batch, kv head): 262144
constexpr int kMaxPages = 2048;   // pages per (batch, kv head)
constexpr int kBatch = 8;         // 16-byte units of K and of V a thread reads before it writes

struct FetchArgs {
  const char* host_k;
  const char* host_v;
  char* pool_k;
  char* pool_v;
  int32_t* page_of_block;  // [bg][cap_blocks + 1]
  int32_t* page_block;     // [bg][n_pages]
  int32_t* page_rows;      // [bg][n_pages]
  int32_t* page_used;      // [bg][n_pages]
  int32_t* fetched;        // [bg] or null
  const int32_t* idx;
  int idx_heads, kk, hkv;
  int n_pages, B, N, nb, nbt, sink_end, win_start, cap_blocks1, step;
  int64_t slice_bytes_mem, slice_bytes_pool;
  int row_bytes;
};

__global__ __launch_bounds__(kThreads) void cache_reset_kernel(int32_t* page_of_block, int32_t* page_block,
                                                               int32_t* page_rows, int32_t* page_used,
                                                               int64_t n_tab, int64_t n_pg) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n_tab) page_of_block[i] = -1;
  if (i < n_pg) {
    page_block[i] = -1;
    page_rows[i] = 0;
    page_used[i] = -1;
  }
}

__device__ __forceinline__ bool bit_of(const uint32_t* w, int i) { return (w[i >> 5] >> (i & 31)) & 1u; }

__global__ __launch_bounds__(kThreads) void cache_fetch_kernel(FetchArgs a) {
  __shared__ uint32_t need[kNeedWords];
  __shared__ uint64_t keys[kMaxPages];  // victim candidates: (last use + 1, page), sorted
  __shared__ int4 jobs[kMaxPages];      // (block, page, first row, end row) to copy
  __shared__ int wave_tot[16];
  __shared__ int s_n[4];
  const int tid = threadIdx.x;
  const int bg = blockIdx.x;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  int32_t* pob = a.page_of_block + (int64_t)bg * a.cap_blocks1;
  int32_t* pblk = a.page_block + (int64_t)bg * a.n_pages;
  int32_t* prow = a.page_rows + (int64_t)bg * a.n_pages;
  int32_t* pused = a.page_used + (int64_t)bg * a.n_pages;
  const int words = (a.nbt + 31) >> 5;
  const int B = a.B, S = a.sink_end, ws = a.win_start;

  // the blocks this step reads: those holding sinks or window tokens, and the
  // selected blocks that hold tokens outside both (as the attention clips)
  for (int w = tid; w < words; w += kThreads) need[w] = 0u;
  if (tid == 0) {
    s_n[0] = 0;  // candidates
    s_n[1] = 0;  // jobs
  }
  __syncthreads();
  const int sink_blocks = (S + B - 1) / B;
  const int win_block0 = ws < a.N ? ws / B : a.nbt;
  for (int x = tid; x < a.nbt; x += kThreads)
    if (x < sink_blocks || x >= win_block0) atomicOr(&need[x >> 5], 1u << (x & 31));
  const int lists = sel_lists(a.idx_heads, a.hkv);
  const int E = lists * a.kk;
  for (int e = tid; e < E; e += kThreads) {
    const int j = e / a.kk;
    const int x = a.idx[sel_row(a.idx_heads, a.hkv, b, g, j) * a.kk + (e - j * a.kk)];
    if (x >= 0 && x < a.nb && max(x * B, S) < min(x * B + B, ws)) atomicOr(&need[x >> 5], 1u << (x & 31));
  }
  __syncthreads();

  // pages holding a needed block stay (the rows the block gained since it
  // was copied are copied now); the others are victim candidates
  for (int p = tid; p < a.n_pages; p += kThreads) {
    const int x = pblk[p];
    if (x >= 0 && x < a.nbt && bit_of(need, x)) {
      const int rows = min(B, a.N - x * B);
      if (prow[p] < rows) {
        const int j = atomicAdd(&s_n[1], 1);
        jobs[j] = make_int4(x, p, prow[p], rows);
        prow[p] = rows;
      }
      pused[p] = a.step;
    } else {
      const int c = atomicAdd(&s_n[0], 1);
      keys[c] = ((uint64_t)(uint32_t)(pused[p] + 1) << 32) | (uint32_t)p;
    }
  }
  __syncthreads();
  const int n_cand = s_n[0];
  // candidates in (last use, page) order: free pages (last use -1) first
  int np2 = 1;
  while (np2 < n_cand) np2 <<= 1;
  for (int i = n_cand + tid; i < np2; i += kThreads) keys[i] = ~0ull;
  __syncthreads();
  for (int size = 2; size <= np2; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < np2; i += kThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint64_t x = keys[i], y = keys[j];
          if ((x > y) == up) {
            keys[i] = y;
            keys[j] = x;
          }
        }
      }
      __syncthreads();
    }

  // needed blocks without a page, in block order, take the candidates in order
  int base = 0;
  for (int w0 = 0; w0 < words; w0 += kThreads) {
    const int w = w0 + tid;
    uint32_t miss = 0u;
    if (w < words) {
      uint32_t u = need[w];
      while (u) {
        const int bit = __builtin_ctz(u);
        u &= u - 1u;
        const int x = w * 32 + bit;
        if (pob[x] < 0) miss |= 1u << bit;
      }
    }
    const int cnt = __popc(miss);
    const int incl = block_inclusive_scan(cnt, wave_tot);
    int r = base + incl - cnt;
    while (miss) {
      const int bit = __builtin_ctz(miss);
      miss &= miss - 1u;
      const int x = w * 32 + bit;
      if (r < n_cand) {
        const int p = (int)(uint32_t)keys[r];
        const int old = pblk[p];
        if (old >= 0) pob[old] = -1;
        const int rows = min(B, a.N - x * B);
        pblk[p] = x;
        pob[x] = p;
        prow[p] = rows;
        pused[p] = a.step;
        const int j = atomicAdd(&s_n[1], 1);
        jobs[j] = make_int4(x, p, 0, rows);
      }
      ++r;
    }
    if (tid == kThreads - 1) s_n[2] = incl;
    __syncthreads();
    base += s_n[2];
    __syncthreads();
  }
  const int n_jobs = s_n[1];
  if (tid == 0 && a.fetched) a.fetched[bg] += n_jobs;

  // The copies: 16-byte units of every job's rows, K and V.  Each thread
  // issues the loads of kBatch units of K and of V before any store, so
  // that 2 kBatch host reads per thread are in flight across the link (a
  // load-store pair at a time would leave the link idle for most of each
  // round trip).
  const int units_row = a.row_bytes / 16;
  const char* __restrict__ hk = a.host_k + (int64_t)bg * a.slice_bytes_mem;
  const char* __restrict__ hv = a.host_v + (int64_t)bg * a.slice_bytes_mem;
  char* __restrict__ pk = a.pool_k + (int64_t)bg * a.slice_bytes_pool;
  char* __restrict__ pv = a.pool_v + (int64_t)bg * a.slice_bytes_pool;
  for (int j = 0; j < n_jobs; ++j) {
    const int4 jb = jobs[j];
    const int n_units = (jb.w - jb.z) * units_row;
    const int64_t src0 = ((int64_t)jb.x * B + jb.z) * a.row_bytes;
    const int64_t dst0 = ((int64_t)jb.y * B + jb.z) * a.row_bytes;
    for (int u0 = tid; u0 < n_units; u0 += kBatch * kThreads) {
      uint4 kv[kBatch], vv[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        // past the job's end a lane re-reads unit u0 (no branch around the loads)
        const int u = u0 + i * kThreads < n_units ? u0 + i * kThreads : u0;
        kv[i] = *reinterpret_cast<const uint4*>(hk + src0 + (int64_t)u * 16);
        vv[i] = *reinterpret_cast<const uint4*>(hv + src0 + (int64_t)u * 16);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int u = u0 + i * kThreads;
        if (u < n_units) {
          *reinterpret_cast<uint4*>(pk + dst0 + (int64_t)u * 16) = kv[i];
          *reinterpret_cast<uint4*>(pv + dst0 + (int64_t)u * 16) = vv[i];
        }
      }
    }
  }
}

}  // namespace

int cache_max_pages() { return kMaxPages; }
int64_t cache_max_blocks() { return (int64_t)kNeedWords * 32; }

hipError_t launch_cache_reset(const brs_memory& m, const brs_page_cache& c, hipStream_t s) {
  const int64_t bgs = (int64_t)m.batch * m.n_kv_heads;
  const int64_t n_tab = bgs * (m.capacity / m.block_size + 1);
  const int64_t n_pg = bgs * c.n_pages;
  const int64_t n = n_tab > n_pg ? n_tab : n_pg;
  hipLaunchKernelGGL(cache_reset_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     c.page_of_block, c.page_block, c.page_rows, c.page_used, n_tab, n_pg);
  return hipGetLastError();
}

hipError_t launch_cache_fetch(const brs_memory& m, const brs_page_cache& c, const int32_t* idx, int idx_heads,
                              int k, int64_t sink_end, int64_t win_start, int step, int32_t* fetched,
                              hipStream_t s) {
  FetchArgs a;
  const int es = elem_bytes(m.dtype);
  a.host_k = (const char*)m.k;
  a.host_v = (const char*)m.v;
  a.pool_k = (char*)c.k;
  a.pool_v = (char*)c.v;
  a.page_of_block = c.page_of_block;
  a.page_block = c.page_block;
  a.page_rows = c.page_rows;
  a.page_used = c.page_used;
  a.fetched = fetched;
  a.idx = idx;
  a.idx_heads = idx_heads;
  a.kk = idx ? k : 0;
  a.hkv = m.n_kv_heads;
  a.n_pages = c.n_pages;
  a.B = m.block_size;
  a.N = (int)m.length;
  a.nb = (int)(m.length / m.block_size);
  a.nbt = (int)((m.length + m.block_size - 1) / m.block_size);
  a.sink_end = (int)sink_end;
  a.win_start = (int)win_start;
  a.cap_blocks1 = (int)(m.capacity / m.block_size + 1);
  a.step = step;
  a.row_bytes = m.row_stride * es;
  a.slice_bytes_mem = m.capacity * (int64_t)a.row_bytes;
  a.slice_bytes_pool = (int64_t)c.n_pages * m.block_size * a.row_bytes;
  hipLaunchKernelGGL(cache_fetch_kernel, dim3((unsigned)(m.batch * m.n_kv_heads)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace brs

// Retrieval counters and memory pruning (MemLong 2.3.2, dynamic memory
// update: when the memory overflows, the newest tenth is kept, the oldest
// tenth dropped, and the least retrieved of the middle are evicted until half
// the memory is in use).
//
// count: one atomic add per valid selection entry (integer sums, so the
// order of the adds does not matter).
// plan: one workgroup sorts the middle blocks by (hits summed over the batch
// rows, block index) with a bitonic sort in LDS; the first n_evict are
// evicted; a prefix count gives every kept block its new index.
// copy: one workgroup per (old block, batch x kv head) moves the block's K/V
// rows, representatives and count to the new index of a second memory; the
// partial tail block goes behind the kept blocks.
#include "brs_internal.h"

namespace brs {
namespace {

__global__ __launch_bounds__(256) void count_hits_kernel(const int32_t* __restrict__ idx, int idx_heads, int k,
                                                         int64_t n_lists, int nb, int64_t capB,
                                                         int32_t* __restrict__ hits) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n_lists * k) return;
  const int b = (int)(i / ((int64_t)idx_heads * k));
  const int blk = idx[i];
  if (blk >= 0 && blk < nb) atomicAdd(hits + (int64_t)b * capB + blk, 1);
}

constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxMid = 16384;  // middle blocks one workgroup sorts in LDS
constexpr int kPlanMaxBlocks = kPlanMaxMid + kPlanMaxMid / 4 + 64;  // nb <= n_mid / 0.8 + 2

__global__ __launch_bounds__(kPlanThreads) void prune_plan_kernel(const int32_t* __restrict__ hits, int batch,
                                                                  int64_t capB, int nb, int n10, int n_evict,
                                                                  int P, int32_t* __restrict__ plan) {
  __shared__ uint64_t keys[kPlanMaxMid];  // (hits, block) of the middle blocks, padded to P
  __shared__ uint8_t kept[kPlanMaxBlocks];
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x;
  const int n_mid = nb - 2 * n10;
  for (int i = tid; i < P; i += kPlanThreads) {
    uint64_t key = ~0ull;  // padding sorts last
    if (i < n_mid) {
      const int blk = n10 + i;
      uint32_t h = 0;
      for (int b = 0; b < batch; ++b) h += (uint32_t)max(hits[(int64_t)b * capB + blk], 0);
      key = ((uint64_t)h << 32) | (uint32_t)blk;
    }
    keys[i] = key;
  }
  for (int i = tid; i < nb; i += kPlanThreads) kept[i] = i >= n10;
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kPlanThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t a = keys[i], c = keys[j];
          const bool up = (i & size) == 0;
          if ((a > c) == up) {
            keys[i] = c;
            keys[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n_evict; i += kPlanThreads) kept[(int)(uint32_t)keys[i]] = 0;
  __syncthreads();
  // new index = kept blocks before it: each thread takes a contiguous run
  const int per = (nb + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(tid * per, nb), b1 = min(b0 + per, nb);
  int cnt = 0;
  for (int i = b0; i < b1; ++i) cnt += kept[i];
  int next = block_inclusive_scan(cnt, wave_tot) - cnt;
  for (int i = b0; i < b1; ++i) plan[i] = kept[i] ? next++ : -1;
}

struct PruneArgs {
  const uint32_t* sk;  // source K / V as 32-bit words
  const uint32_t* sv;
  uint32_t* dk;
  uint32_t* dv;
  const uint16_t* sr;  // representatives as 16-bit units
  uint16_t* dr;
  const int32_t* hits;
  int32_t* dhits;
  const int32_t* plan;
  int64_t cap, capB;
  int row_words;  // 32-bit words per token row
  int rep_units;  // 16-bit units per block of representatives (all R)
  int B, nb, tail, kept;
  int batch, hkv, rep_heads;
};

// VEC: token rows are whole 16-byte units (row_words % 4 == 0): copy uint4s
template <bool VEC>
__global__ __launch_bounds__(256) void prune_copy_kernel(PruneArgs a) {
  const int i = blockIdx.x;  // old block; i == nb is the partial tail
  const int y = blockIdx.y;  // (batch, kv head)
  const int nb_new = i < a.nb ? a.plan[i] : a.kept;
  if (nb_new < 0) return;
  const int rows = i < a.nb ? a.B : a.tail;
  const int64_t src0 = ((int64_t)y * a.cap + (int64_t)i * a.B) * a.row_words;
  const int64_t dst0 = ((int64_t)y * a.cap + (int64_t)nb_new * a.B) * a.row_words;
  const int64_t n = (int64_t)rows * a.row_words;
  if constexpr (VEC) {
    const uint4* sk = reinterpret_cast<const uint4*>(a.sk + src0);
    const uint4* sv = reinterpret_cast<const uint4*>(a.sv + src0);
    uint4* dk = reinterpret_cast<uint4*>(a.dk + dst0);
    uint4* dv = reinterpret_cast<uint4*>(a.dv + dst0);
    for (int64_t e = threadIdx.x; e < n / 4; e += blockDim.x) {
      const uint4 x = sk[e], z = sv[e];
      dk[e] = x;
      dv[e] = z;
    }
  } else {
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
      a.dk[dst0 + e] = a.sk[src0 + e];
      a.dv[dst0 + e] = a.sv[src0 + e];
    }
  }
  if (i == a.nb) return;
  if (y < a.batch * a.rep_heads) {
    const int64_t r0 = ((int64_t)y * a.capB + i) * a.rep_units, r1 = ((int64_t)y * a.capB + nb_new) * a.rep_units;
    for (int e = threadIdx.x; e < a.rep_units; e += blockDim.x) a.dr[r1 + e] = a.sr[r0 + e];
  }
  if (y < a.batch && a.dhits && threadIdx.x == 0) a.dhits[(int64_t)y * a.capB + nb_new] = a.hits[(int64_t)y * a.capB + i];
}

}  // namespace

hipError_t launch_count_hits(const brs_memory& m, const int32_t* idx, int idx_heads, int k, int32_t* hits,
                             hipStream_t s) {
  const int64_t n = (int64_t)m.batch * idx_heads * k;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(count_hits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, idx_heads, k,
                     (int64_t)m.batch * idx_heads, (int)(m.length / m.block_size), m.capacity / m.block_size, hits);
  return hipGetLastError();
}

int prune_max_middle() { return kPlanMaxMid; }
int prune_max_blocks() { return kPlanMaxBlocks; }

hipError_t launch_prune(const brs_memory& src, const brs_memory& dst, const int32_t* hits, int32_t* dst_hits,
                        int32_t* plan, int nb, int n10, int n_evict, int kept, int tail, hipStream_t s) {
  const int n_mid = nb - 2 * n10;
  int P = 1;
  while (P < n_mid) P <<= 1;
  if (nb > 0) {
    hipLaunchKernelGGL(prune_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, hits, src.batch,
                       src.capacity / src.block_size, nb, n10, n_evict, P, plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  PruneArgs a;
  a.sk = (const uint32_t*)src.k;
  a.sv = (const uint32_t*)src.v;
  a.dk = (uint32_t*)dst.k;
  a.dv = (uint32_t*)dst.v;
  a.sr = (const uint16_t*)src.reps;
  a.dr = (uint16_t*)dst.reps;
  a.hits = hits;
  a.dhits = dst_hits;
  a.plan = plan;
  a.cap = src.capacity;
  a.capB = src.capacity / src.block_size;
  a.row_words = src.row_stride * elem_bytes(src.dtype) / 4;
  a.rep_units = src.reps_per_block * src.rep_dim * elem_bytes(src.rep_dtype) / 2;
  a.B = src.block_size;
  a.nb = nb;
  a.tail = tail;
  a.kept = kept;
  a.batch = src.batch;
  a.hkv = src.n_kv_heads;
  a.rep_heads = src.rep_heads;
  const dim3 grid((unsigned)(nb + 1), (unsigned)(src.batch * src.n_kv_heads));
  // k, v are 16-byte aligned (memory check), so whole-unit rows keep uint4 alignment
  if (a.row_words % 4 == 0)
    hipLaunchKernelGGL(prune_copy_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prune_copy_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace brs

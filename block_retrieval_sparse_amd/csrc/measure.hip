// Read-bandwidth reference kernels (measurement only; not part of the method).
//
// They read device memory the way the attention kernels do and nothing
// else, so their rate is the "achievable" read bandwidth a kernel of the
// path can be compared with:
//   - contiguous: one long span, 16-byte loads, a grid-stride loop with four
//     loads in flight per thread;
//   - gathered: a list of equal chunks at arbitrary offsets (a retrieved
//     block of one kv head is one such chunk), one workgroup per chunk.
// The loaded words are folded with XOR and written only if the fold equals a
// value the caller passes (never, for the data used), so the loads cannot be
// dropped and the kernel writes nothing in practice.
#include "brs_internal.h"
#include "brs_measure.h"

namespace brs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ uint32_t fold(const uint4& u) { return u.x ^ u.y ^ u.z ^ u.w; }

__global__ __launch_bounds__(kThreads) void read_contiguous_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                   uint32_t never, uint32_t* __restrict__ sink) {
  uint32_t acc = 0u;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(p[i]);
  if (acc == never) sink[blockIdx.x & 1023] = acc;
}

__global__ __launch_bounds__(kThreads) void read_gather_kernel(const char* __restrict__ base, int64_t chunk_bytes,
                                                               const int64_t* __restrict__ offsets,
                                                               uint32_t never, uint32_t* __restrict__ sink) {
  const uint4* p = reinterpret_cast<const uint4*>(base + offsets[blockIdx.x]);
  const int64_t n16 = chunk_bytes / 16;
  uint32_t acc = 0u;
  int64_t i = threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n16; i += kUnroll * kThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += kThreads) acc ^= fold(p[i]);
  if (acc == never) sink[blockIdx.x & 1023] = acc;
}

}  // namespace
}  // namespace brs

extern "C" int brs_measure_read(const void* base, int64_t chunk_bytes, const int64_t* offsets, int64_t n_chunks,
                                uint32_t never, uint32_t* sink, void* stream) {
  if (!base || !sink || chunk_bytes < 16 || chunk_bytes % 16 != 0 || n_chunks < 1) return BRS_E_INVAL;
  if (((uintptr_t)base % 16) != 0) return BRS_E_INVAL;
  hipStream_t s = (hipStream_t)stream;
  if (!offsets) {
    if (n_chunks != 1) return BRS_E_INVAL;
    const int64_t n16 = chunk_bytes / 16;
    int64_t blocks = (n16 + brs::kThreads * brs::kUnroll - 1) / (brs::kThreads * brs::kUnroll);
    blocks = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
    hipLaunchKernelGGL(brs::read_contiguous_kernel, dim3((unsigned)blocks), dim3(brs::kThreads), 0, s,
                       (const uint4*)base, n16, never, sink);
  } else {
    if (n_chunks > INT32_MAX) return BRS_E_INVAL;
    hipLaunchKernelGGL(brs::read_gather_kernel, dim3((unsigned)n_chunks), dim3(brs::kThreads), 0, s,
                       (const char*)base, chunk_bytes, offsets, never, sink);
  }
  return hipGetLastError() == hipSuccess ? BRS_OK : BRS_E_HIP;
}

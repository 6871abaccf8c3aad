// Read-bandwidth reference kernels (measurement only; not part of the method).
//
// They read device memory and nothing else, so their rate is the read
// bandwidth a kernel of this GPU can reach; the attention kernels are
// compared with it.  Both use the fastest form measured here: one workgroup
// per chunk, buffer loads of 16 bytes per lane (each instruction reads whole
// cache lines), four in flight per thread, with the non-temporal cache policy
// (on gfx950 7.1-7.3 TB/s, against 6.2-6.5 TB/s with the default policy and
// 5.7 TB/s for a grid-stride loop of plain global loads over the same bytes):
//   - contiguous: one long span cut into 256 KB chunks;
//   - gathered: a list of equal chunks at arbitrary offsets (a retrieved
//     block of one kv head is one such chunk).
// The loaded words are folded with XOR and written only if the fold equals a
// value the caller passes (never, for the data used), so the loads cannot be
// dropped and the kernel writes nothing in practice.
#include "brs_internal.h"
#include "brs_measure.h"

namespace brs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kSpanChunk = 256 << 10;  // bytes per workgroup of the contiguous read
constexpr int kNonTemporal = 2;            // buffer-load cache policy: nt
constexpr int kRsrcFlags = 0x00020000;     // raw buffer resource word 3 (32-bit data, no swizzle)

__device__ __forceinline__ uint32_t fold(const uint4& u) { return u.x ^ u.y ^ u.z ^ u.w; }

// Reads [p, p + bytes) (bytes a multiple of 16, below 2^31) and folds it.
__device__ __forceinline__ uint32_t read_chunk(const char* p, int bytes) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, bytes, kRsrcFlags);
  const int n16 = bytes / 16;
  uint32_t acc = 0u;
  int i = threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n16; i += kUnroll * kThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_bit_cast(uint4,
                                __builtin_amdgcn_raw_buffer_load_b128(rs, (i + u * kThreads) * 16, 0, kNonTemporal));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += kThreads)
    acc ^= fold(__builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16, 0, kNonTemporal)));
  return acc;
}

__global__ __launch_bounds__(kThreads) void read_contiguous_kernel(const char* __restrict__ base, int64_t bytes,
                                                                   uint32_t never, uint32_t* __restrict__ sink) {
  const int64_t lo = (int64_t)blockIdx.x * kSpanChunk;
  const int64_t len = bytes - lo < kSpanChunk ? bytes - lo : kSpanChunk;
  const uint32_t acc = read_chunk(base + lo, (int)len);
  if (acc == never) sink[blockIdx.x & 1023] = acc;
}

__global__ __launch_bounds__(kThreads) void read_gather_kernel(const char* __restrict__ base, int64_t chunk_bytes,
                                                               const int64_t* __restrict__ offsets,
                                                               uint32_t never, uint32_t* __restrict__ sink) {
  const uint32_t acc = read_chunk(base + offsets[blockIdx.x], (int)chunk_bytes);
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
    const int64_t blocks = (chunk_bytes + brs::kSpanChunk - 1) / brs::kSpanChunk;
    if (blocks > INT32_MAX) return BRS_E_INVAL;
    hipLaunchKernelGGL(brs::read_contiguous_kernel, dim3((unsigned)blocks), dim3(brs::kThreads), 0, s,
                       (const char*)base, chunk_bytes, never, sink);
  } else {
    if (n_chunks > INT32_MAX || chunk_bytes > INT32_MAX - 15) return BRS_E_INVAL;
    hipLaunchKernelGGL(brs::read_gather_kernel, dim3((unsigned)n_chunks), dim3(brs::kThreads), 0, s,
                       (const char*)base, chunk_bytes, offsets, never, sink);
  }
  return hipGetLastError() == hipSuccess ? BRS_OK : BRS_E_HIP;
}

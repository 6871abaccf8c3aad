/*
 * brs_measure.h -- measurement helpers of libbrs.  They are not part of the
 * method; they give the reference numbers the attention kernels are judged
 * against (the read bandwidth a kernel of this GPU actually reaches) and the
 * per-kernel timing hook.
 */
#ifndef BRS_MEASURE_H_
#define BRS_MEASURE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read n_chunks chunks of chunk_bytes bytes each from device memory and
 * discard them (a read-bandwidth reference).
 *   base    : device pointer, 16-byte aligned.
 *   offsets : device array of n_chunks byte offsets from base (each a
 *             multiple of 16), one workgroup per chunk -- the access pattern
 *             of retrieved blocks; or NULL with n_chunks = 1 to read
 *             [base, base + chunk_bytes) as one contiguous span, one
 *             workgroup per 256 KB of it.  Non-temporal 16-byte buffer loads
 *             that read whole cache lines per instruction (the fastest read
 *             form measured on gfx950).
 *   never   : a value the XOR of all words read is compared with; only on
 *             equality is anything written (to sink), so the loads stay in
 *             the kernel but nothing is written in practice.
 *   sink    : device buffer of 1024 uint32.
 * chunk_bytes must be a positive multiple of 16 (below 2^31 with offsets).
 * Enqueued on stream;
 * returns BRS_OK, BRS_E_INVAL or BRS_E_HIP (no message is recorded). */
int brs_measure_read(const void* base, int64_t chunk_bytes, const int64_t* offsets, int64_t n_chunks,
                     uint32_t never, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BRS_MEASURE_H_ */

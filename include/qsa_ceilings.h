/*
 * qsa_ceilings.h - memory-system ceilings of the part under the access
 * patterns of the QSA path, for benchmarks (not part of the method).
 * Library: libqsa.so.  Status codes as in qsa.h.
 *
 * Both calls only read the given memory (the kernels fold what they read
 * into one word and store it to *sink only in a practically impossible
 * case), enqueue one kernel on `stream` and return at once.  Nothing is
 * allocated or synchronised.  Every pointer is a device pointer owned by the
 * caller.
 */
#ifndef QSA_CEILINGS_H_
#define QSA_CEILINGS_H_

#include <stddef.h>
#include <stdint.h>

#include "qsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a multiple
 * of 16; QSA_ERR_ALIGN otherwise): workgroup w of `workgroups` (1 .. 2^20,
 * 512 threads each) reads the w-th of equal contiguous pieces.  The decode
 * step's compressed-key scan is such a read of every candidate block's
 * 128-byte key. */
qsa_status qsa_ceil_stream_read(const void* buf, size_t bytes, int32_t workgroups,
                                uint32_t* sink, void* stream);

/* Random gather: piece i is the row_bytes bytes at byte offset
 * row_index[i] * row_bytes from base (row_bytes a power of two in
 * 16 .. 16384; base 16-byte and row_index 8-byte aligned).  The caller
 * guarantees every row_index[i] * row_bytes + row_bytes lies inside its
 * allocation.  `workgroups` (1 .. 2^20) workgroups of 256 threads.  The
 * sparse attention gathers 256-byte pieces (one KV head's row of one token),
 * 1 KiB rows (one token, all KV heads) or 4 KiB pieces (one micro-block). */
qsa_status qsa_ceil_gather(const void* base, const int64_t* row_index, int64_t n_rows,
                           int32_t row_bytes, int32_t workgroups, uint32_t* sink, void* stream);

/* LDS atomic adds (a cost the kernels' reductions are designed around, not a
 * memory ceiling): `workgroups` (1 .. 2^20) workgroups of 256 threads each
 * issue `iters` (1 .. 4096) atomic adds of 1 to a 4 KiB LDS array, 32-bit
 * integer (f32 = 0) or float32 (f32 = 1), with `share` (1, 2, 4, 16 or 64)
 * consecutive lanes of a wavefront on one address and the address groups of
 * a wavefront distinct.  Stores one word of the result to sink[blockIdx]
 * only in a practically impossible case; sink must hold `workgroups` words
 * (QSA_ERR_SHAPE for other arguments). */
qsa_status qsa_ceil_lds_atomic(int32_t f32, int32_t share, int32_t workgroups, int32_t iters,
                               uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_CEILINGS_H_ */

/* libpdecode measurement helper: the device's streaming-read ceiling.
 *
 * Not an operation of the decode path. The decode is bound by HBM bandwidth; this call measures
 * how many bytes per second a kernel that only reads can draw from HBM on the same device, so
 * that a decode's KV-read rate can be stated against that ceiling as well as against the
 * published peak.
 *
 * pdecode_bench_stream_read reads `bytes` bytes of `buf` once. Thread t of the
 * workgroups x 256 threads reads the 16-byte vectors t, t + N, t + 2N, ... (N = threads) in rounds
 * of `loads_per_lane` loads, all issued before any is used; adjacent lanes read adjacent vectors.
 *   buf            device pointer, 16-byte aligned; bytes: a multiple of 16, at least 16.
 *   loads_per_lane 1, 2, 4, 8 or 16 (else PDECODE_ERR_UNSUPPORTED).
 *   nontemporal    nonzero: loads carry the nontemporal hint.
 *   workgroups     grid size, > 0.
 *   sink           device uint32 [workgroups * 256], written (an XOR of the words each thread
 *                  read, so that no load is dropped).
 *   stream         hipStream_t (NULL = default stream); the call is asynchronous.
 * Nothing is allocated. Errors: PDECODE_ERR_INVALID_ARG (null pointer, bad size or alignment,
 * workgroups <= 0; nothing launched), PDECODE_ERR_UNSUPPORTED, PDECODE_ERR_HIP (launch failure).
 */
#ifndef PDECODE_BENCH_H
#define PDECODE_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "pdecode.h"

#ifdef __cplusplus
extern "C" {
#endif

pdecode_status pdecode_bench_stream_read(const void *buf, size_t bytes, int32_t loads_per_lane,
                                         int32_t nontemporal, int32_t workgroups, uint32_t *sink,
                                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PDECODE_BENCH_H */

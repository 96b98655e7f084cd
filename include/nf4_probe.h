/*
 * nf4_probe.h -- bandwidth probes of libnf4 (measurement helpers, not part of
 * the NF4 method).  They move bytes with the same access patterns as the hot
 * path's kernels and no arithmetic, so that the hot path's achieved
 * bandwidth can be set against what plain streaming reaches on the same GPU.
 * Device pointers; asynchronous on `stream`; they allocate nothing.
 */
#ifndef NF4_PROBE_H_
#define NF4_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "nf4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * nf4_probe_stream_read -- reads `bytes` bytes at src once (16-byte streaming
 * loads, one contiguous range per wave, four loads in flight per lane: the
 * GEMV's weight stream without the decode).  Writes one dword to *sink only
 * for a data pattern that does not occur in practice (it keeps the loads
 * alive).  src 16-byte aligned, bytes a multiple of 16; sink 4 bytes.
 * Returns NF4_EINVAL for NULL or misaligned pointers or sizes.
 */
nf4_status nf4_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * nf4_probe_expand_copy -- reads `src_bytes` bytes and writes four times as
 * many: dst dword-quad i = (w, w ^ 1, w ^ 2, w ^ 3) for w = src dword i,
 * with 16-byte streaming stores (the dequant's 1 : 4 read : write stream
 * without the decode).  src 4-byte aligned, dst 16-byte aligned, src_bytes a
 * multiple of 4.  Returns NF4_EINVAL for NULL or misaligned pointers or sizes.
 */
nf4_status nf4_probe_expand_copy(const void* src, size_t src_bytes, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_PROBE_H_ */

/*
 * sketchssm_measure.h -- measurement aid shipped with the SketchSSM library.
 *
 * Not part of the decode path.  The decode read is bound by HBM bandwidth, and
 * the rate a kernel can reach depends on its mix of reads and writes and on
 * the machine; the vendor peak (8 TB/s on MI355X) is never reached by any
 * access pattern.  This call streams a buffer through the GPU in a chosen
 * read:write proportion with the simplest possible access pattern (whole
 * 16-byte pieces, every wave reading 1 KB contiguous runs), so a benchmark can
 * measure, on the machine it runs on and in the same process, the practical
 * ceiling against which a decode kernel with the same mix is judged.
 */
#ifndef SKETCHSSM_MEASURE_H
#define SKETCHSSM_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "sketchssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming probe.  Reads every byte of src once and writes dst:
 *   src          device, read_bytes bytes, 16-byte aligned
 *   read_bytes   a multiple of unroll * 4096
 *   dst          device, 16-byte aligned, at least write_bytes bytes; with
 *                write_bytes = 0 it must hold blocks * 4096 bytes
 *   write_bytes  0 (read only: each thread writes one 16-byte sum at the end),
 *                or read_bytes / m where m divides unroll (each thread writes
 *                one 16-byte sum of m consecutive 16-byte pieces it read)
 *   unroll       16-byte pieces each thread has in flight: 4, 8 or 16
 *   blocks       256-thread blocks; 0 = one block per unroll * 4 KB chunk
 *                (not allowed with write_bytes = 0), else each block loops
 *                over chunks blocks apart
 *   flags        bit 0: non-temporal (streaming) loads and stores; other
 *                bits must be 0
 * The values written are fp32 sums of the values read.  Asynchronous on
 * `stream`; returns SKSSM_EINVAL / SKSSM_EALIGN / SKSSM_ESHAPE for arguments
 * outside the rules above and SKSSM_ELAUNCH if the launch fails.
 */
sketchssm_status sketchssm_stream_probe(const void* src, size_t read_bytes, void* dst,
                                        size_t write_bytes, int32_t unroll, int32_t blocks,
                                        int32_t flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SKETCHSSM_MEASURE_H */

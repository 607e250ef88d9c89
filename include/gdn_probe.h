/*
 * gdn_probe.h -- HBM bandwidth probe of the MI355X verify-and-commit library.
 *
 * A measurement aid, not a step of the method: plain streaming kernels that
 * read, write or copy a buffer with the same access pattern as the all-layer
 * commit (16-byte non-temporal vector accesses, each load or store instruction
 * of a 256-thread workgroup covering 4 KiB of contiguous memory, 16 KiB per
 * workgroup, workgroup ids remapped so that each XCD streams a contiguous
 * range). Timing them gives the bandwidth this access pattern can reach on the
 * device, the ceiling that the replay kernels' achieved bandwidth is read
 * against; the bandwidth the method itself must move is set by the RecoverSSM
 * PR's commit running at the memory floor ([vLLM] Test Result).
 *
 * Same conventions as gdn_replay.h: device pointers owned by the caller,
 * asynchronous on `stream` (a hipStream_t; NULL = default stream), nothing
 * allocated, host-checkable errors returned as a negative gdn_status before
 * any launch.
 */
#ifndef GDN_PROBE_H
#define GDN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_PROBE_CHUNK 16384  /* bytes streamed by one workgroup */

typedef enum {
    GDN_PROBE_READ = 0,   /* read src; write one 16-byte word per chunk to dst */
    GDN_PROBE_WRITE = 1,  /* write dst (every 32-bit word set to its chunk index) */
    GDN_PROBE_COPY = 2    /* copy src to dst */
} gdn_probe_kind;

/* Stream `bytes` bytes through HBM.
 *   kind   one of gdn_probe_kind (else GDN_ERR_SHAPE)
 *   src    device, `bytes` bytes, 16-byte aligned (READ, COPY; ignored by WRITE)
 *   dst    device, 16-byte aligned: READ needs bytes / GDN_PROBE_CHUNK * 16
 *          bytes (one word per chunk, the XOR of the chunk's 16-byte words,
 *          so that the loads cannot be dropped); WRITE and COPY need `bytes`
 *   bytes  a positive multiple of GDN_PROBE_CHUNK, at most
 *          2^31 - 1 chunks (else GDN_ERR_SHAPE)
 * Returns GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_ALIGN or
 * GDN_ERR_LAUNCH (gdn_replay.h). */
int32_t gdn_bandwidth_probe(int32_t kind, const void* src, void* dst, int64_t bytes,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PROBE_H */

/*
 * confk_probe.h -- measurement aid beside the CONF-KV decode step, built as a
 * library of its own (libconfk_probe.so) so that the product library holds
 * only the step.
 */
#ifndef CONFK_PROBE_H
#define CONFK_PROBE_H

#include <stdint.h>

#include "confk.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * confk_read_probe -- a measurement aid beside the five calls, not a step of
 * the method: reads `bytes` of device memory at `buf` once, with the 16-byte
 * non-temporal loads (whole 128-byte lines per instruction) that
 * confk_attn_decode streams its cache with, so that a timed launch measures
 * the streaming-read rate HBM sustains for that load form (the ceiling the
 * attention kernel is compared with, beside the 8 TB/s peak).
 *   buf    device, 16-byte aligned, read only
 *   bytes  a positive multiple of 65536
 *   sink   device uint32 [1]: XOR-ed (atomically) with the XOR of every
 *          little-endian 32-bit word of the buffer; a zeroed sink ends up
 *          holding that checksum
 * Errors: CONFK_ERR_INVALID_ARG for a null pointer, a misaligned buffer or a
 * size that is not a positive multiple of 65536.
 */
int confk_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONFK_PROBE_H */

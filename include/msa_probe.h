/*
 * msa_probe.h - measurement aid of libmsa.so (not a step of the MSA method).
 *
 * The decode path's indexer and gather are bound by HBM bandwidth, and their roofline fractions
 * are taken against the MI355X's published 8 TB/s. This probe measures what a plain streaming
 * read achieves on the same GPU for a given working set, so that a kernel's fraction can also be
 * read against the rate the memory system actually delivers at that size.
 */
#ifndef MSA_PROBE_H
#define MSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at `buf` (device memory, 16-byte aligned, bytes a multiple of 16) once, each
 * of the workgroups streaming one contiguous share with coalesced 16-byte loads, four workgroups
 * per compute unit, and write one 32-bit word per workgroup (an
 * XOR of the data, so the loads cannot be skipped) to `sink` (device, at least
 * msa_probe_sink_words() words). Asynchronous on `stream`, like the library's other calls.
 * Returns 0 (MSA_OK), or -1 for a NULL pointer or a misaligned size, -4 for a launch error.
 */
int msa_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Words msa_probe_stream_read writes to `sink`. */
size_t msa_probe_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PROBE_H */

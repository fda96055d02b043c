/*
 * msa_debug.h - diagnostics of the checked build of the library (a debugging aid, not a step of
 * the MSA method).
 *
 * The library is built twice from the same sources: libmsa.so, and libmsa_checked.so compiled
 * with MSA_CHECKED, whose kernels also check, as they run, the values they read from device
 * memory against their contract and the indexes they compute against the extents of their
 * arguments. Every build clamps or skips the device-memory values outside their contract, so a
 * failed check never changes where a kernel reads or writes; it is counted, the lowest failing
 * site is kept, and the kernel goes on. The checked build's results equal the normal build's
 * (bit for bit) whenever no check fails.
 *
 * Sites (the value of *site below):
 *   1   MSA_CHECK_CTX_LEN    a context length outside q_len .. max_blocks * 128 (the kernels
 *                            clamp it to that range; tokens past the table are unreachable)
 *   101 MSA_CHECK_SELECTION  a row's selected ids not strictly ascending within its eligible
 *                            blocks, or without the block of its query token (a kernel error)
 *   102 MSA_CHECK_WORKSPACE  a split partial or counter index past the call's workspace
 *   103 MSA_CHECK_LDS        a list or table index past its on-chip array
 *   104 MSA_CHECK_OUTPUT     a row, score or output index past its array
 */
#ifndef MSA_DEBUG_H
#define MSA_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MSA_CHECK_CTX_LEN = 1,
    MSA_CHECK_SELECTION = 101,
    MSA_CHECK_WORKSPACE = 102,
    MSA_CHECK_LDS = 103,
    MSA_CHECK_OUTPUT = 104,
};

/*
 * Failed checks on the current device since the previous call (or since the library was
 * loaded), and the lowest failing site (0 when none failed); both are reset. Waits for the
 * device's queued work to finish first (the counters are read with a synchronous copy), so call
 * it between steps, not inside a captured graph.
 *   count, site : host pointers, both required.
 * Returns MSA_OK; MSA_ERR_INVALID_ARG for a NULL pointer; MSA_ERR_UNSUPPORTED from libmsa.so
 * (built without the checks: nothing is counted); MSA_ERR_HIP when a copy fails.
 */
int msa_debug_checks(uint32_t *count, uint32_t *site);

#ifdef __cplusplus
}
#endif

#endif /* MSA_DEBUG_H */

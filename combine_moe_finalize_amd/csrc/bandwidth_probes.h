/*
 * bandwidth_probes.h - streaming read and copy kernels that measure the
 * HBM rates one MI355X reaches in the same session as a benchmark, so the
 * finalize kernels can be reported against a measured ceiling beside the
 * 8 TB/s specification, and an empty kernel for the per-launch floor.
 * Measurement infrastructure: the finalize library does not use them.
 *
 * Both kernels read `bytes` from `src` as 16-byte vectors with non-temporal
 * loads, each lane keeping four loads in flight; one workgroup covers 16 KiB.
 *
 *  src, dst  device pointers, 16-byte aligned, `bytes` long each.
 *  bytes     a positive multiple of MOEF_PROBE_GRAIN, at most
 *            MOEF_PROBE_MAX_GRAINS of them (one launch covers at most
 *            2^32 - 1 work-items, 256 per grain).
 *  sink      device uint32 (read probe): written only when the XOR of a
 *            lane's 64 bytes equals 0x9E3779B9, which keeps the loads from
 *            being optimized away; with all-zero input it is never written.
 *  stream    hipStream_t as void* (NULL: the null stream); the call returns
 *            without waiting.
 *
 * Return value: 0, or 1 (a NULL pointer), 2 (bytes not a positive multiple
 * of MOEF_PROBE_GRAIN, or more than MOEF_PROBE_MAX_GRAINS grains), 4 (src or
 * dst not 16-byte aligned, sink not 4-byte aligned), 6 (dst overlaps src),
 * 7 (the HIP runtime rejected the launch). Checks run before any HIP call.
 */
#ifndef MOEF_BANDWIDTH_PROBES_H
#define MOEF_BANDWIDTH_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEF_PROBE_GRAIN 16384
#define MOEF_PROBE_MAX_GRAINS 16777215LL /* 2^24 - 1 */

/* Reads every byte of src once. */
int moef_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* dst = src, byte for byte, with non-temporal loads and stores. */
int moef_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* One 64-lane workgroup that does nothing: the cost of a launch itself, the
 * floor under any kernel's time per call. Returns 0, or 7. */
int moef_probe_empty(void* stream);

/* The same empty kernel on two workgroups: a marker a benchmark launches
 * between the cases it times, so that a kernel trace splits into one block
 * per case (its grid tells it apart from moef_probe_empty). Returns 0, or 7. */
int moef_probe_mark(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEF_BANDWIDTH_PROBES_H */

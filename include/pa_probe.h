/*
 * pa_probe.h - measurement aid of libpa: the achievable HBM read rate.
 *
 * Not part of the attention method.  Decode attention reads every K/V byte
 * once and writes almost nothing, so its ceiling on a given GPU is the rate
 * at which plain streaming reads can leave HBM, which is below the 8 TB/s
 * vendor figure.  This probe measures that rate with the same loads the
 * decode kernels use (16 bytes per lane, optionally non-temporal), so that a
 * benchmark can quote decode against a measured ceiling as well as against
 * the nominal peak.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_PROBE_NONTEMPORAL 1u /* non-temporal loads (the decode kernels' streaming loads) */
#define PA_PROBE_SCATTERED 2u   /* runs visited in a scattered order, as paged blocks lie in the
                                   pool: run r read in place of run (r * 0x9E3779B1) mod (number
                                   of runs); needs run_bytes > 0 dividing bytes into a power-of-two
                                   number of runs */

/*
 * pa_hbm_read_probe - read `bytes` bytes of device memory once.
 *
 *   src            device memory, 16-byte aligned; bytes a positive multiple of 16
 *   sink           device memory of num_workgroups uint32 values; a workgroup
 *                  writes its slot only when its running XOR of the data equals
 *                  `magic` (so the loads cannot be optimised away while the
 *                  writes stay negligible); contents otherwise untouched
 *   num_workgroups 1 .. 65535 workgroups of 512 threads, four 16-byte loads
 *                  in flight per lane
 *   run_bytes      0: the workgroups stride over the whole buffer together
 *                  (consecutive lanes on consecutive 16-byte chunks); else a
 *                  multiple of 8192: the buffer is cut into runs of this many
 *                  bytes and workgroup w reads runs w, w + num_workgroups, ...
 *                  each from start to end, as a decode workgroup reads whole
 *                  K/V blocks
 *   flags          PA_PROBE_NONTEMPORAL and/or PA_PROBE_SCATTERED (other bits:
 *                  PA_ERR_INVALID; SCATTERED with run_bytes 0, or with a run
 *                  count that is not a power of two: PA_ERR_INVALID)
 *
 * Enqueued on `stream` (a hipStream_t); nothing allocated or synchronised.
 * Returns PA_OK, PA_ERR_NULL, PA_ERR_INVALID (sizes, alignment, run length, flags) or
 * PA_ERR_HIP.
 */
int pa_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t num_workgroups, size_t run_bytes,
                      uint32_t magic, uint32_t flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */

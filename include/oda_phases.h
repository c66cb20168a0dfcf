/*
 * oda_phases.h -- the profiling build of the ODA library (liboda_phases.so).
 *
 * The same library as liboda.so (include/oda.h, every entry point and
 * kernel), built with ODA_PHASE_STAMPS: thread 0 of every attention workgroup
 * records the chip's 100 MHz real-time counter at eight points of its work
 * and the XCD it ran on.  This is measurement support for the split-K passes
 * of the picx.dev summary's "Local-First Decoding" (the Local pass over S^L_t,
 * the Full pass over S^F_t): where a launch spends its time, and how evenly
 * its workgroups finish.  Nothing here is part of the product library.
 *
 * Phase k of slot w (w = the workgroup's linear id,
 * (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x, modulo
 * 65536): 0 entry, 1 request state known (Full: its length; Local: seq_len),
 * 2 first tile reduced, 3 static rows done, 4 tail pool done, 5 fold barrier
 * passed, 6 partial stored (once the stores completed; ticket merges: the
 * ticket taken), 7 merge done (merging workgroup only).  Stamps are raw
 * counter values (10 ns apart); a phase a workgroup did not reach keeps the
 * value an earlier launch left (clear first, and compare with phase 0).
 */
#ifndef ODA_PHASES_H_
#define ODA_PHASES_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host.  Copies the stamps of slots 0..groups-1 (stamps: host [groups][8],
 * xcc: host [groups]) after the work that wrote them has completed.
 * Returns 0, or a HIP error code (groups > 65536 or a null pointer: invalid
 * value). */
int oda_phase_stamps_read(unsigned long long* stamps, unsigned* xcc, size_t groups);

/* Host.  Zeroes every stamp (synchronous). */
int oda_phase_stamps_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* ODA_PHASES_H_ */

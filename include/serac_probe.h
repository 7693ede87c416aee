/*
 * serac_probe.h - measurement entry point of libserac_probe.so, used by the
 * benchmark to price the matcher's sweep against the hardware (not part of
 * the matcher; libserac.so does not depend on it).
 */
#ifndef SERAC_PROBE_H
#define SERAC_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Back-to-back v_mfma_i32_32x32x32_i8 (the matcher's contraction
 * instruction) on four independent accumulators per wave, `nv` independent
 * v_max3_u32 after each MFMA (nv in {0, 4, 8, 12, 16}), `iters` rounds, in
 * `blocks` workgroups of four waves (256 workgroups: one wave per SIMD on a
 * 256-CU device; 512: two).  Runs once to warm up, then once timed with HIP
 * events on the null stream; synchronous.
 *   ms    device time of the timed launch
 *   tops  int8 ops per second / 1e12 (65536 ops per MFMA)
 *   ghz   shader clock seen by workgroup 0: its shader-clock counter ticks
 *         over the constant 100 MHz real-time counter
 * Allocates and frees its own device buffers.  Returns 0, -1 for a bad
 * argument, -5 for a HIP error.
 */
int serac_probe_mfma(int32_t blocks, int32_t iters, int32_t nv, double *ms,
                     double *tops, double *ghz);

#ifdef __cplusplus
}
#endif

#endif /* SERAC_PROBE_H */

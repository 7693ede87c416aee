/*
 * serac_bench.h - benchmark instrumentation exported by libserac.so.
 *
 * Not part of the matching interface (serac.h): these calls keep process-wide
 * state and exist so that a benchmark can time the dominant kernel of the
 * matcher, the tile sweep that does the int8 contraction and the on-the-fly
 * reductions, on the stream its launches run on.
 */
#ifndef SERAC_BENCH_H
#define SERAC_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * serac_profile_start arms up to max_launches pairs of HIP events; from then
 * on one tile-kernel launch in `every` (the first, then every `every`-th)
 * made by serac_match_pair, serac_match_pairs or serac_top2_pair is
 * dispatched with hipExtLaunchKernel carrying one pair as its start and stop
 * events, recorded by the dispatch itself on the call's stream.  The events
 * carry no system-scope fence, so a timed dispatch ends like an untimed one
 * (a default event adds a cache write-back for the host to its dispatch).
 * The event handling slows the enqueueing host; timing a fraction of the
 * launches keeps the queue as full as without it.
 *
 * serac_profile_stop waits for the recorded events and returns:
 *   tile_kernel_ms  the summed device time of the timed launches (ms)
 *   launches        how many launches were timed
 *   per_launch_ms   (may be NULL when capacity is 0) the first `capacity`
 *                   launches' device times, in launch order
 *   kernel          (may be NULL) static text naming the tile kernel timed,
 *                   e.g. "serac_tiles_fused<true, true>"; "mixed" if
 *                   launches of several kernels were timed, "none" if none
 * and disarms.  Not thread-safe against concurrent matching calls from other
 * threads.
 * Errors: SERAC_ERR_INVALID_ARG (max_launches or every outside [1, 1048576],
 * NULL outputs, capacity < 0, stop without start), SERAC_ERR_HIP.
 */
int serac_profile_start(int32_t max_launches, int32_t every);
int serac_profile_stop(double *tile_kernel_ms, int32_t *launches, float *per_launch_ms,
                       int32_t capacity, const char **kernel);

/*
 * The current device's angle slack: the finishing kernel of a single pair
 * takes the ratio and distance gates from the device's double acos where an
 * interval of this half-width around it settles them, and from the host-built
 * table (the oracle's libm values) otherwise.  The slack is twice the largest
 * distance between the two over every attainable score, measured once per
 * device at set-up, plus 1e-15; +INFINITY (table only) if that check could
 * not run or while SERAC_TEST_ANGLE_TABLE is set at set-up.
 * Errors: SERAC_ERR_INVALID_ARG (NULL), those of the device set-up.
 */
int serac_angle_slack(double *slack);

/*
 * Bytes of device memory the library's workspaces on the current device hold
 * now (accumulators and scratch of every stream's workspace; not the angle
 * table, the fixed scratch of serac_match_pair_noalloc, or pinned host
 * memory).  Workspaces only grow, so after a call this is that call's peak.
 * Errors: SERAC_ERR_INVALID_ARG (NULL), SERAC_ERR_HIP.
 */
int serac_workspace_bytes(int64_t *bytes);

#ifdef __cplusplus
}
#endif

#endif /* SERAC_BENCH_H */

/*
 * serac.h - C ABI of the MI355X (gfx950) SIFT descriptor matcher.
 *
 * The library matches 128-dimensional unsigned 8-bit SIFT descriptors
 * between image pairs by brute force, as the SERAC README describes (its
 * introduction and the sections "What changed" and "Exactness"):
 *
 *   S[i][j] = sum_k A[i][k] * B[j][k]           exact integer inner product
 *   row i   : (best, idx, second) over all j    identity (0, -1, 0), lowest
 *                                                column on a tie, second
 *                                                counted with multiplicity
 *   col j   : (best, idx) over all i            lowest row on a tie
 *   accept  : idx >= 0 and d1 <= max_distance and d1 < max_ratio * d2 and
 *             (cross_check == 0 or col_idx[idx] == i),
 *             where d = acos(min(s, 512^2) / 512^2) in IEEE double.
 *
 * The S matrix is never written to memory: the kernels reduce it to the
 * row top-2 and the column best as they compute it.
 *
 * Conventions for every entry point:
 *   - Descriptor arrays are device pointers to n rows of exactly 128 bytes,
 *     row-major, 16-byte aligned.  The caller owns them; the library only
 *     reads them.
 *   - Output arrays are device pointers owned by the caller: match arrays
 *     8-byte aligned, int32 arrays and counts 4-byte aligned.  A pointer
 *     that is NULL where data is needed, or misaligned, is
 *     SERAC_ERR_INVALID_ARG.
 *   - Work is enqueued on the given HIP stream (NULL = the null stream) and
 *     is asynchronous: results are valid once that stream has synchronised.
 *     Temporary device memory is taken from the device's stream-ordered
 *     pool on that stream and returned on it.
 *   - Results are deterministic: they do not depend on occupancy, launch
 *     order or the number of compute units.
 *   - Calls may come from several host threads.  Calls on one stream share
 *     that stream's device workspace and are serialized by the library;
 *     their order on the stream is the order in which they acquire it.
 *   - Arguments are validated before any HIP call; on an error nothing is
 *     enqueued and no output is written.
 *   - Only gfx950 devices are supported; any other device is refused with
 *     SERAC_ERR_UNSUPPORTED_DEVICE (there is no fallback path).
 *   - A failed allocation returns SERAC_ERR_OUT_OF_MEMORY; no kernel that
 *     writes the caller's outputs has been enqueued, and the next call
 *     tries again.  (For tests, the environment
 *     variable SERAC_TEST_FAIL_ALLOC, while set, makes every allocation
 *     the library attempts fail this way.)
 *   - No C++ exception crosses this interface.
 */
#ifndef SERAC_H
#define SERAC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SERAC_OK 0
#define SERAC_ERR_INVALID_ARG (-1)        /* NULL with n > 0, n < 0, n too large, bad params */
#define SERAC_ERR_CAPACITY (-2)           /* output capacity smaller than nA (after the cap) */
#define SERAC_ERR_UNSUPPORTED_DEVICE (-3) /* current device is not gfx950 */
#define SERAC_ERR_OUT_OF_MEMORY (-4)      /* device workspace allocation failed */
#define SERAC_ERR_HIP (-5)                /* any other HIP runtime error */
#define SERAC_ERR_TOO_LARGE (-6)          /* pair beyond serac_match_pair_noalloc's fixed scratch */
#define SERAC_ERR_NOT_INITIALIZED (-7)    /* serac_match_pair_noalloc before the device's set-up */

/* Largest descriptor count per image the library accepts. */
#define SERAC_MAX_DESCRIPTORS 262144

/* Matching parameters.
 *   max_ratio    ratio test on angles, accept iff d1 < max_ratio * d2;
 *                finite and > 0 (0.8 is the README's default; values above
 *                1 are allowed and then a top-1 tie can pass).
 *   max_distance accept iff d1 <= max_distance (radians); >= 0, +INFINITY
 *                disables the gate; NaN is an error.
 *   cross_check  0 or 1: require row i to be the best row of its best
 *                column (lowest row on a tie).
 *   flags        0, or SERAC_FLAG_SYMMETRIC; other bits are an error.
 *   stream       hipStream_t to enqueue on; NULL selects the null stream.
 *   max_features the match cap: when > 0, only the first max_features
 *                descriptors of each set take part (the rest are ignored,
 *                as if the sets were that long; output indices are
 *                unchanged).  The SERAC README ("Memory") describes
 *                lowering COLMAP's cap as clamping the lower-scale features
 *                away, i.e. features stored largest scale first are kept up
 *                to the cap.  0: no cap; negative is an error.  Output
 *                capacity is then needed for min(nA, max_features) rows.
 *   reserved     must be 0. */
typedef struct serac_params {
    double max_ratio;
    double max_distance;
    int32_t cross_check;
    int32_t flags;
    void *stream;
    int32_t max_features;
    int32_t reserved;
} serac_params;

/* Symmetric column gates (an option the pages name without defining it;
 * this is its plainest reading): column j must pass the same gates as row
 * i, on its own best and second-best score over all rows (lowest row on a
 * tie, second counted with multiplicity), and the two must be each other's
 * best:
 *   accept (i, j) iff row i passes, j = idx_i, col j passes, col_idx[j] == i.
 * It implies the cross-check (cross_check is then ignored).  The library
 * runs it as two sweeps, of (A, B) and of (B, A), without column bests: about
 * twice the work of one call.  serac_match_pair and serac_match_pairs take
 * it; serac_match_pair_noalloc refuses it (SERAC_ERR_INVALID_ARG). */
#define SERAC_FLAG_SYMMETRIC 1

/* One correspondence: row a of the first set, row b of the second. */
typedef struct serac_match {
    uint32_t a;
    uint32_t b;
} serac_match;

/* Output of one pair.  matches: device array of capacity entries, filled in
 * ascending order of a; count: device int32 receiving the number written,
 * or -1 if the device-side ordering hand-off between workgroups did not
 * complete (a bounded wait that only a malfunctioning device exhausts; the
 * match list is then invalid).  The bound is 2^22 polls; for tests, the
 * environment variable SERAC_LOOKBACK_SPIN_LIMIT read at the first call on
 * a device replaces it (-1: give up at once).  capacity must be at least nA,
 * or min(nA, max_features) under a match cap (each row yields at most one
 * match). */
typedef struct serac_matches {
    serac_match *matches;
    int64_t capacity;
    int32_t *count;
} serac_matches;

/* A pair of image indices into a batch. */
typedef struct serac_pair {
    int32_t a;
    int32_t b;
} serac_pair;

/*
 * Match one pair: descA [nA][128] against descB [nB][128] (device).
 * Implements the README's fused matcher (sections "What changed" and
 * "Exactness"): the ratio test on the best and second-best score of each
 * row, the optional max-distance gate and the optional mutual cross-check
 * against the best of each column.
 * nA or nB may be 0 (then *count is set to 0).  0 <= n <= SERAC_MAX_DESCRIPTORS.
 * Errors: SERAC_ERR_INVALID_ARG, SERAC_ERR_CAPACITY, SERAC_ERR_UNSUPPORTED_DEVICE,
 * SERAC_ERR_OUT_OF_MEMORY, SERAC_ERR_HIP.
 */
int serac_match_pair(const uint8_t *descA, int32_t nA, const uint8_t *descB,
                     int32_t nB, const serac_params *params,
                     const serac_matches *out_matches);

/*
 * The unfused arm, for comparison: the structure the SERAC README measures
 * its fused kernel against ("GPU kernel time", "Memory").  The score matrix
 * S is written to device memory (int32 [nA][nB]: the per-pair intermediate
 * the README removes), then read back by a row pass (row top-2) and a column
 * pass (column best); the finishing step is serac_match_pair's, so the list
 * is the same, byte for byte.  Same arguments and errors as serac_match_pair,
 * plus SERAC_ERR_TOO_LARGE above nA * nB = 2^32 (16 GiB of scores); the
 * workspace grows by 4 * nA * nB bytes.  SERAC_FLAG_SYMMETRIC is refused
 * (SERAC_ERR_INVALID_ARG); the match cap applies.
 */
int serac_match_pair_unfused(const uint8_t *descA, int32_t nA, const uint8_t *descB,
                             int32_t nB, const serac_params *params,
                             const serac_matches *out_matches);

/*
 * Release the current device's workspace for `stream` (device scratch and
 * pinned staging memory the library keeps per stream; NULL = the null
 * stream), e.g. before destroying a stream that will not be used again.
 * Device memory is freed in stream order behind the work already enqueued
 * on `stream`; the call waits for the copies out of the pinned staging
 * memory that are still pending.  A later call on the stream allocates a
 * new workspace.  No-op if the stream has none.  Must not overlap a call on
 * the same stream from another thread.
 * Errors: SERAC_ERR_HIP.
 */
int serac_release_stream(void *stream);

/*
 * Set up the current device for the library (architecture check, the angle
 * table, the fixed scratch of serac_match_pair_noalloc): the work every
 * other entry point does on its first call on a device, done now.  It
 * allocates device memory.  Idempotent; after a transient failure the next
 * call tries again.
 * Errors: SERAC_ERR_UNSUPPORTED_DEVICE, SERAC_ERR_OUT_OF_MEMORY, SERAC_ERR_HIP.
 */
int serac_init(void);

/*
 * serac_match_pair for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, semantics and results as serac_match_pair; it
 * makes no allocation and no free, and works in a fixed 4 MiB array of
 * device memory that the library holds on each device until the process
 * ends.  Each call leaves that array's accumulators zero again (a kernel at
 * its end clears them), so a captured call can be replayed.  The device must
 * have been set up first (serac_init, or any other entry point called on
 * it), else SERAC_ERR_NOT_INITIALIZED.
 * Limit: the single-kernel sweep (nA * nB <= 2^28) with a working set that
 * fits the array: every pair of sets of up to 16384 descriptors does; nB
 * above about 20000 does not.  Other pairs return SERAC_ERR_TOO_LARGE.
 * All calls on one device share its array: calls that overlap on one
 * device (two streams, or two threads on different streams) race and give
 * wrong results; calls on one stream run in order.
 * Errors: those of serac_match_pair, SERAC_ERR_TOO_LARGE,
 * SERAC_ERR_NOT_INITIALIZED.
 */
int serac_match_pair_noalloc(const uint8_t *descA, int32_t nA, const uint8_t *descB,
                             int32_t nB, const serac_params *params,
                             const serac_matches *out_matches);

/*
 * Match many pairs of one image set in one call, as exhaustive matching
 * over all image pairs does (README introduction: 589 images matched over
 * all 173,166 pairs).
 *   desc      host array [num_images] of device pointers to [n[k]][128]
 *   n         host array [num_images] of descriptor counts
 *   pairs     host array [num_pairs] of image index pairs (a, b)
 *   out_matches host array [num_pairs]; out_matches[p] receives pair p's
 *             matches (capacity >= n[pairs[p].a], or the cap if smaller).
 * Every pair gets exactly the result serac_match_pair would give it.
 * Pairs that share their first image may be swept together (cross-pair
 * reuse of that image's rows, used where the second images are small, up
 * to 2048 descriptors on average, and the batch is large enough to keep
 * the device busy); this changes no result, only the kernel that runs.
 * Asynchronous on params->stream like the other entry points: the host
 * arrays are read before the call returns (they may be released at once);
 * the library copies what the device needs through pinned memory of its
 * own, a ring of four buffers per stream.  A call blocks only when the
 * copy made by the batch call four calls earlier on the same stream has
 * not run yet.  Results are valid once the stream has synchronised.
 * Device scratch grows with the batch: about 16 bytes per column and 12
 * per row of each pair (about 230 KiB per 8192 x 8192 pair), plus ~132
 * bytes per descriptor and role (first or second image of a pair) of each
 * image used.  Very large pair lists are best
 * split, or given to serac_match_pairs_host, which runs them in stages.
 */
int serac_match_pairs(const uint8_t *const *desc, const int32_t *n,
                      int32_t num_images, const serac_pair *pairs,
                      int32_t num_pairs, const serac_params *params,
                      const serac_matches *out_matches);

/*
 * Match many pairs and deliver every match list to host memory, the way an
 * exhaustive matching stage consumes them (README "GPU kernel time": at stage level
 * much of the wall clock is host-side work around the kernels).  The pairs
 * run in stages of pairs_per_stage (0: 64) through serac_match_pairs on
 * params->stream; while the device matches stage s, stage s-1's lists are
 * copied to pinned host memory on a copy stream of the library's and the
 * host copies stage s-2's lists out to the caller's arrays.
 *   desc, n, num_images, pairs, num_pairs, params: as serac_match_pairs.
 *   host_matches host array [num_pairs] of host pointers; host_matches[p]
 *                receives pair p's matches, ascending a, and must hold
 *                n[pairs[p].a] entries (it may be NULL when that is 0).
 *   host_counts  host int32 [num_pairs]: each pair's count, or -1 where its
 *                device-side ordering hand-off failed (see serac_matches;
 *                that pair's list is then not written).
 * Synchronous: returns once every list is in host memory; the results are
 * identical to serac_match_pairs'.  Device memory for two stages' results
 * (at capacity) comes from the stream-ordered pool on params->stream;
 * pinned host memory for two stages is kept per device between calls.
 * Calls for one device are serialized by the library.
 * Errors: those of serac_match_pairs, plus SERAC_ERR_INVALID_ARG for
 * pairs_per_stage < 0 or missing host arrays.  Argument errors are found
 * before anything is enqueued.  A runtime error in a stage is returned once
 * the copies already enqueued have finished: the lists and counts of the
 * stages before it are written, host_counts of the rest is untouched.
 */
int serac_match_pairs_host(const uint8_t *const *desc, const int32_t *n,
                           int32_t num_images, const serac_pair *pairs,
                           int32_t num_pairs, const serac_params *params,
                           int32_t pairs_per_stage, serac_match *const *host_matches,
                           int32_t *host_counts);

/*
 * The reductions behind the match list, exported for inspection:
 *   row_top2 device int32 [nA][3] = (best, idx, second) per row of A
 *   col_best device int32 [nB][2] = (best, idx) per row of B
 * with the semantics in the header comment above.  Same ownership, stream
 * and error rules as serac_match_pair; nA or nB may be 0.
 */
int serac_top2_pair(const uint8_t *descA, int32_t nA, const uint8_t *descB,
                    int32_t nB, void *stream, int32_t *row_top2,
                    int32_t *col_best);

/* Human-readable text for a status code (static storage). */
const char *serac_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SERAC_H */

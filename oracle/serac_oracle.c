/*
 * Oracle: a plain, slow, CPU full-matrix matcher for 128-d uint8 SIFT
 * descriptors.  TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it; the matching library
 * never calls it, includes it or links it, and it shares no code with the
 * library.
 *
 * What it computes (the SERAC README, sections "What changed" and
 * "Exactness"):
 *
 *   S[i][j]  = sum_k A[i][k] * B[j][k], exact in 32-bit integers (each
 *              product of two bytes is at most 255^2; 128 of them stay below
 *              2^23, so no overflow is possible).
 *   per row  (best, idx, second), scanned over ascending j from the identity
 *            (0, -1, 0) with strictly-greater updates: a score of 0 never
 *            becomes best, the earliest (lowest) column keeps a top-1 tie,
 *            and a tie pushes the tied score into second, so second counts
 *            equal scores with multiplicity.
 *   per col  (best, idx) over ascending i from (0, -1), strictly greater:
 *            the column direction the README's matcher keeps with per-block
 *            partials, used for the mutual cross-check; ties go to the
 *            lowest row.
 *   gates    angle(s) = acos(min(s, 512^2) / 512^2): SIFT vectors have
 *            norm 512, so s / 512^2 is the cosine of the angle between them.
 *            A row i with idx >= 0 is accepted iff
 *              d1 <= max_distance  and  d1 < max_ratio * d2
 *              and (cross_check == 0 or colidx[idx] == i).
 *            The strict ratio test rejects every top-1 tie for max_ratio
 *            <= 1 (README, "Exactness": a tie makes second equal best).
 *   output   (i, idx) as two little-endian uint32 per accepted row, rows in
 *            ascending order; the README stores one correspondence blob per
 *            pair of about 8 bytes per correspondence.
 *   symmetric (an option the pages do not define; the plainest reading of
 *            "symmetric column gates"): the column side passes the same
 *            gates as the row side.  Column j's (best, idx, second) is its
 *            scan over ascending i with the row rules (ties to the lowest
 *            row, second with multiplicity), i.e. row j of the scores of the
 *            swapped pair (B, A).  Row i with idx = j >= 0 is accepted iff
 *            row i passes the gates, column j passes them on its own best
 *            and second, and column j's idx is i (the cross-check).
 *
 * Everything is in int32 / IEEE double with no fast-math and no FMA
 * contraction (built with -O2 -ffp-contract=off).  The scores are computed
 * block by block (RB rows at a time); blocking only bounds memory, every
 * scan still visits rows and columns in ascending order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DIM 128
#define RB 256
#define NORM2 262144   /* 512 * 512 */

static int32_t dot(const uint8_t *a, const uint8_t *b)
{
    int32_t s = 0;
    for (int k = 0; k < DIM; ++k)
        s += (int32_t)a[k] * (int32_t)b[k];
    return s;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The row scan of one row of S: identity (0, -1, 0), strictly greater. */
static void row_scan(const int32_t *srow, int32_t nB, int32_t *out3)
{
    int32_t best = 0, idx = -1, second = 0;
    for (int32_t j = 0; j < nB; ++j) {
        int32_t s = srow[j];
        if (s > best) {
            second = best;
            best = s;
            idx = j;
        } else if (s > second) {
            second = s;
        }
    }
    out3[0] = best;
    out3[1] = idx;
    out3[2] = second;
}

/*
 * row_top2 [nA][3] = (best, idx, second); col_best [nB][2] = (best, idx).
 * Either output may be NULL.  Returns 0, or -1 on bad arguments or
 * allocation failure.
 */
int oracle_top2(const uint8_t *A, int32_t nA, const uint8_t *B, int32_t nB,
                int32_t *row_top2, int32_t *col_best, int nthreads)
{
    if (nA < 0 || nB < 0 || (nA > 0 && !A) || (nB > 0 && !B))
        return -1;
    set_threads(nthreads);
    if (col_best)
        for (int32_t j = 0; j < nB; ++j) {
            col_best[2 * j] = 0;
            col_best[2 * j + 1] = -1;
        }
    if (row_top2)
        for (int32_t i = 0; i < nA; ++i) {
            row_top2[3 * i] = 0;
            row_top2[3 * i + 1] = -1;
            row_top2[3 * i + 2] = 0;
        }
    if (nA == 0 || nB == 0)
        return 0;

    int32_t *S = (int32_t *)malloc((size_t)RB * (size_t)nB * sizeof(int32_t));
    if (!S)
        return -1;
    for (int32_t i0 = 0; i0 < nA; i0 += RB) {
        int32_t rows = (nA - i0 < RB) ? nA - i0 : RB;
        /* the scores of this block of rows */
#pragma omp parallel for schedule(static)
        for (int32_t r = 0; r < rows; ++r) {
            const uint8_t *a = A + (size_t)(i0 + r) * DIM;
            int32_t *srow = S + (size_t)r * nB;
            for (int32_t j = 0; j < nB; ++j)
                srow[j] = dot(a, B + (size_t)j * DIM);
        }
        if (row_top2) {
#pragma omp parallel for schedule(static)
            for (int32_t r = 0; r < rows; ++r)
                row_scan(S + (size_t)r * nB, nB, row_top2 + 3 * (size_t)(i0 + r));
        }
        if (col_best) {
            /* blocks are visited in ascending row order, rows within a block
             * too, so the column scan sees rows in ascending order overall */
#pragma omp parallel for schedule(static)
            for (int32_t j = 0; j < nB; ++j) {
                int32_t best = col_best[2 * j], idx = col_best[2 * j + 1];
                for (int32_t r = 0; r < rows; ++r) {
                    int32_t s = S[(size_t)r * nB + j];
                    if (s > best) {
                        best = s;
                        idx = i0 + r;
                    }
                }
                col_best[2 * j] = best;
                col_best[2 * j + 1] = idx;
            }
        }
    }
    free(S);
    return 0;
}

/* Row top-2 for a chosen subset of rows (full rows of S, same scan). */
int oracle_rows(const uint8_t *A, int32_t nA, const uint8_t *B, int32_t nB,
                const int32_t *rows, int32_t nrows, int32_t *out3, int nthreads)
{
    if (nA < 0 || nB < 0 || nrows < 0)
        return -1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int32_t t = 0; t < nrows; ++t) {
        int32_t i = rows[t];
        if (i < 0 || i >= nA) {
            bad = 1;
            continue;
        }
        int32_t *srow = (int32_t *)malloc((size_t)(nB ? nB : 1) * sizeof(int32_t));
        if (!srow) {
            bad = 1;
            continue;
        }
        for (int32_t j = 0; j < nB; ++j)
            srow[j] = dot(A + (size_t)i * DIM, B + (size_t)j * DIM);
        row_scan(srow, nB, out3 + 3 * (size_t)t);
        free(srow);
    }
    return bad ? -1 : 0;
}

/* Column best for a chosen subset of columns (ascending rows, strict >). */
int oracle_cols(const uint8_t *A, int32_t nA, const uint8_t *B, int32_t nB,
                const int32_t *cols, int32_t ncols, int32_t *out2, int nthreads)
{
    if (nA < 0 || nB < 0 || ncols < 0)
        return -1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int32_t t = 0; t < ncols; ++t) {
        int32_t j = cols[t];
        if (j < 0 || j >= nB) {
            bad = 1;
            continue;
        }
        int32_t best = 0, idx = -1;
        for (int32_t i = 0; i < nA; ++i) {
            int32_t s = dot(A + (size_t)i * DIM, B + (size_t)j * DIM);
            if (s > best) {
                best = s;
                idx = i;
            }
        }
        out2[2 * (size_t)t] = best;
        out2[2 * (size_t)t + 1] = idx;
    }
    return bad ? -1 : 0;
}

/* The angle between two norm-512 descriptors with inner product s. */
double oracle_angle(int32_t s)
{
    double c = (s >= NORM2) ? 1.0 : (double)s / (double)NORM2;
    return acos(c);
}

/* The acceptance test of one row, given its top-2 and its best column's
 * best row (colidx_of_best; ignored when cross_check is 0). */
int oracle_accept(int32_t i, int32_t best, int32_t idx, int32_t second,
                  int32_t colidx_of_best, double max_ratio,
                  double max_distance, int32_t cross_check)
{
    if (idx < 0)
        return 0;
    double d1 = oracle_angle(best);
    double d2 = oracle_angle(second);
    if (!(d1 <= max_distance))
        return 0;
    if (!(d1 < max_ratio * d2))
        return 0;
    if (cross_check && colidx_of_best != i)
        return 0;
    return 1;
}

/*
 * The matcher with symmetric column gates (header: "symmetric").  The
 * column top-2 is the row top-2 of the swapped pair: S(B, A)[j][i] =
 * S(A, B)[i][j], scanned over ascending i.  out_pairs has room for nA
 * pairs; *count receives the number written.  Returns 0 or -1.
 */
int oracle_match_pair_sym(const uint8_t *A, int32_t nA, const uint8_t *B,
                          int32_t nB, double max_ratio, double max_distance,
                          uint32_t *out_pairs, int32_t *count, int nthreads)
{
    if (!count || nA < 0 || nB < 0 || (nA > 0 && !out_pairs))
        return -1;
    *count = 0;
    if (nA == 0 || nB == 0)
        return 0;
    int32_t *row = (int32_t *)malloc((size_t)nA * 3 * sizeof(int32_t));
    int32_t *col = (int32_t *)malloc((size_t)nB * 3 * sizeof(int32_t));
    if (!row || !col) {
        free(row);
        free(col);
        return -1;
    }
    int rc = oracle_top2(A, nA, B, nB, row, NULL, nthreads);
    if (rc == 0)
        rc = oracle_top2(B, nB, A, nA, col, NULL, nthreads);
    if (rc == 0) {
        int32_t n = 0;
        for (int32_t i = 0; i < nA; ++i) {
            int32_t best = row[3 * i], j = row[3 * i + 1], second = row[3 * i + 2];
            if (!oracle_accept(i, best, j, second, -1, max_ratio, max_distance, 0))
                continue;
            /* column j: its own best row, best score and second */
            int32_t cbest = col[3 * j], ci = col[3 * j + 1], csecond = col[3 * j + 2];
            if (ci != i)
                continue;
            if (!oracle_accept(j, cbest, ci, csecond, -1, max_ratio, max_distance, 0))
                continue;
            out_pairs[2 * n] = (uint32_t)i;
            out_pairs[2 * n + 1] = (uint32_t)j;
            ++n;
        }
        *count = n;
    }
    free(row);
    free(col);
    return rc;
}

/*
 * The whole matcher for one pair.  out_pairs has room for nA (a, b) uint32
 * pairs; *count receives the number written.  Returns 0 or -1.
 */
int oracle_match_pair(const uint8_t *A, int32_t nA, const uint8_t *B,
                      int32_t nB, double max_ratio, double max_distance,
                      int32_t cross_check, uint32_t *out_pairs,
                      int32_t *count, int nthreads)
{
    if (!count || nA < 0 || nB < 0 || (nA > 0 && !out_pairs))
        return -1;
    *count = 0;
    if (nA == 0 || nB == 0)
        return 0;
    int32_t *row = (int32_t *)malloc((size_t)nA * 3 * sizeof(int32_t));
    int32_t *col = (int32_t *)malloc((size_t)nB * 2 * sizeof(int32_t));
    if (!row || !col) {
        free(row);
        free(col);
        return -1;
    }
    int rc = oracle_top2(A, nA, B, nB, row, col, nthreads);
    if (rc == 0) {
        int32_t n = 0;
        for (int32_t i = 0; i < nA; ++i) {
            int32_t best = row[3 * i], idx = row[3 * i + 1], second = row[3 * i + 2];
            int32_t cidx = (idx >= 0) ? col[2 * idx + 1] : -1;
            if (oracle_accept(i, best, idx, second, cidx, max_ratio,
                              max_distance, cross_check)) {
                out_pairs[2 * n] = (uint32_t)i;
                out_pairs[2 * n + 1] = (uint32_t)idx;
                ++n;
            }
        }
        *count = n;
    }
    free(row);
    free(col);
    return rc;
}

// serac.hip - fused brute-force SIFT descriptor matcher for MI355X (gfx950).
//
// What is computed (SERAC README, introduction and the sections "What
// changed" and "Exactness"): for descriptor sets A [nA][128] and B [nB][128]
// of unsigned bytes, the exact inner products S[i][j] = sum_k A[i][k]*B[j][k],
// reduced on the fly, without ever storing S, to
//   * per row of A: the best score, its column (lowest on a tie) and the
//     second-best score (ties counted), from the identity (0, -1, 0);
//   * per row of B ("column"): the best score and its row (lowest on a tie);
// then the ratio test, the max-distance gate and the mutual cross-check, and
// an ordered match list.
//
// How it maps to gfx950:
//   * The contraction runs on v_mfma_i32_16x16x64_i8.  The MFMA is signed,
//     so bytes enter as a' = a ^ 0x80 = a - 128 (exact) and the product is
//     corrected with per-descriptor byte sums:
//       S = sum a'b' + 128*SA_i + 128*SB_j - 2^21,
//     every term exact in int32 (|sum a'b'| <= 2^21, S < 2^23).
//     The row term 128*SA_i - 2^21 enters through the MFMA accumulator input,
//     so it costs no vector instruction.
//   * A wave keeps the operand fragments of 64 rows of A in registers and
//     sweeps 16-column tiles of B staged in LDS (512 columns per chunk).
//     Each score becomes one packed 32-bit key
//       key = (S << 9) | (511 - local column),
//     in one v_lshl_add (the column term 128*SB_j is folded into the addend),
//     and a key comparison orders by score, then by lowest column.  Scores
//     stay below 2^23, so the key is exact.
//   * Row top-2: per lane and row, max3/med3 over two new keys at a time.
//     Keys are unique per column, so a tie on score leaves the tied score in
//     second place (multiplicity) and the lowest column in first.
//   * Column best: a max3 tree over the 16 rows a lane holds in one tile
//     gives the column maximum of those rows; the key's low 9 bits are then
//     replaced by the 16-row slice number (lowest slice wins) and merged with
//     an LDS atomic max.  The exact lowest row inside the winning slice is
//     settled afterwards from the 15 rows that precede it (rarely more than
//     a filter check).
//   * All merges (across lanes, waves, chunks, workgroups) compare packed
//     keys or scan in ascending index order, so the result does not depend
//     on scheduling (MASDA part 3, section 6: an order-independent key).
//   * The angle gate reads a table of acos(s / 512^2) built on the host with
//     the C library's acos, so the double-precision decision is the same
//     one a CPU makes; the ratio test is one IEEE multiply and compare.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "serac.h"

namespace {

constexpr int DIM = 128;
constexpr int THREADS = 256;            // 4 waves of 64
constexpr int ROWS_PER_WAVE = 64;
constexpr int ROWS_PER_BLOCK = 256;     // rows of A per workgroup pass
constexpr int CHUNK = 512;              // columns of B per LDS chunk (9-bit index)
constexpr int TILES = CHUNK / 16;       // 16-column tiles per chunk
constexpr int MAX_CC_PER_WG = 4;        // chunks one workgroup sweeps
constexpr int MAX_RB_PER_WG = 32;       // 32 blocks * 16 slices = 512 slice ids
constexpr int NORM2 = 262144;           // 512^2
constexpr int FIN_THREADS = 256;
constexpr int MAX_FIN = SERAC_MAX_DESCRIPTORS / FIN_THREADS;

typedef int v4i __attribute__((ext_vector_type(4)));

// One pair's work description and workspace.
struct Job {
    const uint8_t *A;
    const uint8_t *B;
    int32_t nA, nB;
    int32_t nRB, nCC;        // row blocks of 256, column chunks of 512
    int32_t rbPer, ccPer;    // per workgroup
    int32_t Gr, Gc;          // workgroup grid (row groups x column groups)
    int32_t nFin;            // finishing workgroups (256 rows each)
    int32_t pad;
    int4 *rowpart;           // [Gc][nA]   (best, idx, second, 0) per column group
    uint32_t *colpart;       // [Gr][nB]   (best << 9) | (511 - slice)
    uint2 *staging;          // [nFin][256] accepted (a, b) per finishing group
    int32_t *wgcount;        // [nFin]
    uint32_t *ticket;        // 1
    serac_match *out;        // [>= nA]
    int32_t *count;          // 1
};

struct Gate {
    const double *table;     // acos(min(s, 512^2) / 512^2), s = 0 .. 512^2
    double max_ratio;
    double max_distance;
    int32_t cross_check;
};

__device__ __forceinline__ uint32_t umax3(uint32_t a, uint32_t b, uint32_t c)
{
    return max(max(a, b), c);
}

// Median of three, as the single VALU instruction (the compiler otherwise
// expands it into a min/max chain of four).
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c)
{
    uint32_t r;
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ uint32_t bytesum16(uint4 v)
{
    uint32_t s = __builtin_amdgcn_udot4(v.x, 0x01010101u, 0u, false);
    s = __builtin_amdgcn_udot4(v.y, 0x01010101u, s, false);
    s = __builtin_amdgcn_udot4(v.z, 0x01010101u, s, false);
    return __builtin_amdgcn_udot4(v.w, 0x01010101u, s, false);
}

__device__ __forceinline__ v4i to_i8(uint4 v)
{
    v4i r;
    r[0] = (int)(v.x ^ 0x80808080u);
    r[1] = (int)(v.y ^ 0x80808080u);
    r[2] = (int)(v.z ^ 0x80808080u);
    r[3] = (int)(v.w ^ 0x80808080u);
    return r;
}

// Byte offset of 16-byte part `part` of column `col` in the LDS chunk.  The
// XOR spreads eight consecutive columns over distinct bank groups.
__device__ __forceinline__ int lds_off(int col, int part)
{
    return col * DIM + ((part ^ (col & 7)) << 4);
}

// Stage columns [cbase, cbase + 512) of B into LDS as int8 (a ^ 0x80), and
// for each column the key addend P = ((128 * SB) << 9) + (511 - col).
__device__ __forceinline__ void stage_chunk(const uint8_t *__restrict__ B, int nB,
                                            int cbase, uint8_t *sB, uint32_t *sP,
                                            int tid)
{
    constexpr int PARTS = CHUNK * DIM / 16 / THREADS;   // 16 per thread
    uint4 v[PARTS];
#pragma unroll
    for (int q = 0; q < PARTS; ++q) {
        const int e = q * THREADS + tid;
        const int col = e >> 3, part = e & 7;
        const int gcol = cbase + col;
        v[q] = make_uint4(0u, 0u, 0u, 0u);
        if (gcol < nB)
            v[q] = *reinterpret_cast<const uint4 *>(B + (size_t)gcol * DIM + part * 16);
    }
#pragma unroll
    for (int q = 0; q < PARTS; ++q) {
        const int e = q * THREADS + tid;
        const int col = e >> 3, part = e & 7;
        uint32_t s = bytesum16(v[q]);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        if (part == 0)
            sP[col] = ((s * 128u) << 9) + (uint32_t)(511 - col);
        v4i x = to_i8(v[q]);
        *reinterpret_cast<v4i *>(sB + lds_off(col, part)) = x;
    }
}

// The fused tile sweep of one workgroup: row groups [rb0, rb1) of 256 rows
// by column chunks [cc0, cc1) of 512 columns.
template <bool COLS>
__device__ __forceinline__ void tiles_body(const Job &J, int wgi)
{
    __shared__ __attribute__((aligned(16))) uint8_t sB[CHUNK * DIM];   // 64 KiB
    __shared__ uint32_t sP[CHUNK];
    __shared__ uint32_t sCol[COLS ? MAX_CC_PER_WG * CHUNK : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r = wgi % J.Gr, c = wgi / J.Gr;
    const int rb0 = r * J.rbPer, rb1 = min(rb0 + J.rbPer, J.nRB);
    const int cc0 = c * J.ccPer, cc1 = min(cc0 + J.ccPer, J.nCC);
    if (rb0 >= rb1 || cc0 >= cc1)
        return;
    const int nA = J.nA, nB = J.nB;

    if (wgi == 0 && tid == 0)
        *J.ticket = 0u;   // the finishing kernel's arrival counter
    if (COLS) {
        for (int k = tid; k < (cc1 - cc0) * CHUNK; k += THREADS)
            sCol[k] = 0u;
    }

    for (int rb = rb0; rb < rb1; ++rb) {
        // ---- this wave's 64 rows of A: operand fragments and the row term
        // The MFMA row m = 4*grp + reg of tile rt holds wave row
        // 16*grp + 4*rt + reg, so lane group grp of the accumulator covers
        // the 16 consecutive rows [16*grp, 16*grp + 16).
        v4i af[4][2];
        v4i ci[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int q = 16 * (n >> 2) + 4 * rt + (n & 3);
            const int row = rb * ROWS_PER_BLOCK + w * ROWS_PER_WAVE + q;
            uint4 x0 = make_uint4(0u, 0u, 0u, 0u), x1 = x0;
            if (row < nA) {
                const uint8_t *a = J.A + (size_t)row * DIM;
                x0 = *reinterpret_cast<const uint4 *>(a + g * 16);
                x1 = *reinterpret_cast<const uint4 *>(a + 64 + g * 16);
            }
            uint32_t s = bytesum16(x0) + bytesum16(x1);
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            af[rt][0] = to_i8(x0);
            af[rt][1] = to_i8(x1);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                ci[rt][rr] = (int)(128u * (uint32_t)__shfl((int)s, 4 * g + rr)) - 2097152;
        }

        // running (best, idx, second) of wave row `lane` over the chunks
        uint32_t S1 = 0u, S2 = 0u;
        int32_t I1 = -1;
        const int slice = (rb - rb0) * 16 + w * 4 + g;

        for (int cc = cc0; cc < cc1; ++cc) {
            __syncthreads();                 // sB / sP free
            stage_chunk(J.B, nB, cc * CHUNK, sB, sP, tid);
            __syncthreads();

            uint32_t b1[16], b2[16];
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                b1[x] = 0u;
                b2[x] = 0u;
            }
            uint32_t *colbase = sCol + (COLS ? (cc - cc0) * CHUNK : 0);

            for (int u = 0; u < TILES; u += 2) {
                const int col0 = u * 16 + n, col1 = col0 + 16;
                const v4i bf00 = *reinterpret_cast<const v4i *>(sB + lds_off(col0, g));
                const v4i bf01 = *reinterpret_cast<const v4i *>(sB + lds_off(col0, 4 + g));
                const v4i bf10 = *reinterpret_cast<const v4i *>(sB + lds_off(col1, g));
                const v4i bf11 = *reinterpret_cast<const v4i *>(sB + lds_off(col1, 4 + g));
                const uint32_t P0 = sP[col0], P1 = sP[col1];
                v4i acc0[4], acc1[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    acc0[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[rt][0], bf00, ci[rt], 0, 0, 0);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    acc1[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[rt][0], bf10, ci[rt], 0, 0, 0);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    acc0[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[rt][1], bf01, acc0[rt], 0, 0, 0);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    acc1[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[rt][1], bf11, acc1[rt], 0, 0, 0);

                uint32_t cm0 = 0u, cm1 = 0u;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int x = rt * 4 + rr;
                        const uint32_t k0 = ((uint32_t)acc0[rt][rr] << 9) + P0;
                        const uint32_t k1 = ((uint32_t)acc1[rt][rr] << 9) + P1;
                        const uint32_t md = umed3(b1[x], k0, k1);
                        b1[x] = umax3(b1[x], k0, k1);
                        b2[x] = max(b2[x], md);
                        if (COLS) {
                            cm0 = max(cm0, k0);
                            cm1 = max(cm1, k1);
                        }
                    }
                }
                if (COLS) {
                    const uint32_t tag = (uint32_t)(511 - slice);
                    atomicMax(colbase + col0, (cm0 & ~511u) | tag);
                    atomicMax(colbase + col1, (cm1 & ~511u) | tag);
                }
            }

            // ---- merge the 16 lanes that share each row (via LDS)
            __syncthreads();                 // everyone done with sB
            uint2 *scr = reinterpret_cast<uint2 *>(sB) + w * (ROWS_PER_WAVE * 16);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int q = 16 * g + 4 * rt + rr;
                    scr[q * 16 + ((n + q) & 15)] = make_uint2(b1[rt * 4 + rr], b2[rt * 4 + rr]);
                }
            }
            __syncthreads();
            uint32_t K1 = 0u, K2 = 0u;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint2 e = scr[lane * 16 + ((k + lane) & 15)];
                const uint32_t lo = min(K1, e.x);
                K1 = max(K1, e.x);
                K2 = umax3(lo, K2, e.y);
            }
            const uint32_t s1 = K1 >> 9, s2 = K2 >> 9;
            const uint32_t lo = min(S1, s1);
            S2 = umax3(lo, S2, s2);
            if (s1 > S1) {
                S1 = s1;
                I1 = cc * CHUNK + 511 - (int)(K1 & 511u);
            }
        }

        const int row = rb * ROWS_PER_BLOCK + w * ROWS_PER_WAVE + lane;
        if (row < nA)
            J.rowpart[(size_t)c * nA + row] = make_int4((int)S1, I1, (int)S2, 0);
    }

    if (COLS) {
        __syncthreads();
        const int base = cc0 * CHUNK;
        for (int k = tid; k < (cc1 - cc0) * CHUNK; k += THREADS) {
            const int col = base + k;
            if (col < nB)
                J.colpart[(size_t)r * nB + col] = sCol[k];
        }
    }
}

template <bool COLS>
__global__ __launch_bounds__(THREADS, 2) void serac_tiles_one(Job J)
{
    tiles_body<COLS>(J, blockIdx.x);
}

template <bool COLS>
__global__ __launch_bounds__(THREADS, 2) void serac_tiles_many(const Job *__restrict__ jobs,
                                                               int wgPerJob)
{
    const Job J = jobs[blockIdx.x / wgPerJob];
    const int wgi = blockIdx.x % wgPerJob;
    if (wgi >= J.Gr * J.Gc)
        return;
    tiles_body<COLS>(J, wgi);
}

// Exact inner product of two descriptors (used only to settle column ties
// inside one 16-row slice).
__device__ int32_t dot_exact(const uint8_t *a, const uint8_t *b)
{
    uint32_t s = 0u;
    for (int k = 0; k < DIM; k += 16) {
        const uint4 x = *reinterpret_cast<const uint4 *>(a + k);
        const uint4 y = *reinterpret_cast<const uint4 *>(b + k);
        // unsigned bytes: exact byte-wise products summed in 32 bits
        s = __builtin_amdgcn_udot4(x.x, y.x, s, false);
        s = __builtin_amdgcn_udot4(x.y, y.y, s, false);
        s = __builtin_amdgcn_udot4(x.z, y.z, s, false);
        s = __builtin_amdgcn_udot4(x.w, y.w, s, false);
    }
    return (int32_t)s;
}

// Merge the column-group partials of row i (ascending column groups, so a
// strictly greater score is needed to move the index: lowest column wins).
__device__ __forceinline__ void merge_row(const Job &J, int i, uint32_t &S1, int32_t &I1,
                                          uint32_t &S2)
{
    S1 = 0u;
    S2 = 0u;
    I1 = -1;
    for (int c = 0; c < J.Gc; ++c) {
        const int4 p = J.rowpart[(size_t)c * J.nA + i];
        const uint32_t s1 = (uint32_t)p.x, s2 = (uint32_t)p.z;
        const uint32_t lo = min(S1, s1);
        S2 = umax3(lo, S2, s2);
        if (s1 > S1) {
            S1 = s1;
            I1 = p.y;
        }
    }
}

// Best score of column j and the first 16-row slice reaching it.
__device__ __forceinline__ void merge_col(const Job &J, int j, uint32_t &C1, int32_t &slice)
{
    C1 = 0u;
    slice = -1;
    for (int r = 0; r < J.Gr; ++r) {
        const uint32_t key = J.colpart[(size_t)r * J.nB + j];
        const uint32_t s = key >> 9;
        if (s > C1) {
            C1 = s;
            slice = r * J.rbPer * 16 + 511 - (int)(key & 511u);
        }
    }
}

// Gates, cross-check and ordered compaction of one group of 256 rows; the
// last group to arrive concatenates all groups' matches in row order.
__device__ __forceinline__ void finish_body(const Job &J, int wg, const Gate &G)
{
    __shared__ uint32_t sS1[FIN_THREADS];
    __shared__ int32_t sWave[FIN_THREADS / 64];
    __shared__ int32_t sOff[MAX_FIN + 1];
    __shared__ int32_t sLast;

    const int tid = threadIdx.x;
    const int i = wg * FIN_THREADS + tid;
    uint32_t S1 = 0u, S2 = 0u;
    int32_t I1 = -1;
    if (i < J.nA)
        merge_row(J, i, S1, I1, S2);
    sS1[tid] = S1;
    __syncthreads();

    bool acc = false;
    if (i < J.nA && I1 >= 0 && I1 < J.nB) {
        const double d1 = G.table[min(S1, (uint32_t)NORM2)];
        const double d2 = G.table[min(S2, (uint32_t)NORM2)];
        acc = (d1 <= G.max_distance) && (d1 < G.max_ratio * d2);
        if (acc && G.cross_check) {
            uint32_t C1;
            int32_t slice;
            merge_col(J, I1, C1, slice);
            if (C1 != S1 || slice != (i >> 4)) {
                acc = false;
            } else {
                // a lower row of the same slice reaching the same score wins
                const uint8_t *b = J.B + (size_t)I1 * DIM;
                for (int i2 = i & ~15; i2 < i; ++i2) {
                    if (sS1[i2 - wg * FIN_THREADS] >= C1 &&
                        (uint32_t)dot_exact(J.A + (size_t)i2 * DIM, b) == C1) {
                        acc = false;
                        break;
                    }
                }
            }
        }
    }

    // ordered compaction within the group
    const int lane = tid & 63, wv = tid >> 6;
    const uint64_t mask = __ballot(acc);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0)
        sWave[wv] = __popcll(mask);
    __syncthreads();
    int base = 0, total = 0;
    for (int k = 0; k < FIN_THREADS / 64; ++k) {
        base += (k < wv) ? sWave[k] : 0;
        total += sWave[k];
    }
    if (acc)
        J.staging[(size_t)wg * FIN_THREADS + base + before] = make_uint2((uint32_t)i, (uint32_t)I1);
    if (tid == 0)
        J.wgcount[wg] = total;

    // arrival; the last group concatenates
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t t = atomicAdd(J.ticket, 1u);
        sLast = (t == (uint32_t)(J.nFin - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!sLast)
        return;
    __threadfence();
    if (tid == 0) {
        int run = 0;
        for (int k = 0; k < J.nFin; ++k) {
            sOff[k] = run;
            run += __hip_atomic_load(J.wgcount + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        sOff[J.nFin] = run;
    }
    __syncthreads();
    const int all = sOff[J.nFin];
    for (int p = tid; p < all; p += FIN_THREADS) {
        // group holding output position p: last k with sOff[k] <= p
        int lo = 0, hi = J.nFin - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sOff[mid] <= p)
                lo = mid;
            else
                hi = mid - 1;
        }
        const uint2 m = J.staging[(size_t)lo * FIN_THREADS + (p - sOff[lo])];
        J.out[p].a = m.x;
        J.out[p].b = m.y;
    }
    if (tid == 0) {
        *J.count = all;
        *J.ticket = 0u;
    }
}

__global__ __launch_bounds__(FIN_THREADS) void serac_finish_one(Job J, Gate G)
{
    finish_body(J, blockIdx.x, G);
}

__global__ __launch_bounds__(FIN_THREADS) void serac_finish_many(const Job *__restrict__ jobs,
                                                                 int finPerJob, Gate G)
{
    const Job J = jobs[blockIdx.x / finPerJob];
    const int wg = blockIdx.x % finPerJob;
    if (wg >= J.nFin)
        return;
    finish_body(J, wg, G);
}

__global__ void serac_zero_counts(int32_t *const *counts, int32_t *count, int n)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (counts) {
        if (t < n)
            *counts[t] = 0;
    } else if (t == 0) {
        *count = 0;
    }
}

// Export of the row reduction: row_top2[i] = (best, idx, second).
__global__ void serac_export_rows(Job J, int32_t *row_top2, uint32_t *s1_out)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= J.nA)
        return;
    uint32_t S1, S2;
    int32_t I1;
    merge_row(J, i, S1, I1, S2);
    row_top2[3 * (size_t)i] = (int32_t)S1;
    row_top2[3 * (size_t)i + 1] = I1;
    row_top2[3 * (size_t)i + 2] = (int32_t)S2;
    s1_out[i] = S1;
}

// Export of the column reduction: col_best[j] = (best, lowest row).  The
// winning 16-row slice is known; its first row reaching the best score is
// found among the rows whose own best is at least that score.
__global__ void serac_export_cols(Job J, const uint32_t *s1, int32_t *col_best)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= J.nB)
        return;
    uint32_t C1;
    int32_t slice;
    merge_col(J, j, C1, slice);
    int32_t idx = -1;
    if (C1 > 0u) {
        const uint8_t *b = J.B + (size_t)j * DIM;
        for (int i = slice * 16; i < min(slice * 16 + 16, J.nA); ++i) {
            if (s1[i] >= C1 && (uint32_t)dot_exact(J.A + (size_t)i * DIM, b) == C1) {
                idx = i;
                break;
            }
        }
    }
    col_best[2 * (size_t)j] = (int32_t)C1;
    col_best[2 * (size_t)j + 1] = idx;
}

// ------------------------------------------------------------------ host

struct Device {
    bool init = false;
    int status = SERAC_OK;
    int cus = 0;
    double *table = nullptr;
};

std::mutex g_mutex;
Device g_devices[64];

int hip_fail()
{
    (void)hipGetLastError();
    return SERAC_ERR_HIP;
}

// Per-device set-up: architecture check, acos table, pool threshold.
int device_setup(Device **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return hip_fail();
    if (dev < 0 || dev >= 64)
        return SERAC_ERR_UNSUPPORTED_DEVICE;
    std::lock_guard<std::mutex> lock(g_mutex);
    Device &d = g_devices[dev];
    if (!d.init) {
        d.init = true;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            d.status = hip_fail();
            return d.status;
        }
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            d.status = SERAC_ERR_UNSUPPORTED_DEVICE;
            return d.status;
        }
        d.cus = prop.multiProcessorCount;
        // angle of every attainable clamped score, with the C library's acos
        std::vector<double> t(NORM2 + 1);
        for (int s = 0; s <= NORM2; ++s)
            t[s] = std::acos(s >= NORM2 ? 1.0 : (double)s / (double)NORM2);
        if (hipMalloc(&d.table, t.size() * sizeof(double)) != hipSuccess) {
            d.status = SERAC_ERR_OUT_OF_MEMORY;
            (void)hipGetLastError();
            return d.status;
        }
        if (hipMemcpy(d.table, t.data(), t.size() * sizeof(double), hipMemcpyHostToDevice) !=
            hipSuccess) {
            d.status = hip_fail();
            return d.status;
        }
        hipMemPool_t pool;
        if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
            uint64_t keep = UINT64_MAX;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        }
        (void)hipGetLastError();
        d.status = SERAC_OK;
    }
    *out = &d;
    return d.status;
}

struct Plan {
    int nRB, nCC, rbPer, ccPer, Gr, Gc, nFin;
    size_t rowpart, colpart, staging, wgcount;   // bytes
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Choose how many 256 x 512 sub-tiles each workgroup sweeps so that about
// `target` workgroups cover the pair.
Plan make_plan(int nA, int nB, int target)
{
    Plan p;
    p.nRB = (nA + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    p.nCC = (nB + CHUNK - 1) / CHUNK;
    p.rbPer = 1;
    p.ccPer = 1;
    auto groups = [&](int rb, int cc) {
        return (long long)((p.nRB + rb - 1) / rb) * ((p.nCC + cc - 1) / cc);
    };
    while (groups(p.rbPer, p.ccPer) > target) {
        const bool can_c = p.ccPer < MAX_CC_PER_WG && p.ccPer < p.nCC;
        const bool can_r = p.rbPer < MAX_RB_PER_WG && p.rbPer < p.nRB;
        if (can_c && (p.ccPer <= p.rbPer || !can_r))
            ++p.ccPer;
        else if (can_r)
            ++p.rbPer;
        else
            break;
    }
    p.Gr = (p.nRB + p.rbPer - 1) / p.rbPer;
    p.Gc = (p.nCC + p.ccPer - 1) / p.ccPer;
    p.nFin = (nA + FIN_THREADS - 1) / FIN_THREADS;
    p.rowpart = align256((size_t)p.Gc * nA * sizeof(int4));
    p.colpart = align256((size_t)p.Gr * nB * sizeof(uint32_t));
    p.staging = align256((size_t)p.nFin * FIN_THREADS * sizeof(uint2));
    p.wgcount = align256((size_t)p.nFin * sizeof(int32_t) + 64);   // + ticket
    return p;
}

size_t plan_bytes(const Plan &p)
{
    return p.rowpart + p.colpart + p.staging + p.wgcount;
}

void fill_job(Job &J, const Plan &p, const uint8_t *A, int nA, const uint8_t *B, int nB,
              uint8_t *ws, serac_match *out, int32_t *count)
{
    J.A = A;
    J.B = B;
    J.nA = nA;
    J.nB = nB;
    J.nRB = p.nRB;
    J.nCC = p.nCC;
    J.rbPer = p.rbPer;
    J.ccPer = p.ccPer;
    J.Gr = p.Gr;
    J.Gc = p.Gc;
    J.nFin = p.nFin;
    J.pad = 0;
    uint8_t *q = ws;
    J.rowpart = reinterpret_cast<int4 *>(q);
    q += p.rowpart;
    J.colpart = reinterpret_cast<uint32_t *>(q);
    q += p.colpart;
    J.staging = reinterpret_cast<uint2 *>(q);
    q += p.staging;
    J.wgcount = reinterpret_cast<int32_t *>(q);
    J.ticket = reinterpret_cast<uint32_t *>(q + p.wgcount - 64);
    J.out = out;
    J.count = count;
}

bool bad_params(const serac_params *p)
{
    if (!p)
        return true;
    if (!std::isfinite(p->max_ratio) || !(p->max_ratio > 0.0))
        return true;
    if (std::isnan(p->max_distance) || p->max_distance < 0.0)
        return true;
    if (p->cross_check != 0 && p->cross_check != 1)
        return true;
    return p->flags != 0;
}

bool bad_set(const uint8_t *d, int32_t n)
{
    return n < 0 || n > SERAC_MAX_DESCRIPTORS || (n > 0 && d == nullptr);
}

Gate make_gate(const Device *d, const serac_params *p)
{
    Gate G;
    G.table = d->table;
    G.max_ratio = p->max_ratio;
    G.max_distance = p->max_distance;
    G.cross_check = p->cross_check;
    return G;
}

}  // namespace

extern "C" {

const char *serac_status_string(int status)
{
    switch (status) {
    case SERAC_OK:
        return "ok";
    case SERAC_ERR_INVALID_ARG:
        return "invalid argument";
    case SERAC_ERR_CAPACITY:
        return "output capacity smaller than the number of query descriptors";
    case SERAC_ERR_UNSUPPORTED_DEVICE:
        return "unsupported device (gfx950 required)";
    case SERAC_ERR_OUT_OF_MEMORY:
        return "device memory allocation failed";
    case SERAC_ERR_HIP:
        return "HIP runtime error";
    default:
        return "unknown status";
    }
}

int serac_match_pair(const uint8_t *descA, int32_t nA, const uint8_t *descB, int32_t nB,
                     const serac_params *params, const serac_matches *out)
{
    if (bad_set(descA, nA) || bad_set(descB, nB) || bad_params(params) || !out ||
        !out->count || (nA > 0 && !out->matches))
        return SERAC_ERR_INVALID_ARG;
    if (out->capacity < nA)
        return SERAC_ERR_CAPACITY;
    Device *d = nullptr;
    int st = device_setup(&d);
    if (st != SERAC_OK)
        return st;
    hipStream_t stream = static_cast<hipStream_t>(params->stream);
    if (nA == 0 || nB == 0) {
        serac_zero_counts<<<1, 64, 0, stream>>>(nullptr, out->count, 1);
        return hipGetLastError() == hipSuccess ? SERAC_OK : SERAC_ERR_HIP;
    }
    const Plan p = make_plan(nA, nB, 2 * d->cus);
    uint8_t *ws = nullptr;
    if (hipMallocAsync(reinterpret_cast<void **>(&ws), plan_bytes(p), stream) != hipSuccess) {
        (void)hipGetLastError();
        return SERAC_ERR_OUT_OF_MEMORY;
    }
    Job J;
    fill_job(J, p, descA, nA, descB, nB, ws, out->matches, out->count);
    const Gate G = make_gate(d, params);
    if (params->cross_check)
        serac_tiles_one<true><<<p.Gr * p.Gc, THREADS, 0, stream>>>(J);
    else
        serac_tiles_one<false><<<p.Gr * p.Gc, THREADS, 0, stream>>>(J);
    serac_finish_one<<<p.nFin, FIN_THREADS, 0, stream>>>(J, G);
    const hipError_t e = hipGetLastError();
    (void)hipFreeAsync(ws, stream);
    return e == hipSuccess ? SERAC_OK : SERAC_ERR_HIP;
}

int serac_match_pairs(const uint8_t *const *desc, const int32_t *n, int32_t num_images,
                      const serac_pair *pairs, int32_t num_pairs, const serac_params *params,
                      const serac_matches *out)
{
    if (num_images < 0 || num_pairs < 0 || bad_params(params))
        return SERAC_ERR_INVALID_ARG;
    if (num_pairs == 0)
        return SERAC_OK;
    if (!desc || !n || !pairs || !out)
        return SERAC_ERR_INVALID_ARG;
    for (int k = 0; k < num_images; ++k)
        if (bad_set(desc[k], n[k]))
            return SERAC_ERR_INVALID_ARG;
    for (int q = 0; q < num_pairs; ++q) {
        const serac_pair pr = pairs[q];
        if (pr.a < 0 || pr.a >= num_images || pr.b < 0 || pr.b >= num_images)
            return SERAC_ERR_INVALID_ARG;
        if (!out[q].count || (n[pr.a] > 0 && !out[q].matches))
            return SERAC_ERR_INVALID_ARG;
        if (out[q].capacity < n[pr.a])
            return SERAC_ERR_CAPACITY;
    }
    Device *d = nullptr;
    int st = device_setup(&d);
    if (st != SERAC_OK)
        return st;
    hipStream_t stream = static_cast<hipStream_t>(params->stream);

    // pairs with an empty side only get a zero count
    std::vector<int32_t *> zero;
    std::vector<int> live;
    for (int q = 0; q < num_pairs; ++q) {
        if (n[pairs[q].a] == 0 || n[pairs[q].b] == 0)
            zero.push_back(out[q].count);
        else
            live.push_back(q);
    }
    // workgroups per pair: enough to fill the device a few times over
    const int nlive = (int)live.size();
    const int target = nlive ? std::max(1, (8 * d->cus + nlive - 1) / nlive) : 1;
    std::vector<Plan> plans(nlive);
    size_t bytes = align256(sizeof(Job) * (size_t)std::max(nlive, 1)) +
                   align256(sizeof(int32_t *) * zero.size() + 8);
    int wgPerJob = 1, finPerJob = 1;
    for (int k = 0; k < nlive; ++k) {
        const serac_pair pr = pairs[live[k]];
        plans[k] = make_plan(n[pr.a], n[pr.b], target);
        bytes += plan_bytes(plans[k]);
        wgPerJob = std::max(wgPerJob, plans[k].Gr * plans[k].Gc);
        finPerJob = std::max(finPerJob, plans[k].nFin);
    }
    uint8_t *ws = nullptr;
    if (hipMallocAsync(reinterpret_cast<void **>(&ws), bytes, stream) != hipSuccess) {
        (void)hipGetLastError();
        return SERAC_ERR_OUT_OF_MEMORY;
    }
    std::vector<uint8_t> host(align256(sizeof(Job) * (size_t)std::max(nlive, 1)) +
                              align256(sizeof(int32_t *) * zero.size() + 8));
    Job *jobs = reinterpret_cast<Job *>(host.data());
    int32_t **zp = reinterpret_cast<int32_t **>(host.data() +
                                                align256(sizeof(Job) * (size_t)std::max(nlive, 1)));
    uint8_t *q = ws + host.size();
    for (int k = 0; k < nlive; ++k) {
        const serac_pair pr = pairs[live[k]];
        fill_job(jobs[k], plans[k], desc[pr.a], n[pr.a], desc[pr.b], n[pr.b], q,
                 out[live[k]].matches, out[live[k]].count);
        q += plan_bytes(plans[k]);
    }
    for (size_t k = 0; k < zero.size(); ++k)
        zp[k] = zero[k];
    hipError_t e = hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, stream);
    const Job *djobs = reinterpret_cast<const Job *>(ws);
    int32_t *const *dzero = reinterpret_cast<int32_t *const *>(
        ws + align256(sizeof(Job) * (size_t)std::max(nlive, 1)));
    if (e == hipSuccess && !zero.empty())
        serac_zero_counts<<<((int)zero.size() + 255) / 256, 256, 0, stream>>>(dzero, nullptr,
                                                                         (int)zero.size());
    if (e == hipSuccess && nlive) {
        const Gate G = make_gate(d, params);
        if (params->cross_check)
            serac_tiles_many<true><<<nlive * wgPerJob, THREADS, 0, stream>>>(djobs, wgPerJob);
        else
            serac_tiles_many<false><<<nlive * wgPerJob, THREADS, 0, stream>>>(djobs, wgPerJob);
        serac_finish_many<<<nlive * finPerJob, FIN_THREADS, 0, stream>>>(djobs, finPerJob, G);
    }
    if (e == hipSuccess)
        e = hipGetLastError();
    (void)hipFreeAsync(ws, stream);
    if (e == hipSuccess) {
        // the staging buffer `host` must outlive the copy
        e = hipStreamSynchronize(stream);
    }
    return e == hipSuccess ? SERAC_OK : hip_fail();
}

int serac_top2_pair(const uint8_t *descA, int32_t nA, const uint8_t *descB, int32_t nB,
                    void *stream_, int32_t *row_top2, int32_t *col_best)
{
    if (bad_set(descA, nA) || bad_set(descB, nB) || (nA > 0 && !row_top2) ||
        (nB > 0 && !col_best))
        return SERAC_ERR_INVALID_ARG;
    Device *d = nullptr;
    int st = device_setup(&d);
    if (st != SERAC_OK)
        return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (nA == 0 && nB == 0)
        return SERAC_OK;
    const Plan p = make_plan(std::max(nA, 1), std::max(nB, 1), 2 * d->cus);
    size_t bytes = plan_bytes(p) + align256((size_t)std::max(nA, 1) * sizeof(uint32_t));
    uint8_t *ws = nullptr;
    if (hipMallocAsync(reinterpret_cast<void **>(&ws), bytes, stream) != hipSuccess) {
        (void)hipGetLastError();
        return SERAC_ERR_OUT_OF_MEMORY;
    }
    Job J;
    fill_job(J, p, descA, nA, descB, nB, ws, nullptr, nullptr);
    uint32_t *s1 = reinterpret_cast<uint32_t *>(ws + plan_bytes(p));
    if (nA > 0 && nB > 0)
        serac_tiles_one<true><<<p.Gr * p.Gc, THREADS, 0, stream>>>(J);
    // with an empty side the partial tables are never read: rows report
    // (0, -1, 0) and columns (0, -1) through Gc = Gr = 0
    Job E = J;
    if (nA == 0 || nB == 0) {
        E.Gc = 0;
        E.Gr = 0;
    }
    if (nA > 0)
        serac_export_rows<<<(nA + 255) / 256, 256, 0, stream>>>(E, row_top2, s1);
    if (nB > 0)
        serac_export_cols<<<(nB + 255) / 256, 256, 0, stream>>>(E, s1, col_best);
    const hipError_t e = hipGetLastError();
    (void)hipFreeAsync(ws, stream);
    return e == hipSuccess ? SERAC_OK : SERAC_ERR_HIP;
}

}  // extern "C"

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
//   * The contraction runs on v_mfma_i32_32x32x32_i8.  The MFMA is signed,
//     so bytes enter as a' = a ^ 0x80 = a - 128 (exact) and the product is
//     corrected with per-descriptor byte sums:
//       S = sum a'b' + 128*SA_i + 128*SB_j - 2^21,
//     every term exact in int32 (|sum a'b'| <= 2^21, S < 2^23).
//     The row term 128*SA_i - 2^21 enters through the MFMA accumulator input,
//     so it costs no vector instruction.
//   * A wave keeps the operand fragments of 64 rows of A in registers and
//     sweeps 32-column tiles of B staged in LDS (512 columns per chunk).
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
#include <algorithm>
#include <mutex>
#include <vector>

#include "serac.h"

namespace {

constexpr int DIM = 128;
constexpr int THREADS = 512;            // 8 waves of 64
constexpr int ROWS_PER_WAVE = 32;       // one 32-row MFMA tile
constexpr int ROWS_PER_BLOCK = 256;     // rows of A per workgroup pass
constexpr int SLICE = 16;               // rows per column tie-break slice
constexpr int CHUNK = 512;              // columns of B per LDS chunk (9-bit index)
constexpr int SUB = 128;                // columns per staged sub-chunk
constexpr int NSUB = CHUNK / SUB;
constexpr int MAX_CC_PER_WG = 4;        // chunks one workgroup sweeps
constexpr int MAX_RB_PER_WG = 32;       // 32 blocks * 16 slices = 512 slice ids
constexpr int NORM2 = 262144;           // 512^2
constexpr int GATE_THREADS = 256;
constexpr int COMPACT_THREADS = 1024;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// One pair's work description and its accumulators.  The accumulators
// are zero between calls: the tile kernel raises them with atomic maxima and
// the finishing kernel reads them and clears them again.
struct Job {
    const uint8_t *A;
    const uint8_t *B;
    int32_t nA, nB;
    int32_t nRB, nCC;        // row blocks of 256, column chunks of 512
    int32_t rbPer, ccPer;    // per workgroup
    int32_t Gr, Gc;          // workgroup grid (row groups x column groups)
    unsigned long long *rbest;  // [nA] (best << 32) | ~column   (max: lowest column)
    uint32_t *rsec;             // [nA] second-best score
    unsigned long long *cbest;  // [nB] (best << 32) | ~slice    (max: lowest slice)
    int32_t *res;            // [nA] accepted column of each row, or -1 (scratch)
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

// LDS layout of a chunk: eight planes, one per 16-byte part of the
// descriptors, each holding that part of all 512 columns back to back.  A
// wave's 32-column MFMA operand read is then 512 contiguous bytes per lane
// half; the 32-byte pad per plane keeps the staging writes (four parts of
// four columns per 16 lanes) on distinct banks.
constexpr int PLANE = CHUNK * 16 + 32;
constexpr int CHUNK_LDS = 8 * PLANE;

__device__ __forceinline__ int lds_off(int col, int part)
{
    return part * PLANE + col * 16;
}

// A quarter of a chunk of B (SUB columns) in flight from global memory:
// each thread holds 32 bytes (a quarter) of one column.
struct SubRegs {
    uint4 lo, hi;
};

__device__ __forceinline__ SubRegs load_sub(const uint8_t *__restrict__ B, int nB, int gcol0,
                                            int tid)
{
    const int col = tid >> 2, q = tid & 3;
    const int gcol = gcol0 + col;
    SubRegs r;
    r.lo = make_uint4(0u, 0u, 0u, 0u);
    r.hi = r.lo;
    if (gcol < nB) {
        const uint8_t *p = B + (size_t)gcol * DIM + q * 32;
        r.lo = *reinterpret_cast<const uint4 *>(p);
        r.hi = *reinterpret_cast<const uint4 *>(p + 16);
    }
    return r;
}

// Write a quarter chunk into LDS as int8 (a ^ 0x80) at chunk columns
// [col0, col0 + SUB), with each column's key addend
//   P = ((128 * SB) << 9) + (511 - t),
// t being the index of the column's 32-column tile among the tiles this
// workgroup sweeps (t0 = index of the chunk's first tile).
__device__ __forceinline__ void store_sub(const SubRegs &r, int col0, int t0, uint8_t *sB,
                                          uint32_t *sP, int tid)
{
    const int col = col0 + (tid >> 2), q = tid & 3;
    uint32_t s = bytesum16(r.lo) + bytesum16(r.hi);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (q == 0)
        sP[col] = ((s * 128u) << 9) + (uint32_t)(511 - (t0 + (col >> 5)));
    *reinterpret_cast<v4i *>(sB + lds_off(col, 2 * q)) = to_i8(r.lo);
    *reinterpret_cast<v4i *>(sB + lds_off(col, 2 * q + 1)) = to_i8(r.hi);
}

// The fused tile sweep of one workgroup: row blocks [rb0, rb1) of 256 rows
// by column chunks [cc0, cc1) of 512 columns.  Each of the 8 waves owns 32
// rows as one tile of v_mfma_i32_32x32x32_i8 (on gfx950 this MFMA leaves the
// vector ALU free far more of the time than the 16x16x64 form does).  B is
// double-buffered in LDS: while one chunk is swept, the next one (of this
// row block, or the first of the next row block) is loaded a quarter at a
// time into the other buffer.
//
// Accumulator layout of the 32x32 MFMA: lane l, register r holds output row
// 8*(r/4) + 4*(l/32) + r%4 of column l%32.  The operand row that feeds
// output row m is wave row 16*((m/4)%2) + 4*(m/8) + m%4, so lane half h,
// register r is wave row 16*h + r: each lane half covers 16 consecutive
// rows (one column tie-break slice).
//
// A lane only ever sees columns l%32 + 32*t of its workgroup's range, so
// its running top-2 keys carry t (at most 64 tiles) in their low 9 bits and
// stay valid across chunks; the 32 lanes sharing a row are merged once per
// row block.
template <bool COLS>
__device__ __forceinline__ void tiles_body(const Job &J, int wgi)
{
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][CHUNK_LDS];   // 2 x 64.25 KiB
    __shared__ uint32_t sP[2][CHUNK];
    __shared__ uint32_t sCol[COLS ? MAX_CC_PER_WG * CHUNK : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int r = wgi % J.Gr, c = wgi / J.Gr;
    const int rb0 = r * J.rbPer, rb1 = min(rb0 + J.rbPer, J.nRB);
    const int cc0 = c * J.ccPer, cc1 = min(cc0 + J.ccPer, J.nCC);
    if (rb0 >= rb1 || cc0 >= cc1)
        return;
    const int nA = J.nA, nB = J.nB;
    const int nchunks = cc1 - cc0;

    if (COLS) {
        for (int k = tid; k < nchunks * CHUNK; k += THREADS)
            sCol[k] = 0u;
    }

    // stage the first chunk
    {
        SubRegs q[NSUB];
#pragma unroll
        for (int sq = 0; sq < NSUB; ++sq)
            q[sq] = load_sub(J.B, nB, cc0 * CHUNK + sq * SUB, tid);
#pragma unroll
        for (int sq = 0; sq < NSUB; ++sq)
            store_sub(q[sq], sq * SUB, 0, sB[0], sP[0], tid);
    }
    int buf = 0;

    for (int rb = rb0; rb < rb1; ++rb) {
        // ---- this wave's 32 rows of A: operand fragments and the row term
        v4i af[4];
        v16i ci;
        {
            const int m = n;
            const int q = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
            const int row = rb * ROWS_PER_BLOCK + w * ROWS_PER_WAVE + q;
            uint4 x[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                x[kc] = make_uint4(0u, 0u, 0u, 0u);
            if (row < nA) {
                const uint8_t *a = J.A + (size_t)row * DIM + 16 * h;
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    x[kc] = *reinterpret_cast<const uint4 *>(a + 32 * kc);
            }
            uint32_t s = bytesum16(x[0]) + bytesum16(x[1]) + bytesum16(x[2]) + bytesum16(x[3]);
            s += __shfl_xor(s, 32);
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                af[kc] = to_i8(x[kc]);
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int mo = 8 * (rr >> 2) + 4 * h + (rr & 3);
                ci[rr] = (int)(128u * (uint32_t)__shfl((int)s, mo)) - 2097152;
            }
        }
        __syncthreads();                     // the chunk in sB[buf] is complete

        uint32_t b1[16], b2[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            b1[x] = 0u;
            b2[x] = 0u;
        }
        const int slice = (rb - rb0) * (ROWS_PER_BLOCK / SLICE) + w * 2 + h;
        const uint32_t tag = (uint32_t)(511 - slice);

        for (int cc = cc0; cc < cc1; ++cc) {
            // the chunk that follows this one in the sweep, if any
            int ncc = cc + 1, nrb = rb;
            if (ncc == cc1) {
                ncc = cc0;
                nrb = rb + 1;
            }
            const bool pre = nrb < rb1;
            const uint8_t *curB = sB[buf];
            const uint32_t *curP = sP[buf];
            uint32_t *colbase = sCol + (COLS ? (cc - cc0) * CHUNK : 0);

            // pipeline over the chunk's 8 pairs of 32-column tiles: step p
            // loads the B operands of pair p + 1 while it runs the MFMAs and
            // the VALU epilogue of pair p, so LDS latency is covered by a
            // whole step (the other wave on the SIMD overlaps MFMA and VALU).
            v4i bf[2][2][4];           // [pair parity][tile][k chunk]
            uint32_t pp[2][2];         // [pair parity][tile] key addends
            v16i acc[1][2];            // [tile]
            SubRegs nq;
            auto load_pair = [&](int pr, int slot) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int col = pr * 64 + 32 * t + n;
                    pp[slot][t] = curP[col];
#pragma unroll
                    for (int kc = 0; kc < 4; ++kc)
                        bf[slot][t][kc] =
                            *reinterpret_cast<const v4i *>(curB + lds_off(col, 2 * kc + h));
                }
            };
            auto mfma_pair = [&](int slot) {
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        acc[0][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            af[kc], bf[slot][t][kc], kc == 0 ? ci : acc[0][t], 0, 0, 0);
                }
            };
            auto epi_pair = [&](int pr, int slot) {
                const uint32_t P0 = pp[slot][0], P1 = pp[slot][1];
                uint32_t cm0 = 0u, cm1 = 0u;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const uint32_t k0 = ((uint32_t)acc[0][0][rr] << 9) + P0;
                    const uint32_t k1 = ((uint32_t)acc[0][1][rr] << 9) + P1;
                    const uint32_t md = umed3(b1[rr], k0, k1);
                    b1[rr] = umax3(b1[rr], k0, k1);
                    b2[rr] = max(b2[rr], md);
                    if (COLS) {
                        cm0 = max(cm0, k0);
                        cm1 = max(cm1, k1);
                    }
                }
                if (COLS) {
                    const int col0 = pr * 64 + n;
                    atomicMax(colbase + col0, (cm0 & ~511u) | tag);
                    atomicMax(colbase + col0 + 32, (cm1 & ~511u) | tag);
                }
            };

            load_pair(0, 0);
#pragma unroll 1
            for (int sq = 0; sq < NSUB; ++sq) {
                // two pairs per quarter: the even one in slot 0, the odd in 1
                if (pre)
                    nq = load_sub(J.B, nB, ncc * CHUNK + sq * SUB, tid);
                load_pair(2 * sq + 1, 1);
                mfma_pair(0);
                epi_pair(2 * sq, 0);
                if (sq + 1 < NSUB)
                    load_pair(2 * sq + 2, 0);
                mfma_pair(1);
                epi_pair(2 * sq + 1, 1);
                if (pre)
                    store_sub(nq, sq * SUB, nrb == rb ? (ncc - cc0) * (CHUNK / 32) : 0,
                              sB[buf ^ 1], sP[buf ^ 1], tid);
            }
            __syncthreads();                 // next chunk complete, this one free
            buf ^= 1;
        }

        // ---- merge the 32 lanes that share each row (via LDS, in the free
        // buffer): lane pair (q, q + 32) folds 16 of the 32 entries of row q
        // each; key ties (same score, same tile) go to the lower lane, which
        // is the lower column.
        uint2 *scr = reinterpret_cast<uint2 *>(sB[buf ^ 1]) + w * (ROWS_PER_WAVE * 32);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int q = 16 * h + rr;
            scr[q * 32 + ((n + q) & 31)] = make_uint2(b1[rr], b2[rr]);
        }
        __syncthreads();
        uint32_t K1 = 0u, K2 = 0u;
        int L1 = 64;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int src = (16 * h + k) & 31;              // source lane (column)
            const uint2 e = scr[n * 32 + ((src + n) & 31)];
            const uint32_t lo = min(K1, e.x);
            if (e.x > K1 || (e.x == K1 && src < L1))
                L1 = src;
            K1 = max(K1, e.x);
            K2 = umax3(lo, K2, e.y);
        }
        {
            const uint32_t o1 = __shfl_xor(K1, 32), o2 = __shfl_xor(K2, 32);
            const int oL = __shfl_xor(L1, 32);
            const uint32_t lo = min(K1, o1);
            if (o1 > K1 || (o1 == K1 && oL < L1))
                L1 = oL;
            K1 = max(K1, o1);
            K2 = umax3(lo, K2, o2);
        }
        __syncthreads();                     // scratch free
        // publish this row block's top-2 over the workgroup's columns: the
        // atomic max keeps the best key over all workgroups; whichever key
        // loses an exchange (or this group's own second) raises the row's
        // second score, so the second ends as the runner-up of all
        // candidates, ties counted.
        const uint32_t S1 = K1 >> 9, S2 = K2 >> 9;
        const int row = rb * ROWS_PER_BLOCK + w * ROWS_PER_WAVE + n;
        if (h == 0 && row < nA && S1 > 0u) {
            const uint32_t col = (uint32_t)(cc0 * CHUNK + 32 * (511 - (int)(K1 & 511u)) + L1);
            const unsigned long long key = ((unsigned long long)S1 << 32) | (0xFFFFFFFFu - col);
            const unsigned long long old = atomicMax(J.rbest + row, key);
            const uint32_t loser = (uint32_t)(min(old, key) >> 32);
            atomicMax(J.rsec + row, max(loser, S2));
        }
    }

    if (COLS) {
        __syncthreads();
        const int base = cc0 * CHUNK;
        for (int k = tid; k < nchunks * CHUNK; k += THREADS) {
            const int col = base + k;
            const uint32_t key = sCol[k];
            if (col < nB && (key >> 9) > 0u) {
                const uint32_t slice = (uint32_t)(r * J.rbPer * (ROWS_PER_BLOCK / SLICE) + 511 -
                                                  (int)(key & 511u));
                atomicMax(J.cbest + col,
                          ((unsigned long long)(key >> 9) << 32) | (0xFFFFFFFFu - slice));
            }
        }
    }
}

template <bool COLS>
__global__ __launch_bounds__(THREADS, 1) void serac_tiles_one(Job J)
{
    tiles_body<COLS>(J, blockIdx.x);
}

template <bool COLS>
__global__ __launch_bounds__(THREADS, 1) void serac_tiles_many(const Job *__restrict__ jobs,
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

// Row i's published result: best score, its column (-1 below the zero
// floor) and the second score.
__device__ __forceinline__ void row_result(const Job &J, unsigned long long key, uint32_t sec,
                                           uint32_t &S1, int32_t &I1, uint32_t &S2)
{
    S1 = (uint32_t)(key >> 32);
    I1 = S1 ? (int32_t)(0xFFFFFFFFu - (uint32_t)key) : -1;
    S2 = sec;
}

// Gates and cross-check of 256 rows: res[i] = the accepted column of row i,
// or -1.  The row accumulators are cleared as they are consumed.
__device__ __forceinline__ void gate_body(const Job &J, int wg, const Gate &G)
{
    __shared__ uint32_t sS1[GATE_THREADS];
    const int tid = threadIdx.x;
    const int i = wg * GATE_THREADS + tid;
    uint32_t S1 = 0u, S2 = 0u;
    int32_t I1 = -1;
    if (i < J.nA) {
        row_result(J, J.rbest[i], J.rsec[i], S1, I1, S2);
        J.rbest[i] = 0ull;
        J.rsec[i] = 0u;
    }
    sS1[tid] = S1;
    const bool cand = I1 >= 0 && I1 < J.nB;
    double d1 = 0.0, d2 = 0.0;
    unsigned long long cb = 0ull;
    if (cand) {
        d1 = G.table[min(S1, (uint32_t)NORM2)];
        d2 = G.table[min(S2, (uint32_t)NORM2)];
        if (G.cross_check)
            cb = J.cbest[I1];
    }
    __syncthreads();                         // sS1 complete
    if (i >= J.nA)
        return;
    bool acc = cand && (d1 <= G.max_distance) && (d1 < G.max_ratio * d2);
    if (acc && G.cross_check) {
        const uint32_t C1 = (uint32_t)(cb >> 32);
        const int32_t slice = (int32_t)(0xFFFFFFFFu - (uint32_t)cb);
        if (C1 != S1 || slice != i / SLICE) {
            acc = false;
        } else {
            // a lower row of the same slice reaching the same score wins
            const uint8_t *b = J.B + (size_t)I1 * DIM;
            for (int i2 = i - i % SLICE; i2 < i; ++i2) {
                if (sS1[i2 - wg * GATE_THREADS] >= C1 &&
                    (uint32_t)dot_exact(J.A + (size_t)i2 * DIM, b) == C1) {
                    acc = false;
                    break;
                }
            }
        }
    }
    J.res[i] = acc ? I1 : -1;
}

__global__ __launch_bounds__(GATE_THREADS) void serac_gate_one(Job J, Gate G)
{
    gate_body(J, blockIdx.x, G);
}

__global__ __launch_bounds__(GATE_THREADS) void serac_gate_many(const Job *__restrict__ jobs,
                                                                int gatePerJob, Gate G)
{
    const Job J = jobs[blockIdx.x / gatePerJob];
    const int wg = blockIdx.x % gatePerJob;
    if (wg * GATE_THREADS >= J.nA)
        return;
    gate_body(J, wg, G);
}

// Ordered compaction of one pair by one workgroup: rows are taken 8192 at a
// time, eight consecutive rows per thread, and a workgroup-wide exclusive
// scan of the per-thread counts places each thread's matches.  The column
// accumulators, read by every gate group, are cleared here.
__device__ __forceinline__ void compact_body(const Job &J)
{
    __shared__ int32_t sWave[COMPACT_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t run = 0;
    for (int base = 0; base < J.nA; base += 8 * COMPACT_THREADS) {
        const int i0 = base + 8 * tid;
        int32_t v[8];
        if (i0 + 8 <= J.nA) {
            const int4 lo = *reinterpret_cast<const int4 *>(J.res + i0);
            const int4 hi = *reinterpret_cast<const int4 *>(J.res + i0 + 4);
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                v[k] = (i0 + k < J.nA) ? J.res[i0 + k] : -1;
        }
        int32_t cnt = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            cnt += v[k] >= 0;
        int32_t inc = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t t = __shfl_up(inc, d);
            if (lane >= d)
                inc += t;
        }
        if (lane == 63)
            sWave[wv] = inc;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int k = 0; k < COMPACT_THREADS / 64; ++k) {
            before += (k < wv) ? sWave[k] : 0;
            total += sWave[k];
        }
        int32_t o = run + before + inc - cnt;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (v[k] >= 0) {
                J.out[o].a = (uint32_t)(i0 + k);
                J.out[o].b = (uint32_t)v[k];
                ++o;
            }
        }
        run += total;
        __syncthreads();                     // sWave reused by the next tile
    }
    for (int j = tid; j < J.nB; j += COMPACT_THREADS)
        J.cbest[j] = 0ull;
    if (tid == 0)
        *J.count = run;
}

__global__ __launch_bounds__(COMPACT_THREADS) void serac_compact_one(Job J)
{
    compact_body(J);
}

__global__ __launch_bounds__(COMPACT_THREADS) void serac_compact_many(const Job *__restrict__ jobs)
{
    const Job J = jobs[blockIdx.x];
    compact_body(J);
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

// Clears a freshly allocated accumulator buffer (n 16-byte words).
__global__ void serac_clear(uint4 *p, size_t n)
{
    for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < n;
         k += (size_t)gridDim.x * blockDim.x)
        p[k] = make_uint4(0u, 0u, 0u, 0u);
}

// Export of the row reduction: row_top2[i] = (best, idx, second).  The best
// score is kept in rsec for the column export, rbest is cleared.
__global__ void serac_export_rows(Job J, int32_t *row_top2)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= J.nA)
        return;
    uint32_t S1, S2;
    int32_t I1;
    row_result(J, J.rbest[i], J.rsec[i], S1, I1, S2);
    row_top2[3 * (size_t)i] = (int32_t)S1;
    row_top2[3 * (size_t)i + 1] = I1;
    row_top2[3 * (size_t)i + 2] = (int32_t)S2;
    J.rbest[i] = 0ull;
    J.rsec[i] = S1;
}

// Export of the column reduction: col_best[j] = (best, lowest row).  The
// winning 16-row slice is known; its first row reaching the best score is
// found among the rows whose own best is at least that score.  cbest is
// cleared.
__global__ void serac_export_cols(Job J, int32_t *col_best)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= J.nB)
        return;
    const unsigned long long key = J.cbest[j];
    const uint32_t C1 = (uint32_t)(key >> 32);
    const int32_t slice = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    int32_t idx = -1;
    if (C1 > 0u) {
        const uint8_t *b = J.B + (size_t)j * DIM;
        for (int i = slice * SLICE; i < min(slice * SLICE + SLICE, J.nA); ++i) {
            if (J.rsec[i] >= C1 && (uint32_t)dot_exact(J.A + (size_t)i * DIM, b) == C1) {
                idx = i;
                break;
            }
        }
    }
    col_best[2 * (size_t)j] = (int32_t)C1;
    col_best[2 * (size_t)j + 1] = idx;
    J.cbest[j] = 0ull;
}

// Clears rsec after the column export has used it.
__global__ void serac_export_clear(Job J)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < J.nA)
        J.rsec[i] = 0u;
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

// Event pairs around tile-kernel launches while profiling is armed.
struct Profile {
    bool armed = false;
    int used = 0;
    std::vector<hipEvent_t> ev;   // [2 * max]: begin, end
};
std::mutex g_prof_mutex;
Profile g_prof;

int prof_begin(hipStream_t s)
{
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    if (!g_prof.armed || 2 * (g_prof.used + 1) > (int)g_prof.ev.size())
        return -1;
    const int slot = g_prof.used++;
    (void)hipEventRecord(g_prof.ev[2 * slot], s);
    return slot;
}

void prof_end(hipStream_t s, int slot)
{
    if (slot < 0)
        return;
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    (void)hipEventRecord(g_prof.ev[2 * slot + 1], s);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

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

// Grow-only workspace per (device, stream).  Work on one stream runs in
// order, so consecutive calls on a stream can share one workspace; calls on
// different streams get different ones.  Growth frees the old buffers and
// allocates new ones on the same stream, both stream-ordered.
//   acc  the accumulators of the jobs; all zero between calls (each call
//        clears what it raised), cleared by a kernel when (re)allocated or
//        after a failed call;
//   aux  per-call scratch (the job table of a batch).
struct Workspace {
    int dev;
    hipStream_t stream;
    uint8_t *acc;
    size_t acc_bytes;
    uint8_t *aux;
    size_t aux_bytes;
    bool dirty;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;

int grow(uint8_t *&ptr, size_t &have, size_t need, hipStream_t stream, bool clear)
{
    if (have >= need && ptr)
        return SERAC_OK;
    if (ptr)
        (void)hipFreeAsync(ptr, stream);
    ptr = nullptr;
    have = 0;
    const size_t want = std::max(align256(need), (size_t)1 << 20);
    if (hipMallocAsync(reinterpret_cast<void **>(&ptr), want, stream) != hipSuccess) {
        (void)hipGetLastError();
        ptr = nullptr;
        return SERAC_ERR_OUT_OF_MEMORY;
    }
    have = want;
    if (clear) {
        serac_clear<<<1024, 256, 0, stream>>>(reinterpret_cast<uint4 *>(ptr), want / 16);
        if (hipGetLastError() != hipSuccess)
            return SERAC_ERR_HIP;
    }
    return SERAC_OK;
}

// The workspace of the current device and `stream`, with at least the
// given sizes; returns it locked to the caller's use via *out.
int get_workspace(hipStream_t stream, size_t acc_bytes, size_t aux_bytes, Workspace **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return hip_fail();
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace *w = nullptr;
    for (auto &e : g_ws)
        if (e.dev == dev && e.stream == stream)
            w = &e;
    if (!w) {
        g_ws.push_back(Workspace{dev, stream, nullptr, 0, nullptr, 0, false});
        w = &g_ws.back();
    }
    int st = grow(w->acc, w->acc_bytes, acc_bytes, stream, true);
    if (st == SERAC_OK && w->dirty) {
        serac_clear<<<1024, 256, 0, stream>>>(reinterpret_cast<uint4 *>(w->acc),
                                              w->acc_bytes / 16);
        st = hipGetLastError() == hipSuccess ? SERAC_OK : SERAC_ERR_HIP;
        if (st == SERAC_OK)
            w->dirty = false;
    }
    if (st == SERAC_OK && aux_bytes)
        st = grow(w->aux, w->aux_bytes, aux_bytes, stream, false);
    *out = w;
    return st;
}

// A call that enqueued work on the accumulators and then failed may have
// left them raised: have the next call clear them first.
void mark_dirty(Workspace *w)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    w->dirty = true;
}

struct Plan {
    int nRB, nCC, rbPer, ccPer, Gr, Gc;
    size_t acc;   // bytes of accumulators
};

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
    p.acc = align256((size_t)nA * 8) + align256((size_t)nA * 4) + align256((size_t)nB * 8);
    return p;
}

void fill_job(Job &J, const Plan &p, const uint8_t *A, int nA, const uint8_t *B, int nB,
              uint8_t *acc, int32_t *res, serac_match *out, int32_t *count)
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
    uint8_t *q = acc;
    J.rbest = reinterpret_cast<unsigned long long *>(q);
    q += align256((size_t)nA * 8);
    J.rsec = reinterpret_cast<uint32_t *>(q);
    q += align256((size_t)nA * 4);
    J.cbest = reinterpret_cast<unsigned long long *>(q);
    J.res = res;
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
    const Plan p = make_plan(nA, nB, d->cus);
    Workspace *w = nullptr;
    st = get_workspace(stream, p.acc, (size_t)nA * 4, &w);
    if (st != SERAC_OK)
        return st;
    Job J;
    fill_job(J, p, descA, nA, descB, nB, w->acc, reinterpret_cast<int32_t *>(w->aux),
             out->matches, out->count);
    const Gate G = make_gate(d, params);
    const int slot = prof_begin(stream);
    if (params->cross_check)
        serac_tiles_one<true><<<p.Gr * p.Gc, THREADS, 0, stream>>>(J);
    else
        serac_tiles_one<false><<<p.Gr * p.Gc, THREADS, 0, stream>>>(J);
    prof_end(stream, slot);
    serac_gate_one<<<(nA + GATE_THREADS - 1) / GATE_THREADS, GATE_THREADS, 0, stream>>>(J, G);
    serac_compact_one<<<1, COMPACT_THREADS, 0, stream>>>(J);
    if (hipGetLastError() != hipSuccess) {
        mark_dirty(w);
        return SERAC_ERR_HIP;
    }
    return SERAC_OK;
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
    const int target = nlive ? std::max(1, (4 * d->cus + nlive - 1) / nlive) : 1;
    std::vector<Plan> plans(nlive);
    size_t acc_bytes = 0, res_bytes = 0;
    int wgPerJob = 1, gatePerJob = 1;
    for (int k = 0; k < nlive; ++k) {
        const serac_pair pr = pairs[live[k]];
        plans[k] = make_plan(n[pr.a], n[pr.b], target);
        acc_bytes += plans[k].acc;
        res_bytes += align256((size_t)n[pr.a] * 4);
        wgPerJob = std::max(wgPerJob, plans[k].Gr * plans[k].Gc);
        gatePerJob = std::max(gatePerJob, (n[pr.a] + GATE_THREADS - 1) / GATE_THREADS);
    }
    const size_t jobs_bytes = align256(sizeof(Job) * (size_t)std::max(nlive, 1));
    std::vector<uint8_t> host(jobs_bytes + align256(sizeof(int32_t *) * zero.size() + 8));
    Workspace *w = nullptr;
    st = get_workspace(stream, acc_bytes, host.size() + res_bytes, &w);
    if (st != SERAC_OK)
        return st;
    Job *jobs = reinterpret_cast<Job *>(host.data());
    int32_t **zp = reinterpret_cast<int32_t **>(host.data() + jobs_bytes);
    uint8_t *q = w->acc, *rq = w->aux + host.size();
    for (int k = 0; k < nlive; ++k) {
        const serac_pair pr = pairs[live[k]];
        fill_job(jobs[k], plans[k], desc[pr.a], n[pr.a], desc[pr.b], n[pr.b], q,
                 reinterpret_cast<int32_t *>(rq), out[live[k]].matches, out[live[k]].count);
        q += plans[k].acc;
        rq += align256((size_t)n[pr.a] * 4);
    }
    for (size_t k = 0; k < zero.size(); ++k)
        zp[k] = zero[k];
    hipError_t e = hipMemcpyAsync(w->aux, host.data(), host.size(), hipMemcpyHostToDevice, stream);
    const Job *djobs = reinterpret_cast<const Job *>(w->aux);
    int32_t *const *dzero = reinterpret_cast<int32_t *const *>(w->aux + jobs_bytes);
    if (e == hipSuccess && !zero.empty())
        serac_zero_counts<<<((int)zero.size() + 255) / 256, 256, 0, stream>>>(dzero, nullptr,
                                                                         (int)zero.size());
    if (e == hipSuccess && nlive) {
        const Gate G = make_gate(d, params);
        const int slot = prof_begin(stream);
        if (params->cross_check)
            serac_tiles_many<true><<<nlive * wgPerJob, THREADS, 0, stream>>>(djobs, wgPerJob);
        else
            serac_tiles_many<false><<<nlive * wgPerJob, THREADS, 0, stream>>>(djobs, wgPerJob);
        prof_end(stream, slot);
        serac_gate_many<<<nlive * gatePerJob, GATE_THREADS, 0, stream>>>(djobs, gatePerJob, G);
        serac_compact_many<<<nlive, COMPACT_THREADS, 0, stream>>>(djobs);
    }
    if (e == hipSuccess)
        e = hipGetLastError();
    if (e == hipSuccess) {
        // the staging buffer `host` must outlive the copy
        e = hipStreamSynchronize(stream);
    }
    if (e != hipSuccess) {
        mark_dirty(w);
        return hip_fail();
    }
    return SERAC_OK;
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
    const Plan p = make_plan(std::max(nA, 1), std::max(nB, 1), d->cus);
    Workspace *w = nullptr;
    st = get_workspace(stream, p.acc, 0, &w);
    if (st != SERAC_OK)
        return st;
    Job J;
    fill_job(J, p, descA, nA, descB, nB, w->acc, nullptr, nullptr, nullptr);
    // with an empty side nothing is raised: rows report (0, -1, 0) and
    // columns (0, -1) from the cleared accumulators
    if (nA > 0 && nB > 0)
        serac_tiles_one<true><<<p.Gr * p.Gc, THREADS, 0, stream>>>(J);
    if (nA > 0)
        serac_export_rows<<<(nA + 255) / 256, 256, 0, stream>>>(J, row_top2);
    if (nB > 0)
        serac_export_cols<<<(nB + 255) / 256, 256, 0, stream>>>(J, col_best);
    if (nA > 0)
        serac_export_clear<<<(nA + 255) / 256, 256, 0, stream>>>(J);
    if (hipGetLastError() != hipSuccess) {
        mark_dirty(w);
        return SERAC_ERR_HIP;
    }
    return SERAC_OK;
}

int serac_profile_start(int32_t max_launches)
{
    if (max_launches < 1 || max_launches > (1 << 20))
        return SERAC_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    for (hipEvent_t e : g_prof.ev)
        (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.used = 0;
    g_prof.armed = false;
    g_prof.ev.resize(2 * (size_t)max_launches);
    for (auto &e : g_prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            return hip_fail();
        }
    }
    g_prof.armed = true;
    return SERAC_OK;
}

int serac_profile_stop(double *tile_kernel_ms, int32_t *launches)
{
    if (!tile_kernel_ms || !launches)
        return SERAC_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    if (!g_prof.armed)
        return SERAC_ERR_INVALID_ARG;
    double total = 0.0;
    int st = SERAC_OK;
    for (int k = 0; k < g_prof.used; ++k) {
        float ms = 0.f;
        if (hipEventSynchronize(g_prof.ev[2 * k + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_prof.ev[2 * k], g_prof.ev[2 * k + 1]) != hipSuccess) {
            st = hip_fail();
            break;
        }
        total += ms;
    }
    *tile_kernel_ms = total;
    *launches = g_prof.used;
    for (hipEvent_t e : g_prof.ev)
        if (e)
            (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.used = 0;
    g_prof.armed = false;
    return st;
}

}  // extern "C"

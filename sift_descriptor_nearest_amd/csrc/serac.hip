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
//   * The tile kernel reads A as per-lane MFMA operand fragments plus the
//     row terms, and B as 256-column chunks of eight 16-byte "planes" plus
//     each column's key addend, double-buffered in LDS.  For one pair up to
//     2^28 products it builds these itself from the raw descriptors: A in
//     its prologue, each B chunk copied raw into LDS (global_load_lds) and
//     converted during the chunk before.  Larger pairs and batches get a
//     preparation kernel that converts each set once; the tile kernel then
//     streams the prepared chunks straight into LDS (no registers, no
//     vector instructions).
//   * A workgroup is eight waves, two per SIMD, 256 rows of A by up to 16384
//     columns of B, one workgroup per CU: the eight waves share every staged
//     B chunk and the per-chunk barrier keeps them in step (two smaller
//     workgroups on one CU drift apart, the older one taking the issue
//     slots, and the younger then finishes alone).  Each wave keeps the operand
//     fragments of its 32 rows in registers and sweeps 32-column tiles two at
//     a time, software-pipelined: the MFMAs of one tile pair are issued while
//     the vector epilogue of the previous pair runs in the same wave, so the
//     matrix core and the vector ALU work side by side.
//   * Each score becomes one packed 32-bit key
//       key = (S << 9) | (511 - t),
//     t being the index of its 32-column tile in the 16384-column window, in
//     one v_lshl_add (the column term 128*SB_j is folded into the addend).
//     A key comparison orders by score, then by lowest column.  Scores stay
//     below 2^23, so the key is exact.
//   * Row top-2: per lane and row, max3/med3 over two new keys at a time; the
//     second-best update is deferred to every other pair (the runner-up of
//     the two pairs is folded in with one max3).  Keys are unique per column,
//     so a tie on score leaves the tied score in second place (multiplicity)
//     and the lowest column in first.
//   * Column best: a max3 tree over the 16 rows a lane holds in one tile
//     gives the column maximum of those rows; the key's low 9 bits are then
//     replaced by the 16-row slice number (lowest slice wins) and merged with
//     an LDS atomic max into a ring of eight chunks, which goes out to the
//     global column bests (an atomic max, 32-bit up to 8192 rows of A, else
//     64-bit) during the sweep.  The exact
//     lowest row inside the winning slice is settled afterwards from the 15
//     rows that precede it, compared in registers (an exact product only in
//     the rare case the bounds leave open).
//   * All merges (across lanes, waves, workgroups) compare packed keys or
//     scan in ascending index order, so the result does not depend on
//     scheduling (MASDA part 3, section 6: an order-independent key).
//   * The angle gates take the C library's acos of s / 512^2 (a table built
//     on the host), so each double-precision decision is the one a CPU
//     makes; a single pair's finishing kernel first evaluates the device's
//     own acos and trusts it only where a bracket measured against the
//     table at set-up settles the decision.  The ratio test is one IEEE
//     multiply and compare.
//   * In a batch of many pairs with small second images, the pairs that
//     share their first image are swept in strips: one workgroup keeps a row
//     block of that image in registers and runs through the second images
//     of up to 16 pairs as one stream of chunks, its reductions segmented
//     at the pairs' boundaries, so each pair after the first skips the wait
//     for its first chunk.
//   * Variants: symmetric column gates run the sweep of the swapped pair as
//     well and compare each row's best column's accepted row; the match cap
//     takes the first descriptors of each set; an unfused comparison arm
//     writes the score matrix and reduces it in separate passes; a
//     non-allocating entry point works in a fixed device array.
//   * Host side: one workspace per (device, stream), grow-only and
//     stream-ordered, releasable per stream; a batch stages its job tables
//     through a ring of pinned buffers, each behind an event;
//     serac_match_pairs_host runs a batch in stages and overlaps the copy of
//     each stage's lists to the host with the matching of the next.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <deque>
#include <mutex>
#include <numeric>
#include <atomic>
#include <new>
#include <type_traits>
#include <unordered_map>
#include <utility>
#include <vector>

#include "serac.h"
#include "serac_bench.h"

#include <cstddef>

static_assert(sizeof(serac_params) == 40 && offsetof(serac_params, stream) == 24 &&
                  offsetof(serac_params, max_features) == 32,
              "serac_params layout (the Python binding mirrors it)");

namespace {

constexpr int DIM = 128;
constexpr int TILE_WAVES = 8;           // two per SIMD
constexpr int TILE_THREADS = 64 * TILE_WAVES;
constexpr int WAVE_ROWS = 32;           // one 32-row MFMA tile per wave
constexpr int BLOCK_ROWS = WAVE_ROWS * TILE_WAVES;   // rows of A per workgroup
constexpr int SLICE = 16;               // rows per column tie-break slice
constexpr int CHUNK = 256;              // columns of B per LDS chunk
constexpr int CHUNK_BYTES = CHUNK * DIM;
constexpr int PLANE_BYTES = CHUNK * 16; // one 16-byte part of every column
constexpr int GROUP_MAX = 16384;        // columns per workgroup: 512 tiles (the keys' 9-bit index)
constexpr int MAX_GCH = GROUP_MAX / CHUNK;
constexpr int COL_RING = 8;             // chunks of column maxima a workgroup keeps in LDS
constexpr int STRIP_MAX_SEG = 16;       // pairs one workgroup of a strip sweeps (see serac_tiles_strip)
constexpr int SCR_ROW = 33;              // lane-merge scratch: 32 entries per row plus one of padding
constexpr int SCR_WAVE = WAVE_ROWS * SCR_ROW;   // entries per wave (8448 bytes)
// LDS chunk buffer stride: a chunk plus 1 KiB, so that a buffer the chunks no
// longer use holds the lane-merge scratch of four waves
constexpr int BUF_BYTES = CHUNK_BYTES + 1024;
static_assert(4 * SCR_WAVE * 8 <= BUF_BYTES, "merge scratch of four waves in one chunk buffer");
constexpr int PREP_THREADS = 256;
constexpr int NORM2 = 262144;           // 512^2
constexpr int GATE_THREADS = 256;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// One set prepared for the tile kernel (either role or both).
//   Af  [rowsA/256][8 waves][4 k-slices][64 lanes][16 B]: the MFMA A operand
//       of every lane, bytes a ^ 0x80.  Lane (n, h) of wave w holds bytes
//       [32*kc + 16*h, +16) of wave row q(n) = 16*((n>>2)&1) + 4*(n>>3) + n%4.
//   RT  [rowsA] row term 128*SA - 2^21.
//   Bp  [rowsB/256][8 parts][256 columns][16 B]: part p of column j holds
//       bytes [16*p, +16) of that descriptor, ^ 0x80.
//   P   [rowsB] key addend ((128*SB) << 9) + (511 - ((j >> 5) & 511)).
// Rows beyond n are all-zero descriptors: their score against anything is 0.
struct PrepJob {
    const uint8_t *X;
    int32_t n;
    int32_t rowsA, rowsB;    // padded row counts of the two roles (0 = role unused)
    uint8_t *Af;
    int32_t *RT;
    uint8_t *Bp;
    uint32_t *P;
};

struct PrepPair {
    PrepJob q[2];
};

// Words of the accumulator region the previous call on this stream left
// raised; the first kernel of this call clears them, `stride` threads of it
// (the blocks of its first grid row).
struct Clear {
    uint4 *p;
    size_t words;
    uint32_t stride;
};

// One pair's work description and its accumulators.  The accumulators
// (column bests, finishing status words) are zero when a sweep starts: the
// tile kernel raises the column bests with atomic maxima, the finishing
// kernel reads them and publishes its status words, and the next call's
// preparation kernel on the stream clears what was left raised.
struct Job {
    const uint8_t *A;        // raw descriptors (exact tie checks)
    const uint8_t *B;
    const uint8_t *Af;       // prepared A (see PrepJob)
    const int32_t *RT;
    const uint8_t *Bp;       // prepared B
    const uint32_t *P;
    int32_t nA, nB;
    int32_t nRB, nBC;        // 128-row blocks of A, 256-column chunks of B
    int32_t gch, Gc;         // chunks per workgroup (a power of two up to 64), column groups
    unsigned long long *rslot;  // [Gc][nA] one row result per column group (see pack_slot)
    uint32_t *rs1;              // [nA] best score per row (column export scratch)
    unsigned long long *cbest;  // [nB] column bests (see col_best_at), raised by atomic maxima
    int32_t cb32;            // 1: 32-bit column bests (at most 512 slices, nA <= 8192)
    unsigned long long *status;  // [ceil(nA / 256)] finishing hand-off (zero before the finish)
    serac_match *out;        // [>= nA]
    int32_t *count;          // 1
};

// What a strip's sweep needs of one of its pairs (see serac_tiles_strip).
struct SegRef {
    const uint8_t *Bp;
    const uint32_t *P;
    unsigned long long *cbest;
    unsigned long long *rslot;
    int32_t nB, nBC;
};

struct Gate {
    const double *table;     // acos(min(s, 512^2) / 512^2), s = 0 .. 512^2
    double max_ratio;
    double max_distance;
    double slack;            // the device angle is within `slack` of the table (angle_bounds)
    int32_t cross_check;
    int32_t spin_limit;      // look-back polls before giving up (< 0: give up at once)
};

// Angle of a clamped score computed on the device: the same expression the
// host table is built from, evaluated with the device's double acos.
__device__ __forceinline__ double angle_dev(uint32_t s)
{
    return acos(s >= (uint32_t)NORM2 ? 1.0 : (double)s / (double)NORM2);
}

// Deviation of the device angle from the host table over the whole domain
// (s = 0 .. 512^2): raised into *err as the bits of a non-negative double
// (which order like the double itself); a NaN counts as infinite.
__global__ void serac_angle_check(const double *table, unsigned long long *err)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s > NORM2)
        return;
    double e = fabs(angle_dev((uint32_t)s) - table[s]);
    if (!(e == e))
        e = INFINITY;
    atomicMax(err, (unsigned long long)__double_as_longlong(e));
}

// The gates without the table where the device angle settles them: with
// every device angle within E of the table's, T in [a - slack, a + slack]
// for slack = 2E + 1e-15 (which also covers the rounding of a +- slack), and
// the ratio and distance decisions are taken only where the whole interval
// agrees (max_ratio * x is monotone in x).  1: accept, 0: reject, -1: the
// table decides.  A NaN angle or slack leaves every comparison false.
__device__ __forceinline__ int gates_sure(uint32_t S1, uint32_t S2, const Gate &G)
{
    const double a1 = angle_dev(S1), a2 = angle_dev(S2);
    const double lo1 = a1 - G.slack, hi1 = a1 + G.slack;
    const double lo2 = a2 - G.slack, hi2 = a2 + G.slack;
    if (lo1 > G.max_distance || lo1 >= G.max_ratio * hi2)
        return 0;
    if (hi1 <= G.max_distance && hi1 < G.max_ratio * lo2)
        return 1;
    return -1;
}



// A row's result over one column group packed into 64 bits, ordered like
// the key (score first, then lowest column):
//   bits 63..41  best score S1 (< 2^23)
//   bits 40..23  2^18 - 1 - column of S1 (columns < 2^18)
//   bits 22..0   second score S2 (< 2^23)
// A group whose best score is 0 stores 0.
constexpr int SLOT_COL_BITS = 18;
constexpr uint32_t SLOT_COL_MAX = (1u << SLOT_COL_BITS) - 1;

__host__ __device__ __forceinline__ unsigned long long pack_slot(uint32_t S1, uint32_t col,
                                                                 uint32_t S2)
{
    if (S1 == 0u)
        return 0ull;
    return ((unsigned long long)S1 << 41) |
           ((unsigned long long)(SLOT_COL_MAX - col) << 23) | (unsigned long long)S2;
}

// A column's best: its score and the 16-row slice holding the first row
// that reaches it (lowest slice on a tie), raised by atomic maxima.  With at
// most 512 slices (nA <= 8192) it takes 32 bits, (S << 9) | (511 - slice);
// otherwise 64, (S << 32) | ~slice.  Both order by score, then lowest
// slice, and are 0 for a column no row scores above 0 on.  The 64-bit
// atomic maximum costs ~0.6 us more per 8192 x 8192 sweep than the 32-bit
// one (measured), hence the narrow form where it fits.
__device__ __forceinline__ void col_best_at(const Job &J, int j, uint32_t &C1, int32_t &slice)
{
    if (J.cb32) {
        const uint32_t v = reinterpret_cast<const uint32_t *>(J.cbest)[j];
        C1 = v >> 9;
        slice = 511 - (int32_t)(v & 511u);
    } else {
        const unsigned long long v = J.cbest[j];
        C1 = (uint32_t)(v >> 32);
        slice = (int32_t)(0xFFFFFFFFu - (uint32_t)v);
    }
}

// 128 zero bytes: the descriptor a fused sweep reads for columns past the end
// of B (an all-zero descriptor scores 0 against anything).
__device__ const uint8_t g_zero_desc[DIM] = {};

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

// Wait until at most `N` vector-memory loads of this wave are outstanding.
// Loads complete in issue order, so this waits for all but the last N
// issued.  Written as inline assembly with a memory clobber, so that the
// compiler moves no memory access across it: it is what orders the LDS
// reads of a chunk after that chunk's copy into LDS (see load_lds16).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, not for its global stores (the release fence of
// __syncthreads() would wait for those as well).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void *lds_void_ptr;

// The lane's index in its wave, computed where it is used: volatile, so
// that the compiler neither hoists it nor keeps an address derived from it
// live across a loop (for blocks that run rarely inside a register-bound
// loop).
__device__ __forceinline__ int lane_here()
{
    int id;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(id));
    return id;
}

// 16 bytes through a global-address-space pointer: a generic pointer that
// may point at a __device__ array (the zero descriptor) would otherwise be
// read with a flat load, which also waits on and counts as an LDS access.
__device__ __forceinline__ uint4 load_global16(const void *p)
{
    typedef uint32_t gv4 __attribute__((ext_vector_type(4)));
    const gv4 x = *(const __attribute__((address_space(1))) gv4 *)p;
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the
// wave writes bytes [16*l, 16*l + 16) after `lds_wave_base`, which must be
// the same for the whole wave.
//
// Issued as inline assembly so that the compiler does not track the LDS
// write: its tracking of such copies does not survive the branches of the
// chunk loop, and it would then wait for the prefetch of the next chunk
// before LDS reads of the other buffer.  The LDS base goes in through an
// input operand bound to M0, so the compiler itself loads M0 and knows
// what it holds (nothing is clobbered behind its back).  Callers order the
// write themselves: wait_vmcnt (a compiler barrier as well) before the
// reads, and a barrier where other waves read it; the compiler's own vmcnt
// waits stay safe, as extra loads in flight only make them wait longer.
__device__ __forceinline__ void load_lds16(const void *src, void *lds_wave_base)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_ptr)lds_wave_base;
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The same from a wave-uniform base (in SGPRs) plus a 32-bit per-lane byte
// offset: no per-lane address arithmetic when only the base moves.  The
// base goes through readfirstlane, so that it is in SGPRs even where the
// compiler cannot prove it uniform (where it can, that costs nothing).
__device__ __forceinline__ void load_lds16(const void *sbase, uint32_t voff, void *lds_wave_base)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_ptr)lds_wave_base;
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32);
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(u), "{m0}"(m0) : "memory");
}

// ------------------------------------------------------------ preparation

// Converts one set: one thread per (row, 16-byte part), eight threads per
// row in consecutive lanes.
__device__ __forceinline__ void prep_body(const PrepJob &Q, int blk)
{
    const int t = blk * PREP_THREADS + (int)threadIdx.x;
    const int r = t >> 3, part = t & 7;
    if (r >= max(Q.rowsA, Q.rowsB))
        return;                              // whole rows (row counts are multiples of 256)
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < Q.n)
        v = *reinterpret_cast<const uint4 *>(Q.X + (size_t)r * DIM + 16 * part);
    uint32_t s = bytesum16(v);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    const uint4 x = make_uint4(v.x ^ 0x80808080u, v.y ^ 0x80808080u, v.z ^ 0x80808080u,
                               v.w ^ 0x80808080u);
    if (r < Q.rowsA) {
        const int b = r / BLOCK_ROWS, w = (r % BLOCK_ROWS) / WAVE_ROWS, qr = r & 31;
        const int nn = 8 * ((qr >> 2) & 3) + 4 * (qr >> 4) + (qr & 3);   // q(nn) = qr
        const int kc = part >> 1, hh = part & 1;
        const size_t off = ((((size_t)b * TILE_WAVES + w) * 4 + kc) * 64 + 32 * hh + nn) * 16;
        *reinterpret_cast<uint4 *>(Q.Af + off) = x;
        if (part == 0)
            Q.RT[r] = (int32_t)(128u * s) - 2097152;
    }
    if (r < Q.rowsB) {
        const int c = r >> 8, j = r & 255;
        const size_t off = (((size_t)c * 8 + part) * CHUNK + j) * 16;
        *reinterpret_cast<uint4 *>(Q.Bp + off) = x;
        if (part == 0)
            Q.P[r] = ((128u * s) << 9) + (uint32_t)(511 - ((r >> 5) & 511));
    }
}

// (The block size is a template argument: reading blockDim or gridDim costs
// a load from the dispatch packet at kernel start.)
template <int BS>
__device__ __forceinline__ void clear_body(const Clear &C)
{
    if (blockIdx.y != 0)
        return;
    for (size_t k = (size_t)blockIdx.x * BS + threadIdx.x; k < C.words; k += C.stride)
        C.p[k] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ __launch_bounds__(PREP_THREADS) void serac_prep_pair(PrepPair Q, Clear C)
{
    clear_body<PREP_THREADS>(C);
    prep_body(Q.q[blockIdx.y], blockIdx.x);
}

__global__ __launch_bounds__(PREP_THREADS) void serac_prep_many(const PrepJob *__restrict__ Q,
                                                                Clear C)
{
    clear_body<PREP_THREADS>(C);
    prep_body(Q[blockIdx.y], blockIdx.x);
}

// ------------------------------------------------------------ tile sweep

// The fused sweep of one workgroup: 256 rows of A (row block rb) against
// chunks [c0, c0 + nch) of B.
//
// Accumulator layout of the 32x32 MFMA: lane l, register r holds output row
// 8*(r/4) + 4*(l/32) + r%4 of column l%32.  The operand row that feeds
// output row m is wave row q(m) = 16*((m/4)%2) + 4*(m/8) + m%4, so lane half
// h, register r is wave row 16*h + r: each lane half covers 16 consecutive
// rows (one column tie-break slice).
//
// A lane only ever sees columns l%32 + 32*t of the workgroup's range, so
// its running top-2 keys carry t in their low 9 bits and stay valid across
// chunks; the 32 lanes sharing a row are merged once at the end.
//
// Schedule per chunk (4 tile pairs, k = 0..3): step k issues the MFMAs of
// pair k, runs the epilogue of pair k-1 (pair 3 of the previous chunk for
// k = 0) and reads the operands of pair k+1 from LDS; the accumulators
// alternate between two register sets.  Chunk c+1 is fetched into the other
// LDS buffer while chunk c is swept.
//
// Each workgroup writes, per row and column group, one packed slot (best,
// column, second) with a plain store, and raises the column best of its
// columns with 64-bit atomic maxima; nothing is read back.
//
// FUSED sweeps read the raw descriptors and convert them on the way (what
// the preparation kernel does otherwise): the wave's A operands and row
// terms in the prologue, and each chunk of B in two stages, a copy of the
// raw chunk into LDS and, during the chunk before the one that needs it,
// its conversion into the operand planes and the columns' key addends.
// Workgroup order: the tile a workgroup sweeps is (a * x + b) mod n of its
// dispatch index x, a bijection for gcd(a, n) = 1 (the host keeps
// a * (n - 1) + b below 2^32).  The library launches
// with a = 1, b = 0 (the XCD-aware map below); other values only come from a
// test hook that checks that results do not depend on the order in which
// workgroups run (their merges are all order-independent maxima).
struct WgOrder {
    uint32_t a, b;
};

__device__ __forceinline__ int wg_index(uint32_t x, WgOrder o, uint32_t n)
{
    if (o.a == 1u && o.b == 0u)
        return (int)x;
    return (int)((o.a * x + o.b) % n);
}

template <bool COLS, bool FUSED, bool NARROW, bool STRIP = false>
__device__ __forceinline__ void tiles_body(const Job &J, int u, const Job *__restrict__ jobs = nullptr,
                                           const int32_t *__restrict__ segJob = nullptr,
                                           int nseg = 1)
{
    static_assert(!(STRIP && FUSED), "a strip sweeps prepared sets");
    // chunk buffers (operand planes), and for a fused sweep the raw chunk;
    // for a strip, its tables of chunks and of segments after them
    constexpr int STRIP_TABLE = STRIP ? 4 * STRIP_MAX_SEG * MAX_GCH + sizeof(SegRef) * STRIP_MAX_SEG : 0;
    __shared__ __attribute__((aligned(16))) uint8_t sB[(FUSED ? 3 : 2) * BUF_BYTES + STRIP_TABLE];
    __shared__ __attribute__((aligned(16))) uint32_t sP[2 * CHUNK];
    __shared__ uint32_t sCol[COLS ? COL_RING * CHUNK : 1];   // ring of chunks: chunk c at c % 8
    // lane-merge scratch, 8448 bytes per wave; a fused sweep merges in the LDS
    // its chunks no longer use
    __shared__ uint2 sScr[FUSED ? 1 : TILE_WAVES * SCR_WAVE];
    __shared__ __attribute__((aligned(16))) int32_t sRT[FUSED ? BLOCK_ROWS : 1];
    uint8_t *const sRaw = sB + 2 * BUF_BYTES;

    // a strip's stream of chunks (segment << 8 | chunk inside it) and what
    // the sweep needs of each segment's pair, in the space past the two
    // chunk buffers that a fused sweep uses for its raw chunk (a strip is
    // never fused)
    int32_t *const sChunk = reinterpret_cast<int32_t *>(sB + 2 * BUF_BYTES);
    SegRef *const sSeg =
        reinterpret_cast<SegRef *>(sB + 2 * BUF_BYTES + 4 * STRIP_MAX_SEG * MAX_GCH);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int rb = STRIP ? u : u % J.nRB, cg = STRIP ? 0 : u / J.nRB;
    const int c0 = cg * J.gch;
    const int nch = [&]() {
        if constexpr (STRIP) {
            // every segment is one pair's whole B (one column group), so the
            // stream has sum(nBC) chunks; the table is read after the
            // barrier that ends the prologue (chunk 0 is segment 0's chunk 0)
            int start = 0;
            for (int s = 0; s < nseg; ++s) {
                const Job &Js = jobs[segJob[s]];
                const int m = Js.nBC;
                for (int k = tid; k < m; k += TILE_THREADS)
                    sChunk[start + k] = (s << 8) | k;
                if (tid == 0)
                    sSeg[s] = SegRef{Js.Bp, Js.P, Js.cbest, Js.rslot, Js.nB, Js.nBC};
                start += m;
            }
            return start;
        } else {
            return min(J.gch, J.nBC - c0);
        }
    }();
    // a segment's entry, read at a uniform LDS address into scalars
    auto seg_ref = [&](int s) {
        SegRef r;
        const uint64_t *q = reinterpret_cast<const uint64_t *>(sSeg + s);
        auto u64 = [](uint64_t v) {
            return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v) |
                   ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32);
        };
        r.Bp = reinterpret_cast<const uint8_t *>(u64(q[0]));
        r.P = reinterpret_cast<const uint32_t *>(u64(q[1]));
        r.cbest = reinterpret_cast<unsigned long long *>(u64(q[2]));
        r.rslot = reinterpret_cast<unsigned long long *>(u64(q[3]));
        r.nB = __builtin_amdgcn_readfirstlane(sSeg[s].nB);
        r.nBC = __builtin_amdgcn_readfirstlane(sSeg[s].nBC);
        return r;
    };
    // STRIP: a position in the stream of chunks (segment, chunk inside it,
    // the segment's chunk count), kept in scalars.  next() moves it on by
    // one chunk and reads the segment table, an LDS read the wave has to
    // wait for together with all its LDS traffic in flight, only when it
    // enters a new segment (once per pair, not once per chunk); it returns
    // whether it did.
    struct Pos {
        int s, lc, nbc;
    };
    auto next = [&](Pos &p) {
        if (++p.lc < p.nbc)
            return false;
        p.lc = 0;
        if (++p.s < nseg)
            p.nbc = __builtin_amdgcn_readfirstlane(sSeg[p.s].nBC);
        return true;
    };
    // segment and chunk (inside its column group) of stream chunk c
    auto chunk_at = [&](int c, int &s, int &lc) {
        if constexpr (STRIP) {
            const int v = __builtin_amdgcn_readfirstlane(sChunk[c]);
            s = v >> 8;
            lc = v & 255;
        } else {
            s = 0;
            lc = c0 + c;
        }
    };

    // ---- fused sweep: raw chunk copy (contiguous, like the chunk itself) and
    // its conversion.  Each wave converts only bytes it copied itself (no
    // barrier needed): lane l takes half l&1 of column 64*(l>>4) + 8*w +
    // ((l>>1)&7).
    const int hf = lane & 1;
    const int hcol = 64 * (lane >> 4) + 8 * w + ((lane >> 1) & 7);
    auto fetch_raw = [&](int c) {
        const int col0 = (c0 + c) * CHUNK;
        if (col0 + CHUNK <= J.nB) {
            // a whole chunk: 32 KiB from one scalar base, the lane offsets fixed
            const uint8_t *base = J.B + (size_t)col0 * DIM;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                load_lds16(base + k * (TILE_THREADS * 16), (uint32_t)tid * 16u,
                           sRaw + k * (TILE_THREADS * 16) + w * 1024);
        } else {
            // the ragged last chunk: columns past the set read the zero descriptor
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int off = k * (TILE_THREADS * 16) + tid * 16;    // byte of the chunk
                const int col = col0 + off / DIM;
                const uint8_t *src = col < J.nB ? J.B + (size_t)col * DIM + off % DIM
                                                : g_zero_desc + off % DIM;
                load_lds16(src, sRaw + k * (TILE_THREADS * 16) + w * 1024);
            }
        }
    };
    auto convert = [&](int c, int buf) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            v[k] = *reinterpret_cast<const uint4 *>(sRaw + hcol * DIM + 64 * hf + 16 * k);
        uint32_t sum = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            sum += bytesum16(v[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<uint4 *>(sB + buf * BUF_BYTES + (4 * hf + k) * PLANE_BYTES +
                                       hcol * 16) =
                make_uint4(v[k].x ^ 0x80808080u, v[k].y ^ 0x80808080u, v[k].z ^ 0x80808080u,
                           v[k].w ^ 0x80808080u);
        // the other half of the column is in the neighbouring lane
        sum += (uint32_t)__builtin_amdgcn_mov_dpp((int)sum, 0xB1, 0xF, 0xF, false);
        const int col = (c0 + c) * CHUNK + hcol;
        if (hf == 0)
            sP[buf * CHUNK + hcol] = ((128u * sum) << 9) + (uint32_t)(511 - ((col >> 5) & 511));
    };

    // ---- this wave's rows of A: operand fragments and the row terms
    v4i af[4];
    v16i ci;
    if (FUSED) {
        fetch_raw(0);
        // lane (n, h) holds bytes [32*kc + 16*h, +16) of wave row q(n)
        const int qn = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
        const int row = rb * BLOCK_ROWS + w * WAVE_ROWS + qn;
        const uint8_t *ra = (row < J.nA ? J.A + (size_t)row * DIM : g_zero_desc) + 16 * h;
        uint4 v4[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
            v4[kc] = load_global16(ra + 32 * kc);
        uint32_t sa = 0u;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const uint4 v = v4[kc];
            sa += bytesum16(v);
            af[kc] = (v4i){(int)(v.x ^ 0x80808080u), (int)(v.y ^ 0x80808080u),
                           (int)(v.z ^ 0x80808080u), (int)(v.w ^ 0x80808080u)};
        }
        sa += __shfl_xor(sa, 32);             // the row's other 64 bytes
        // row terms into the C-input order: lane half h, register r <- wave
        // row 16*h + r (through this wave's slice of sRT)
        if (h == 0)
            sRT[w * WAVE_ROWS + qn] = (int32_t)(128u * sa) - 2097152;
        __builtin_amdgcn_wave_barrier();
        const v4i *pr = reinterpret_cast<const v4i *>(sRT + w * WAVE_ROWS + 16 * h);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const v4i x = pr[g];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ci[4 * g + e] = x[e];
        }
    } else {
        const v4i *pa =
            reinterpret_cast<const v4i *>(J.Af) + (size_t)(rb * TILE_WAVES + w) * 256 + lane;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
            af[kc] = pa[64 * kc];
        const v4i *pr = reinterpret_cast<const v4i *>(J.RT + rb * BLOCK_ROWS + w * WAVE_ROWS +
                                                      16 * h);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const v4i x = pr[g];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ci[4 * g + e] = x[e];
        }
    }

    // ---- column maxima of chunk cc raised into the global column bests,
    // column k.  A FlushRef holds the column bests, first column and width
    // of the pair chunk cc belongs to: the job's, or for a strip its
    // segment's.
    struct FlushRef {
        unsigned long long *cbest;
        int col0, nB;
    };
    auto flush_ref = [&](int cc) {
        if constexpr (STRIP) {
            int s, lc;
            chunk_at(cc, s, lc);
            const SegRef r = seg_ref(s);
            return FlushRef{r.cbest, lc * CHUNK, r.nB};
        } else {
            return FlushRef{J.cbest, (c0 + cc) * CHUNK, J.nB};
        }
    };
    auto flush_col = [&](const FlushRef &f, int cc, int k) {
        const int col = f.col0 + k;
        const uint32_t key = sCol[(cc & (COL_RING - 1)) * CHUNK + k];
        if (col < f.nB && (key >> 9) > 0u) {
            const uint32_t slice = (uint32_t)(rb * (BLOCK_ROWS / SLICE) + 511 - (int)(key & 511u));
            if constexpr (NARROW)
                atomicMax(reinterpret_cast<uint32_t *>(f.cbest) + col, (key & ~511u) | (511u - slice));
            else
                atomicMax(f.cbest + col,
                          ((unsigned long long)(key >> 9) << 32) | (0xFFFFFFFFu - slice));
        }
    };

    // ---- chunk staging of prepared sets: 8 + (wave 0) 1 loads per thread
    // STRIP: the chunk the next stage() copies (segment 0's first chunk
    // to begin with, from the job itself) and its segment's operands
    Pos fpos{0, 0, J.nBC};
    const uint8_t *fB = J.Bp;
    const uint32_t *fP = J.P;
    auto stage = [&](int c, int buf) {
        uint8_t *dst = sB + buf * BUF_BYTES + w * 1024;
        if constexpr (STRIP) {
            // uniform bases plus fixed lane offsets
            const uint8_t *base = fB + (size_t)fpos.lc * CHUNK_BYTES;
#pragma unroll
            for (int k = 0; k < CHUNK_BYTES / (TILE_THREADS * 16); ++k)
                load_lds16(base + k * (TILE_THREADS * 16), (uint32_t)tid * 16u,
                           dst + k * (TILE_THREADS * 16));
            if (w == 0)                      // 16 bytes (four addends) per lane
                load_lds16(fP + (size_t)fpos.lc * CHUNK, (uint32_t)lane_here() * 16u,
                           sP + buf * CHUNK);
            // on to the next chunk (chunk 0's successor is set up after the
            // barrier that makes the tables readable)
            if (c > 0 && next(fpos) && fpos.s < nseg) {
                const SegRef r = seg_ref(fpos.s);
                fB = r.Bp;
                fP = r.P;
            }
        } else {
            const uint8_t *src = J.Bp + (size_t)(c0 + c) * CHUNK_BYTES + tid * 16;
#pragma unroll
            for (int k = 0; k < CHUNK_BYTES / (TILE_THREADS * 16); ++k)
                load_lds16(src + k * (TILE_THREADS * 16), dst + k * (TILE_THREADS * 16));
            if (w == 0)
                load_lds16(J.P + (size_t)(c0 + c) * CHUNK + lane * 4, sP + buf * CHUNK);
        }
    };
    if (!FUSED)
        stage(0, 0);
    if (COLS) {
        for (int k = tid; k < min(nch, COL_RING) * CHUNK; k += TILE_THREADS)
            sCol[k] = 0u;
    }
    wait_vmcnt<0>();                         // chunk 0 and the A operands landed
    if (FUSED) {
        convert(0, 0);
        if (nch > 1)
            fetch_raw(1);                    // after the read-back (the plane stores use it)
    }
    __syncthreads();
    if constexpr (STRIP) {
        if (nch > 1) {
            int s1, lc1;
            chunk_at(1, s1, lc1);
            const SegRef r = seg_ref(s1);
            fpos = Pos{s1, lc1, r.nBC};
            fB = r.Bp;
            fP = r.P;
        }
    }
    if (!FUSED && nch > 1)
        stage(1, 1);                         // needed one chunk from now

    v4i bf[2][4];        // [tile][k-slice]: operands of the next pair
    uint32_t pk[2][2];   // [set][tile] key addends
    v16i acc[2][2];      // [set][tile]
    // The running top-2 starts from a zero the compiler cannot see through:
    // with a literal 0 the gfx950 register coalescer merged one of these
    // initial values into the zero upper half of a 64-bit address and lost
    // it (the machine verifier reports "no live subrange at use").
    uint32_t zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    uint32_t b1[16], b2[16], tk[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        b1[x] = zero;
        b2[x] = zero;
        tk[x] = zero;
    }
    const uint32_t tag = (uint32_t)(511 - (2 * w + h));

    auto frags = [&](int buf, int pr, int set) {
        const uint8_t *base = sB + buf * BUF_BYTES + h * PLANE_BYTES + n * 16 + pr * 1024;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                bf[tt][kc] =
                    *reinterpret_cast<const v4i *>(base + kc * 2 * PLANE_BYTES + tt * 512);
            pk[set][tt] = sP[buf * CHUNK + pr * 64 + tt * 32 + n];
        }
    };
    auto mfma = [&](int set) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                acc[set][tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    af[kc], bf[tt][kc], kc == 0 ? ci : acc[set][tt], 0, 0, 0);
        }
    };
    // epilogue of tile pair `pr` of chunk `c`, held in register set `set`;
    // `odd` pairs close the deferred second-best update
    auto epi = [&](int set, int c, int pr, auto odd) {
        uint32_t k0[16], k1[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            k0[rr] = ((uint32_t)acc[set][0][rr] << 9) + pk[set][0];
            k1[rr] = ((uint32_t)acc[set][1][rr] << 9) + pk[set][1];
        }
        if (COLS) {
            uint32_t m0[5], m1[5];
#pragma unroll
            for (int g = 0; g < 5; ++g) {
                m0[g] = umax3(k0[3 * g], k0[3 * g + 1], k0[3 * g + 2]);
                m1[g] = umax3(k1[3 * g], k1[3 * g + 1], k1[3 * g + 2]);
            }
            const uint32_t cm0 = max(umax3(m0[0], m0[1], m0[2]), umax3(m0[3], m0[4], k0[15]));
            const uint32_t cm1 = max(umax3(m1[0], m1[1], m1[2]), umax3(m1[3], m1[4], k1[15]));
            uint32_t *cp = sCol + (c & (COL_RING - 1)) * CHUNK + pr * 64 + n;
            atomicMax(cp, (cm0 & ~511u) | tag);
            atomicMax(cp + 32, (cm1 & ~511u) | tag);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const uint32_t md = umed3(b1[rr], k0[rr], k1[rr]);
            b1[rr] = umax3(b1[rr], k0[rr], k1[rr]);
            if (decltype(odd)::value)
                b2[rr] = umax3(b2[rr], tk[rr], md);
            else
                tk[rr] = md;
        }
    };
    using Even = std::integral_constant<bool, false>;
    using Odd = std::integral_constant<bool, true>;

    // Steps do not mix: each step's MFMAs, epilogue and operand reads are
    // scheduled among themselves.
    auto step_end = [&]() { __builtin_amdgcn_sched_barrier(0); };

    // ---- merge the 32 lanes that share each row, through this wave's own
    // LDS scratch (no barrier: only this wave writes and reads it): lane pair
    // (q, q + 32) merges the entries of source lanes 0..15 and 16..31 of row
    // q pairwise in a four-level tree (dependency depth 4 instead of a
    // 16-step chain), the lower source lane first in every pair, so on a
    // key tie (same score, same tile) the lowest lane, which is the lowest
    // column, stays.
    // Entry e of row r sits at 33*r + e (rows padded by one entry): the
    // stores of one row and the loads of one entry from 32 rows both fall on
    // distinct banks, and every access is a fixed offset from a per-lane
    // base.  A fused sweep uses the buffers its chunks left free (every wave
    // is past the last chunk barrier): the buffer of chunk nch-2 for waves
    // 0..3, the raw copy for waves 4..7.
    // STRIP: also at every segment boundary, for the pair the segment ended
    // (a fused sweep never has one); there, inside the loop, the 16 entries
    // are merged in a chain in lane order instead (the same keys and the
    // same lowest lane on a tie, with fewer registers live beside the
    // accumulators).
    auto publish = [&](unsigned long long *rslot, int cgs, int c0s, auto chain) {
        // the lane's row and half; inside the loop taken afresh from the
        // lane id (volatile, so that the compiler keeps this block's
        // addresses out of the registers live across the whole loop)
        int nl = n, hl = h;
        if constexpr (decltype(chain)::value) {
            const int id = lane_here();
            nl = id & 31;
            hl = id >> 5;
        }
        uint2 *scr;
        if (FUSED)
            scr = reinterpret_cast<uint2 *>((w < 4 ? sB + (nch & 1) * BUF_BYTES : sRaw)) +
                  (w & 3) * SCR_WAVE;
        else
            scr = sScr + w * SCR_WAVE;
        // Row 16h + rr, entry n is at wb + SCR_ROW*rr, and row n, entry 16h + k
        // at rb + k.
        uint2 *const wb = scr + SCR_ROW * 16 * hl + nl;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            wb[SCR_ROW * rr] = make_uint2(b1[rr], b2[rr]);
        const uint2 *const rbp = scr + SCR_ROW * nl + 16 * hl;
        uint32_t K1, K2;
        int L1;                                              // source lane (column in the tile)
        if constexpr (decltype(chain)::value) {
            K1 = 0u;
            K2 = 0u;
            int k1 = 0;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint2 e = rbp[k];
                k1 = e.x > K1 ? k : k1;
                K2 = umax3(min(K1, e.x), K2, e.y);
                K1 = max(K1, e.x);
            }
            L1 = 16 * hl + k1;
        } else {
            uint32_t t1[16], t2[16];
            int tl[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint2 e = rbp[k];
                t1[k] = e.x;
                t2[k] = e.y;
                tl[k] = k;
            }
#pragma unroll
            for (int s = 1; s < 16; s *= 2) {
#pragma unroll
                for (int k = 0; k < 16; k += 2 * s) {
                    const uint32_t a1 = t1[k], b1 = t1[k + s];
                    tl[k] = b1 > a1 ? tl[k + s] : tl[k];
                    t2[k] = umax3(min(a1, b1), t2[k], t2[k + s]);
                    t1[k] = max(a1, b1);
                }
            }
            K1 = t1[0];
            K2 = t2[0];
            L1 = 16 * hl + tl[0];
        }
        {
            // lane half 0 holds the lower source lanes: it keeps its own on a tie
            const uint32_t o1 = __shfl_xor(K1, 32), o2 = __shfl_xor(K2, 32);
            const int oL = __shfl_xor(L1, 32);
            L1 = (o1 > K1 || (hl == 1 && o1 == K1)) ? oL : L1;
            K2 = umax3(min(K1, o1), K2, o2);
            K1 = max(K1, o1);
        }
        // publish this row block's top-2 over the workgroup's columns as one
        // packed slot per (row, column group); the finishing kernel merges the
        // groups
        const int row = rb * BLOCK_ROWS + w * WAVE_ROWS + nl;
        if (hl == 0 && row < J.nA) {
            const uint32_t S1 = K1 >> 9, S2 = K2 >> 9;
            const int window = (c0s * CHUNK) & ~(GROUP_MAX - 1);
            const uint32_t col = (uint32_t)(window + 32 * (511 - (int)(K1 & 511u)) + L1);
            rslot[(size_t)cgs * J.nA + row] = pack_slot(S1, col, S2);
        }
    };

    // chunk c: pairs 1..3 of the chunk and pair 0 of the next one (pair 0
    // of chunk 0 is issued before the loop)
    // Issue priority of the two waves sharing a SIMD: with equal priorities
    // the older wave is always issued first and the other finishes every
    // chunk alone.  The younger wave takes the higher priority in steps 0..2
    // (and the conversion after step 1), the older one in step 3; with this
    // split both arrive at the chunk barrier about together (measured: an
    // even split still left the younger wave ~0.5 us behind per chunk).
    const bool second = (w >> 2) & 1;        // waves w and w + 4 share a SIMD
    auto turn = [&](int k) {
        if ((k != 3) == second)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
    };
    // STRIP: positions of the chunk being swept and of the chunk whose
    // column maxima are flushed next, with that chunk's column bests
    Pos cpos{0, 0, J.nBC}, xpos{0, 0, J.nBC};
    FlushRef xref{J.cbest, 0, J.nB};
    // `when`: whether chunk c is the last, known at compile time in a strip
    // (its last chunk is peeled off the loop: with a branch on it in the
    // loop body the compiler hoisted the last pair's key construction, common
    // to both arms, above the branch, which then waited for the step's MFMAs
    // before the chunk barrier), tested at run time otherwise
    auto chunk = [&](int c, auto when) {
        const int buf = c & 1;
        if constexpr (STRIP) {
            // chunk c starts a new segment: the previous pair's rows are
            // complete (a chunk's last pair closes the deferred fold), so
            // they are published and the running top-2 starts again.  Done
            // before the step's MFMAs are issued, so that the step stays one
            // block in which the compiler interleaves them with the
            // epilogue.
            if (c > 0 && cpos.lc == 0) {
                publish(seg_ref(cpos.s - 1).rslot, 0, 0, std::true_type{});
                // a fresh opaque zero (see above), not one kept live across
                // the loop
                uint32_t z;
                asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    b1[x] = z;
                    b2[x] = z;
                }
            }
        }
        turn(1);
        mfma(1);
        epi(0, c, 0, Even{});
        frags(buf, 2, 0);
        step_end();
        if (FUSED && c + 1 < nch) {
            // chunk c+1 into the buffer chunk c-1 used; then the raw copy of
            // chunk c+2 (the reads of this thread's part of the raw copy have
            // returned: the plane stores before it use their data)
            wait_vmcnt<0>();
            convert(c + 1, buf ^ 1);
            if (c + 2 < nch)
                fetch_raw(c + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (COLS && c >= COL_RING - 1) {
            // chunk c-7's column maxima are final (every wave is past two
            // chunk barriers since); its ring slot is chunk c+1's
            if constexpr (STRIP) {
                // waves 0..3 (the test on the wave index keeps the flush
                // position in scalars)
                if (w < CHUNK / 64) {
                    flush_col(xref, c - (COL_RING - 1), tid);
                    sCol[((c + 1) & (COL_RING - 1)) * CHUNK + tid] = 0u;
                    if (next(xpos) && xpos.s < nseg) {
                        const SegRef r = seg_ref(xpos.s);
                        xref = FlushRef{r.cbest, 0, r.nB};
                    }
                    xref.col0 = xpos.lc * CHUNK;
                }
            } else if (tid < CHUNK) {
                flush_col(flush_ref(c - (COL_RING - 1)), c - (COL_RING - 1), tid);
                sCol[((c + 1) & (COL_RING - 1)) * CHUNK + tid] = 0u;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        turn(2);
        mfma(0);
        epi(1, c, 1, Odd{});
        frags(buf, 3, 1);
        step_end();
        turn(3);
        mfma(1);
        epi(0, c, 2, Even{});
        step_end();
        constexpr int WHEN = decltype(when)::value;   // 0: not last, 1: last, 2: test
        if (WHEN == 2 ? c + 1 < nch : WHEN == 0) {
            if (!FUSED)
                wait_vmcnt<0>();             // chunk c+1 landed (this wave's part)
            __syncthreads();                 // ... all parts; chunk c no longer read
            if (!FUSED && c + 2 < nch)
                stage(c + 2, buf);
            frags(buf ^ 1, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            turn(0);
            mfma(0);
            epi(1, c, 3, Odd{});
            frags(buf ^ 1, 1, 1);
            step_end();
        } else {
            epi(1, c, 3, Odd{});
        }
        if constexpr (STRIP)
            next(cpos);
    };

    frags(0, 0, 0);
    mfma(0);
    frags(0, 1, 1);
    step_end();
    if constexpr (STRIP) {
        for (int c = 0; c < nch - 1; ++c)
            chunk(c, std::integral_constant<int, 0>{});
        chunk(nch - 1, std::integral_constant<int, 1>{});
    } else {
        for (int c = 0; c < nch; ++c)
            chunk(c, std::integral_constant<int, 2>{});
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- column maxima out first: their atomics complete behind the merge
    if (COLS) {
        lds_barrier();                       // every wave's column maxima are in
        // the chunks still in the ring (a strip's table read is convergent:
        // that loop is not unrolled)
        const uint32_t k0 = (uint32_t)(max(nch - (COL_RING - 1), 0) * CHUNK + tid);
        if constexpr (STRIP) {
            for (uint32_t k = k0; k < (uint32_t)(nch * CHUNK); k += TILE_THREADS)
                flush_col(flush_ref((int)(k / CHUNK)), (int)(k / CHUNK), (int)(k % CHUNK));
        } else {
#pragma unroll 2
            for (uint32_t k = k0; k < (uint32_t)(nch * CHUNK); k += TILE_THREADS)
                flush_col(flush_ref((int)(k / CHUNK)), (int)(k / CHUNK), (int)(k % CHUNK));
        }
    }

    if constexpr (STRIP)
        publish(seg_ref(nseg - 1).rslot, 0, 0, std::false_type{});
    else
        publish(J.rslot, cg, c0, std::false_type{});
}

// NARROW: the column bests take 32 bits (J.cb32; see col_best_at).
template <bool COLS, bool NARROW>
__global__ __launch_bounds__(TILE_THREADS, 2) void serac_tiles_one(Job J, WgOrder o)
{
    tiles_body<COLS, false, NARROW>(J, wg_index(blockIdx.x, o, (uint32_t)(J.nRB * J.Gc)));
}

// One pair straight from the raw descriptors (no preparation kernel); also
// clears what the previous call on the stream left raised (the other
// accumulator region, which this call does not touch).
//
// The fields the sweep needs first are also passed as leading scalar
// arguments: the build preloads the first 16 argument dwords into SGPRs at
// wave launch, while a struct argument is read from the argument buffer in
// memory before the first load can be addressed.  They override the copies
// in J.
template <bool COLS, bool NARROW>
__global__ __launch_bounds__(TILE_THREADS, 2) void serac_tiles_fused(
    const uint8_t *A, const uint8_t *B, int32_t nA, int32_t nB, int32_t nRB, int32_t nBC,
    int32_t gch, uint4 *clear_p, uint32_t clear_words, uint32_t clear_stride, uint32_t order_a,
    uint32_t order_b, uint32_t units, Job J)
{
    J.A = A;
    J.B = B;
    J.nA = nA;
    J.nB = nB;
    J.nRB = nRB;
    J.nBC = nBC;
    J.gch = gch;
    clear_body<TILE_THREADS>(Clear{clear_p, clear_words, clear_stride});
    tiles_body<COLS, true, NARROW>(J, wg_index(blockIdx.x, WgOrder{order_a, order_b}, units));
}

template <bool COLS, bool NARROW>
__global__ __launch_bounds__(TILE_THREADS, 2) void serac_tiles_many(const Job *__restrict__ jobs,
                                                                    int unitsPerJob, WgOrder o,
                                                                    uint32_t blocks)
{
    const int x = wg_index(blockIdx.x, o, blocks);
    const Job J = jobs[x / unitsPerJob];
    const int u = x % unitsPerJob;
    if (u >= J.nRB * J.Gc)
        return;
    tiles_body<COLS, false, NARROW>(J, u);
}

// Cross-pair reuse of a staged row block in a batch (an exhaustive image
// set matches each image as A against many others).  One workgroup sweeps
// row block rb of an image against the B sides of up to STRIP_MAX_SEG pairs
// that share that image as A, as one stream of chunks: the A operands and
// row terms are loaded once, and the software pipeline runs on across the
// pairs, the first chunks of the next pair staged while the last ones of
// the current pair are swept, so only one prologue is paid per strip.  The
// reductions are segmented at the pairs' boundaries: when a chunk starts a
// new pair, the finished pair's row top-2 goes through the lane merge into
// its slots and the running keys start again from zero; column maxima go
// to the column bests of the pair their chunk belongs to.  Every pair of a
// strip has its whole B in one column group (at most 16384 columns, the
// keys' tile index), so its slots and column bests are the same as a
// single-pair sweep's and the finishing kernel is unchanged.
//   strips[s] = (first entry in stripJobs, number of pairs), the pairs'
//   jobs listed in stripJobs, all with the same A; workgroup x sweeps row
//   block x % rbPerStrip of strip x / rbPerStrip.
struct StripRef {
    int32_t first, count;
};

template <bool COLS, bool NARROW>
__global__ __launch_bounds__(TILE_THREADS, 2) void serac_tiles_strip(
    const Job *__restrict__ jobs, const int32_t *__restrict__ stripJobs,
    const StripRef *__restrict__ strips, int rbPerStrip, WgOrder o, uint32_t blocks)
{
    const int x = wg_index(blockIdx.x, o, blocks);
    const StripRef S = strips[x / rbPerStrip];
    const int rb = x % rbPerStrip;
    const Job J = jobs[stripJobs[S.first]];
    if (rb >= J.nRB)
        return;
    tiles_body<COLS, false, NARROW, true>(J, rb, jobs, stripJobs + S.first, S.count);
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

// Row i's result over all column groups: best score, its column (-1 below
// the zero floor) and the second score.  The best slot wins (highest score,
// then lowest column); the second is the largest of every group's second
// and every other group's best, ties counted.
__device__ __forceinline__ void row_result(const Job &J, int i, uint32_t &S1, int32_t &I1,
                                           uint32_t &S2)
{
    unsigned long long best = 0ull;
    uint32_t sec = 0u, loser = 0u;
    const int groups = J.nB > 0 ? J.Gc : 0;   // no sweep ran against an empty set
    for (int g0 = 0; g0 < groups; g0 += 8) {
        // eight groups' slots in flight at once
        unsigned long long v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = g0 + k < groups ? J.rslot[(size_t)(g0 + k) * J.nA + i] : 0ull;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const unsigned long long lo = min(best, v[k]);
            loser = max(loser, (uint32_t)(lo >> 41));
            best = max(best, v[k]);
            sec = max(sec, (uint32_t)(v[k] & 0x7FFFFFu));
        }
    }
    S1 = (uint32_t)(best >> 41);
    I1 = S1 ? (int32_t)(SLOT_COL_MAX - (uint32_t)((best >> 23) & SLOT_COL_MAX)) : -1;
    S2 = max(sec, loser);
}

// Row results of the lane `D` places lower in the same 16-lane row (one
// 16-row slice), `fill` where there is none.
template <int D>
__device__ __forceinline__ uint32_t slice_below(uint32_t v, uint32_t fill)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, 0x110 | D, 0xF, 0xF, false);
}

// Column-tie test of the cross-check for a row whose best score S1 equals
// its column's maximum C1: a lower row i2 of the slice scores S(i2, I1) <=
// S1(i2); when I1 is i2's best column S(i2, I1) = S1(i2) (a tie when equal
// to C1), and otherwise S(i2, I1) <= S2(i2), so the exact product is needed
// only when S1(i2) and S2(i2) both reach C1 (bit D of `dots`).  All lanes
// of the wave take part.
template <int D>
__device__ __forceinline__ void slice_ties(uint32_t S1, uint32_t S2, int32_t I1, uint32_t C1,
                                           bool &tie, uint32_t &dots)
{
    const uint32_t s1 = slice_below<D>(S1, 0u);
    const uint32_t s2 = slice_below<D>(S2, 0u);
    const int32_t i1 = (int32_t)slice_below<D>((uint32_t)I1, 0xFFFFFFFFu);
    const bool same = i1 == I1;
    tie = tie | (same & (s1 == C1));
    dots |= (uint32_t)(!same & (s1 >= C1) & (s2 >= C1)) << D;
    if constexpr (D < SLICE - 1)
        slice_ties<D + 1>(S1, S2, I1, C1, tie, dots);
}

// Cross-workgroup hand-off of the finishing kernel: one 64-bit status word
// per finishing workgroup, bits 63..62 the state and bits 31..0 a count.
constexpr unsigned long long ST_OWN = 1ull << 62;        // own match count published
constexpr unsigned long long ST_INCL = 2ull << 62;       // inclusive prefix published
constexpr unsigned long long ST_ERR = 3ull << 62;        // look-back gave up
constexpr int FINISH_SPIN_LIMIT = 1 << 22;   // default look-back polls

__device__ __forceinline__ unsigned long long status_load(unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void status_store(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Gates, cross-check and ordered output of 256 rows, one kernel for the
// whole pair.  Each workgroup decides its rows, publishes its match count
// and sums the counts of the groups before it (decoupled look-back: a group
// only waits for groups dispatched before it, so every wait ends), then
// writes its own matches at that offset.  Only atomic status words cross
// workgroups, so no device-scope fence (an L2 write-back on gfx950) is
// needed.  The last group in the chain writes the count.  The column
// accumulators and the status words are left raised: the next call's
// preparation kernel on this stream clears them before its sweep.  A
// look-back that does not see its predecessors within the spin limit marks
// the pair failed: count -1.
//
// DEV_ANGLE: the ratio and distance gates are taken from the device's angle
// where it settles them (gates_sure), computed while the column best of the
// row's best column is being loaded, so that the table is read only for the
// rare row the device angle leaves open.
//
// SYM: symmetric column gates, in two passes over two sweeps without column
// bests.  SYM_COLUMNS finishes the sweep of the swapped pair (B, A): row r
// of it is column r of the pair, and the kernel writes, densely, the row of
// A that column r accepts under the gates (its best row, lowest on a tie),
// or -1, into that sweep's rs1 (which only the top-2 export uses
// otherwise).  SYM_ROWS finishes the sweep of (A, B): row i passes if it
// passes the gates and its best column accepts exactly row i, which is the
// mutual check and the column's own gates in one comparison.
constexpr int SYM_NONE = 0, SYM_COLUMNS = 1, SYM_ROWS = 2;

template <bool DEV_ANGLE, bool NARROW = false, int SYM = SYM_NONE>
__device__ __forceinline__ void finish_body(const Job &J, int wg, int nwg, const Gate &G,
                                            const int32_t *partner = nullptr)
{
    __shared__ int32_t sWave[GATE_THREADS / 64];
    __shared__ long long sBase;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int i = wg * GATE_THREADS + tid;
    uint32_t S1 = 0u, S2 = 0u;
    int32_t I1 = -1;
    if (i < J.nA)
        row_result(J, i, S1, I1, S2);
    const bool cand = I1 >= 0 && I1 < J.nB;
    uint32_t C1 = 0u;
    int32_t slice = -1;
    bool acc = false;
    const bool cross = SYM == SYM_NONE && G.cross_check;
    if (DEV_ANGLE) {
        // the column best is loaded first and decoded last: the device angles
        // are computed while it is in flight (its width is a template
        // argument, so the load is issued without a branch)
        unsigned long long raw = 0ull;
        if (cross) {
            const int j = cand ? I1 : 0;
            raw = NARROW ? (unsigned long long)reinterpret_cast<const uint32_t *>(J.cbest)[j]
                         : J.cbest[j];
        }
        int sure = gates_sure(S1, S2, G);
        if (cand && sure < 0) {
            const double d1 = G.table[min(S1, (uint32_t)NORM2)];
            const double d2 = G.table[min(S2, (uint32_t)NORM2)];
            sure = (d1 <= G.max_distance) && (d1 < G.max_ratio * d2);
        }
        acc = cand && sure > 0;
        if (NARROW) {
            C1 = (uint32_t)raw >> 9;
            slice = 511 - (int32_t)(raw & 511u);
        } else {
            C1 = (uint32_t)(raw >> 32);
            slice = (int32_t)(0xFFFFFFFFu - (uint32_t)raw);
        }
    } else if (cand) {
        const double d1 = G.table[min(S1, (uint32_t)NORM2)];
        const double d2 = G.table[min(S2, (uint32_t)NORM2)];
        if (cross)
            col_best_at(J, I1, C1, slice);
        acc = (d1 <= G.max_distance) && (d1 < G.max_ratio * d2);
    }
    if (SYM == SYM_COLUMNS) {
        // every thread of the group leaves here: no barrier follows
        if (i < J.nA)
            J.rs1[i] = acc ? (uint32_t)I1 : 0xFFFFFFFFu;
        return;
    }
    if (SYM == SYM_ROWS && acc)
        acc = partner[I1] == i;
    if (cross) {
        acc = acc && C1 == S1 && slice == i / SLICE;
        // Row i is its column's best only if no lower row of its 16-row
        // slice (the lanes below it in its 16-lane row) reaches C1 on that
        // column too; tested in registers for the whole wave at once.
        if (__ballot(acc) != 0ull) {
            bool tie = false;
            uint32_t dots = 0u;
            slice_ties<1>(S1, S2, I1, C1, tie, dots);
            acc = acc && !tie;
            const uint8_t *b = J.B + (size_t)max(I1, 0) * DIM;
            while (acc && dots != 0u) {
                const int d = __ffs(dots) - 1;
                dots &= dots - 1u;
                if ((uint32_t)dot_exact(J.A + (size_t)(i - d) * DIM, b) == C1)
                    acc = false;
            }
        }
    }

    // rank of this row's match inside the group
    const unsigned long long ball = __ballot(acc);
    const int in_wave = __popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0)
        sWave[wv] = __popcll(ball);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < GATE_THREADS / 64; ++k) {
        before += k < wv ? sWave[k] : 0;
        tot += sWave[k];
    }

    // offset of this group's matches: wave 0 looks back over the groups
    // before it, 64 status words at a time, folding own counts until the
    // nearest inclusive prefix
    unsigned long long *st = J.status;
    if (wv == 0) {
        long long base = 0;
        bool failed = false;
        if (wg == 0) {
            if (lane == 0)
                status_store(st, ST_INCL | (unsigned)tot);
        } else {
            if (lane == 0)
                status_store(st + wg, ST_OWN | (unsigned)tot);
            int k0 = wg - 1, spins = 0;
            failed = G.spin_limit < 0;
            // The groups publish within ~0.4 us of each other, and a poll
            // that finds a predecessor still unpublished costs a whole
            // round trip: waiting ~0.4 us first (12 x 64 clocks) lets most
            // look-backs end with their first poll (measured: -0.45 us per
            // 8192 x 8192 call; 32 finishing groups).
            __builtin_amdgcn_s_sleep(12);
            while (!failed) {
                const int k = k0 - lane;
                // before group 0 there is an inclusive prefix of 0
                const unsigned long long v = k >= 0 ? status_load(st + k) : ST_INCL;
                const unsigned long long state = v & ST_ERR;
                const unsigned long long incl = __ballot(state == ST_INCL);
                const int stop = incl ? __ffsll(incl) - 1 : 64;   // nearest inclusive lane
                const unsigned long long upto = stop >= 63 ? ~0ull : ((2ull << stop) - 1ull);
                if (__ballot(state == ST_ERR) & upto) {
                    failed = true;
                    break;
                }
                if (__ballot(state == 0ull) & upto) {
                    if (++spins > G.spin_limit) {
                        failed = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                uint32_t c = lane <= stop ? (uint32_t)v : 0u;
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1)
                    c += __shfl_xor(c, d);
                base += c;
                if (stop < 64)
                    break;
                k0 -= 64;
            }
            if (lane == 0)
                status_store(st + wg, failed ? ST_ERR : (ST_INCL | (unsigned)(base + tot)));
        }
        if (lane == 0) {
            sBase = failed ? -1 : base;
            if (wg == nwg - 1)
                *J.count = failed ? -1 : (int32_t)(base + tot);
        }
    }
    __syncthreads();
    const long long base = sBase;
    if (acc && base >= 0) {
        serac_match m;
        m.a = (uint32_t)i;
        m.b = (uint32_t)I1;
        J.out[base + before + in_wave] = m;
    }
}

// The fields read first as leading scalar arguments (preloaded into SGPRs,
// like the fused sweep's); they override the copies in J and G.
template <bool NARROW>
__global__ __launch_bounds__(GATE_THREADS) void serac_finish_one(
    const unsigned long long *rslot, int32_t nA, int32_t nB, int32_t Gc,
    unsigned long long *cbest, const double *table, int32_t cross_check, Job J, Gate G)
{
    J.rslot = const_cast<unsigned long long *>(rslot);
    J.nA = nA;
    J.nB = nB;
    J.Gc = Gc;
    J.cbest = cbest;
    G.table = table;
    G.cross_check = cross_check;
    finish_body<true, NARROW>(J, blockIdx.x, (J.nA + GATE_THREADS - 1) / GATE_THREADS, G);
}

// The two passes of the symmetric column gates for one pair: SYM_COLUMNS on
// the job of the swapped pair, then SYM_ROWS on the pair's own job with the
// first pass's output as `partner`.
template <int SYM>
__global__ __launch_bounds__(GATE_THREADS) void serac_finish_sym(Job J, Gate G,
                                                                 const int32_t *partner)
{
    finish_body<true, false, SYM>(J, blockIdx.x, (J.nA + GATE_THREADS - 1) / GATE_THREADS, G,
                                  partner);
}

// The same for a batch: jobs [0, npairs) are the pairs, jobs [npairs,
// 2 npairs) the swapped pairs in the same order.
template <int SYM>
__global__ __launch_bounds__(GATE_THREADS) void serac_finish_many_sym(
    const Job *__restrict__ jobs, int gatePerJob, int npairs, Gate G)
{
    const int k = blockIdx.x / gatePerJob;
    const Job J = jobs[SYM == SYM_COLUMNS ? npairs + k : k];
    const int wg = blockIdx.x % gatePerJob;
    const int nwg = (J.nA + GATE_THREADS - 1) / GATE_THREADS;
    if (wg >= nwg)
        return;
    const int32_t *partner =
        SYM == SYM_ROWS ? reinterpret_cast<const int32_t *>(jobs[npairs + k].rs1) : nullptr;
    finish_body<false, false, SYM>(J, wg, nwg, G, partner);
}

__global__ __launch_bounds__(GATE_THREADS) void serac_finish_many(const Job *__restrict__ jobs,
                                                                  int gatePerJob, Gate G)
{
    const Job J = jobs[blockIdx.x / gatePerJob];
    const int wg = blockIdx.x % gatePerJob;
    const int nwg = (J.nA + GATE_THREADS - 1) / GATE_THREADS;
    if (wg >= nwg)
        return;
    finish_body<false>(J, wg, nwg, G);
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
// score is kept in rs1 for the column export.
__global__ void serac_export_rows(Job J, int32_t *row_top2)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= J.nA)
        return;
    uint32_t S1, S2;
    int32_t I1;
    row_result(J, i, S1, I1, S2);
    row_top2[3 * (size_t)i] = (int32_t)S1;
    row_top2[3 * (size_t)i + 1] = I1;
    row_top2[3 * (size_t)i + 2] = (int32_t)S2;
    J.rs1[i] = S1;
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
    uint32_t C1;
    int32_t slice;
    col_best_at(J, j, C1, slice);
    int32_t idx = -1;
    if (C1 > 0u) {
        const uint8_t *b = J.B + (size_t)j * DIM;
        for (int i = slice * SLICE; i < min(slice * SLICE + SLICE, J.nA); ++i) {
            if (J.rs1[i] >= C1 && (uint32_t)dot_exact(J.A + (size_t)i * DIM, b) == C1) {
                idx = i;
                break;
            }
        }
    }
    col_best[2 * (size_t)j] = (int32_t)C1;
    col_best[2 * (size_t)j + 1] = idx;
    if (J.cb32)
        reinterpret_cast<uint32_t *>(J.cbest)[j] = 0u;
    else
        J.cbest[j] = 0ull;
}

// ------------------------------------------------------------ unfused arm
//
// The structure the SERAC README measures its fused kernel against
// ("GPU kernel time", "Memory"): the whole score matrix written to memory,
// then separate row and column passes over it.  Here S (int32 [nA][nB],
// the exact scores) is written by an MFMA kernel, read back by a row pass
// (row top-2, one slot per row) and a column pass (column best, as the
// sweep's atomic maxima leave it), and the finishing kernel does the rest,
// so its lists equal the fused path's.  It is a comparison arm: its memory
// grows as nA * nB and every score crosses HBM three times.

constexpr long long UNFUSED_MAX_SCORES = 1ll << 32;   // nA * nB (16 GiB of scores)
constexpr int SCORE_ROWS = 128;        // rows of A per workgroup (4 waves x 32)
constexpr int SCORE_COLS = 256;        // columns of B per workgroup (8 tiles of 32)
constexpr int SCORE_THREADS = 256;

// S[i][j] for a 128 x 256 block: each wave holds the operand fragments of
// its 32 rows (lane (n, h): bytes [32 kc + 16 h, +16) of row n) and sweeps
// eight 32-column tiles, reading B's fragments straight from memory; the
// row term enters as the MFMA's C input and the column term is added before
// the store.  Rows and columns past the sets read the zero descriptor and
// are not stored.
__global__ __launch_bounds__(SCORE_THREADS) void serac_scores(const uint8_t *A, const uint8_t *B,
                                                              int32_t nA, int32_t nB, int32_t *S)
{
    __shared__ int32_t sRT[SCORE_ROWS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int row0 = blockIdx.y * SCORE_ROWS + w * WAVE_ROWS;
    const int col0 = blockIdx.x * SCORE_COLS;

    const int ra = row0 + n;
    const uint8_t *pa = (ra < nA ? A + (size_t)ra * DIM : g_zero_desc) + 16 * h;
    v4i af[4];
    uint32_t sa = 0u;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        const uint4 v = load_global16(pa + 32 * kc);
        sa += bytesum16(v);
        af[kc] = (v4i){(int)(v.x ^ 0x80808080u), (int)(v.y ^ 0x80808080u),
                       (int)(v.z ^ 0x80808080u), (int)(v.w ^ 0x80808080u)};
    }
    sa += __shfl_xor(sa, 32);
    if (h == 0)
        sRT[w * WAVE_ROWS + n] = (int32_t)(128u * sa) - 2097152;
    __syncthreads();
    // C input: register r of lane half h is output row (r / 4) * 8 + h * 4 + r % 4
    v16i ci;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        ci[r] = sRT[w * WAVE_ROWS + (r >> 2) * 8 + h * 4 + (r & 3)];

    for (int t = 0; t < SCORE_COLS / 32; ++t) {
        const int cb = col0 + 32 * t + n;
        const uint8_t *pb = (cb < nB ? B + (size_t)cb * DIM : g_zero_desc) + 16 * h;
        v4i bf[4];
        uint32_t sb = 0u;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const uint4 v = load_global16(pb + 32 * kc);
            sb += bytesum16(v);
            bf[kc] = (v4i){(int)(v.x ^ 0x80808080u), (int)(v.y ^ 0x80808080u),
                           (int)(v.z ^ 0x80808080u), (int)(v.w ^ 0x80808080u)};
        }
        sb += __shfl_xor(sb, 32);
        v16i acc = ci;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[kc], bf[kc], acc, 0, 0, 0);
        if (cb < nB) {
            const int32_t colterm = (int32_t)(128u * sb);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = row0 + (r >> 2) * 8 + h * 4 + (r & 3);
                if (i < nA)
                    S[(size_t)i * nB + cb] = acc[r] + colterm;
            }
        }
    }
}

// Row pass: one workgroup per row, its threads over the columns in
// ascending steps; each keeps the top two of the 64-bit keys
// (S << 32 | ~j) (largest score, then lowest column; a tie leaves the tied
// score second), merged across the workgroup the same way.  The row's
// result goes out as the single slot of one column group.
__global__ __launch_bounds__(256) void serac_score_rows(const int32_t *S, int32_t nA, int32_t nB,
                                                        unsigned long long *rslot)
{
    __shared__ unsigned long long sK[2][256 / 64];
    const int i = blockIdx.x;
    const int32_t *row = S + (size_t)i * nB;
    unsigned long long k1 = 0ull, k2 = 0ull;
#pragma unroll 8
    for (int j = threadIdx.x; j < nB; j += 256) {
        const unsigned long long k =
            ((unsigned long long)(uint32_t)row[j] << 32) | (0xFFFFFFFFu - (uint32_t)j);
        k2 = max(k2, min(k1, k));
        k1 = max(k1, k);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const unsigned long long o1 = __shfl_xor(k1, d), o2 = __shfl_xor(k2, d);
        k2 = max(max(k2, o2), min(k1, o1));
        k1 = max(k1, o1);
    }
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sK[0][wv] = k1;
        sK[1][wv] = k2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        k1 = sK[0][0];
        k2 = sK[1][0];
        for (int v = 1; v < 256 / 64; ++v) {
            k2 = max(max(k2, sK[1][v]), min(k1, sK[0][v]));
            k1 = max(k1, sK[0][v]);
        }
        const uint32_t S1 = (uint32_t)(k1 >> 32), S2 = (uint32_t)(k2 >> 32);
        const uint32_t col = 0xFFFFFFFFu - (uint32_t)k1;
        rslot[i] = pack_slot(S1, col, S2);
    }
}

// Column pass: a thread per column over a band of rows in ascending order
// (consecutive threads read consecutive columns of a row); the band's best
// goes to the column bests as the sweep leaves them, (S << 32) | ~slice
// raised by an atomic maximum (highest score, then lowest 16-row slice).
constexpr int SCORE_BAND = 512;        // rows per column-pass workgroup

__global__ __launch_bounds__(256) void serac_score_cols(const int32_t *S, int32_t nA, int32_t nB,
                                                        unsigned long long *cbest)
{
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= nB)
        return;
    const int i0 = blockIdx.y * SCORE_BAND, i1 = min(i0 + SCORE_BAND, nA);
    int32_t best = 0, at = -1;
#pragma unroll 16
    for (int i = i0; i < i1; ++i) {
        const int32_t v = S[(size_t)i * nB + j];
        if (v > best) {
            best = v;
            at = i;
        }
    }
    if (at >= 0)
        atomicMax(cbest + j, ((unsigned long long)(uint32_t)best << 32) |
                                 (0xFFFFFFFFu - (uint32_t)(at / SLICE)));
}


// ------------------------------------------------------------------ host

struct Device {
    bool init = false;
    int status = SERAC_OK;
    int cus = 0;
    double *table = nullptr;
    double slack = INFINITY;     // device angles are within this of the table (finish_body)
    int spin_limit = FINISH_SPIN_LIMIT;
};

std::mutex g_mutex;
Device g_devices[64];

// Dispatch-attached timing of tile-kernel launches while profiling is armed:
// each launch carries its own start and stop events (hipExtLaunchKernel), so
// the queue gets no extra marker packets and the launches stay back to back.
struct Profile {
    bool armed = false;
    int used = 0;
    int every = 1;                // time one launch in `every`
    long long seen = 0;           // tile launches since arming
    std::vector<hipEvent_t> ev;   // [2 * max]: start, stop
    const char *kernel = nullptr; // the kernel timed ("mixed" if several)
};
std::mutex g_prof_mutex;
Profile g_prof;

// Per-device state of serac_match_pairs_host, reused across its calls (one
// call at a time per device: `busy`): a copy stream, two events per half of
// the double buffer and the pinned host memory the results land in.
struct HostPipe {
    std::mutex busy;
    bool ready = false;
    hipStream_t copy = nullptr;
    hipEvent_t done[2] = {nullptr, nullptr};     // a stage's matching has run
    hipEvent_t copied[2] = {nullptr, nullptr};   // its results are in pinned memory
    uint8_t *pinned = nullptr;
    size_t pinned_bytes = 0;
};
HostPipe g_pipes[64];
constexpr int HOST_STAGE_PAIRS = 64;     // pairs per pipeline stage unless the caller says

// Event pair for the next tile launch (a launch of the kernel `kernel`),
// or nulls when not armed / full.
void prof_slot(hipEvent_t &start, hipEvent_t &stop, const char *kernel)
{
    start = stop = nullptr;
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    if (!g_prof.armed || 2 * (g_prof.used + 1) > (int)g_prof.ev.size())
        return;
    if (g_prof.seen++ % g_prof.every != 0)
        return;
    start = g_prof.ev[2 * g_prof.used];
    stop = g_prof.ev[2 * g_prof.used + 1];
    ++g_prof.used;
    if (!g_prof.kernel)
        g_prof.kernel = kernel;
    else if (std::strcmp(g_prof.kernel, kernel) != 0)
        g_prof.kernel = "mixed";
}

// Names of the tile kernels as the profiler reports them.
template <bool COLS, bool NARROW>
const char *tile_name(bool fused)
{
    if (fused)
        return COLS ? (NARROW ? "serac_tiles_fused<true, true>" : "serac_tiles_fused<true, false>")
                    : "serac_tiles_fused<false, false>";
    return COLS ? (NARROW ? "serac_tiles_one<true, true>" : "serac_tiles_one<true, false>")
                : "serac_tiles_one<false, false>";
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Test hook: while the environment variable SERAC_TEST_FAIL_ALLOC is set,
// every allocation of device or pinned memory the library would make
// reports failure instead (SERAC_ERR_OUT_OF_MEMORY), so that tests can
// check that such a call enqueues nothing and that a later call recovers.
// Read at each allocation, which only happens when a workspace grows.
bool fail_alloc()
{
    return std::getenv("SERAC_TEST_FAIL_ALLOC") != nullptr;
}

int hip_fail()
{
    (void)hipGetLastError();
    return SERAC_ERR_HIP;
}

// How far the device angle (angle_dev) can be from the host table: the
// largest deviation over the whole domain, measured once on this device,
// doubled, plus 1e-15 for the rounding of a +- slack (finish_body).
// Infinite (every gate decision from the table) if the check cannot run or
// while the environment variable SERAC_TEST_ANGLE_TABLE is set (a test
// hook for the table path).
double angle_slack(const double *table)
{
    if (std::getenv("SERAC_TEST_ANGLE_TABLE") || fail_alloc())
        return INFINITY;
    unsigned long long *err = nullptr, h = 0;
    double slack = INFINITY;
    if (hipMalloc(&err, sizeof(h)) == hipSuccess && hipMemset(err, 0, sizeof(h)) == hipSuccess) {
        serac_angle_check<<<(NORM2 + 1 + 255) / 256, 256>>>(table, err);
        if (hipMemcpy(&h, err, sizeof(h), hipMemcpyDeviceToHost) == hipSuccess) {
            double e;
            std::memcpy(&e, &h, sizeof(e));
            if (std::isfinite(e))
                slack = 2.0 * e + 1e-15;
        }
    }
    if (err)
        (void)hipFree(err);
    (void)hipGetLastError();
    return slack;
}

int fixed_setup(int dev);

// Test hook SERAC_TEST_STRIP_PAIRS=<m> (read at a device's set-up): 1 turns
// a batch's strips off; 2..STRIP_MAX_SEG puts up to m pairs in each strip
// whatever number of workgroups that leaves (see make_strips).
std::atomic<int> g_strip_pairs{0};
constexpr int STRIP_ROUNDS = 8;         // workgroups per compute unit a strip plan keeps
constexpr int STRIP_MAX_CHUNKS = 8;     // mean chunks of B per pair up to which strips pay


// Test hook SERAC_TEST_WG_ORDER=<seed> (read at a device's set-up; 0 or
// unset: the library's own order): the tile kernels sweep their tiles in a
// permuted workgroup order (see WgOrder).
std::atomic<uint32_t> g_order_seed{0};

WgOrder wg_order(uint32_t n)
{
    const uint32_t seed = g_order_seed.load(std::memory_order_relaxed);
    if (seed == 0u || n <= 1u)
        return WgOrder{1u, 0u};
    const uint32_t b = (uint32_t)((seed * 40503ull) % n);
    uint32_t a = (uint32_t)((seed * 2654435761ull) % n) | 1u;
    while (std::gcd(a % n, n) != 1u)
        a += 2u;
    a %= n;
    // (a * x + b) must not wrap in 32 bits; a rotation always fits
    if ((unsigned long long)a * (n - 1) + b >= (1ull << 32))
        a = 1u;
    return WgOrder{a, b};
}

// Per-device set-up: architecture check, acos table and the device angle's
// distance from it, the fixed scratch of the non-allocating entry point,
// pool threshold.
int device_setup(Device **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return hip_fail();
    if (dev < 0 || dev >= 64)
        return SERAC_ERR_UNSUPPORTED_DEVICE;
    std::lock_guard<std::mutex> lock(g_mutex);
    Device &d = g_devices[dev];
    // Only success and an unsupported device are final; after a transient
    // failure (a HIP error, the table's allocation) the next call tries again.
    if (!d.init) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return hip_fail();
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            d.init = true;
            d.status = SERAC_ERR_UNSUPPORTED_DEVICE;
            return d.status;
        }
        d.cus = prop.multiProcessorCount;
        // test hook: SERAC_LOOKBACK_SPIN_LIMIT bounds the finishing kernel's
        // look-back polls (negative: give up at once, so count = -1)
        if (const char *e = std::getenv("SERAC_LOOKBACK_SPIN_LIMIT")) {
            char *end = nullptr;
            const long v = std::strtol(e, &end, 10);
            if (end != e && v >= -1 && v <= (1L << 30))
                d.spin_limit = (int)v;
        }
        if (const char *e = std::getenv("SERAC_TEST_WG_ORDER")) {
            char *end = nullptr;
            const unsigned long v = std::strtoul(e, &end, 10);
            if (end != e && v <= 0xFFFFFFFFul)
                g_order_seed.store((uint32_t)v, std::memory_order_relaxed);
        }
        if (const char *e = std::getenv("SERAC_TEST_STRIP_PAIRS")) {
            char *end = nullptr;
            const long v = std::strtol(e, &end, 10);
            if (end != e && v >= 1 && v <= STRIP_MAX_SEG)
                g_strip_pairs.store((int)v, std::memory_order_relaxed);
        }
        // angle of every attainable clamped score, with the C library's acos
        std::vector<double> t(NORM2 + 1);
        for (int s = 0; s <= NORM2; ++s)
            t[s] = std::acos(s >= NORM2 ? 1.0 : (double)s / (double)NORM2);
        if (!d.table && (fail_alloc() || hipMalloc(&d.table, t.size() * sizeof(double)) != hipSuccess)) {
            (void)hipGetLastError();
            d.table = nullptr;
            return SERAC_ERR_OUT_OF_MEMORY;
        }
        if (hipMemcpy(d.table, t.data(), t.size() * sizeof(double), hipMemcpyHostToDevice) !=
            hipSuccess)
            return hip_fail();
        d.slack = angle_slack(d.table);
        if (const int st = fixed_setup(dev); st != SERAC_OK)
            return st;
        hipMemPool_t pool;
        if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
            uint64_t keep = UINT64_MAX;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        }
        (void)hipGetLastError();
        d.status = SERAC_OK;
        d.init = true;
    }
    *out = &d;
    return d.status;
}

// The current device if it has been set up (no set-up work here), else null.
Device *device_ready(int *dev_out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (dev < 0 || dev >= 64)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    Device &d = g_devices[dev];
    *dev_out = dev;
    return d.init && d.status == SERAC_OK ? &d : nullptr;
}

// Grow-only workspace per (device, stream).  Work on one stream runs in
// order, so consecutive calls on a stream can share one workspace; calls on
// different streams get different ones.  A call holds its workspace's lock
// while it enqueues, so calls on one stream from several host threads are
// serialized (their enqueue order is their stream order).  Growth frees the
// old buffers and allocates new ones on the same stream, both stream-ordered.
//   acc  the accumulators of the jobs, in two equal regions that calls use
//        in turn; a call's region is zero when it starts: the first kernel
//        of each call clears the leading bytes the previous call left
//        raised in the other region (which this call does not touch); the
//        whole buffer is cleared by a kernel when (re)allocated or after a
//        failed call;
//   aux  per-call scratch (the job table of a batch, prepared sets);
//   stage a ring of pinned host buffers the job tables of batches are
//        copied from, each with an event recorded after its copy: a batch
//        call rewrites the buffer used STAGE_RING calls before, so it waits
//        only if that call's copy has not run yet (the stream is then at
//        least STAGE_RING batch calls behind the host).
constexpr int STAGE_RING = 4;       // pinned staging buffers per workspace

struct Workspace {
    int dev = 0;
    hipStream_t stream = nullptr;
    uint8_t *acc = nullptr;
    size_t acc_bytes = 0;            // both regions
    size_t acc_used[2] = {0, 0};     // leading bytes of each region the last call on it left raised
    int region = 0;                  // the region the next call uses (zero)
    uint8_t *aux = nullptr;
    size_t aux_bytes = 0;
    bool dirty = false;
    uint8_t *stage[STAGE_RING] = {};
    size_t stage_bytes[STAGE_RING] = {};
    hipEvent_t staged[STAGE_RING] = {};   // recorded after the copy out of stage[k] (or null)
    int stage_next = 0;                   // the ring entry the next batch call uses
    std::mutex busy;                 // held by the call enqueueing on this workspace
    bool released = false;           // freed by serac_release_stream; free for reuse
};
std::mutex g_ws_mutex;          // guards the list itself
std::deque<Workspace> g_ws;     // a deque: workspaces keep their addresses as others are added

int grow(uint8_t *&ptr, size_t &have, size_t need, hipStream_t stream, bool clear)
{
    if (have >= need && ptr)
        return SERAC_OK;
    if (ptr)
        (void)hipFreeAsync(ptr, stream);
    ptr = nullptr;
    have = 0;
    const size_t want = std::max(align256(need), (size_t)1 << 20);
    if (fail_alloc() || hipMallocAsync(reinterpret_cast<void **>(&ptr), want, stream) != hipSuccess) {
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
// given sizes, in *out; `hold` receives its lock, which the caller keeps
// until it has enqueued its work (also when this returns an error).
int get_workspace(hipStream_t stream, size_t acc_bytes, size_t aux_bytes, Workspace **out,
                  std::unique_lock<std::mutex> &hold)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return hip_fail();
    Workspace *w = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_ws_mutex);
        for (auto &e : g_ws)
            if (!e.released && e.dev == dev && e.stream == stream)
                w = &e;
        // a released entry is reused for a new stream (the list never shrinks:
        // entries keep their addresses)
        for (auto &e : g_ws)
            if (!w && e.released && e.busy.try_lock()) {
                if (e.released) {
                    e.released = false;
                    e.dev = dev;
                    e.stream = stream;
                    w = &e;
                }
                e.busy.unlock();
            }
        if (!w) {
            w = &g_ws.emplace_back();
            w->dev = dev;
            w->stream = stream;
        }
    }
    hold = std::unique_lock<std::mutex>(w->busy);
    const uint8_t *before = w->acc;
    // two regions of at least acc_bytes each (grow's minimum keeps halves
    // 256-byte aligned)
    int st = grow(w->acc, w->acc_bytes, 2 * align256(acc_bytes), stream, true);
    if (w->acc != before) {
        w->acc_used[0] = w->acc_used[1] = 0;   // a fresh buffer is cleared
        w->region = 0;
    }
    if (st == SERAC_OK && w->dirty) {
        serac_clear<<<1024, 256, 0, stream>>>(reinterpret_cast<uint4 *>(w->acc),
                                              w->acc_bytes / 16);
        st = hipGetLastError() == hipSuccess ? SERAC_OK : SERAC_ERR_HIP;
        if (st == SERAC_OK) {
            w->dirty = false;
            w->acc_used[0] = w->acc_used[1] = 0;
        }
    }
    if (st == SERAC_OK && aux_bytes)
        st = grow(w->aux, w->aux_bytes, aux_bytes, stream, false);
    *out = w;
    return st;
}

// The next ring entry of pinned staging memory, at least `bytes`, free to
// be written: the copy out of it enqueued STAGE_RING batch calls ago has
// run (waited for here only if it has not).  *ev is to be recorded behind
// this call's copy out of it.
int get_stage(Workspace *w, size_t bytes, uint8_t **out, hipEvent_t *ev)
{
    const int k = w->stage_next;
    if (w->staged[k] && hipEventSynchronize(w->staged[k]) != hipSuccess)
        return hip_fail();
    if (w->stage_bytes[k] < bytes) {
        if (w->stage[k])
            (void)hipHostFree(w->stage[k]);
        w->stage[k] = nullptr;
        w->stage_bytes[k] = 0;
        const size_t want = std::max(align256(bytes), (size_t)1 << 16);
        if (fail_alloc() ||
            hipHostMalloc(reinterpret_cast<void **>(&w->stage[k]), want, hipHostMallocDefault) !=
                hipSuccess) {
            (void)hipGetLastError();
            w->stage[k] = nullptr;
            return SERAC_ERR_OUT_OF_MEMORY;
        }
        w->stage_bytes[k] = want;
    }
    if (!w->staged[k] &&
        hipEventCreateWithFlags(&w->staged[k], hipEventDisableTiming) != hipSuccess) {
        w->staged[k] = nullptr;
        return hip_fail();
    }
    w->stage_next = (k + 1) % STAGE_RING;
    *out = w->stage[k];
    *ev = w->staged[k];
    return SERAC_OK;
}

// The accumulator region of the next call (zero).  (This and the two below
// run under the workspace's lock.)
uint8_t *next_region(Workspace *w)
{
    return w->acc + (size_t)w->region * (w->acc_bytes / 2);
}

// Takes the next region for this call: returns what the previous call left
// raised in the other region, for this call's first kernel to clear, and
// records what this call will leave in its own.
Clear take_clear(Workspace *w, size_t leaves)
{
    const int cur = w->region, other = 1 - cur;
    Clear C;
    C.stride = 1;                            // set by the launch
    C.p = reinterpret_cast<uint4 *>(w->acc + (size_t)other * (w->acc_bytes / 2));
    C.words = w->acc_used[other] / 16;
    w->acc_used[other] = 0;
    w->acc_used[cur] = leaves;
    w->region = other;
    return C;
}

// A call that enqueued work on the accumulators and then failed may have
// left them raised: have the next call clear them first.
void mark_dirty(Workspace *w)
{
    w->dirty = true;
}

// ---- fixed scratch of serac_match_pair_noalloc
//
// One array per device, in the code object's device memory: the
// accumulators (NOALLOC_REGION bytes; each call clears what it raised there
// with a kernel at its end) and the per-call scratch after them.  It is
// never allocated or freed; each device's copy lives at its own address,
// taken once per device at set-up with hipGetSymbolAddress (the array's
// name in host code is not a device address).  Every call on a device
// shares that device's copy.  With 256 compute units every pair of sets of
// up to 16384 descriptors fits (at most 2.1 MB of per-call scratch).
constexpr size_t NOALLOC_REGION = 160u << 10;   // >= the accumulators of any accepted pair
constexpr size_t NOALLOC_BYTES = 4u << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_BYTES];

struct FixedScratch {
    bool ready = false;
    Workspace w;          // acc, aux point into this device's copy of `scratch`
};
FixedScratch g_fixed[64];

// Set-up of device `dev`'s fixed scratch (under g_mutex, device current):
// its address, and a clear by a kernel (its contents start at zero).  A
// failure fails the device's set-up, which the next call then retries.
int fixed_setup(int dev)
{
    FixedScratch &f = g_fixed[dev];
    if (f.ready)
        return SERAC_OK;
    uint8_t *ptr = nullptr;
    if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return hip_fail();
    serac_clear<<<256, 256>>>(reinterpret_cast<uint4 *>(ptr), NOALLOC_BYTES / 16);
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        return hip_fail();
    f.w.dev = dev;
    f.w.acc = ptr;
    f.w.acc_bytes = NOALLOC_REGION;
    f.w.aux = f.w.acc + NOALLOC_REGION;
    f.w.aux_bytes = NOALLOC_BYTES - NOALLOC_REGION;
    f.ready = true;
    return SERAC_OK;
}

struct Plan {
    int nRB, nBC, gch, Gc;
    size_t acc;       // bytes of accumulators: cbest, then the finishing status words
    size_t scratch;   // bytes of per-call scratch: rs1, then rslot
    int units() const { return nRB * Gc; }
};

// Workgroups of 256 rows by gch chunks of 256 columns; gch is a power of
// two, at most 64, so a workgroup's columns stay inside one aligned
// 16384-column window.
//   - A batch (cus = 0): the largest gch that still yields about `target`
//     workgroups for the pair (the batch's pairs fill the device together).
//   - One pair on a device of `cus` compute units (one workgroup each): the
//     gch with the shortest estimated sweep, the larger on a tie.  A
//     workgroup of c chunks takes about 1.25 + c chunk times (prologue and
//     end of the sweep, measured); the full groups run in rounds of `cus`
//     workgroups, and the workgroups of a ragged last group run in the
//     last round's idle units if they fit, else after it.  At 10400 x 10400
//     this takes one round of 8-chunk workgroups instead of two rounds of
//     4-chunk ones (-8%), at 12000 x 12000 three rounds of 4 chunks instead
//     of two of 8 plus a ragged round (-8%).
//
// Workgroup u sweeps row block u % nRB against column group u / nRB.
// Consecutive workgroups go to the eight XCDs in turn, so with nRB a
// multiple of 8 all sweeps of a row block share one XCD, and so does the
// finishing workgroup of that row block (256 rows each).  Every XCD's L2
// then fetches all of B; a map giving each XCD a 2-D block of the grid cut
// the fetched bytes by a third but made both kernels slower (measured).
Plan make_plan(int nA, int nB, long long target, int cus = 0)
{
    Plan p;
    p.nRB = (nA + BLOCK_ROWS - 1) / BLOCK_ROWS;
    p.nBC = (nB + CHUNK - 1) / CHUNK;
    p.gch = MAX_GCH;
    auto groups = [&](int g) { return (p.nBC + g - 1) / g; };
    if (cus > 0) {
        double best = 0.0;
        for (int g = MAX_GCH; g >= 1; g >>= 1) {
            const long long full = (long long)p.nRB * (p.nBC / g);   // workgroups of g chunks
            const int r = p.nBC % g;                                  // chunks of the ragged group
            const long long rounds = (full + cus - 1) / cus;
            double t = (double)rounds * (1.25 + g);
            if (r > 0 && rounds * cus - full < p.nRB)
                t += 1.25 + r;
            if (g == MAX_GCH || t < best) {
                best = t;
                p.gch = g;
            }
        }
    } else {
        while (p.gch > 1 && (long long)p.nRB * groups(p.gch) < target)
            p.gch >>= 1;
    }
    p.Gc = groups(p.gch);
    const size_t gates = (size_t)(nA + GATE_THREADS - 1) / GATE_THREADS;
    p.acc = align256((size_t)nB * 8) + align256(gates * 8);
    p.scratch = align256((size_t)nA * 4) + align256((size_t)p.Gc * nA * 8);
    return p;
}

// Strips of a batch (serac_tiles_strip): the jobs of each A image, in job
// order, cut into runs of nearly equal length of at most m jobs.  Used when
// every job's B is one column group and the pairs' B sides average at most
// STRIP_MAX_CHUNKS chunks; m is the largest value up to STRIP_MAX_SEG that
// still leaves STRIP_ROUNDS workgroups per compute unit, and at m = 1 (a
// strip per pair, nothing to reuse) the batch keeps serac_tiles_many.
// Strips save each pair after a strip's first the latency of its first
// chunk and the workgroup's start and drain, but not its lane merge or
// column flush: measured on exhaustive image sets, the tile kernel took
// 13.5% less time with 512-descriptor images (2 chunks per pair), 8.6% less
// with 1024, 3% less with 2048, and 1-3% more with 4096 and 10400, about
// the same with 8192 (one MI355X; strips of up to 16 pairs).  Strips with
// more chunks come first, so that the last workgroups to start are the
// short ones.  Returns the row blocks per strip (the grid's stride), or 0
// for no strips.
int make_strips(const std::vector<int> &jobA, const std::vector<Plan> &plans, int cus,
                std::vector<int32_t> &stripJobs, std::vector<StripRef> &strips)
{
    stripJobs.clear();
    strips.clear();
    const int njobs = (int)jobA.size();
    if (njobs < 2)
        return 0;
    for (const Plan &p : plans)
        if (p.Gc != 1)
            return 0;
    // jobs per A image, images in order of their first job
    std::vector<std::vector<int>> runs;
    std::unordered_map<int, int> at;
    for (int k = 0; k < njobs; ++k) {
        auto it = at.find(jobA[k]);
        if (it == at.end()) {
            at.emplace(jobA[k], (int)runs.size());
            runs.push_back({k});
        } else {
            runs[it->second].push_back(k);
        }
    }
    auto workgroups = [&](int m) {
        long long wg = 0;
        for (const auto &r : runs)
            wg += (long long)(((int)r.size() + m - 1) / m) * plans[r[0]].nRB;
        return wg;
    };
    int m = g_strip_pairs.load(std::memory_order_relaxed);
    if (m == 0) {
        long long chunks = 0;
        for (const Plan &p : plans)
            chunks += p.nBC;
        if (chunks > (long long)STRIP_MAX_CHUNKS * njobs)
            return 0;
        m = 1;
        for (int t = STRIP_MAX_SEG; t >= 2; --t)
            if (workgroups(t) >= (long long)STRIP_ROUNDS * cus) {
                m = t;
                break;
            }
    }
    if (m < 2)
        return 0;
    std::vector<std::pair<long long, StripRef>> order;
    int rbPerStrip = 0;
    for (const auto &r : runs) {
        const int c = (int)r.size(), k = (c + m - 1) / m;
        int pos = 0;
        for (int q = 0; q < k; ++q) {
            const int len = c / k + (q < c % k ? 1 : 0);
            long long chunks = 0;
            StripRef S{(int32_t)stripJobs.size(), len};
            for (int e = 0; e < len; ++e) {
                stripJobs.push_back(r[pos + e]);
                chunks += plans[r[pos + e]].nBC;
            }
            pos += len;
            order.push_back({chunks, S});
        }
        rbPerStrip = std::max(rbPerStrip, plans[r[0]].nRB);
    }
    std::stable_sort(order.begin(), order.end(),
                     [](const auto &a, const auto &b) { return a.first > b.first; });
    for (const auto &o : order)
        strips.push_back(o.second);
    return rbPerStrip;
}

int round_up(int n, int m) { return (n + m - 1) / m * m; }

// Bytes of one set prepared in the requested roles.
size_t prep_bytes(int n, bool asA, bool asB)
{
    size_t b = 0;
    if (asA) {
        const size_t r = (size_t)round_up(n, BLOCK_ROWS);
        b += align256(r * DIM) + align256(r * 4);
    }
    if (asB) {
        const size_t r = (size_t)round_up(n, CHUNK);
        b += align256(r * DIM) + align256(r * 4);
    }
    return b;
}

// Places the prepared buffers of one set at q (advancing q).
PrepJob make_prep(const uint8_t *X, int n, bool asA, bool asB, uint8_t *&q)
{
    PrepJob Q{};
    Q.X = X;
    Q.n = n;
    if (asA) {
        Q.rowsA = round_up(n, BLOCK_ROWS);
        Q.Af = q;
        q += align256((size_t)Q.rowsA * DIM);
        Q.RT = reinterpret_cast<int32_t *>(q);
        q += align256((size_t)Q.rowsA * 4);
    }
    if (asB) {
        Q.rowsB = round_up(n, CHUNK);
        Q.Bp = q;
        q += align256((size_t)Q.rowsB * DIM);
        Q.P = reinterpret_cast<uint32_t *>(q);
        q += align256((size_t)Q.rowsB * 4);
    }
    return Q;
}

int prep_blocks(const PrepJob &Q)
{
    return (std::max(Q.rowsA, Q.rowsB) * 8 + PREP_THREADS - 1) / PREP_THREADS;
}

void fill_job(Job &J, const Plan &p, const uint8_t *A, int nA, const PrepJob &QA,
              const uint8_t *B, int nB, const PrepJob &QB, uint8_t *acc, uint8_t *scratch,
              serac_match *out, int32_t *count)
{
    J.A = A;
    J.B = B;
    J.Af = QA.Af;
    J.RT = QA.RT;
    J.Bp = QB.Bp;
    J.P = QB.P;
    J.nA = nA;
    J.nB = nB;
    J.nRB = p.nRB;
    J.nBC = p.nBC;
    J.gch = p.gch;
    J.Gc = p.Gc;
    J.cb32 = p.nRB * (BLOCK_ROWS / SLICE) <= 512 ? 1 : 0;
    J.cbest = reinterpret_cast<unsigned long long *>(acc);
    J.status = reinterpret_cast<unsigned long long *>(acc + align256((size_t)nB * 8));
    J.rs1 = reinterpret_cast<uint32_t *>(scratch);
    J.rslot = reinterpret_cast<unsigned long long *>(scratch + align256((size_t)nA * 4));
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
    if (p->max_features < 0 || p->reserved != 0)
        return true;
    return (p->flags & ~SERAC_FLAG_SYMMETRIC) != 0;
}

// A set's descriptor count under the match cap.
int32_t capped(int32_t n, const serac_params *p)
{
    return p->max_features > 0 ? std::min(n, p->max_features) : n;
}

bool symmetric(const serac_params *p)
{
    return (p->flags & SERAC_FLAG_SYMMETRIC) != 0;
}

bool misaligned(const void *p, uintptr_t align)
{
    return ((uintptr_t)p & (align - 1)) != 0;
}

// A descriptor set: 0 <= n <= the maximum, and for n > 0 a pointer aligned
// to 16 bytes (the kernels read 16-byte words).
bool bad_set(const uint8_t *d, int32_t n)
{
    return n < 0 || n > SERAC_MAX_DESCRIPTORS || (n > 0 && (d == nullptr || misaligned(d, 16)));
}

// One pair's output: a count (4-byte aligned) and, when the pair can match,
// a match array (8-byte aligned: a match is written as one 8-byte word).
bool bad_out(const serac_matches &o, int32_t nA)
{
    return !o.count || misaligned(o.count, 4) ||
           (nA > 0 && (!o.matches || misaligned(o.matches, 8)));
}

Gate make_gate(const Device *d, const serac_params *p)
{
    Gate G;
    G.table = d->table;
    G.max_ratio = p->max_ratio;
    G.max_distance = p->max_distance;
    G.slack = d->slack;
    G.cross_check = p->cross_check;
    G.spin_limit = d->spin_limit;
    return G;
}

template <bool COLS, bool NARROW>
void launch_one(const Job &J, int units, hipStream_t stream)
{
    hipEvent_t e0, e1;
    prof_slot(e0, e1, tile_name<COLS, NARROW>(false));
    const WgOrder o = wg_order((uint32_t)units);
    if (e0)
        hipExtLaunchKernelGGL(serac_tiles_one<COLS, NARROW>, dim3(units), dim3(TILE_THREADS), 0,
                              stream, e0, e1, 0, J, o);
    else
        serac_tiles_one<COLS, NARROW><<<units, TILE_THREADS, 0, stream>>>(J, o);
}

void launch_tiles(const Job &J, const Plan &p, bool cols, hipStream_t stream)
{
    if (!cols)
        launch_one<false, false>(J, p.units(), stream);
    else if (J.cb32)
        launch_one<true, true>(J, p.units(), stream);
    else
        launch_one<true, false>(J, p.units(), stream);
}

// A pair small enough that converting the raw descriptors inside the sweep
// (every workgroup converts the chunks it reads) costs less than the
// separate preparation kernel and the launch boundary after it (measured:
// the fused sweep is 1-3% faster from 12000^2 to 16384^2 and 8192 x 32768,
// 2% slower at 20000^2).
constexpr long long FUSED_MAX_WORK = 1ll << 28;    // nA * nB

bool fused_pair(int nA, int nB)
{
    return (long long)nA * nB <= FUSED_MAX_WORK;
}

// Bytes of prepared sets one pair needs (none for a fused sweep).
size_t pair_prep_bytes(int nA, int nB)
{
    return fused_pair(nA, nB) ? 0 : prep_bytes(nA, true, false) + prep_bytes(nB, false, true);
}

// The fused sweep, with the timing events e0/e1 attached when not null.
template <bool COLS, bool NARROW>
void launch_fused(const Job &J, uint4 *clear_p, uint32_t clear_words, uint32_t clear_stride,
                  int units, hipStream_t stream)
{
    hipEvent_t e0, e1;
    prof_slot(e0, e1, tile_name<COLS, NARROW>(true));
    const WgOrder o = wg_order((uint32_t)units);
    if (e0)
        hipExtLaunchKernelGGL(serac_tiles_fused<COLS, NARROW>, dim3(units), dim3(TILE_THREADS), 0,
                              stream, e0, e1, 0, J.A, J.B, J.nA, J.nB, J.nRB, J.nBC, J.gch,
                              clear_p, clear_words, clear_stride, o.a, o.b, (uint32_t)units, J);
    else
        serac_tiles_fused<COLS, NARROW><<<units, TILE_THREADS, 0, stream>>>(
            J.A, J.B, J.nA, J.nB, J.nRB, J.nBC, J.gch, clear_p, clear_words, clear_stride, o.a,
            o.b, (uint32_t)units, J);
}

// Preparation and tile sweep of one pair (nA, nB > 0) on `stream`; the
// prepared sets go to `prep` (pair_prep_bytes(nA, nB)).
void launch_pair(Job &J, const Plan &p, const uint8_t *A, int nA, const uint8_t *B, int nB,
                 uint8_t *prep, Clear C, bool cols, hipStream_t stream)
{
    if (fused_pair(nA, nB)) {
        C.stride = (uint32_t)p.units() * TILE_THREADS;
        // (the cleared region is a few MiB at most: its 16-byte word count
        // fits 32 bits)
        const uint32_t words = (uint32_t)C.words;
        if (!cols)
            launch_fused<false, false>(J, C.p, words, C.stride, p.units(), stream);
        else if (J.cb32)
            launch_fused<true, true>(J, C.p, words, C.stride, p.units(), stream);
        else
            launch_fused<true, false>(J, C.p, words, C.stride, p.units(), stream);
        return;
    }
    uint8_t *q = prep;
    PrepPair Q;
    Q.q[0] = make_prep(A, nA, true, false, q);
    Q.q[1] = make_prep(B, nB, false, true, q);
    J.Af = Q.q[0].Af;
    J.RT = Q.q[0].RT;
    J.Bp = Q.q[1].Bp;
    J.P = Q.q[1].P;
    const dim3 pg(std::max(prep_blocks(Q.q[0]), prep_blocks(Q.q[1])), 2);
    C.stride = pg.x * PREP_THREADS;
    serac_prep_pair<<<pg, PREP_THREADS, 0, stream>>>(Q, C);
    launch_tiles(J, p, cols, stream);
}

// The kernels of one pair (nA, nB > 0) on `stream`, with w's accumulators
// and w's scratch (p.scratch, then the prepared sets): the sweep (after the
// preparation kernel for a large pair) and the finishing kernel.  The caller
// holds w's lock and has sized w for p.
// Accumulators: by default the call takes w's next region and its first
// kernel clears what the previous call left in the other one (host-side
// bookkeeping).  With `self_clear` it always takes the first region and a
// kernel after the finishing kernel clears what this call raised there, so
// the region is zero whenever a call starts without the host tracking
// anything, also when a captured graph of the call is replayed.
// Clears the whole accumulator buffer of w if a failed call may have left it
// raised (get_workspace does the same for the workspaces it hands out).
int clear_if_dirty(Workspace *w, hipStream_t stream)
{
    if (!w->dirty)
        return SERAC_OK;
    serac_clear<<<1024, 256, 0, stream>>>(reinterpret_cast<uint4 *>(w->acc), w->acc_bytes / 16);
    if (hipGetLastError() != hipSuccess)
        return SERAC_ERR_HIP;
    w->dirty = false;
    w->acc_used[0] = w->acc_used[1] = 0;
    return SERAC_OK;
}

int enqueue_pair(const Device *d, const Plan &p, Workspace *w, const uint8_t *A, int nA,
                 const uint8_t *B, int nB, const serac_params *params, const serac_matches *out,
                 hipStream_t stream, bool self_clear = false)
{
    if (clear_if_dirty(w, stream) != SERAC_OK)
        return SERAC_ERR_HIP;
    Job J;
    const PrepJob none{};
    uint8_t *const region = self_clear ? w->acc : next_region(w);
    fill_job(J, p, A, nA, none, B, nB, none, region, w->aux, out->matches, out->count);
    const Clear C = self_clear ? Clear{reinterpret_cast<uint4 *>(w->acc), 0, 1}
                               : take_clear(w, p.acc);
    launch_pair(J, p, A, nA, B, nB, w->aux + p.scratch, C, params->cross_check != 0, stream);
    const Gate G = make_gate(d, params);
    const dim3 fg((nA + GATE_THREADS - 1) / GATE_THREADS);
    if (J.cb32)
        serac_finish_one<true><<<fg, GATE_THREADS, 0, stream>>>(
            J.rslot, J.nA, J.nB, J.Gc, J.cbest, G.table, G.cross_check, J, G);
    else
        serac_finish_one<false><<<fg, GATE_THREADS, 0, stream>>>(
            J.rslot, J.nA, J.nB, J.Gc, J.cbest, G.table, G.cross_check, J, G);
    if (self_clear) {
        const size_t words = p.acc / 16;
        serac_clear<<<(unsigned)std::min<size_t>((words + 255) / 256, 1024), 256, 0, stream>>>(
            reinterpret_cast<uint4 *>(region), words);
    }
    if (hipGetLastError() != hipSuccess) {
        mark_dirty(w);
        return SERAC_ERR_HIP;
    }
    return SERAC_OK;
}

// Scratch of a pair under symmetric column gates: that of the pair (A, B)
// with its prepared sets, then that of the swapped pair (B, A), whose rs1
// holds the columns' accepted rows between the two finishing passes.
size_t sym_aux_bytes(const Plan &pf, const Plan &pr, int nA, int nB)
{
    return align256(pf.scratch + pair_prep_bytes(nA, nB)) + pr.scratch + pair_prep_bytes(nB, nA);
}

// A pair under symmetric column gates (nA, nB > 0): the sweep of (B, A) and
// its finishing pass, which writes each column's accepted row, then the
// sweep of (A, B) and its finishing pass, which keeps row i where its best
// column accepts i.  Neither sweep keeps column bests.  Each sweep takes an
// accumulator region of its own in turn, like two calls.
int enqueue_sym(const Device *d, const Plan &pf, const Plan &pr, Workspace *w, const uint8_t *A,
                int nA, const uint8_t *B, int nB, const serac_params *params,
                const serac_matches *out, hipStream_t stream)
{
    if (clear_if_dirty(w, stream) != SERAC_OK)
        return SERAC_ERR_HIP;
    const PrepJob none{};
    uint8_t *const fa = w->aux;
    uint8_t *const ra = w->aux + align256(pf.scratch + pair_prep_bytes(nA, nB));
    Gate G = make_gate(d, params);
    G.cross_check = 0;
    Job Jr;
    fill_job(Jr, pr, B, nB, none, A, nA, none, next_region(w), ra, nullptr, nullptr);
    launch_pair(Jr, pr, B, nB, A, nA, ra + pr.scratch, take_clear(w, pr.acc), false, stream);
    serac_finish_sym<SYM_COLUMNS>
        <<<(nB + GATE_THREADS - 1) / GATE_THREADS, GATE_THREADS, 0, stream>>>(Jr, G, nullptr);
    Job Jf;
    fill_job(Jf, pf, A, nA, none, B, nB, none, next_region(w), fa, out->matches, out->count);
    launch_pair(Jf, pf, A, nA, B, nB, fa + pf.scratch, take_clear(w, pf.acc), false, stream);
    serac_finish_sym<SYM_ROWS><<<(nA + GATE_THREADS - 1) / GATE_THREADS, GATE_THREADS, 0, stream>>>(
        Jf, G, reinterpret_cast<const int32_t *>(Jr.rs1));
    if (hipGetLastError() != hipSuccess) {
        mark_dirty(w);
        return SERAC_ERR_HIP;
    }
    return SERAC_OK;
}

// Runs an entry point's body: no C++ exception crosses the C interface (a
// failed host allocation is reported as out of memory, anything else as a
// runtime error).
template <class F>
int guarded(F &&body) noexcept
{
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return SERAC_ERR_OUT_OF_MEMORY;
    } catch (...) {
        return SERAC_ERR_HIP;
    }
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
    case SERAC_ERR_TOO_LARGE:
        return "pair too large for the fixed scratch of the non-allocating entry point";
    case SERAC_ERR_NOT_INITIALIZED:
        return "device not set up (call serac_init first)";
    default:
        return "unknown status";
    }
}

int serac_match_pair(const uint8_t *descA, int32_t nA, const uint8_t *descB, int32_t nB,
                     const serac_params *params, const serac_matches *out)
{
    return guarded([&]() -> int {
        if (bad_set(descA, nA) || bad_set(descB, nB) || bad_params(params) || !out)
            return SERAC_ERR_INVALID_ARG;
        nA = capped(nA, params);
        nB = capped(nB, params);
        if (bad_out(*out, nA))
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
        const Plan p = make_plan(nA, nB, 0, d->cus);
        Workspace *w = nullptr;
        std::unique_lock<std::mutex> hold;
        if (symmetric(params)) {
            const Plan pr = make_plan(nB, nA, 0, d->cus);
            st = get_workspace(stream, std::max(p.acc, pr.acc), sym_aux_bytes(p, pr, nA, nB), &w,
                               hold);
            if (st != SERAC_OK)
                return st;
            return enqueue_sym(d, p, pr, w, descA, nA, descB, nB, params, out, stream);
        }
        st = get_workspace(stream, p.acc, p.scratch + pair_prep_bytes(nA, nB), &w, hold);
        if (st != SERAC_OK)
            return st;
        return enqueue_pair(d, p, w, descA, nA, descB, nB, params, out, stream);
    });
}

int serac_init(void)
{
    return guarded([&]() -> int {
        Device *d = nullptr;
        return device_setup(&d);
    });
}

int serac_match_pair_noalloc(const uint8_t *descA, int32_t nA, const uint8_t *descB, int32_t nB,
                             const serac_params *params, const serac_matches *out)
{
    return guarded([&]() -> int {
        if (bad_set(descA, nA) || bad_set(descB, nB) || bad_params(params) || !out ||
            symmetric(params))
            return SERAC_ERR_INVALID_ARG;
        nA = capped(nA, params);
        nB = capped(nB, params);
        if (bad_out(*out, nA))
            return SERAC_ERR_INVALID_ARG;
        if (out->capacity < nA)
            return SERAC_ERR_CAPACITY;
        if (!fused_pair(nA, nB))
            return SERAC_ERR_TOO_LARGE;
        int dev = 0;
        Device *d = device_ready(&dev);
        if (!d)
            return SERAC_ERR_NOT_INITIALIZED;
        FixedScratch &f = g_fixed[dev];
        if (!f.ready)
            return SERAC_ERR_NOT_INITIALIZED;
        hipStream_t stream = static_cast<hipStream_t>(params->stream);
        if (nA == 0 || nB == 0) {
            serac_zero_counts<<<1, 64, 0, stream>>>(nullptr, out->count, 1);
            return hipGetLastError() == hipSuccess ? SERAC_OK : SERAC_ERR_HIP;
        }
        const Plan p = make_plan(nA, nB, 0, d->cus);
        if (p.acc > NOALLOC_REGION || p.scratch > f.w.aux_bytes)
            return SERAC_ERR_TOO_LARGE;
        std::lock_guard<std::mutex> hold(f.w.busy);
        return enqueue_pair(d, p, &f.w, descA, nA, descB, nB, params, out, stream, true);
    });
}

int serac_match_pairs(const uint8_t *const *desc, const int32_t *n, int32_t num_images,
                      const serac_pair *pairs, int32_t num_pairs, const serac_params *params,
                      const serac_matches *out)
{
    return guarded([&]() -> int {
        if (num_images < 0 || num_pairs < 0 || bad_params(params))
            return SERAC_ERR_INVALID_ARG;
        if (num_pairs == 0)
            return SERAC_OK;
        if (!desc || !n || !pairs || !out)
            return SERAC_ERR_INVALID_ARG;
        for (int k = 0; k < num_images; ++k)
            if (bad_set(desc[k], n[k]))
                return SERAC_ERR_INVALID_ARG;
        // the counts under the match cap (the caller's n is not modified)
        std::vector<int32_t> nc(num_images);
        for (int k = 0; k < num_images; ++k)
            nc[k] = capped(n[k], params);
        for (int q = 0; q < num_pairs; ++q) {
            const serac_pair pr = pairs[q];
            if (pr.a < 0 || pr.a >= num_images || pr.b < 0 || pr.b >= num_images)
                return SERAC_ERR_INVALID_ARG;
            if (bad_out(out[q], nc[pr.a]))
                return SERAC_ERR_INVALID_ARG;
            if (out[q].capacity < nc[pr.a])
                return SERAC_ERR_CAPACITY;
        }
        Device *d = nullptr;
        int st = device_setup(&d);
        if (st != SERAC_OK)
            return st;
        hipStream_t stream = static_cast<hipStream_t>(params->stream);
        const bool sym = symmetric(params);

        // pairs with an empty side only get a zero count
        std::vector<int32_t *> zero;
        std::vector<int> live;
        std::vector<char> asA(num_images, 0), asB(num_images, 0);
        for (int q = 0; q < num_pairs; ++q) {
            const serac_pair pr = pairs[q];
            if (nc[pr.a] == 0 || nc[pr.b] == 0) {
                zero.push_back(out[q].count);
            } else {
                live.push_back(q);
                asA[pr.a] = asB[pr.b] = 1;
                if (sym)                          // and the swapped pair
                    asA[pr.b] = asB[pr.a] = 1;
            }
        }
        // every image is prepared once, in the roles its pairs use
        std::vector<int> prepped;
        size_t prep_total = 0;
        for (int k = 0; k < num_images; ++k) {
            if (asA[k] || asB[k]) {
                prepped.push_back(k);
                prep_total += prep_bytes(nc[k], asA[k], asB[k]);
            }
        }
        // Jobs: the live pairs, then (symmetric gates) the swapped pairs in
        // the same order.  Workgroups per job: enough to fill the device a
        // few times over.
        const int nlive = (int)live.size();
        const int njobs = sym ? 2 * nlive : nlive;
        auto job_sets = [&](int k, int &a, int &b) {
            const serac_pair pr = pairs[live[k % std::max(nlive, 1)]];
            a = k < nlive ? pr.a : pr.b;
            b = k < nlive ? pr.b : pr.a;
        };
        const long long target = njobs ? std::max(1LL, (4LL * d->cus + njobs - 1) / njobs) : 1;
        std::vector<Plan> plans(njobs), whole(njobs);
        std::vector<int> jobA(njobs);
        for (int k = 0; k < njobs; ++k) {
            int b;
            job_sets(k, jobA[k], b);
            plans[k] = make_plan(nc[jobA[k]], nc[b], target);
            whole[k] = make_plan(nc[jobA[k]], nc[b], 1);   // B in as few column groups as fit
        }
        // Strips (cross-pair reuse of A) take every pair's B in one column
        // group; when they are used, those plans replace the ones that split
        // columns for parallelism.
        std::vector<int32_t> stripJobs;
        std::vector<StripRef> strips;
        const int rbPerStrip = make_strips(jobA, whole, d->cus, stripJobs, strips);
        if (rbPerStrip > 0)
            plans.swap(whole);
        size_t acc_bytes = 0, res_bytes = 0;
        int unitsPerJob = 1, gatePerJob = 1;
        for (int k = 0; k < njobs; ++k) {
            acc_bytes += plans[k].acc;
            res_bytes += plans[k].scratch;
            unitsPerJob = std::max(unitsPerJob, plans[k].units());
            gatePerJob = std::max(gatePerJob, (nc[jobA[k]] + GATE_THREADS - 1) / GATE_THREADS);
        }
        const size_t jobs_bytes = align256(sizeof(Job) * (size_t)std::max(njobs, 1));
        const size_t prepjobs_bytes = align256(sizeof(PrepJob) * std::max<size_t>(prepped.size(), 1));
        const size_t zero_bytes = align256(sizeof(int32_t *) * zero.size() + 8);
        const size_t sjobs_bytes = align256(sizeof(int32_t) * stripJobs.size() + 8);
        const size_t strips_bytes = align256(sizeof(StripRef) * strips.size() + 8);
        const size_t host_bytes = jobs_bytes + prepjobs_bytes + zero_bytes + sjobs_bytes +
                                  strips_bytes;
        Workspace *w = nullptr;
        std::unique_lock<std::mutex> hold;
        st = get_workspace(stream, acc_bytes, host_bytes + res_bytes + prep_total, &w, hold);
        if (st != SERAC_OK)
            return st;
        uint8_t *host = nullptr;
        hipEvent_t staged = nullptr;
        st = get_stage(w, host_bytes, &host, &staged);
        if (st != SERAC_OK)
            return st;
        Job *jobs = reinterpret_cast<Job *>(host);
        PrepJob *pjobs = reinterpret_cast<PrepJob *>(host + jobs_bytes);
        int32_t **zp = reinterpret_cast<int32_t **>(host + jobs_bytes + prepjobs_bytes);
        uint8_t *rq = w->aux + host_bytes;
        uint8_t *pq = rq + res_bytes;
        std::vector<int> slot(num_images, -1);
        int prepBlocks = 1;
        for (size_t k = 0; k < prepped.size(); ++k) {
            const int im = prepped[k];
            pjobs[k] = make_prep(desc[im], nc[im], asA[im], asB[im], pq);
            slot[im] = (int)k;
            prepBlocks = std::max(prepBlocks, prep_blocks(pjobs[k]));
        }
        uint8_t *q = next_region(w);
        bool narrow = true;                      // 32-bit column bests for every pair of the batch
        for (int k = 0; k < njobs; ++k) {
            int a, b;
            job_sets(k, a, b);
            const bool own = k < nlive;
            fill_job(jobs[k], plans[k], desc[a], nc[a], pjobs[slot[a]], desc[b], nc[b],
                     pjobs[slot[b]], q, rq, own ? out[live[k]].matches : nullptr,
                     own ? out[live[k]].count : nullptr);
            narrow = narrow && jobs[k].cb32;
            q += plans[k].acc;
            rq += plans[k].scratch;
        }
        for (int k = 0; k < njobs; ++k)          // one sweep kernel: one format for all pairs
            jobs[k].cb32 = narrow ? 1 : 0;
        for (size_t k = 0; k < zero.size(); ++k)
            zp[k] = zero[k];
        const size_t sjobs_at = jobs_bytes + prepjobs_bytes + zero_bytes;
        const size_t strips_at = sjobs_at + sjobs_bytes;
        if (!stripJobs.empty())
            std::memcpy(host + sjobs_at, stripJobs.data(), sizeof(int32_t) * stripJobs.size());
        if (!strips.empty())
            std::memcpy(host + strips_at, strips.data(), sizeof(StripRef) * strips.size());
        hipError_t e = hipMemcpyAsync(w->aux, host, host_bytes, hipMemcpyHostToDevice, stream);
        if (e == hipSuccess)
            e = hipEventRecord(staged, stream);   // the staging buffer is reusable once this has run
        const Job *djobs = reinterpret_cast<const Job *>(w->aux);
        const PrepJob *dpjobs = reinterpret_cast<const PrepJob *>(w->aux + jobs_bytes);
        int32_t *const *dzero =
            reinterpret_cast<int32_t *const *>(w->aux + jobs_bytes + prepjobs_bytes);
        if (e == hipSuccess && !zero.empty())
            serac_zero_counts<<<((int)zero.size() + 255) / 256, 256, 0, stream>>>(dzero, nullptr,
                                                                             (int)zero.size());
        if (e == hipSuccess && nlive) {
            Clear C = take_clear(w, acc_bytes);
            C.stride = (uint32_t)prepBlocks * PREP_THREADS;
            serac_prep_many<<<dim3(prepBlocks, (unsigned)prepped.size()), PREP_THREADS, 0, stream>>>(
                dpjobs, C);
            Gate G = make_gate(d, params);
            const bool cols = params->cross_check && !sym;
            hipEvent_t e0, e1;
            if (rbPerStrip > 0) {
                // cross-pair reuse of A: strips of pairs sharing their A image
                prof_slot(e0, e1,
                          !cols    ? "serac_tiles_strip<false, false>"
                          : narrow ? "serac_tiles_strip<true, true>"
                                   : "serac_tiles_strip<true, false>");
                const int32_t *dsj = reinterpret_cast<const int32_t *>(w->aux + sjobs_at);
                const StripRef *dst = reinterpret_cast<const StripRef *>(w->aux + strips_at);
                const dim3 grid((unsigned)strips.size() * rbPerStrip);
                const WgOrder o = wg_order(grid.x);
                if (!cols)
                    hipExtLaunchKernelGGL(serac_tiles_strip<false, false>, grid, dim3(TILE_THREADS),
                                          0, stream, e0, e1, 0, djobs, dsj, dst, rbPerStrip, o,
                                          grid.x);
                else if (narrow)
                    hipExtLaunchKernelGGL(serac_tiles_strip<true, true>, grid, dim3(TILE_THREADS),
                                          0, stream, e0, e1, 0, djobs, dsj, dst, rbPerStrip, o,
                                          grid.x);
                else
                    hipExtLaunchKernelGGL(serac_tiles_strip<true, false>, grid, dim3(TILE_THREADS),
                                          0, stream, e0, e1, 0, djobs, dsj, dst, rbPerStrip, o,
                                          grid.x);
            } else {
                prof_slot(e0, e1,
                          !cols    ? "serac_tiles_many<false, false>"
                          : narrow ? "serac_tiles_many<true, true>"
                                   : "serac_tiles_many<true, false>");
                const dim3 grid(njobs * unitsPerJob);
                const WgOrder o = wg_order(grid.x);
                if (!cols)
                    hipExtLaunchKernelGGL(serac_tiles_many<false, false>, grid, dim3(TILE_THREADS),
                                          0, stream, e0, e1, 0, djobs, unitsPerJob, o, grid.x);
                else if (narrow)
                    hipExtLaunchKernelGGL(serac_tiles_many<true, true>, grid, dim3(TILE_THREADS), 0,
                                          stream, e0, e1, 0, djobs, unitsPerJob, o, grid.x);
                else
                    hipExtLaunchKernelGGL(serac_tiles_many<true, false>, grid, dim3(TILE_THREADS),
                                          0, stream, e0, e1, 0, djobs, unitsPerJob, o, grid.x);
            }
            if (sym) {
                G.cross_check = 0;
                serac_finish_many_sym<SYM_COLUMNS><<<nlive * gatePerJob, GATE_THREADS, 0, stream>>>(
                    djobs, gatePerJob, nlive, G);
                serac_finish_many_sym<SYM_ROWS><<<nlive * gatePerJob, GATE_THREADS, 0, stream>>>(
                    djobs, gatePerJob, nlive, G);
            } else {
                serac_finish_many<<<nlive * gatePerJob, GATE_THREADS, 0, stream>>>(djobs,
                                                                                  gatePerJob, G);
            }
        }
        if (e == hipSuccess)
            e = hipGetLastError();
        if (e != hipSuccess) {
            mark_dirty(w);
            return hip_fail();
        }
        return SERAC_OK;
    });
}

int serac_match_pairs_host(const uint8_t *const *desc, const int32_t *n, int32_t num_images,
                           const serac_pair *pairs, int32_t num_pairs,
                           const serac_params *params, int32_t pairs_per_stage,
                           serac_match *const *host_matches, int32_t *host_counts)
{
    return guarded([&]() -> int {
        if (num_images < 0 || num_pairs < 0 || pairs_per_stage < 0 || bad_params(params))
            return SERAC_ERR_INVALID_ARG;
        if (num_pairs == 0)
            return SERAC_OK;
        if (!desc || !n || !pairs || !host_matches || !host_counts)
            return SERAC_ERR_INVALID_ARG;
        for (int k = 0; k < num_images; ++k)
            if (bad_set(desc[k], n[k]))
                return SERAC_ERR_INVALID_ARG;
        for (int q = 0; q < num_pairs; ++q) {
            const serac_pair pr = pairs[q];
            if (pr.a < 0 || pr.a >= num_images || pr.b < 0 || pr.b >= num_images)
                return SERAC_ERR_INVALID_ARG;
            if (n[pr.a] > 0 && !host_matches[q])
                return SERAC_ERR_INVALID_ARG;
        }
        Device *d = nullptr;
        int st = device_setup(&d);
        if (st != SERAC_OK)
            return st;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return hip_fail();
        HostPipe &P = g_pipes[dev];
        std::lock_guard<std::mutex> lock(P.busy);
        if (!P.ready) {
            // default priority, like every stream of the library
            if (hipStreamCreateWithFlags(&P.copy, hipStreamNonBlocking) != hipSuccess)
                return hip_fail();
            for (int b = 0; b < 2; ++b)
                if (hipEventCreateWithFlags(&P.done[b], hipEventDisableTiming) != hipSuccess ||
                    hipEventCreateWithFlags(&P.copied[b], hipEventDisableTiming) != hipSuccess)
                    return hip_fail();
            P.ready = true;
        }
        hipStream_t stream = static_cast<hipStream_t>(params->stream);
        const int per = std::min(pairs_per_stage ? pairs_per_stage : HOST_STAGE_PAIRS, num_pairs);
        const int stages = (num_pairs + per - 1) / per;

        // A stage's results in one block: the counts, then each pair's matches
        // at capacity n[a] (the counts are not known when the copy is enqueued).
        const size_t counts_bytes = align256((size_t)per * 4);
        std::vector<size_t> off(num_pairs + 1);     // byte offset of each pair's matches in its stage
        size_t half = 0;
        for (int s0 = 0; s0 < num_pairs; s0 += per) {
            size_t o = counts_bytes;
            for (int q = s0; q < std::min(num_pairs, s0 + per); ++q) {
                off[q] = o;
                o += (size_t)n[pairs[q].a] * sizeof(serac_match);
            }
            half = std::max(half, align256(o));
        }
        if (P.pinned_bytes < 2 * half) {
            if (P.pinned)
                (void)hipHostFree(P.pinned);
            P.pinned = nullptr;
            P.pinned_bytes = 0;
            if (fail_alloc() ||
                hipHostMalloc(reinterpret_cast<void **>(&P.pinned), 2 * half, hipHostMallocDefault) !=
                hipSuccess) {
                (void)hipGetLastError();
                P.pinned = nullptr;
                return SERAC_ERR_OUT_OF_MEMORY;
            }
            P.pinned_bytes = 2 * half;
        }
        uint8_t *dbuf = nullptr;
        if (fail_alloc() ||
            hipMallocAsync(reinterpret_cast<void **>(&dbuf), 2 * half, stream) != hipSuccess) {
            (void)hipGetLastError();
            return SERAC_ERR_OUT_OF_MEMORY;
        }

        // Stage s runs in half s % 2 of the device and pinned buffers.  The
        // host enqueues stage s, then waits for stage s-1's copy and unpacks
        // it, so the device matches stage s while stage s-1 crosses the bus and
        // the host copies stage s-2's lists out.
        auto unpack = [&](int s) {
            const uint8_t *h = P.pinned + (size_t)(s & 1) * half;
            const int32_t *cnt = reinterpret_cast<const int32_t *>(h);
            for (int q = s * per; q < std::min(num_pairs, (s + 1) * per); ++q) {
                const int32_t c = cnt[q - s * per];
                host_counts[q] = c;
                if (c > 0)
                    std::memcpy(host_matches[q], h + off[q], (size_t)c * sizeof(serac_match));
            }
        };
        std::vector<serac_matches> outs(per);
        int rc = SERAC_OK;
        int copied = 0, unpacked = 0;   // stages whose copy is enqueued / whose lists are out
        for (int s = 0; s < stages && rc == SERAC_OK; ++s) {
            const int b = s & 1, q0 = s * per, m = std::min(per, num_pairs - q0);
            uint8_t *dst = dbuf + (size_t)b * half;
            hipError_t e = hipSuccess;
            if (s >= 2)   // stage s-2's copy out of this half has run
                e = hipStreamWaitEvent(stream, P.copied[b], 0);
            for (int k = 0; k < m; ++k) {
                outs[k].matches = reinterpret_cast<serac_match *>(dst + off[q0 + k]);
                outs[k].capacity = n[pairs[q0 + k].a];
                outs[k].count = reinterpret_cast<int32_t *>(dst) + k;
            }
            if (e == hipSuccess)
                rc = serac_match_pairs(desc, n, num_images, pairs + q0, m, params, outs.data());
            else
                rc = hip_fail();
            if (rc != SERAC_OK)
                break;
            const size_t used = off[q0 + m - 1] + (size_t)n[pairs[q0 + m - 1].a] * sizeof(serac_match);
            e = hipEventRecord(P.done[b], stream);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(P.copy, P.done[b], 0);
            if (e == hipSuccess)
                e = hipMemcpyAsync(P.pinned + (size_t)b * half, dst, used, hipMemcpyDeviceToHost,
                                   P.copy);
            if (e == hipSuccess)
                e = hipEventRecord(P.copied[b], P.copy);
            if (e == hipSuccess)
                copied = s + 1;
            if (e == hipSuccess && s >= 1)
                e = hipEventSynchronize(P.copied[1 - b]);
            if (e != hipSuccess) {
                rc = hip_fail();
                break;
            }
            if (s >= 1)
                unpack(unpacked++);
        }
        if (rc == SERAC_OK) {
            if (hipEventSynchronize(P.copied[(stages - 1) & 1]) == hipSuccess)
                unpack(unpacked++);
            else
                rc = hip_fail();
        } else if (hipStreamSynchronize(P.copy) == hipSuccess) {
            // a later stage failed: the lists of the stages copied before it
            // are complete
            while (unpacked < copied)
                unpack(unpacked++);
        }
        // the device buffer is freed behind every copy out of it
        if (hipEventRecord(P.done[0], P.copy) != hipSuccess ||
            hipStreamWaitEvent(stream, P.done[0], 0) != hipSuccess ||
            hipFreeAsync(dbuf, stream) != hipSuccess) {
            (void)hipGetLastError();
            if (rc == SERAC_OK)
                rc = SERAC_ERR_HIP;
        }
        return rc;
    });
}

int serac_match_pair_unfused(const uint8_t *descA, int32_t nA, const uint8_t *descB,
                             int32_t nB, const serac_params *params, const serac_matches *out)
{
    return guarded([&]() -> int {
        if (bad_set(descA, nA) || bad_set(descB, nB) || bad_params(params) || !out ||
            symmetric(params))
            return SERAC_ERR_INVALID_ARG;
        nA = capped(nA, params);
        nB = capped(nB, params);
        if (bad_out(*out, nA))
            return SERAC_ERR_INVALID_ARG;
        if (out->capacity < nA)
            return SERAC_ERR_CAPACITY;
        if ((long long)nA * nB > UNFUSED_MAX_SCORES)
            return SERAC_ERR_TOO_LARGE;
        Device *d = nullptr;
        int st = device_setup(&d);
        if (st != SERAC_OK)
            return st;
        hipStream_t stream = static_cast<hipStream_t>(params->stream);
        if (nA == 0 || nB == 0) {
            serac_zero_counts<<<1, 64, 0, stream>>>(nullptr, out->count, 1);
            return hipGetLastError() == hipSuccess ? SERAC_OK : SERAC_ERR_HIP;
        }
        // accumulators: column bests (64-bit) and finishing status words;
        // scratch: the score matrix, then one slot per row
        const size_t gates = (size_t)(nA + GATE_THREADS - 1) / GATE_THREADS;
        const size_t acc = align256((size_t)nB * 8) + align256(gates * 8);
        const size_t sbytes = align256((size_t)nA * nB * 4);
        Workspace *w = nullptr;
        std::unique_lock<std::mutex> hold;
        st = get_workspace(stream, acc, sbytes + align256((size_t)nA * 8), &w, hold);
        if (st != SERAC_OK)
            return st;
        uint8_t *const region = next_region(w);
        const Clear C = take_clear(w, acc);
        if (C.words)
            serac_clear<<<(unsigned)std::min<size_t>((C.words + 255) / 256, 1024), 256, 0,
                          stream>>>(C.p, C.words);
        int32_t *S = reinterpret_cast<int32_t *>(w->aux);
        unsigned long long *rslot = reinterpret_cast<unsigned long long *>(w->aux + sbytes);
        unsigned long long *cbest = reinterpret_cast<unsigned long long *>(region);
        serac_scores<<<dim3((nB + SCORE_COLS - 1) / SCORE_COLS, (nA + SCORE_ROWS - 1) / SCORE_ROWS),
                       SCORE_THREADS, 0, stream>>>(descA, descB, nA, nB, S);
        serac_score_rows<<<nA, 256, 0, stream>>>(S, nA, nB, rslot);
        if (params->cross_check)
            serac_score_cols<<<dim3((nB + 255) / 256, (nA + SCORE_BAND - 1) / SCORE_BAND), 256, 0,
                               stream>>>(S, nA, nB, cbest);
        Job J;
        J.A = descA;
        J.B = descB;
        J.nA = nA;
        J.nB = nB;
        J.Gc = 1;
        J.rslot = rslot;
        J.rs1 = nullptr;
        J.cbest = cbest;
        J.cb32 = 0;
        J.status = reinterpret_cast<unsigned long long *>(region + align256((size_t)nB * 8));
        J.out = out->matches;
        J.count = out->count;
        const Gate G = make_gate(d, params);
        serac_finish_one<false><<<(nA + GATE_THREADS - 1) / GATE_THREADS, GATE_THREADS, 0, stream>>>(
            J.rslot, J.nA, J.nB, J.Gc, J.cbest, G.table, G.cross_check, J, G);
        if (hipGetLastError() != hipSuccess) {
            mark_dirty(w);
            return SERAC_ERR_HIP;
        }
        return SERAC_OK;
    });
}

int serac_release_stream(void *stream_)
{
    return guarded([&]() -> int {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return hip_fail();
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        Workspace *w = nullptr;
        {
            std::lock_guard<std::mutex> lock(g_ws_mutex);
            for (auto &e : g_ws)
                if (!e.released && e.dev == dev && e.stream == stream)
                    w = &e;
        }
        if (!w)
            return SERAC_OK;
        std::lock_guard<std::mutex> hold(w->busy);
        int st = SERAC_OK;
        // device buffers: freed in stream order, behind the work that uses them
        if (w->acc && hipFreeAsync(w->acc, stream) != hipSuccess)
            st = SERAC_ERR_HIP;
        if (w->aux && hipFreeAsync(w->aux, stream) != hipSuccess)
            st = SERAC_ERR_HIP;
        // pinned staging: freed once the copies out of it have run
        for (int k = 0; k < STAGE_RING; ++k) {
            if (w->staged[k]) {
                if (hipEventSynchronize(w->staged[k]) != hipSuccess)
                    st = SERAC_ERR_HIP;
                (void)hipEventDestroy(w->staged[k]);
            }
            if (w->stage[k])
                (void)hipHostFree(w->stage[k]);
            w->staged[k] = nullptr;
            w->stage[k] = nullptr;
            w->stage_bytes[k] = 0;
        }
        (void)hipGetLastError();
        w->acc = w->aux = nullptr;
        w->acc_bytes = w->aux_bytes = 0;
        w->acc_used[0] = w->acc_used[1] = 0;
        w->region = 0;
        w->dirty = false;
        w->stage_next = 0;
        {
            std::lock_guard<std::mutex> lock(g_ws_mutex);
            w->released = true;
            w->stream = nullptr;
        }
        return st;
    });
}

int serac_workspace_bytes(int64_t *bytes)
{
    return guarded([&]() -> int {
        if (!bytes)
            return SERAC_ERR_INVALID_ARG;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return hip_fail();
        size_t total = 0;
        std::lock_guard<std::mutex> lock(g_ws_mutex);
        for (auto &e : g_ws)
            if (e.dev == dev && !e.released)
                total += e.acc_bytes + e.aux_bytes;
        *bytes = (int64_t)total;
        return SERAC_OK;
    });
}

int serac_top2_pair(const uint8_t *descA, int32_t nA, const uint8_t *descB, int32_t nB,
                    void *stream_, int32_t *row_top2, int32_t *col_best)
{
    return guarded([&]() -> int {
        if (bad_set(descA, nA) || bad_set(descB, nB) ||
            (nA > 0 && (!row_top2 || misaligned(row_top2, 4))) ||
            (nB > 0 && (!col_best || misaligned(col_best, 4))))
            return SERAC_ERR_INVALID_ARG;
        Device *d = nullptr;
        int st = device_setup(&d);
        if (st != SERAC_OK)
            return st;
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        if (nA == 0 && nB == 0)
            return SERAC_OK;
        const Plan p = make_plan(std::max(nA, 1), std::max(nB, 1), 0, d->cus);
        Workspace *w = nullptr;
        std::unique_lock<std::mutex> hold;
        st = get_workspace(stream, p.acc, p.scratch + pair_prep_bytes(std::max(nA, 1), std::max(nB, 1)),
                           &w, hold);
        if (st != SERAC_OK)
            return st;
        Job J;
        const PrepJob none{};
        fill_job(J, p, descA, nA, none, descB, nB, none, next_region(w), w->aux, nullptr, nullptr);
        // with an empty side nothing is raised: rows report (0, -1, 0) and
        // columns (0, -1) from the cleared accumulators
        if (nA > 0 && nB > 0)
            // the export clears the column accumulators: nothing stays raised
            launch_pair(J, p, descA, nA, descB, nB, w->aux + p.scratch, take_clear(w, 0), true,
                        stream);
        if (nA > 0)
            serac_export_rows<<<(nA + 255) / 256, 256, 0, stream>>>(J, row_top2);
        if (nB > 0)
            serac_export_cols<<<(nB + 255) / 256, 256, 0, stream>>>(J, col_best);
        if (hipGetLastError() != hipSuccess) {
            mark_dirty(w);
            return SERAC_ERR_HIP;
        }
        return SERAC_OK;
    });
}

int serac_angle_slack(double *slack)
{
    return guarded([&]() -> int {
        if (!slack)
            return SERAC_ERR_INVALID_ARG;
        Device *d = nullptr;
        const int st = device_setup(&d);
        if (st != SERAC_OK)
            return st;
        *slack = d->slack;
        return SERAC_OK;
    });
}

int serac_profile_start(int32_t max_launches, int32_t every)
{
    return guarded([&]() -> int {
        if (max_launches < 1 || max_launches > (1 << 20) || every < 1 || every > (1 << 20))
            return SERAC_ERR_INVALID_ARG;
        std::lock_guard<std::mutex> lock(g_prof_mutex);
        for (hipEvent_t e : g_prof.ev)
            if (e)
                (void)hipEventDestroy(e);
        g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
        g_prof.used = 0;
        g_prof.seen = 0;
        g_prof.every = every;
        g_prof.armed = false;
        g_prof.kernel = nullptr;
        // Without a system-scope fence: a default event makes its dispatch
        // write the caches back for the host at the end, which lengthened the
        // timed launches by ~1.3 us against the untimed ones (profiler trace).
        for (auto &e : g_prof.ev) {
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
                e = nullptr;
                return hip_fail();
            }
        }
        g_prof.armed = true;
        return SERAC_OK;
    });
}

int serac_profile_stop(double *tile_kernel_ms, int32_t *launches, float *per_launch_ms,
                       int32_t capacity, const char **kernel)
{
    return guarded([&]() -> int {
        if (!tile_kernel_ms || !launches || capacity < 0 || (capacity > 0 && !per_launch_ms))
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
            if (k < capacity)
                per_launch_ms[k] = ms;
        }
        *tile_kernel_ms = total;
        *launches = g_prof.used;
        if (kernel)
            *kernel = g_prof.kernel ? g_prof.kernel : "none";
        for (hipEvent_t e : g_prof.ev)
            if (e)
                (void)hipEventDestroy(e);
        g_prof.ev.clear();
        g_prof.used = 0;
        g_prof.armed = false;
        return st;
    });
}

}  // extern "C"

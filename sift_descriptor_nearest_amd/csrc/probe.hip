// probe.hip - measurement kernels for the benchmark (not part of the matcher).
//
// serac_probe_mfma runs back-to-back v_mfma_i32_32x32x32_i8 on independent
// accumulators, with NV independent v_max3_u32 issued after each MFMA, and
// reports the achieved int8 rate and the shader clock the waves saw (ticks
// of the shader-clock counter against the constant 100 MHz real-time
// counter).  With NV = 0 it measures the matrix-core ceiling; with NV > 0 it
// measures what each vector instruction beside an MFMA costs in issue
// cycles, which is what bounds the matcher's sweep (its epilogue issues
// vector instructions between MFMAs).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "serac_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int PROBE_THREADS = 256;      // four waves: one per SIMD per workgroup
constexpr int CHAINS = 4;               // independent accumulators per wave

template <int NV>
__global__ __launch_bounds__(PROBE_THREADS) void probe_mfma(int iters, int *out,
                                                             unsigned long long *clk)
{
    const int t = threadIdx.x;
    v4i a = {t, 1, 2, 3};
    v4i b = {3, t, 1, 2};
    v16i c[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
        c[j] = v16i{};
    uint32_t x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = (uint32_t)t + j;
    const uint32_t y = (uint32_t)t * 7u, z = (uint32_t)t * 13u;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < CHAINS; ++j) {
            // inline assembly keeps the compiler from folding or reordering
            // the chain: one MFMA, then NV vector instructions independent of it
            asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+v"(c[j]) : "v"(a), "v"(b));
#pragma unroll
            for (int v = 0; v < NV; ++v)
                asm volatile("v_max3_u32 %0, %0, %1, %2" : "+v"(x[v & 7]) : "v"(y), "v"(z));
        }
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    int s = 0;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            s += c[j][e];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        s += (int)x[j];
    out[blockIdx.x * PROBE_THREADS + t] = s;
    if (t == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

template <int NV>
void launch(int blocks, int iters, int *out, unsigned long long *clk, hipStream_t s)
{
    probe_mfma<NV><<<blocks, PROBE_THREADS, 0, s>>>(iters, out, clk);
}

}  // namespace

extern "C" int serac_probe_mfma(int32_t blocks, int32_t iters, int32_t nv, double *ms,
                                double *tops, double *ghz)
{
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24) || !ms || !tops || !ghz)
        return -1;
    if (nv != 0 && nv != 4 && nv != 8 && nv != 12 && nv != 16)
        return -1;
    int *out = nullptr;
    unsigned long long *clk = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = -5;
    auto run = [&](hipStream_t s) {
        switch (nv) {
        case 0: launch<0>(blocks, iters, out, clk, s); break;
        case 4: launch<4>(blocks, iters, out, clk, s); break;
        case 8: launch<8>(blocks, iters, out, clk, s); break;
        case 12: launch<12>(blocks, iters, out, clk, s); break;
        default: launch<16>(blocks, iters, out, clk, s); break;
        }
    };
    if (hipMalloc(&out, (size_t)blocks * PROBE_THREADS * sizeof(int)) == hipSuccess &&
        hipMalloc(&clk, (size_t)blocks * 2 * sizeof(unsigned long long)) == hipSuccess &&
        hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
        run(nullptr);                                 // warm-up launch
        if (hipDeviceSynchronize() == hipSuccess && hipEventRecord(e0, nullptr) == hipSuccess) {
            run(nullptr);
            float f = 0.f;
            if (hipEventRecord(e1, nullptr) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
                hipEventElapsedTime(&f, e0, e1) == hipSuccess) {
                unsigned long long h[2] = {0, 0};
                if (hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost) == hipSuccess && h[1]) {
                    *ms = f;
                    *tops = (double)blocks * (PROBE_THREADS / 64) * iters * CHAINS * 65536.0 /
                            (f * 1e-3) / 1e12;
                    *ghz = (double)h[0] / ((double)h[1] / 100.0) / 1000.0;   // ticks per 10 ns
                    rc = 0;
                }
            }
        }
    }
    (void)hipGetLastError();
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (out) (void)hipFree(out);
    if (clk) (void)hipFree(clk);
    return rc;
}

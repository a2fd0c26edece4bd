// Sustained shader clock under matrix-core load: a measurement aid for the
// roofline fractions (the MI355X peaks are quoted at 2.4 GHz; a fraction at
// the clock the chip actually holds is the published peak scaled by that
// clock over 2.4 GHz).
//
// Every wave of the probe runs 16 independent bf16 MFMA accumulation chains
// (enough to keep its SIMD's matrix core issuing back to back) on operands
// that change every round, and each
// workgroup reads two counters at its start and end: s_memtime, which counts
// shader-clock cycles, and s_memrealtime, the constant 100 MHz real-time
// counter.  Their ratio is the clock the workgroup ran at.

#include <vector>

#include "ctconv_internal.h"
#include "mfma_common.h"

namespace ctconv {

namespace {

constexpr int kProbeWaves = 8;    // waves per workgroup (two per SIMD)
constexpr int kProbeChains = 16;  // independent accumulators per wave

// out[3 * wg + {0, 1, 2}] = shader cycles, real-time start, real-time end
__global__ __launch_bounds__(64 * kProbeWaves) void clock_probe_kernel(uint64_t* out, int iters,
                                                                        float seed) {
    using namespace mfma;
    const int lane = threadIdx.x & 63;
    // operands from the lane index and a run-time seed, so nothing folds
    u32x4 a, b;
    for (int e = 0; e < 4; ++e) {
        a[e] = __float_as_uint(seed * (float)(lane + e)) & 0x3F7F3F7Fu;
        b[e] = __float_as_uint(seed * (float)(lane - e)) & 0x3F7F3F7Fu;
    }
    f32x4 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) Mma<TBF16>::step(acc[c], a, b);
        // fresh operand bits every round (a linear congruential step, kept to
        // finite bf16 values below 2), as real data would toggle them
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (a[e] * 1664525u + 1013904223u) & 0x3F7F3F7Fu;
    }
    __syncthreads();
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][3];
    if (threadIdx.x == 0) {
        out[3 * blockIdx.x] = c1 - c0;
        out[3 * blockIdx.x + 1] = r0;
        out[3 * blockIdx.x + 2] = r1;
    }
    // (keeps the chains live; never true for finite sums)
    if (s != s && threadIdx.x == 1) out[3 * blockIdx.x] = 0;
}

int probe_blocks() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus > 0 ? 2 * cus : 0;  // two workgroups (16 waves) per compute unit
}

}  // namespace

}  // namespace ctconv

extern "C" {

size_t ctconv_clock_probe_bytes(void) {
    const int blocks = ctconv::probe_blocks();
    return blocks > 0 ? (size_t)blocks * 3 * sizeof(uint64_t) : 0;
}

ctconv_status ctconv_clock_probe(void* workspace, size_t workspace_bytes, int iters, double* mhz,
                                 double* tflops, void* stream) {
    using namespace ctconv;
    if (!workspace || !mhz) return CTCONV_ERR_NULL;
    if (iters < 1 || iters > (1 << 24)) return CTCONV_ERR_PARAM;
    const int blocks = probe_blocks();
    if (blocks <= 0) return CTCONV_ERR_HIP;
    const size_t need = (size_t)blocks * 3 * sizeof(uint64_t);
    if (workspace_bytes < need) return CTCONV_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 7u) != 0) return CTCONV_ERR_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)blocks), dim3(64 * kProbeWaves), 0, s,
                       static_cast<uint64_t*>(workspace), iters, 0.03125f);
    if (hipGetLastError() != hipSuccess) return CTCONV_ERR_HIP;
    std::vector<uint64_t> h((size_t)blocks * 3);
    if (hipMemcpyAsync(h.data(), workspace, need, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return CTCONV_ERR_HIP;
    double cyc = 0.0, ticks = 0.0;
    uint64_t first = UINT64_MAX, last = 0;
    for (int b = 0; b < blocks; ++b) {
        const uint64_t dc = h[3 * b], rs = h[3 * b + 1], re = h[3 * b + 2];
        if (re <= rs) return CTCONV_ERR_HIP;
        cyc += (double)dc;
        ticks += (double)(re - rs);
        if (rs < first) first = rs;
        if (re > last) last = re;
    }
    *mhz = cyc / ticks * 100.0;  // real-time counter: 100 MHz
    if (tflops) {
        // 16 x 16 x 32 multiply-adds per MFMA
        const double flops = (double)blocks * kProbeWaves * kProbeChains * (double)iters * 2.0 *
                             16.0 * 16.0 * 32.0;
        *tflops = flops / ((double)(last - first) * 10e-9) / 1e12;
    }
    return CTCONV_OK;
}

}  // extern "C"

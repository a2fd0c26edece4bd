// Phase-major weight prepack.
//
// The polyphase form of a transposed convolution with k = m*s splits the
// kernel into s phases of m taps each, tap r of phase j being w[s*r + j]
// (ExecuTorch PR #25037, Summary formula, with r = m - 1 - u); the phases are
// ordered phase-major, as the page's depth-to-space expects.  This kernel
// writes that split once per weight, in blocks of 32 input channels, so that
// the weights a column tile needs for one block of input channels (all its
// output channels and taps) are one contiguous run:
//
//   packed[j][cb][co][r][cc] = w[ci, co, sH*rH + jH, sW*rW + jW],  ci = 32*cb + cc
//   j = jH*sW + jW,  r = rH*mW + rW,  cb < C_in_pad / 32,
//
// zero where a tap index reaches past the kernel (k not a multiple of s) or
// ci >= C_in.  A pure copy of bit patterns: no arithmetic.

#include "ctconv_internal.h"

namespace ctconv {

template <typename S>
__global__ __launch_bounds__(256) void prepack_kernel(const S* __restrict__ w,
                                                      S* __restrict__ pw, int64_t total,
                                                      int64_t C_in, int64_t C_out,
                                                      int64_t C_in_pad, int64_t T, int64_t kH,
                                                      int64_t kW, int64_t sH, int64_t sW,
                                                      int64_t mW) {
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t cc = idx % kCinAlign;
        int64_t rest = idx / kCinAlign;
        const int64_t r = rest % T;
        rest /= T;
        const int64_t co = rest % C_out;
        rest /= C_out;
        const int64_t cb = rest % (C_in_pad / kCinAlign);
        const int64_t j = rest / (C_in_pad / kCinAlign);
        const int64_t ci = cb * kCinAlign + cc;
        const int64_t ty = sH * (r / mW) + j / sW;
        const int64_t tx = sW * (r % mW) + j % sW;
        S v = S(0);
        if (ci < C_in && ty < kH && tx < kW) v = w[((ci * C_out + co) * kH + ty) * kW + tx];
        pw[idx] = v;
    }
}

hipError_t launch_prepack(const Problem& p, const void* w, void* pw, hipStream_t s) {
    const int64_t total = p.P * p.C_out * p.T * p.C_in_pad;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    if (p.dtype == CTCONV_F32)
        prepack_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
            static_cast<const float*>(w), static_cast<float*>(pw), total, p.C_in, p.C_out,
            p.C_in_pad, p.T, p.kH, p.kW, p.sH, p.sW, p.mW);
    else
        prepack_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
            static_cast<const uint16_t*>(w), static_cast<uint16_t*>(pw), total, p.C_in,
            p.C_out, p.C_in_pad, p.T, p.kH, p.kW, p.sH, p.sW, p.mW);
    return hipGetLastError();
}

}  // namespace ctconv

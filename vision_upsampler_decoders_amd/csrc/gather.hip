// Gather-form transposed convolution: the route for every shape the polyphase
// kernel does not take (k not a multiple of s, output_padding, dilation).
//
// Output (oy, ox) receives tap (ty, tx) from input ((oy + pH - ty*dH)/sH,
// (ox + pW - tx*dW)/sW) when both numerators are non-negative multiples of the
// strides and the quotients fall inside the input -- the tap condition of the
// gather-form "conv_transpose2d.wgsl" in ExecuTorch PR #20849
// ("[ExecuTorch][WebGPU] Add optimized conv2d op", Implementation).  The
// weight is read from the phase-major packed layout (tap t -> phase t % s,
// tap index t / s), as the onnxruntime PR #33978 fallback gathers from X and
// the packed weights ("[WebGPU] optimizations for audio models", the review
// round on packed-filter limits).
//
// Mapping.  Which taps are valid depends only on (oy + pH) mod sH and
// (ox + pW) mod sW, so consecutive lanes take outputs of one column phase
// bx (ox = sW*ax + bx for consecutive ax) in one output row: every lane of a
// wave runs the same tap loop, and the x loads of a tap are consecutive.
// Each thread accumulates kCoT output channels in fp32 and reduces over all of
// C_in itself, so no cross-lane reduction is needed while the output grid
// alone fills the GPU.

#include "ctconv_internal.h"

namespace ctconv {

namespace {

constexpr int kCoT = 8;

template <class TR>
__global__ __launch_bounds__(256) void gather_kernel(
    const typename TR::storage* __restrict__ x, const typename TR::storage* __restrict__ pw,
    const typename TR::storage* __restrict__ bias, typename TR::storage* __restrict__ y,
    int64_t total, int64_t C_in, int64_t C_out, int64_t C_in_pad, int64_t H, int64_t W,
    int64_t Ho, int64_t Wo, int64_t Wq, int64_t n_cot, int64_t kH, int64_t kW, int64_t sH,
    int64_t sW, int64_t pH, int64_t pW, int64_t dH, int64_t dW, int64_t mW, int64_t T, int act) {
    for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < total;
         id += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ax = id % Wq;
        int64_t rest = id / Wq;
        const int64_t bx = rest % sW;
        rest /= sW;
        const int64_t oy = rest % Ho;
        rest /= Ho;
        const int64_t cot = rest % n_cot;
        const int64_t n = rest / n_cot;
        const int64_t ox = ax * sW + bx;
        if (ox >= Wo) continue;
        const int64_t co0 = cot * kCoT;

        float acc[kCoT];
#pragma unroll
        for (int c = 0; c < kCoT; ++c) acc[c] = 0.f;

        // packed layout [j][ci / 32][co][r][ci % 32]: per output channel the
        // offset of its rows inside a 32-channel block (clamped to C_out-1)
        int64_t wrow[kCoT];
#pragma unroll
        for (int c = 0; c < kCoT; ++c) {
            const int64_t co = co0 + c < C_out ? co0 + c : C_out - 1;
            wrow[c] = co * T * kCinAlign;
        }
        const int64_t blk = C_out * T * kCinAlign;  // one 32-channel block of a phase

        for (int64_t ty = 0; ty < kH; ++ty) {
            const int64_t ny = oy + pH - ty * dH;
            if (ny < 0 || ny % sH != 0) continue;
            const int64_t iy = ny / sH;
            if (iy >= H) continue;
            for (int64_t tx = 0; tx < kW; ++tx) {
                const int64_t nx = ox + pW - tx * dW;
                if (nx < 0 || nx % sW != 0) continue;
                const int64_t ix = nx / sW;
                if (ix >= W) continue;
                const int64_t j = (ty % sH) * sW + (tx % sW);
                const int64_t r = (ty / sH) * mW + (tx / sW);
                const typename TR::storage* wj =
                    pw + j * (C_in_pad / kCinAlign) * blk + r * kCinAlign;
                const typename TR::storage* xp = x + ((n * C_in) * H + iy) * W + ix;
                const int64_t HW = H * W;
                for (int64_t ci = 0; ci < C_in; ++ci) {
                    const float xv = TR::to_f32(xp[ci * HW]);
                    const typename TR::storage* wp =
                        wj + (ci / kCinAlign) * blk + (ci % kCinAlign);
#pragma unroll
                    for (int c = 0; c < kCoT; ++c)
                        acc[c] = fmaf(xv, TR::to_f32(wp[wrow[c]]), acc[c]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < kCoT; ++c) {
            const int64_t co = co0 + c;
            if (co < C_out) {
                const float b = bias ? TR::to_f32(bias[co]) : 0.f;
                float v = acc[c] + b;
                if (act == CTCONV_ACT_ELU) v = elu_act<TR>(v);
                y[((n * C_out + co) * Ho + oy) * Wo + ox] = TR::from_f32(v);
            }
        }
    }
}

template <class TR>
hipError_t launch_gather_t(const Problem& p, const void* x, const void* pw, const void* bias,
                           void* y, hipStream_t s) {
    using S = typename TR::storage;
    const int64_t Wq = (p.Wo + p.sW - 1) / p.sW;
    const int64_t n_cot = (p.C_out + kCoT - 1) / kCoT;
    const int64_t total = p.N * n_cot * p.Ho * p.sW * Wq;
    int64_t blocks = (total + 255) / 256;
    if (blocks > (int64_t)1 << 20) blocks = (int64_t)1 << 20;
    if (blocks < 1) blocks = 1;
    gather_kernel<TR><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<const S*>(x), static_cast<const S*>(pw), static_cast<const S*>(bias),
        static_cast<S*>(y), total, p.C_in, p.C_out, p.C_in_pad, p.H, p.W, p.Ho, p.Wo, Wq, n_cot,
        p.kH, p.kW, p.sH, p.sW, p.pH, p.pW, p.dH, p.dW, p.mW, p.T, p.act);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const Problem& p, const void* x, const void* pw, const void* bias,
                         void* y, hipStream_t s) {
    switch (p.dtype) {
        case CTCONV_F32: return launch_gather_t<TF32>(p, x, pw, bias, y, s);
        case CTCONV_BF16: return launch_gather_t<TBF16>(p, x, pw, bias, y, s);
        case CTCONV_F16: return launch_gather_t<TF16>(p, x, pw, bias, y, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ctconv

// Bias fill, ELU and the iSTFT tail (window-envelope normalisation and trim).
//
// fill: every output element gets bias[co] (or 0).  It serves outputs no tap
// reaches -- an empty input with a non-empty output, the case onnxruntime PR
// #33978 ("[WebGPU] optimizations for audio models") fixed by running one
// pass that writes only the bias or zeros -- and it initialises y before a
// split-over-C_in launch accumulates into it.
//
// elu: y = x for x > 0, exp(x) - 1 otherwise (alpha = 1), in fp32, one rounding.
// The fill applies the forward call's activation to what it writes, except
// before a split-over-C_in accumulation (which never carries an activation).

#include "ctconv_internal.h"

namespace ctconv {

namespace {

template <class TR>
__global__ __launch_bounds__(256) void fill_kernel(const typename TR::storage* __restrict__ bias,
                                                   typename TR::storage* __restrict__ y,
                                                   int64_t total, int64_t plane, int64_t C_out,
                                                   int act) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        typename TR::storage v = TR::from_f32(0.f);
        if (bias) v = bias[(i / plane) % C_out];
        if (act == CTCONV_ACT_ELU) v = TR::from_f32(elu_act<TR>(TR::to_f32(v)));
        y[i] = v;
    }
}

template <class TR>
__global__ __launch_bounds__(256) void elu_kernel(const typename TR::storage* x,
                                                  typename TR::storage* y, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        y[i] = TR::from_f32(elu_act<TR>(TR::to_f32(x[i])));
    }
}

// 16-byte vector variant for 16-bit types: 8 elements per thread.
template <class TR>
__global__ __launch_bounds__(256) void elu_kernel_v8(const uint4* x, uint4* y, int64_t nvec) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * blockDim.x) {
        uint4 v = x[i];
        uint16_t* h = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h[e] = TR::from_f32(elu_act<TR>(TR::to_f32(h[e])));
        }
        y[i] = v;
    }
}

// iSTFT tail: out[r, t] = y[r, trim + t] / env[trim + t] (0 where the
// window-square envelope env is below 1e-11, i.e. no frame covers the sample).
template <class TR>
__global__ __launch_bounds__(256) void istft_norm_kernel(const typename TR::storage* __restrict__ y,
                                                         const typename TR::storage* __restrict__ env,
                                                         typename TR::storage* __restrict__ out,
                                                         int64_t rows, int64_t L_in, int64_t trim,
                                                         int64_t L_out) {
    const int64_t total = rows * L_out;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / L_out, t = i - r * L_out;
        const float e = TR::to_f32(env[trim + t]);
        const float v = TR::to_f32(y[r * L_in + trim + t]);
        out[i] = TR::from_f32(e > 1e-11f ? v / e : 0.f);
    }
}

int64_t grid_for(int64_t work) {
    int64_t b = (work + 255) / 256;
    if (b > 65536) b = 65536;
    return b < 1 ? 1 : b;
}

template <class TR>
hipError_t fill_t(const Problem& p, const void* bias, void* y, hipStream_t s) {
    using S = typename TR::storage;
    const int64_t plane = p.Ho * p.Wo;
    const int64_t total = p.N * p.C_out * plane;
    fill_kernel<TR><<<dim3((unsigned)grid_for(total)), dim3(256), 0, s>>>(
        static_cast<const S*>(bias), static_cast<S*>(y), total, plane, p.C_out, p.act);
    return hipGetLastError();
}

template <class TR>
hipError_t elu_t(const void* x, void* y, int64_t n, hipStream_t s) {
    using S = typename TR::storage;
    if (sizeof(S) == 2) {
        const int64_t nvec = n / 8;
        if (nvec > 0)
            elu_kernel_v8<TR><<<dim3((unsigned)grid_for(nvec)), dim3(256), 0, s>>>(
                static_cast<const uint4*>(x), static_cast<uint4*>(y), nvec);
        const int64_t done = nvec * 8;
        if (n > done)
            elu_kernel<TR><<<dim3(1), dim3(256), 0, s>>>(static_cast<const S*>(x) + done,
                                                         static_cast<S*>(y) + done, n - done);
    } else {
        elu_kernel<TR><<<dim3((unsigned)grid_for(n)), dim3(256), 0, s>>>(
            static_cast<const S*>(x), static_cast<S*>(y), n);
    }
    return hipGetLastError();
}

template <class TR>
hipError_t istft_norm_t(const void* y, const void* env, void* out, int64_t rows, int64_t L_in,
                        int64_t trim, int64_t L_out, hipStream_t s) {
    using S = typename TR::storage;
    istft_norm_kernel<TR><<<dim3((unsigned)grid_for(rows * L_out)), dim3(256), 0, s>>>(
        static_cast<const S*>(y), static_cast<const S*>(env), static_cast<S*>(out), rows, L_in,
        trim, L_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_istft_norm(const void* y, const void* env, void* out, int64_t rows,
                             int64_t L_in, int64_t trim, int64_t L_out, ctconv_dtype dt,
                             hipStream_t s) {
    if (rows * L_out <= 0) return hipSuccess;
    switch (dt) {
        case CTCONV_F32: return istft_norm_t<TF32>(y, env, out, rows, L_in, trim, L_out, s);
        case CTCONV_BF16: return istft_norm_t<TBF16>(y, env, out, rows, L_in, trim, L_out, s);
        case CTCONV_F16: return istft_norm_t<TF16>(y, env, out, rows, L_in, trim, L_out, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fill(const Problem& p, const void* bias, void* y, hipStream_t s) {
    switch (p.dtype) {
        case CTCONV_F32: return fill_t<TF32>(p, bias, y, s);
        case CTCONV_BF16: return fill_t<TBF16>(p, bias, y, s);
        case CTCONV_F16: return fill_t<TF16>(p, bias, y, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_elu(const void* x, void* y, int64_t n, ctconv_dtype dt, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    switch (dt) {
        case CTCONV_F32: return elu_t<TF32>(x, y, n, s);
        case CTCONV_BF16: return elu_t<TBF16>(x, y, n, s);
        case CTCONV_F16: return elu_t<TF16>(x, y, n, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ctconv

// Bias fill, ELU and the iSTFT tail (window-envelope normalisation and trim).
//
// fill: every output element gets bias[co] (or 0).  It serves outputs no tap
// reaches -- an empty input with a non-empty output, the case onnxruntime PR
// #33978 ("[WebGPU] optimizations for audio models") fixed by running one
// pass that writes only the bias or zeros -- and the outputs of a dilated
// shape that no tap reaches.  It applies the forward call's activation to
// what it writes.
//
// split reduce: the sum of the partial results of a reduction split over
// input-channel ranges (the first in y, the others in a caller workspace),
// added in a fixed order, so the result is the same bits on every run; then
// the bias and the activation.
//
// elu: y = x for x > 0, exp(x) - 1 otherwise (alpha = 1), in fp32, one rounding.

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

// y[i] = act(((y[i] + ws[0][i]) + ws[1][i]) + ... + bias[co]) in fp32, four
// elements per thread (total is a multiple of 4, as are the slab offsets).
__global__ __launch_bounds__(256) void split_reduce_kernel(float4* __restrict__ y,
                                                           const float4* __restrict__ ws,
                                                           const float* __restrict__ bias,
                                                           int64_t nvec, int64_t slab_vec,
                                                           int nslab, int64_t plane, int64_t C_out,
                                                           int act) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * blockDim.x) {
        float4 v = y[i];
        for (int k = 0; k < nslab; ++k) {
            const float4 w = ws[k * slab_vec + i];
            v.x += w.x;
            v.y += w.y;
            v.z += w.z;
            v.w += w.w;
        }
        float r[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (bias) r[e] += bias[((4 * i + e) / plane) % C_out];
            if (act == CTCONV_ACT_ELU) r[e] = elu_act<TF32>(r[e]);
        }
        y[i] = make_float4(r[0], r[1], r[2], r[3]);
    }
}

// The same for a total that is not a multiple of 4 (one element per thread).
__global__ __launch_bounds__(256) void split_reduce_kernel_1(float* __restrict__ y,
                                                             const float* __restrict__ ws,
                                                             const float* __restrict__ bias,
                                                             int64_t total, int64_t slab, int nslab,
                                                             int64_t plane, int64_t C_out,
                                                             int act) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = y[i];
        for (int k = 0; k < nslab; ++k) v += ws[k * slab + i];
        if (bias) v += bias[(i / plane) % C_out];
        if (act == CTCONV_ACT_ELU) v = elu_act<TF32>(v);
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

hipError_t launch_split_reduce(const Problem& p, const void* bias, void* y, const void* ws,
                               int nslab, hipStream_t s) {
    const int64_t plane = p.Ho * p.Wo;
    const int64_t total = p.N * p.C_out * plane;
    if (total <= 0) return hipSuccess;
    if (total % 4 == 0) {
        split_reduce_kernel<<<dim3((unsigned)grid_for(total / 4)), dim3(256), 0, s>>>(
            static_cast<float4*>(y), static_cast<const float4*>(ws),
            static_cast<const float*>(bias), total / 4, total / 4, nslab, plane, p.C_out, p.act);
    } else {
        split_reduce_kernel_1<<<dim3((unsigned)grid_for(total)), dim3(256), 0, s>>>(
            static_cast<float*>(y), static_cast<const float*>(ws),
            static_cast<const float*>(bias), total, total, nslab, plane, p.C_out, p.act);
    }
    return hipGetLastError();
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

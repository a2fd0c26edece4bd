// Streaming (chunked) 1-D transposed convolution: overlap-add of the held-back
// tail and the final flush.
//
// A decoder that produces audio frame by frame runs the transposed
// convolution on each new chunk of input frames.  Frame i reaches outputs
// [i*s, i*s + k), so after the frames [0, F) the outputs below F*s are final
// and the k - s outputs from F*s on still await later frames (ExecuTorch PR
// #25037: Phonon's StreamingConvTranspose1d holds that tail back between
// 80 ms frames, and feeds the bias both to the conv and to the tail
// bookkeeping).  Here the chunk's convolution is computed without bias into
// an fp32 workspace (no rounding), the tail is kept as fp32 partial sums
// without bias, and the bias and the activation are applied, and the result
// rounded to the storage type, exactly once, when an output is emitted.
//
// overlap: one chunk of L frames, z = convT(chunk) of length L*s + (k - s):
//   y[o]        = act(z[o] + tail_in[o] + bias)      o <  L*s (tail_in[o] = 0 past k - s)
//   tail_out[t] = z[L*s + t] + tail_in[L*s + t]      t <  k - s
// flush (end of the stream): y[t] = act(tail_in[t] + bias), t < k - s.

#include "ctconv_internal.h"

namespace ctconv {

namespace {

template <class TR>
__global__ __launch_bounds__(256) void overlap_kernel(const float* __restrict__ z,
                                                      const float* __restrict__ tail_in,
                                                      const typename TR::storage* __restrict__ bias,
                                                      typename TR::storage* __restrict__ y,
                                                      float* __restrict__ tail_out, int64_t rows,
                                                      int64_t C_out, int64_t Ly, int64_t Tl,
                                                      int act) {
    const int64_t Lz = Ly + Tl;
    const int64_t total = rows * Lz;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / Lz, o = i - row * Lz;
        float v = z[i];
        if (tail_in != nullptr && o < Tl) v += tail_in[row * Tl + o];
        if (o < Ly) {
            if (bias != nullptr) v += TR::to_f32(bias[row % C_out]);
            if (act == CTCONV_ACT_ELU) v = elu_act<TR>(v);
            y[row * Ly + o] = TR::from_f32(v);
        } else {
            tail_out[row * Tl + (o - Ly)] = v;
        }
    }
}

template <class TR>
__global__ __launch_bounds__(256) void flush_kernel(const float* __restrict__ tail_in,
                                                    const typename TR::storage* __restrict__ bias,
                                                    typename TR::storage* __restrict__ y,
                                                    int64_t rows, int64_t C_out, int64_t Tl,
                                                    int act) {
    const int64_t total = rows * Tl;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / Tl;
        float v = tail_in != nullptr ? tail_in[i] : 0.f;
        if (bias != nullptr) v += TR::to_f32(bias[row % C_out]);
        if (act == CTCONV_ACT_ELU) v = elu_act<TR>(v);
        y[i] = TR::from_f32(v);
    }
}

int64_t grid_for(int64_t work) {
    int64_t b = (work + 255) / 256;
    if (b > 65536) b = 65536;
    return b < 1 ? 1 : b;
}

template <class TR>
hipError_t overlap_t(const float* z, const float* tail_in, const void* bias, void* y,
                     float* tail_out, int64_t rows, int64_t C_out, int64_t Ly, int64_t Tl, int act,
                     hipStream_t s) {
    using S = typename TR::storage;
    overlap_kernel<TR><<<dim3((unsigned)grid_for(rows * (Ly + Tl))), dim3(256), 0, s>>>(
        z, tail_in, static_cast<const S*>(bias), static_cast<S*>(y),
        tail_out, rows, C_out, Ly, Tl, act);
    return hipGetLastError();
}

template <class TR>
hipError_t flush_t(const float* tail_in, const void* bias, void* y, int64_t rows, int64_t C_out,
                   int64_t Tl, int act, hipStream_t s) {
    using S = typename TR::storage;
    flush_kernel<TR><<<dim3((unsigned)grid_for(rows * Tl)), dim3(256), 0, s>>>(
        tail_in, static_cast<const S*>(bias), static_cast<S*>(y), rows, C_out, Tl, act);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_overlap(const float* z, const float* tail_in, const void* bias, void* y,
                                 float* tail_out, int64_t rows, int64_t C_out, int64_t Ly,
                                 int64_t Tl, ctconv_dtype dt, int act, hipStream_t s) {
    if (rows * (Ly + Tl) <= 0) return hipSuccess;
    switch (dt) {
        case CTCONV_F32: return overlap_t<TF32>(z, tail_in, bias, y, tail_out, rows, C_out, Ly, Tl, act, s);
        case CTCONV_BF16: return overlap_t<TBF16>(z, tail_in, bias, y, tail_out, rows, C_out, Ly, Tl, act, s);
        case CTCONV_F16: return overlap_t<TF16>(z, tail_in, bias, y, tail_out, rows, C_out, Ly, Tl, act, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_stream_flush(const float* tail_in, const void* bias, void* y, int64_t rows,
                               int64_t C_out, int64_t Tl, ctconv_dtype dt, int act,
                               hipStream_t s) {
    if (rows * Tl <= 0) return hipSuccess;
    switch (dt) {
        case CTCONV_F32: return flush_t<TF32>(tail_in, bias, y, rows, C_out, Tl, act, s);
        case CTCONV_BF16: return flush_t<TBF16>(tail_in, bias, y, rows, C_out, Tl, act, s);
        case CTCONV_F16: return flush_t<TF16>(tail_in, bias, y, rows, C_out, Tl, act, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ctconv

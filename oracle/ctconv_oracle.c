/*
 * ctconv_oracle.c -- CPU reference for dense transposed convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * Everything is plain, single-threaded and computed in double precision.
 * Loops follow the definitions below with no blocking, fusion or reordering.
 *
 * Definition followed (scatter form).  Each input element x[n,ci,i] adds
 * x[n,ci,i] * w[ci,co,t] to the output element at o = i*s - p + t*d, for every
 * output channel co and kernel tap t, and is dropped when o falls outside
 * [0, L_out).  The weight is the un-flipped ConvTranspose layout
 * [C_in, C_out, k...]; this is the layout and the tap condition that the
 * gather-form kernel "conv_transpose2d.wgsl" of ExecuTorch PR #20849
 * ("[ExecuTorch][WebGPU] Add optimized conv2d op", Implementation) inverts.
 * In 2-D the condition holds per dimension.
 *
 *   L_out = (L_in - 1)*s - 2*p + d*(k - 1) + op + 1
 *
 * (the output length of the same page's transposed path; for d = 1 it is the
 * "clean upscale" length of ExecuTorch PR #25037, commit "Decompose depthwise
 * transposed convs", and the inverse of the page's tap condition in general).
 * Padding p is removed from both ends; output_padding op adds op elements at
 * the high end only.  The bias, when present, is added once to every output.
 *
 * Parity pins live in tests/test_oracle_pins.py (torch float64 reference,
 * adjoint identity with an independent direct convolution, the polyphase
 * identity, impulse responses, the k = s matmul special case, hand-computed
 * examples and the inverse-STFT closed forms).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_BAD 1

/* Per-dimension output length; returns -1 when the parameters are invalid. */
static int64_t or_out_len(int64_t L, int64_t k, int64_t s, int64_t p,
                          int64_t op, int64_t d) {
    if (L < 0 || k < 1 || s < 1 || d < 1 || p < 0 || op < 0) return -1;
    return (L - 1) * s - 2 * p + d * (k - 1) + op + 1;
}

/* Expand 1-D or 2-D per-dimension arguments into (H, W) pairs, with the 1-D
 * case as H = 1 and a trivial first dimension. */
static int or_expand(int ndim, const int64_t* v, int64_t fill, int64_t out[2]) {
    if (ndim == 1) {
        out[0] = fill;
        out[1] = v[0];
        return OR_OK;
    }
    if (ndim == 2) {
        out[0] = v[0];
        out[1] = v[1];
        return OR_OK;
    }
    return OR_BAD;
}

int ctconv_oracle_output_shape(int ndim, const int64_t* in_sp, const int64_t* k,
                               const int64_t* s, const int64_t* p, const int64_t* op,
                               const int64_t* d, int64_t* out_sp) {
    if (ndim != 1 && ndim != 2) return OR_BAD;
    for (int i = 0; i < ndim; ++i) {
        int64_t L = or_out_len(in_sp[i], k[i], s[i], p[i], op[i], d[i]);
        if (L < 1) return OR_BAD;
        out_sp[i] = L;
    }
    return OR_OK;
}

/*
 * Full transposed convolution, scatter form.
 *   x    [N, C_in, H, W]          (1-D: [N, C_in, L])
 *   w    [C_in, C_out, kH, kW]    (1-D: [C_in, C_out, k])
 *   bias [C_out] or NULL
 *   y    [N, C_out, Ho, Wo]       written completely
 */
int ctconv_oracle_conv_transpose(int ndim, int64_t N, int64_t C_in, int64_t C_out,
                                 const int64_t* in_sp, const int64_t* kernel,
                                 const int64_t* stride, const int64_t* padding,
                                 const int64_t* output_padding, const int64_t* dilation,
                                 const double* x, const double* w, const double* bias,
                                 double* y) {
    int64_t in2[2], k2[2], s2[2], p2[2], op2[2], d2[2], o2[2];
    if (or_expand(ndim, in_sp, 1, in2) || or_expand(ndim, kernel, 1, k2) ||
        or_expand(ndim, stride, 1, s2) || or_expand(ndim, padding, 0, p2) ||
        or_expand(ndim, output_padding, 0, op2) || or_expand(ndim, dilation, 1, d2))
        return OR_BAD;
    if (N < 0 || C_in < 1 || C_out < 1) return OR_BAD;
    for (int a = 0; a < 2; ++a) {
        o2[a] = or_out_len(in2[a], k2[a], s2[a], p2[a], op2[a], d2[a]);
        if (o2[a] < 1) return OR_BAD;
    }
    const int64_t H = in2[0], W = in2[1], Ho = o2[0], Wo = o2[1];
    const int64_t kH = k2[0], kW = k2[1];

    /* y = bias broadcast (or zero) */
    for (int64_t n = 0; n < N; ++n)
        for (int64_t co = 0; co < C_out; ++co) {
            double b = bias ? bias[co] : 0.0;
            double* yp = y + (n * C_out + co) * Ho * Wo;
            for (int64_t e = 0; e < Ho * Wo; ++e) yp[e] = b;
        }

    /* scatter every input element through every tap */
    for (int64_t n = 0; n < N; ++n)
        for (int64_t ci = 0; ci < C_in; ++ci)
            for (int64_t iy = 0; iy < H; ++iy)
                for (int64_t ix = 0; ix < W; ++ix) {
                    const double xv = x[((n * C_in + ci) * H + iy) * W + ix];
                    for (int64_t co = 0; co < C_out; ++co)
                        for (int64_t ty = 0; ty < kH; ++ty) {
                            const int64_t oy = iy * s2[0] - p2[0] + ty * d2[0];
                            if (oy < 0 || oy >= Ho) continue;
                            for (int64_t tx = 0; tx < kW; ++tx) {
                                const int64_t ox = ix * s2[1] - p2[1] + tx * d2[1];
                                if (ox < 0 || ox >= Wo) continue;
                                const double wv = w[((ci * C_out + co) * kH + ty) * kW + tx];
                                y[((n * C_out + co) * Ho + oy) * Wo + ox] += xv * wv;
                            }
                        }
                }
    return OR_OK;
}

/*
 * Selected output elements, one at a time, from the same definition: output
 * (n, co, oy, ox) collects x[n,ci,iy,ix] * w[ci,co,ty,tx] over every input
 * position and tap whose scatter target i*s - p + t*d equals it.  The input
 * position is solved from the tap (it exists iff o + p - t*d is a
 * non-negative multiple of s below s*L_in), which is the same set of terms.
 *   idx  [n_pts][4] = (n, co, oy, ox); 1-D uses oy = 0.
 */
int ctconv_oracle_points(int ndim, int64_t N, int64_t C_in, int64_t C_out,
                         const int64_t* in_sp, const int64_t* kernel,
                         const int64_t* stride, const int64_t* padding,
                         const int64_t* output_padding, const int64_t* dilation,
                         const double* x, const double* w, const double* bias,
                         const int64_t* idx, int64_t n_pts, double* out) {
    int64_t in2[2], k2[2], s2[2], p2[2], op2[2], d2[2], o2[2];
    if (or_expand(ndim, in_sp, 1, in2) || or_expand(ndim, kernel, 1, k2) ||
        or_expand(ndim, stride, 1, s2) || or_expand(ndim, padding, 0, p2) ||
        or_expand(ndim, output_padding, 0, op2) || or_expand(ndim, dilation, 1, d2))
        return OR_BAD;
    for (int a = 0; a < 2; ++a) {
        o2[a] = or_out_len(in2[a], k2[a], s2[a], p2[a], op2[a], d2[a]);
        if (o2[a] < 1) return OR_BAD;
    }
    const int64_t H = in2[0], W = in2[1];
    const int64_t kH = k2[0], kW = k2[1];
    for (int64_t e = 0; e < n_pts; ++e) {
        const int64_t n = idx[4 * e], co = idx[4 * e + 1];
        const int64_t oy = idx[4 * e + 2], ox = idx[4 * e + 3];
        if (n < 0 || n >= N || co < 0 || co >= C_out || oy < 0 || oy >= o2[0] ||
            ox < 0 || ox >= o2[1])
            return OR_BAD;
        double acc = bias ? bias[co] : 0.0;
        for (int64_t ci = 0; ci < C_in; ++ci)
            for (int64_t ty = 0; ty < kH; ++ty) {
                const int64_t ny = oy + p2[0] - ty * d2[0];
                if (ny < 0 || ny % s2[0] != 0) continue;
                const int64_t iy = ny / s2[0];
                if (iy >= H) continue;
                for (int64_t tx = 0; tx < kW; ++tx) {
                    const int64_t nx = ox + p2[1] - tx * d2[1];
                    if (nx < 0 || nx % s2[1] != 0) continue;
                    const int64_t ix = nx / s2[1];
                    if (ix >= W) continue;
                    acc += x[((n * C_in + ci) * H + iy) * W + ix] *
                           w[((ci * C_out + co) * kH + ty) * kW + tx];
                }
            }
        out[e] = acc;
    }
    return OR_OK;
}

/*
 * Grouped transposed convolution (the groups argument of ConvTranspose), same
 * scatter definition.  The channels split into G equal groups: input channel
 * ci lies in group g = ci / (C_in / G) and reaches only the output channels
 * co = g * (C_out / G) + j, j < C_out / G, through w[ci, j, t]; the weight is
 * [C_in, C_out / G, k...].  G = C_in is the depthwise transposed convolution
 * (one input channel per group) that ExecuTorch PR #25037, commit
 * "Decompose depthwise transposed convs", rewrites into per-phase depthwise
 * stride-1 convolutions and a depth-to-space; G = 1 is the dense case above.
 *   x    [N, C_in, H, W]            (1-D: [N, C_in, L])
 *   w    [C_in, C_out/G, kH, kW]    (1-D: [C_in, C_out/G, k])
 *   bias [C_out] or NULL
 *   y    [N, C_out, Ho, Wo]         written completely
 */
int ctconv_oracle_conv_transpose_grouped(int ndim, int64_t N, int64_t C_in, int64_t C_out,
                                         int64_t groups, const int64_t* in_sp,
                                         const int64_t* kernel, const int64_t* stride,
                                         const int64_t* padding, const int64_t* output_padding,
                                         const int64_t* dilation, const double* x,
                                         const double* w, const double* bias, double* y) {
    int64_t in2[2], k2[2], s2[2], p2[2], op2[2], d2[2], o2[2];
    if (or_expand(ndim, in_sp, 1, in2) || or_expand(ndim, kernel, 1, k2) ||
        or_expand(ndim, stride, 1, s2) || or_expand(ndim, padding, 0, p2) ||
        or_expand(ndim, output_padding, 0, op2) || or_expand(ndim, dilation, 1, d2))
        return OR_BAD;
    if (N < 0 || C_in < 1 || C_out < 1 || groups < 1 || C_in % groups || C_out % groups)
        return OR_BAD;
    for (int a = 0; a < 2; ++a) {
        o2[a] = or_out_len(in2[a], k2[a], s2[a], p2[a], op2[a], d2[a]);
        if (o2[a] < 1) return OR_BAD;
    }
    const int64_t H = in2[0], W = in2[1], Ho = o2[0], Wo = o2[1];
    const int64_t kH = k2[0], kW = k2[1];
    const int64_t cig = C_in / groups, cog = C_out / groups;

    for (int64_t n = 0; n < N; ++n)
        for (int64_t co = 0; co < C_out; ++co) {
            double b = bias ? bias[co] : 0.0;
            double* yp = y + (n * C_out + co) * Ho * Wo;
            for (int64_t e = 0; e < Ho * Wo; ++e) yp[e] = b;
        }

    for (int64_t n = 0; n < N; ++n)
        for (int64_t ci = 0; ci < C_in; ++ci) {
            const int64_t g = ci / cig;
            for (int64_t iy = 0; iy < H; ++iy)
                for (int64_t ix = 0; ix < W; ++ix) {
                    const double xv = x[((n * C_in + ci) * H + iy) * W + ix];
                    for (int64_t j = 0; j < cog; ++j) {
                        const int64_t co = g * cog + j;
                        for (int64_t ty = 0; ty < kH; ++ty) {
                            const int64_t oy = iy * s2[0] - p2[0] + ty * d2[0];
                            if (oy < 0 || oy >= Ho) continue;
                            for (int64_t tx = 0; tx < kW; ++tx) {
                                const int64_t ox = ix * s2[1] - p2[1] + tx * d2[1];
                                if (ox < 0 || ox >= Wo) continue;
                                const double wv = w[((ci * cog + j) * kH + ty) * kW + tx];
                                y[((n * C_out + co) * Ho + oy) * Wo + ox] += xv * wv;
                            }
                        }
                    }
                }
        }
    return OR_OK;
}

/*
 * Selected outputs of the grouped transposed convolution, one at a time:
 * output (n, co, oy, ox) collects the terms of the input channels of co's
 * group, each input position solved from the tap as in ctconv_oracle_points.
 *   idx  [n_pts][4] = (n, co, oy, ox); 1-D uses oy = 0.
 */
int ctconv_oracle_points_grouped(int ndim, int64_t N, int64_t C_in, int64_t C_out,
                                 int64_t groups, const int64_t* in_sp, const int64_t* kernel,
                                 const int64_t* stride, const int64_t* padding,
                                 const int64_t* output_padding, const int64_t* dilation,
                                 const double* x, const double* w, const double* bias,
                                 const int64_t* idx, int64_t n_pts, double* out) {
    int64_t in2[2], k2[2], s2[2], p2[2], op2[2], d2[2], o2[2];
    if (or_expand(ndim, in_sp, 1, in2) || or_expand(ndim, kernel, 1, k2) ||
        or_expand(ndim, stride, 1, s2) || or_expand(ndim, padding, 0, p2) ||
        or_expand(ndim, output_padding, 0, op2) || or_expand(ndim, dilation, 1, d2))
        return OR_BAD;
    if (groups < 1 || C_in % groups || C_out % groups) return OR_BAD;
    for (int a = 0; a < 2; ++a) {
        o2[a] = or_out_len(in2[a], k2[a], s2[a], p2[a], op2[a], d2[a]);
        if (o2[a] < 1) return OR_BAD;
    }
    const int64_t H = in2[0], W = in2[1];
    const int64_t kH = k2[0], kW = k2[1];
    const int64_t cig = C_in / groups, cog = C_out / groups;
    for (int64_t e = 0; e < n_pts; ++e) {
        const int64_t n = idx[4 * e], co = idx[4 * e + 1];
        const int64_t oy = idx[4 * e + 2], ox = idx[4 * e + 3];
        if (n < 0 || n >= N || co < 0 || co >= C_out || oy < 0 || oy >= o2[0] ||
            ox < 0 || ox >= o2[1])
            return OR_BAD;
        const int64_t g = co / cog, j = co % cog;
        double acc = bias ? bias[co] : 0.0;
        for (int64_t ci = g * cig; ci < (g + 1) * cig; ++ci)
            for (int64_t ty = 0; ty < kH; ++ty) {
                const int64_t ny = oy + p2[0] - ty * d2[0];
                if (ny < 0 || ny % s2[0] != 0) continue;
                const int64_t iy = ny / s2[0];
                if (iy >= H) continue;
                for (int64_t tx = 0; tx < kW; ++tx) {
                    const int64_t nx = ox + p2[1] - tx * d2[1];
                    if (nx < 0 || nx % s2[1] != 0) continue;
                    const int64_t ix = nx / s2[1];
                    if (ix >= W) continue;
                    acc += x[((n * C_in + ci) * H + iy) * W + ix] *
                           w[((ci * cog + j) * kH + ty) * kW + tx];
                }
            }
        out[e] = acc;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Inverse STFT by overlap-add, independent of the transposed convolution.  */
/* ------------------------------------------------------------------------ */

/* In-place iterative radix-2 complex FFT of length n (a power of two) with
 * exponent sign `sign` (+1 for the inverse transform, unnormalised). */
static void or_fft(double* re, double* im, int64_t n, int sign) {
    for (int64_t i = 1, j = 0; i < n; ++i) { /* bit reversal */
        int64_t bit = n >> 1;
        for (; j & bit; bit >>= 1) j ^= bit;
        j ^= bit;
        if (i < j) {
            double t = re[i]; re[i] = re[j]; re[j] = t;
            t = im[i]; im[i] = im[j]; im[j] = t;
        }
    }
    for (int64_t len = 2; len <= n; len <<= 1) {
        const int64_t half = len >> 1;
        for (int64_t j = 0; j < half; ++j) {
            /* twiddle exp(sign * 2 pi i j / len), argument reduced exactly */
            const double ang = sign * 2.0 * M_PI * (double)j / (double)len;
            const double wr = cos(ang), wi = sin(ang);
            for (int64_t i = 0; i < n; i += len) {
                double* ar = re + i + j; double* ai = im + i + j;
                double* br = re + i + j + half; double* bi = im + i + j + half;
                const double tr = *br * wr - *bi * wi;
                const double ti = *br * wi + *bi * wr;
                *br = *ar - tr; *bi = *ai - ti;
                *ar += tr; *ai += ti;
            }
        }
    }
}

/*
 * spec [N, 2F, T] with F = n_fft/2 + 1: channels [0, F) hold the real parts
 * and [F, 2F) the imaginary parts of each frame's one-sided spectrum.
 * Per frame: irfft (1/n normalisation; the imaginary parts of the DC and
 * Nyquist bins do not enter a real signal), multiply by the periodic Hann
 * window, overlap-add at hop.  y [N, (T-1)*hop + n_fft].
 */
int ctconv_oracle_istft_ola(int64_t N, int64_t n_fft, int64_t hop, int64_t T,
                            const double* spec, double* y) {
    if (n_fft < 2 || (n_fft & (n_fft - 1)) != 0 || hop < 1 || T < 0 || N < 0)
        return OR_BAD;
    const int64_t F = n_fft / 2 + 1;
    const int64_t Lo = (T - 1) * hop + n_fft;
    if (Lo < 1) return OR_BAD;
    double* re = (double*)malloc(sizeof(double) * n_fft);
    double* im = (double*)malloc(sizeof(double) * n_fft);
    if (!re || !im) { free(re); free(im); return OR_BAD; }
    for (int64_t n = 0; n < N; ++n) {
        double* yn = y + n * Lo;
        for (int64_t e = 0; e < Lo; ++e) yn[e] = 0.0;
        for (int64_t l = 0; l < T; ++l) {
            const double* sp = spec + n * 2 * F * T;
            for (int64_t f = 0; f < F; ++f) {
                re[f] = sp[f * T + l];
                im[f] = (f == 0 || f == n_fft / 2) ? 0.0 : sp[(F + f) * T + l];
            }
            for (int64_t f = 1; f < n_fft / 2; ++f) { /* Hermitian extension */
                re[n_fft - f] = re[f];
                im[n_fft - f] = -im[f];
            }
            or_fft(re, im, n_fft, +1);
            for (int64_t t = 0; t < n_fft; ++t) {
                const double h = 0.5 - 0.5 * cos(2.0 * M_PI * (double)t / (double)n_fft);
                yn[l * hop + t] += re[t] / (double)n_fft * h;
            }
        }
    }
    free(re);
    free(im);
    return OR_OK;
}

/* Forward real FFT of one real frame (used by the reconstruction pin to build
 * spectra): out_re/out_im [n/2 + 1]. */
int ctconv_oracle_rfft(int64_t n, const double* frame, double* out_re, double* out_im) {
    if (n < 2 || (n & (n - 1)) != 0) return OR_BAD;
    double* re = (double*)malloc(sizeof(double) * n);
    double* im = (double*)malloc(sizeof(double) * n);
    if (!re || !im) { free(re); free(im); return OR_BAD; }
    for (int64_t t = 0; t < n; ++t) { re[t] = frame[t]; im[t] = 0.0; }
    or_fft(re, im, n, -1);
    for (int64_t f = 0; f <= n / 2; ++f) { out_re[f] = re[f]; out_im[f] = im[f]; }
    free(re);
    free(im);
    return OR_OK;
}

/* Exponential linear unit with alpha = 1 (x for x > 0, exp(x) - 1 otherwise),
 * applied between the layers of the vocoder-style stack. */
void ctconv_oracle_elu(int64_t n, const double* x, double* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = x[i] > 0.0 ? x[i] : expm1(x[i]);
}

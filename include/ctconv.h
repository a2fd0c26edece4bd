/*
 * ctconv.h -- dense transposed convolution (ConvTranspose1d/2d, groups = 1)
 * and depthwise transposed convolution (groups = C_in) on AMD Instinct MI355X
 * (gfx950).  C ABI.
 *
 * Operation (scatter definition).  Every input element x[n, ci, i] adds
 * x[n, ci, i] * w[ci, co, t] to the output element at o = i*s - p + t*d for
 * each output channel co and tap t, when 0 <= o < L_out; the optional bias is
 * added once to every output.  Per dimension
 *     L_out = (L_in - 1)*s - 2*p + d*(k - 1) + op + 1.
 * The weight layout [C_in, C_out, k...] (un-flipped) and the tap condition are
 * those of the gather-form kernel "conv_transpose2d.wgsl" in ExecuTorch PR
 * #20849 ("[ExecuTorch][WebGPU] Add optimized conv2d op", Implementation).
 *
 * Two routes compute it:
 *  - polyphase: when every kernel size is a multiple of its stride (k = m*s)
 *    the operation is one stride-1 m-tap convolution producing every output
 *    phase, followed by a phase interleave (depth-to-space) and a padding
 *    slice -- ExecuTorch PR #25037 ("[XNNPACK] Lower dense transposed convs
 *    as one polyphase conv + depth to space", Summary formula).  The same
 *    holds for any k with m = ceil(k / s) taps per phase, the taps past k
 *    being zero in the packed weight, and output_padding only lengthens the
 *    output.  It runs as an implicit GEMM on the MFMA matrix cores with the
 *    interleave, slice, bias and activation fused into its epilogue.  A
 *    dilation d is reduced by g = gcd(s, d) per dimension (only outputs
 *    o0 + g*u receive taps: a transposed convolution with stride s / g,
 *    after a bias fill of the other outputs) and the rest d / g expanded
 *    into zero taps.  Compiled kernel instances take at most 4 taps per
 *    phase in 1-D and 1 or 2 per dimension, or 3 x 3, in 2-D; fp32 shapes
 *    without a dilation reduction take any number, as a sequence of
 *    launches over groups of taps that add into y in order.  Column tiles
 *    hold a subset of the phases when there are more than a tile holds
 *    (e.g. 2-D stride 3).  Input rows must be at least 8 bytes (W >= 4 for
 *    bf16/fp16, W >= 2 for fp32).
 *  - gather: every other shape (16-bit shapes with more taps per phase than
 *    an instance, reduced dilations with too many taps, shorter rows): a
 *    gather-form kernel that stages x and the taps' weights in LDS and
 *    reduces over C_in across lanes, or one output and 8 channels per lane
 *    for small problems and shapes past its staging limits.
 *
 * Layouts.  x [N, C_in, L] or [N, C_in, H, W]; y [N, C_out, L_out] or
 * [N, C_out, H_out, W_out]; bias [C_out]; all dense row-major (contiguous).
 * One element type covers x, w, bias and y; products are accumulated in fp32
 * and rounded once (round to nearest even) to the output type.
 *
 * Ownership.  The caller allocates and owns every buffer.  The library never
 * allocates, frees, retains or aliases caller memory.  Its only global
 * mutable state is the fixed per-device scratch of ctconv_forward_noalloc
 * (see there); every other function is thread-safe.
 *
 * Streams.  Device work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) and the call returns without synchronising.  Errors found
 * on the host are returned before anything is enqueued, so outputs are left
 * untouched; CTCONV_ERR_HIP reports a failed launch (hipGetLastError).
 */
#ifndef CTCONV_H
#define CTCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CTCONV_ABI_VERSION 1

typedef enum {
    CTCONV_F32 = 0,  /* float32 storage, fp32 products */
    CTCONV_BF16 = 1, /* bfloat16 storage, fp32 accumulation */
    CTCONV_F16 = 2   /* float16 storage, fp32 accumulation */
} ctconv_dtype;

typedef enum {
    CTCONV_OK = 0,
    CTCONV_ERR_NULL = 1,  /* a required pointer is NULL */
    CTCONV_ERR_SHAPE = 2, /* sizes out of range, or an output size below 1 */
    CTCONV_ERR_PARAM = 3, /* ndim, stride, padding, dilation, output_padding or route invalid */
    CTCONV_ERR_DTYPE = 4, /* unknown dtype */
    CTCONV_ERR_ALIGN = 5, /* a device pointer is not 16-byte aligned */
    CTCONV_ERR_HIP = 6,   /* the HIP runtime reported an error while enqueuing */
    CTCONV_ERR_WORKSPACE = 7, /* workspace NULL or below ctconv_workspace_bytes */
    CTCONV_ERR_SCRATCH = 8    /* ctconv_forward_noalloc: the call needs more than
                                 CTCONV_SCRATCH_BYTES of workspace */
} ctconv_status;

/* Size of the fixed scratch that ctconv_forward_noalloc uses on each device. */
#define CTCONV_SCRATCH_BYTES (64u << 20)

typedef enum {
    CTCONV_ROUTE_AUTO = 0,      /* polyphase when eligible, else gather */
    CTCONV_ROUTE_POLYPHASE = 1, /* force the polyphase route, its kernel chosen by shape
                                   (ERR_PARAM if ineligible) */
    CTCONV_ROUTE_GATHER = 2,    /* force the gather kernel (valid for every shape) */
    CTCONV_ROUTE_POLYPHASE_TILED = 3,  /* force the LDS-tiled polyphase MFMA kernel */
    CTCONV_ROUTE_POLYPHASE_STREAM = 4  /* force the register-weight streaming polyphase
                                          kernel (16-bit 1-D, stride a multiple of 4,
                                          ceil(k/s) * C_in rounded up to 32 <= 256) */
} ctconv_route;

/* Activation applied to every output (after the bias, before the one rounding). */
typedef enum {
    CTCONV_ACT_NONE = 0,
    CTCONV_ACT_ELU = 1 /* x > 0 ? x : exp(x) - 1 (alpha = 1) */
} ctconv_activation;

/* Version of this ABI (CTCONV_ABI_VERSION). */
int ctconv_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* ctconv_status_string(ctconv_status status);

/*
 * Output spatial size (host only, no device call).
 *   ndim            1 or 2
 *   in_spatial[d]   >= 0      kernel[d], stride[d], dilation[d] >= 1
 *   padding[d]      >= 0      0 <= output_padding[d] < max(stride[d], dilation[d])
 *   out_spatial[d]  receives (in-1)*s - 2p + d*(k-1) + op + 1, which must be >= 1
 * Returns CTCONV_ERR_NULL / _PARAM / _SHAPE on invalid input, writing nothing.
 */
ctconv_status ctconv_output_shape(int ndim, const int64_t* in_spatial, const int64_t* kernel,
                                  const int64_t* stride, const int64_t* padding,
                                  const int64_t* output_padding, const int64_t* dilation,
                                  int64_t* out_spatial);

/*
 * Size in bytes of the packed weight that ctconv_prepack writes (host only).
 * The packed layout is phase-major, in blocks of 32 input channels:
 * [P][C_in_pad / 32][C_out][T][32] where
 *   P = prod_d s_d output phases (phase (jy, jx) at jy*s_x + jx),
 *   T = prod_d ceil(k_d / s_d) taps per phase (tap (ry, rx) at ry*m_x + rx),
 *   C_in_pad = C_in rounded up to a multiple of 32,
 * holding w[ci, co, s_y*ry + jy, s_x*rx + jx] for ci = 32*block + index,
 * and zero where a tap index reaches past the kernel or ci >= C_in.
 */
ctconv_status ctconv_packed_bytes(int ndim, int64_t C_in, int64_t C_out, const int64_t* kernel,
                                  const int64_t* stride, ctconv_dtype dtype, size_t* bytes);

/*
 * Rearrange a ConvTranspose weight w [C_in, C_out, k...] (device memory) into
 * the phase-major packed layout above (device memory of ctconv_packed_bytes
 * bytes, caller-allocated).  An exact copy: no arithmetic.  Asynchronous on
 * `stream`.  Both pointers must be 16-byte aligned.
 */
ctconv_status ctconv_prepack(const void* w, void* packed_w, int ndim, int64_t C_in, int64_t C_out,
                             const int64_t* kernel, const int64_t* stride, ctconv_dtype dtype,
                             void* stream);

/*
 * y = ConvTranspose(x, w, bias) on the device.
 *   x          device, [N, C_in, in_spatial...]; may be NULL when it has no
 *              element (N = 0 or an input size of 0)
 *   packed_w   device, written by ctconv_prepack with the same C_in, C_out,
 *              kernel, stride and dtype (a precondition the library cannot check)
 *   bias       device [C_out], or NULL for none
 *   y          device, [N, C_out, out_spatial...] (see ctconv_output_shape);
 *              every element is written (outputs no tap reaches get the bias,
 *              or 0).  Must not overlap x, packed_w or bias.  May be NULL when N = 0.
 *   N >= 0, C_in >= 1, C_out >= 1; other arguments as in ctconv_output_shape.
 * Pointers must be 16-byte aligned.  With N = 0 nothing is enqueued.
 */
ctconv_status ctconv_forward(const void* x, const void* packed_w, const void* bias, void* y,
                             int64_t N, int64_t C_in, int64_t C_out, int ndim,
                             const int64_t* in_spatial, const int64_t* kernel,
                             const int64_t* stride, const int64_t* padding,
                             const int64_t* output_padding, const int64_t* dilation,
                             ctconv_dtype dtype, void* stream);

/*
 * Deterministic forward with a caller workspace.
 *
 * Shapes with few output tiles (the iSTFT of onnxruntime PR #33978, "[WebGPU]
 * optimizations for audio models", whose transposed convolution has a single
 * output channel and a 16392-long reduction) leave most compute units idle
 * unless the reduction over input channels is split across workgroups.
 * ctconv_forward never splits it; ctconv_forward_ws may, in fp32: the first
 * split writes its partial sums to y, each other split to its own slab of
 * the workspace, and a second kernel adds them to y in a fixed order, then
 * the bias and the activation.  Every call with the same arguments gives the
 * same bits (no atomics; the order of the additions is fixed).
 *
 * ctconv_workspace_bytes (host only): the bytes ctconv_forward_ws needs for
 * these arguments (0 when it does not split; then workspace may be NULL).
 * Validates like ctconv_forward.
 *
 * ctconv_forward_ws: ctconv_forward_act with route AUTO and a workspace.
 *   workspace        device, 16-byte aligned, caller-owned, not retained; its
 *                    contents on entry are ignored and on return undefined; it
 *                    must not overlap x, packed_w, bias or y
 *   workspace_bytes  its size; CTCONV_ERR_WORKSPACE when it is below
 *                    ctconv_workspace_bytes for these arguments
 * Two calls must not share a workspace concurrently.  Everything else as in
 * ctconv_forward_act.
 */
ctconv_status ctconv_workspace_bytes(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                     const int64_t* in_spatial, const int64_t* kernel,
                                     const int64_t* stride, const int64_t* padding,
                                     const int64_t* output_padding, const int64_t* dilation,
                                     ctconv_dtype dtype, size_t* bytes);
ctconv_status ctconv_forward_ws(const void* x, const void* packed_w, const void* bias, void* y,
                                int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                const int64_t* in_spatial, const int64_t* kernel,
                                const int64_t* stride, const int64_t* padding,
                                const int64_t* output_padding, const int64_t* dilation,
                                ctconv_dtype dtype, ctconv_activation act, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * ctconv_forward_ws without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is the library's own
 * fixed scratch: one static device array of CTCONV_SCRATCH_BYTES (64 MiB) per
 * device, created with the library's code object and held until the process
 * ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); on its first use on a device it looks up the scratch's
 * address there once.
 *   Every argument as in ctconv_forward_ws (route AUTO, deterministic).
 *   CTCONV_ERR_SCRATCH when ctconv_workspace_bytes for these arguments exceeds
 *   CTCONV_SCRATCH_BYTES (checked on the host before anything is enqueued).
 * All calls on one device share that device's scratch, and every call that
 * uses it overwrites it (nothing in it needs to start at zero): calls that
 * overlap on one device -- on different streams, or from different threads
 * without ordering -- race and must not be issued.  The stream's device is the
 * one whose scratch is used.
 * ctconv_scratch_bytes returns CTCONV_SCRATCH_BYTES.
 */
ctconv_status ctconv_forward_noalloc(const void* x, const void* packed_w, const void* bias,
                                     void* y, int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                     const int64_t* in_spatial, const int64_t* kernel,
                                     const int64_t* stride, const int64_t* padding,
                                     const int64_t* output_padding, const int64_t* dilation,
                                     ctconv_dtype dtype, ctconv_activation act, void* stream);
size_t ctconv_scratch_bytes(void);

/*
 * ctconv_forward with an explicit route, so the two kernels can be checked
 * against each other on shapes both support.  CTCONV_ROUTE_POLYPHASE on a
 * shape outside the polyphase form returns CTCONV_ERR_PARAM.
 */
ctconv_status ctconv_forward_route(const void* x, const void* packed_w, const void* bias, void* y,
                                   int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                   const int64_t* in_spatial, const int64_t* kernel,
                                   const int64_t* stride, const int64_t* padding,
                                   const int64_t* output_padding, const int64_t* dilation,
                                   ctconv_dtype dtype, ctconv_route route, void* stream);

/*
 * ctconv_forward_route with a pointwise activation fused into the epilogue:
 * y = act(conv + bias), computed in fp32 and rounded once to the output
 * type.  The activation is applied where the transposed convolution writes
 * its output instead of in a separate pass that reads and writes y again
 * (ExecuTorch PR #25037 runs its polyphase rewrite before FuseActivationPass
 * for the same reason; its Test plan has two deconvolutions with an ELU
 * between them).  Outputs no tap reaches get act(bias) (or act(0)).
 * act outside ctconv_activation returns CTCONV_ERR_PARAM; everything else
 * as in ctconv_forward_route.
 */
ctconv_status ctconv_forward_act(const void* x, const void* packed_w, const void* bias, void* y,
                                 int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                 const int64_t* in_spatial, const int64_t* kernel,
                                 const int64_t* stride, const int64_t* padding,
                                 const int64_t* output_padding, const int64_t* dilation,
                                 ctconv_dtype dtype, ctconv_activation act, ctconv_route route,
                                 void* stream);

/*
 * Which kernel ctconv_forward would run for these arguments (host only):
 * writes CTCONV_ROUTE_POLYPHASE or CTCONV_ROUTE_GATHER to *route.
 */
ctconv_status ctconv_query_route(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                 const int64_t* in_spatial, const int64_t* kernel,
                                 const int64_t* stride, const int64_t* padding,
                                 const int64_t* output_padding, const int64_t* dilation,
                                 ctconv_dtype dtype, ctconv_route* route);

/*
 * Exponential linear unit with alpha = 1, y = x > 0 ? x : exp(x) - 1,
 * elementwise over n elements (device memory, computed in fp32, rounded once
 * to dtype).  It is the activation between stacked upsampler layers, a case
 * the test plan of ExecuTorch PR #25037 covers (transposed convs in sequence
 * with an ELU between them).
 * x and y may be the same buffer.
 */
ctconv_status ctconv_elu(const void* x, void* y, int64_t n, ctconv_dtype dtype, void* stream);

/*
 * The iSTFT steps after the overlap-add.  onnxruntime PR #33978 ("[WebGPU]
 * optimizations for audio models") serves the iSTFT's inverse DFT and
 * overlap-add with ConvTranspose; the window-square normalisation and the
 * centre trim come after it.  With y [rows, L_in] the overlap-added frames
 * (ctconv_forward of the Hann-windowed inverse-DFT basis, stride hop) and
 * env [L_in] the window-square envelope sum_f h^2[t - f*hop] (itself a
 * transposed convolution of a row of ones with h^2, stride hop):
 *   out[r, t] = y[r, trim + t] / env[trim + t]   for t < L_out
 * (0 where env <= 1e-11: no frame covers the sample).  For a centred STFT,
 * trim = n_fft / 2 and L_out = hop * (frames - 1).  Computed in fp32,
 * rounded once to dtype; all three buffers of dtype, 16-byte aligned, on the
 * device, caller-owned; out must not overlap y or env.  CTCONV_ERR_SHAPE
 * when trim + L_out > L_in.
 */
ctconv_status ctconv_istft_normalize(const void* y, const void* env, void* out, int64_t rows,
                                     int64_t L_in, int64_t trim, int64_t L_out,
                                     ctconv_dtype dtype, void* stream);

/*
 * Streaming 1-D transposed convolution (padding 0, dilation 1, k >= s), for
 * decoders that turn input frames into output samples chunk by chunk: the
 * Phonon TTS example of ExecuTorch PR #25037 decodes one 80 ms frame per
 * call through a StreamingConvTranspose1d that holds back the outputs later
 * frames still add to, and uses the bias for the conv and for that held-back
 * tail (the page's use-after-free fix).  Frame i reaches outputs
 * [i*s, i*s + k), so after frames [0, F) the outputs below F*s are final and
 * the next k - s are partial.
 *
 * Concatenating the y of successive ctconv_stream_step calls and then the y
 * of ctconv_stream_flush gives the one-shot transposed convolution of all the
 * frames with padding 0 (length (F - 1)*s + k), with the bias and the
 * activation applied once to every output.  The chunk's conv output and the
 * tail are kept as fp32 partial sums without bias; each output is rounded to
 * dtype exactly once, after the tail and the bias are added.
 *
 * ctconv_stream_sizes (host only): for a chunk of L_chunk frames, *y_len =
 * L_chunk * s outputs per row, *tail_len = k - s (0 if k <= s) tail values per
 * row, *workspace_bytes = N * C_out * (L_chunk*s + tail_len) * 4 for the
 * chunk's fp32 conv output (0 when L_chunk = 0).
 *
 * ctconv_stream_step: one chunk.
 *   x          device [N, C_in, L_chunk], L_chunk >= 1 frames
 *   packed_w   from ctconv_prepack with kernel = k, stride = s (1-D)
 *   bias       device [C_out] or NULL
 *   y          device [N, C_out, L_chunk*s]: the outputs this chunk completes
 *   tail_in    device fp32 [N, C_out, k - s] from the previous call, or NULL
 *              at the start of the stream (zeros)
 *   tail_out   device fp32 [N, C_out, k - s] (may be NULL when k = s); must
 *              not be tail_in (pass two buffers and swap them per call)
 *   workspace  device, ctconv_stream_sizes' workspace_bytes, caller-owned
 *   act        activation applied to every emitted output (not to the tail)
 * Errors: CTCONV_ERR_PARAM for k < s, tail_in == tail_out or an unknown act;
 * CTCONV_ERR_SHAPE for L_chunk < 1; otherwise as ctconv_forward.  All
 * buffers 16-byte aligned and caller-owned; nothing is retained.
 *
 * ctconv_stream_flush: the end of the stream, y [N, C_out, k - s] =
 * act(tail_in + bias) (tail_in NULL: act(bias)).  Nothing is enqueued when
 * k <= s or N = 0.
 */
ctconv_status ctconv_stream_sizes(int64_t N, int64_t C_out, int64_t L_chunk, int64_t kernel,
                                  int64_t stride, ctconv_dtype dtype, int64_t* y_len,
                                  int64_t* tail_len, int64_t* workspace_bytes);
ctconv_status ctconv_stream_step(const void* x, const void* packed_w, const void* bias, void* y,
                                 const float* tail_in, float* tail_out, void* workspace,
                                 int64_t N, int64_t C_in, int64_t C_out, int64_t L_chunk,
                                 int64_t kernel, int64_t stride, ctconv_dtype dtype,
                                 ctconv_activation act, void* stream);
ctconv_status ctconv_stream_flush(const float* tail_in, const void* bias, void* y, int64_t N,
                                  int64_t C_out, int64_t kernel, int64_t stride,
                                  ctconv_dtype dtype, ctconv_activation act, void* stream);

/* Kernel choice of the depthwise transposed convolution. */
typedef enum {
    CTCONV_DW_AUTO = 0,   /* row-phase kernel when it covers the shape, else element kernel */
    CTCONV_DW_ROW = 1,    /* force the row-phase kernel (CTCONV_ERR_PARAM if it does not apply) */
    CTCONV_DW_ELEMENT = 2 /* force the element kernel (valid for every shape) */
} ctconv_dw_kernel;

/*
 * Depthwise transposed convolution: ConvTranspose with groups = C_in and
 * C_out = M * C_in (M >= 1 outputs per input channel).  Output channel co
 * reads input channel co / M only:
 *     y[n, co, o] = bias[co] + sum_t x[n, co / M, i] * w[co / M, co % M, t]
 * over the taps t and positions i with o = i*s - p + t*d (per dimension in
 * 2-D), the scatter definition of ctconv_forward restricted to one channel.
 * This is the depthwise layer (an upsampling filter applied per channel) that
 * ExecuTorch PR #25037, commit "Decompose depthwise transposed convs",
 * rewrites into one stride-1 depthwise convolution per output phase and a
 * depth-to-space; here the phases are computed in place, each lane writing a
 * run of consecutive (interleaved) outputs.
 *   x      device [N, C_in, in_spatial...]; may be NULL when it has no element
 *   w      device [C_in, M, kernel...], the ConvTranspose weight layout, used
 *          as is (no prepack)
 *   bias   device [C_out] or NULL
 *   y      device [N, C_out, out_spatial...] (ctconv_output_shape), every
 *          element written; must not overlap x, w or bias
 *   act    activation applied after the bias, before the one rounding
 * Products are accumulated in fp32 and rounded once to dtype.  Kernels: the
 * row-phase kernel takes dilation 1, a last-dimension stride of 1, 2 or 4,
 * an H stride (2-D) of at most 4, at most 4 taps per phase in each dimension
 * (ceil(k / s) <= 4) and x below 2 GiB; the element kernel takes every other
 * shape.
 * Errors: as ctconv_forward, plus CTCONV_ERR_SHAPE when C_out is not a
 * multiple of C_in, CTCONV_ERR_PARAM for an unknown act or kernel choice or a
 * forced row-phase kernel that does not apply.  Pointers 16-byte aligned;
 * asynchronous on `stream`; nothing is allocated or retained.
 */
ctconv_status ctconv_depthwise_forward(const void* x, const void* w, const void* bias, void* y,
                                       int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                       const int64_t* in_spatial, const int64_t* kernel,
                                       const int64_t* stride, const int64_t* padding,
                                       const int64_t* output_padding, const int64_t* dilation,
                                       ctconv_dtype dtype, ctconv_activation act, void* stream);
ctconv_status ctconv_depthwise_forward_kernel(const void* x, const void* w, const void* bias,
                                              void* y, int64_t N, int64_t C_in, int64_t C_out,
                                              int ndim, const int64_t* in_spatial,
                                              const int64_t* kernel, const int64_t* stride,
                                              const int64_t* padding,
                                              const int64_t* output_padding,
                                              const int64_t* dilation, ctconv_dtype dtype,
                                              ctconv_activation act, ctconv_dw_kernel which,
                                              void* stream);
/* Which kernel CTCONV_DW_AUTO would run (host only; validates like the forward). */
ctconv_status ctconv_depthwise_query_kernel(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                            const int64_t* in_spatial, const int64_t* kernel,
                                            const int64_t* stride, const int64_t* padding,
                                            const int64_t* output_padding,
                                            const int64_t* dilation, ctconv_dtype dtype,
                                            ctconv_dw_kernel* which);

/*
 * Sustained shader clock (a measurement aid for roofline fractions, not part
 * of the transposed convolution; callers: benchmarks).  The MI355X peaks are
 * quoted at 2.4 GHz; under load the chip may hold a lower clock.  The probe
 * keeps every matrix core issuing bf16 MFMAs (16 independent accumulation
 * chains per wave, two 8-wave workgroups per compute unit, `iters` rounds of
 * 16 MFMAs per wave) and reads, per workgroup, the shader-clock cycle
 * counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime) at
 * its start and end.
 *   workspace        device buffer, 8-byte aligned, of at least
 *                    ctconv_clock_probe_bytes() bytes (overwritten)
 *   workspace_bytes  its size
 *   iters            1 .. 2^24 (4096 runs about 2 ms)
 *   mhz              out: shader cycles / real time over all workgroups, MHz
 *   tflops           out (may be NULL): the probe's bf16 MFMA rate, TFLOP/s
 * Errors: CTCONV_ERR_NULL (workspace or mhz NULL), CTCONV_ERR_PARAM (iters),
 * CTCONV_ERR_WORKSPACE (too small), CTCONV_ERR_ALIGN, CTCONV_ERR_HIP.
 * Synchronous: returns after the probe kernel has finished on `stream`.
 */
size_t ctconv_clock_probe_bytes(void);
ctconv_status ctconv_clock_probe(void* workspace, size_t workspace_bytes, int iters, double* mhz,
                                 double* tflops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CTCONV_H */

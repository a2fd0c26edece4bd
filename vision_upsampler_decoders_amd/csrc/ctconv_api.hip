// C ABI of libctconv: argument validation, shape arithmetic, routing and
// launches.  No allocation, no synchronisation, no global mutable state.

#include <string.h>

#include "ctconv_internal.h"

using namespace ctconv;

namespace {

constexpr int64_t kI64Max = INT64_MAX;

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

size_t esize(ctconv_dtype dt) { return dt == CTCONV_F32 ? 4 : 2; }

bool dtype_ok(int dt) { return dt == CTCONV_F32 || dt == CTCONV_BF16 || dt == CTCONV_F16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-dimension validation and output length (L-1)*s - 2p + d*(k-1) + op + 1.
ctconv_status out_len(int64_t L, int64_t k, int64_t s, int64_t p, int64_t op, int64_t d,
                      int64_t* out) {
    if (L < 0) return CTCONV_ERR_SHAPE;
    if (k < 1 || s < 1 || d < 1 || p < 0 || op < 0) return CTCONV_ERR_PARAM;
    if (op >= (s > d ? s : d)) return CTCONV_ERR_PARAM;
    int64_t a, b;
    if (!mul_ok(L > 0 ? L - 1 : 0, s, &a) || !mul_ok(d, k - 1, &b)) return CTCONV_ERR_SHAPE;
    // L = 0 contributes -s
    __int128 v = (__int128)(L > 0 ? a : -s) - 2 * (__int128)p + b + op + 1;
    if (v < 1) return CTCONV_ERR_SHAPE;
    if (v > kI64Max) return CTCONV_ERR_SHAPE;
    *out = (int64_t)v;
    return CTCONV_OK;
}

ctconv_status geometry(int ndim, const int64_t* in_sp, const int64_t* kernel,
                       const int64_t* stride, const int64_t* padding,
                       const int64_t* output_padding, const int64_t* dilation, Problem* p) {
    if (ndim != 1 && ndim != 2) return CTCONV_ERR_PARAM;
    if (!in_sp || !kernel || !stride || !padding || !output_padding || !dilation)
        return CTCONV_ERR_NULL;
    int64_t in2[2] = {1, 1}, k2[2] = {1, 1}, s2[2] = {1, 1}, p2[2] = {0, 0}, op2[2] = {0, 0},
            d2[2] = {1, 1}, o2[2] = {1, 1};
    for (int i = 0; i < ndim; ++i) {
        const int j = 2 - ndim + i;
        in2[j] = in_sp[i];
        k2[j] = kernel[i];
        s2[j] = stride[i];
        p2[j] = padding[i];
        op2[j] = output_padding[i];
        d2[j] = dilation[i];
    }
    for (int j = 2 - ndim; j < 2; ++j) {
        const ctconv_status st = out_len(in2[j], k2[j], s2[j], p2[j], op2[j], d2[j], &o2[j]);
        if (st != CTCONV_OK) return st;
    }
    p->ndim = ndim;
    p->H = in2[0];
    p->W = in2[1];
    p->Ho = o2[0];
    p->Wo = o2[1];
    p->kH = k2[0];
    p->kW = k2[1];
    p->sH = s2[0];
    p->sW = s2[1];
    p->pH = p2[0];
    p->pW = p2[1];
    p->opH = op2[0];
    p->opW = op2[1];
    p->dH = d2[0];
    p->dW = d2[1];
    p->mH = (p->kH + p->sH - 1) / p->sH;
    p->mW = (p->kW + p->sW - 1) / p->sW;
    return CTCONV_OK;
}

// Channel counts, packed-layout sizes and element counts (all must fit int64).
ctconv_status channels(int64_t N, int64_t C_in, int64_t C_out, ctconv_dtype dt, Problem* p) {
    if (!dtype_ok(dt)) return CTCONV_ERR_DTYPE;
    if (N < 0 || C_in < 1 || C_out < 1) return CTCONV_ERR_SHAPE;
    if (C_in > kI64Max - kCinAlign) return CTCONV_ERR_SHAPE;
    p->N = N;
    p->C_in = C_in;
    p->C_out = C_out;
    p->dtype = dt;
    p->C_in_pad = (C_in + kCinAlign - 1) / kCinAlign * kCinAlign;
    int64_t P, T, t;
    if (!mul_ok(p->sH, p->sW, &P) || !mul_ok(p->mH, p->mW, &T)) return CTCONV_ERR_SHAPE;
    p->P = P;
    p->T = T;
    // packed weight elements and bytes
    if (!mul_ok(P, C_out, &t) || !mul_ok(t, T, &t) || !mul_ok(t, p->C_in_pad, &t) ||
        !mul_ok(t, (int64_t)esize(dt), &t))
        return CTCONV_ERR_SHAPE;
    // x and y element counts
    if (!mul_ok(N, C_in, &t) || !mul_ok(t, p->H, &t) || !mul_ok(t, p->W, &t) ||
        !mul_ok(t, (int64_t)esize(dt), &t))
        return CTCONV_ERR_SHAPE;
    if (!mul_ok(N, C_out, &t) || !mul_ok(t, p->Ho, &t) || !mul_ok(t, p->Wo, &t) ||
        !mul_ok(t, (int64_t)esize(dt), &t))
        return CTCONV_ERR_SHAPE;
    return CTCONV_OK;
}

ctconv_status to_status(hipError_t e) { return e == hipSuccess ? CTCONV_OK : CTCONV_ERR_HIP; }

ctconv_status build_problem(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                            const int64_t* in_spatial, const int64_t* kernel,
                            const int64_t* stride, const int64_t* padding,
                            const int64_t* output_padding, const int64_t* dilation,
                            ctconv_dtype dtype, Problem* p) {
    memset(p, 0, sizeof(*p));
    ctconv_status st =
        geometry(ndim, in_spatial, kernel, stride, padding, output_padding, dilation, p);
    if (st != CTCONV_OK) return st;
    return channels(N, C_in, C_out, dtype, p);
}

bool polyphase_eligible(const Problem& p) {
    // Any k: with m = ceil(k / s) taps per phase the packed weight's taps past
    // k are zero; output_padding only lengthens the output.  Any dilation: the
    // kernel runs the problem reduced by gcd(s, d) with the remaining
    // dilation expanded into zero taps (the planner declines tap counts no
    // kernel instance covers).
    (void)p;
    return true;
}

ctconv_route choose_route(const Problem& p) {
    if (polyphase_eligible(p) && polyphase_supported(p)) return CTCONV_ROUTE_POLYPHASE;
    return CTCONV_ROUTE_GATHER;
}

// The polyphase kernel for a shape on the polyphase route: the streaming
// kernel when it applies (weights in registers: short reductions), else the
// tiled one.
ctconv_route polyphase_kernel(const Problem& p) {
    return polyrw_supported(p) ? CTCONV_ROUTE_POLYPHASE_STREAM : CTCONV_ROUTE_POLYPHASE_TILED;
}

}  // namespace

extern "C" {

int ctconv_abi_version(void) { return CTCONV_ABI_VERSION; }

const char* ctconv_status_string(ctconv_status status) {
    // a C caller may pass any int: read it as one (a C++ enum object must not
    // hold a value outside its enumerators)
    int v;
    memcpy(&v, &status, sizeof v);
    switch (v) {
        case CTCONV_OK: return "ok";
        case CTCONV_ERR_NULL: return "a required pointer is NULL";
        case CTCONV_ERR_SHAPE: return "invalid or overflowing size";
        case CTCONV_ERR_PARAM: return "invalid ndim, stride, padding, dilation, output_padding or route";
        case CTCONV_ERR_DTYPE: return "unknown dtype";
        case CTCONV_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case CTCONV_ERR_HIP: return "HIP runtime error";
        case CTCONV_ERR_WORKSPACE: return "workspace missing or smaller than ctconv_workspace_bytes";
        case CTCONV_ERR_SCRATCH:
            return "the call needs more workspace than the fixed scratch (CTCONV_SCRATCH_BYTES)";
    }
    return "unknown status";
}

ctconv_status ctconv_output_shape(int ndim, const int64_t* in_spatial, const int64_t* kernel,
                                  const int64_t* stride, const int64_t* padding,
                                  const int64_t* output_padding, const int64_t* dilation,
                                  int64_t* out_spatial) {
    if (!out_spatial) return CTCONV_ERR_NULL;
    Problem p;
    memset(&p, 0, sizeof(p));
    const ctconv_status st =
        geometry(ndim, in_spatial, kernel, stride, padding, output_padding, dilation, &p);
    if (st != CTCONV_OK) return st;
    if (ndim == 1) {
        out_spatial[0] = p.Wo;
    } else {
        out_spatial[0] = p.Ho;
        out_spatial[1] = p.Wo;
    }
    return CTCONV_OK;
}

ctconv_status ctconv_packed_bytes(int ndim, int64_t C_in, int64_t C_out, const int64_t* kernel,
                                  const int64_t* stride, ctconv_dtype dtype, size_t* bytes) {
    if (!kernel || !stride || !bytes) return CTCONV_ERR_NULL;
    if (ndim != 1 && ndim != 2) return CTCONV_ERR_PARAM;
    const int64_t zeros[2] = {0, 0}, ones[2] = {1, 1};
    Problem p;
    ctconv_status st = build_problem(0, C_in, C_out, ndim, ones, kernel, stride, zeros, zeros,
                                     ones, dtype, &p);
    if (st != CTCONV_OK) return st;
    int64_t t = p.P * p.C_out;  // overflow already checked in channels()
    t = t * p.T * p.C_in_pad * (int64_t)esize(dtype);
    *bytes = (size_t)t;
    return CTCONV_OK;
}

ctconv_status ctconv_prepack(const void* w, void* packed_w, int ndim, int64_t C_in, int64_t C_out,
                             const int64_t* kernel, const int64_t* stride, ctconv_dtype dtype,
                             void* stream) {
    if (!w || !packed_w || !kernel || !stride) return CTCONV_ERR_NULL;
    if (ndim != 1 && ndim != 2) return CTCONV_ERR_PARAM;
    const int64_t zeros[2] = {0, 0}, ones[2] = {1, 1};
    Problem p;
    ctconv_status st = build_problem(0, C_in, C_out, ndim, ones, kernel, stride, zeros, zeros,
                                     ones, dtype, &p);
    if (st != CTCONV_OK) return st;
    if (!aligned16(w) || !aligned16(packed_w)) return CTCONV_ERR_ALIGN;
    return to_status(launch_prepack(p, w, packed_w, static_cast<hipStream_t>(stream)));
}

ctconv_status ctconv_query_route(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                 const int64_t* in_spatial, const int64_t* kernel,
                                 const int64_t* stride, const int64_t* padding,
                                 const int64_t* output_padding, const int64_t* dilation,
                                 ctconv_dtype dtype, ctconv_route* route) {
    if (!route) return CTCONV_ERR_NULL;
    Problem p;
    const ctconv_status st = build_problem(N, C_in, C_out, ndim, in_spatial, kernel, stride,
                                           padding, output_padding, dilation, dtype, &p);
    if (st != CTCONV_OK) return st;
    *route = choose_route(p);
    return CTCONV_OK;
}

namespace {

// The forward with an optional workspace (ws_bytes bytes at ws): validation,
// routing and launches.  need_ws receives the workspace the plan asks for.
ctconv_status forward_impl(const void* x, const void* packed_w, const void* bias, void* y,
                           int64_t N, int64_t C_in, int64_t C_out, int ndim,
                           const int64_t* in_spatial, const int64_t* kernel,
                           const int64_t* stride, const int64_t* padding,
                           const int64_t* output_padding, const int64_t* dilation,
                           ctconv_dtype dtype, ctconv_activation act, ctconv_route route,
                           void* ws, size_t ws_bytes, bool ws_call, void* stream) {
    if (route != CTCONV_ROUTE_AUTO && route != CTCONV_ROUTE_POLYPHASE &&
        route != CTCONV_ROUTE_GATHER && route != CTCONV_ROUTE_POLYPHASE_TILED &&
        route != CTCONV_ROUTE_POLYPHASE_STREAM)
        return CTCONV_ERR_PARAM;
    if (act != CTCONV_ACT_NONE && act != CTCONV_ACT_ELU) return CTCONV_ERR_PARAM;
    Problem p;
    const ctconv_status st = build_problem(N, C_in, C_out, ndim, in_spatial, kernel, stride,
                                           padding, output_padding, dilation, dtype, &p);
    if (st != CTCONV_OK) return st;
    p.act = (int)act;
    // x may be NULL when it holds no element, y when N = 0 (empty tensors)
    const bool x_empty = p.N == 0 || p.H == 0 || p.W == 0;
    if (!packed_w || (!x && !x_empty) || (!y && p.N != 0)) return CTCONV_ERR_NULL;
    if ((x && !aligned16(x)) || !aligned16(packed_w) || (y && !aligned16(y)) ||
        (bias && !aligned16(bias)) || (ws && !aligned16(ws)))
        return CTCONV_ERR_ALIGN;
    const bool poly_ok = polyphase_eligible(p) && polyphase_supported(p);
    if ((route == CTCONV_ROUTE_POLYPHASE || route == CTCONV_ROUTE_POLYPHASE_TILED) && !poly_ok &&
        !x_empty)
        return CTCONV_ERR_PARAM;
    if (route == CTCONV_ROUTE_POLYPHASE_STREAM && !polyrw_supported(p) && !x_empty)
        return CTCONV_ERR_PARAM;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.N == 0) return CTCONV_OK;
    if (x_empty) return to_status(launch_fill(p, bias, y, s));  // no tap reaches y
    if (route == CTCONV_ROUTE_AUTO) route = choose_route(p);
    if (route == CTCONV_ROUTE_POLYPHASE) route = polyphase_kernel(p);
    if (route == CTCONV_ROUTE_POLYPHASE_STREAM)
        return to_status(launch_polyrw(p, x, packed_w, bias, y, false, s));
    if (route == CTCONV_ROUTE_POLYPHASE_TILED) {
        if (ws_call) {
            const size_t need = polyphase_workspace_bytes(p);
            if (need > 0 && (!ws || ws_bytes < need)) return CTCONV_ERR_WORKSPACE;
        } else {
            ws = nullptr;
            ws_bytes = 0;
        }
        return to_status(launch_polyphase(p, x, packed_w, bias, y, ws, ws_bytes, s));
    }
    return to_status(launch_gather(p, x, packed_w, bias, y, false, s));
}

}  // namespace

ctconv_status ctconv_forward_act(const void* x, const void* packed_w, const void* bias, void* y,
                                 int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                 const int64_t* in_spatial, const int64_t* kernel,
                                 const int64_t* stride, const int64_t* padding,
                                 const int64_t* output_padding, const int64_t* dilation,
                                 ctconv_dtype dtype, ctconv_activation act, ctconv_route route,
                                 void* stream) {
    return forward_impl(x, packed_w, bias, y, N, C_in, C_out, ndim, in_spatial, kernel, stride,
                        padding, output_padding, dilation, dtype, act, route, nullptr, 0, false,
                        stream);
}

ctconv_status ctconv_workspace_bytes(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                     const int64_t* in_spatial, const int64_t* kernel,
                                     const int64_t* stride, const int64_t* padding,
                                     const int64_t* output_padding, const int64_t* dilation,
                                     ctconv_dtype dtype, size_t* bytes) {
    if (!bytes) return CTCONV_ERR_NULL;
    Problem p;
    const ctconv_status st = build_problem(N, C_in, C_out, ndim, in_spatial, kernel, stride,
                                           padding, output_padding, dilation, dtype, &p);
    if (st != CTCONV_OK) return st;
    const bool x_empty = p.N == 0 || p.H == 0 || p.W == 0;
    *bytes = (!x_empty && choose_route(p) == CTCONV_ROUTE_POLYPHASE)
                 ? polyphase_workspace_bytes(p)
                 : 0;
    return CTCONV_OK;
}

ctconv_status ctconv_forward_ws(const void* x, const void* packed_w, const void* bias, void* y,
                                int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                const int64_t* in_spatial, const int64_t* kernel,
                                const int64_t* stride, const int64_t* padding,
                                const int64_t* output_padding, const int64_t* dilation,
                                ctconv_dtype dtype, ctconv_activation act, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return forward_impl(x, packed_w, bias, y, N, C_in, C_out, ndim, in_spatial, kernel, stride,
                        padding, output_padding, dilation, dtype, act, CTCONV_ROUTE_AUTO,
                        workspace, workspace_bytes, true, stream);
}

ctconv_status ctconv_forward_route(const void* x, const void* packed_w, const void* bias, void* y,
                                   int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                   const int64_t* in_spatial, const int64_t* kernel,
                                   const int64_t* stride, const int64_t* padding,
                                   const int64_t* output_padding, const int64_t* dilation,
                                   ctconv_dtype dtype, ctconv_route route, void* stream) {
    return ctconv_forward_act(x, packed_w, bias, y, N, C_in, C_out, ndim, in_spatial, kernel,
                              stride, padding, output_padding, dilation, dtype, CTCONV_ACT_NONE,
                              route, stream);
}

ctconv_status ctconv_forward(const void* x, const void* packed_w, const void* bias, void* y,
                             int64_t N, int64_t C_in, int64_t C_out, int ndim,
                             const int64_t* in_spatial, const int64_t* kernel,
                             const int64_t* stride, const int64_t* padding,
                             const int64_t* output_padding, const int64_t* dilation,
                             ctconv_dtype dtype, void* stream) {
    return ctconv_forward_route(x, packed_w, bias, y, N, C_in, C_out, ndim, in_spatial, kernel,
                                stride, padding, output_padding, dilation, dtype,
                                CTCONV_ROUTE_AUTO, stream);
}

// Streaming geometry: emitted outputs per chunk (L * s), tail length
// (k - s, or 0 when k <= s) and the chunk's full output length L*s + tail.
namespace {
ctconv_status stream_geometry(int64_t N, int64_t C_out, int64_t L, int64_t k, int64_t s,
                              ctconv_dtype dt, int64_t* Ly, int64_t* Tl, int64_t* ws_bytes) {
    if (!dtype_ok(dt)) return CTCONV_ERR_DTYPE;
    if (k < 1 || s < 1) return CTCONV_ERR_PARAM;
    if (N < 0 || C_out < 1 || L < 0) return CTCONV_ERR_SHAPE;
    int64_t ly, t;
    if (!mul_ok(L, s, &ly)) return CTCONV_ERR_SHAPE;
    const int64_t tl = k > s ? k - s : 0;
    if (ly > kI64Max - tl) return CTCONV_ERR_SHAPE;
    // the chunk's conv output is kept in fp32 (rounded once, when emitted)
    if (!mul_ok(N, C_out, &t) || !mul_ok(t, ly + tl, &t) || !mul_ok(t, (int64_t)sizeof(float), &t))
        return CTCONV_ERR_SHAPE;
    *Ly = ly;
    *Tl = tl;
    *ws_bytes = (L > 0 && k >= s) ? t : 0;
    return CTCONV_OK;
}
}  // namespace

ctconv_status ctconv_stream_sizes(int64_t N, int64_t C_out, int64_t L_chunk, int64_t kernel,
                                  int64_t stride, ctconv_dtype dtype, int64_t* y_len,
                                  int64_t* tail_len, int64_t* workspace_bytes) {
    if (!y_len || !tail_len || !workspace_bytes) return CTCONV_ERR_NULL;
    return stream_geometry(N, C_out, L_chunk, kernel, stride, dtype, y_len, tail_len,
                           workspace_bytes);
}

ctconv_status ctconv_stream_step(const void* x, const void* packed_w, const void* bias, void* y,
                                 const float* tail_in, float* tail_out, void* workspace,
                                 int64_t N, int64_t C_in, int64_t C_out, int64_t L_chunk,
                                 int64_t kernel, int64_t stride, ctconv_dtype dtype,
                                 ctconv_activation act, void* stream) {
    if (act != CTCONV_ACT_NONE && act != CTCONV_ACT_ELU) return CTCONV_ERR_PARAM;
    int64_t Ly, Tl, ws;
    ctconv_status st = stream_geometry(N, C_out, L_chunk, kernel, stride, dtype, &Ly, &Tl, &ws);
    if (st != CTCONV_OK) return st;
    // a kernel shorter than its stride leaves gaps between frames: not a stream of this form
    if (kernel < stride) return CTCONV_ERR_PARAM;
    if (L_chunk < 1) return CTCONV_ERR_SHAPE;
    if (C_in < 1) return CTCONV_ERR_SHAPE;
    if (N == 0) return CTCONV_OK;
    if (!x || !packed_w || !y || !workspace || (Tl > 0 && !tail_out)) return CTCONV_ERR_NULL;
    if (tail_in != nullptr && tail_in == tail_out) return CTCONV_ERR_PARAM;  // must not alias
    if (!aligned16(x) || !aligned16(packed_w) || !aligned16(y) || !aligned16(workspace) ||
        (bias && !aligned16(bias)) || (tail_in && !aligned16(tail_in)) ||
        (tail_out && !aligned16(tail_out)))
        return CTCONV_ERR_ALIGN;
    // z = convT(chunk) with padding 0 and no bias, in fp32, into the
    // workspace: fp32 inputs through the ordinary forward; 16-bit inputs
    // through the register-weight streaming kernel where it applies, else the
    // tiled kernel, else the gather kernel, each writing its fp32
    // accumulators unrounded
    const int64_t one = 1, zero = 0;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (dtype == CTCONV_F32) {
        st = ctconv_forward_act(x, packed_w, nullptr, workspace, N, C_in, C_out, 1, &L_chunk,
                                &kernel, &stride, &zero, &zero, &one, dtype, CTCONV_ACT_NONE,
                                CTCONV_ROUTE_AUTO, stream);
        if (st != CTCONV_OK) return st;
    } else {
        Problem p;
        st = build_problem(N, C_in, C_out, 1, &L_chunk, &kernel, &stride, &zero, &zero, &one,
                           dtype, &p);
        if (st != CTCONV_OK) return st;
        p.act = CTCONV_ACT_NONE;
        float* z = static_cast<float*>(workspace);
        const hipError_t e =
            polyrw_supported(p)             ? launch_polyrw(p, x, packed_w, nullptr, z, true, hs)
            : polyphase_f32out_supported(p) ? launch_polyphase_f32out(p, x, packed_w, z, hs)
                                            : launch_gather(p, x, packed_w, nullptr, z, true, hs);
        if (e != hipSuccess) return to_status(e);
    }
    return to_status(launch_stream_overlap(static_cast<const float*>(workspace), tail_in, bias, y,
                                           tail_out, N * C_out, C_out, Ly, Tl, dtype, (int)act, hs));
}

ctconv_status ctconv_stream_flush(const float* tail_in, const void* bias, void* y, int64_t N,
                                  int64_t C_out, int64_t kernel, int64_t stride,
                                  ctconv_dtype dtype, ctconv_activation act, void* stream) {
    if (act != CTCONV_ACT_NONE && act != CTCONV_ACT_ELU) return CTCONV_ERR_PARAM;
    int64_t Ly, Tl, ws;
    const ctconv_status st = stream_geometry(N, C_out, 0, kernel, stride, dtype, &Ly, &Tl, &ws);
    if (st != CTCONV_OK) return st;
    if (N == 0 || Tl == 0) return CTCONV_OK;
    if (!y) return CTCONV_ERR_NULL;
    if (!aligned16(y) || (bias && !aligned16(bias)) || (tail_in && !aligned16(tail_in)))
        return CTCONV_ERR_ALIGN;
    return to_status(launch_stream_flush(tail_in, bias, y, N * C_out, C_out, Tl, dtype, (int)act,
                                         static_cast<hipStream_t>(stream)));
}

ctconv_status ctconv_istft_normalize(const void* y, const void* env, void* out, int64_t rows,
                                     int64_t L_in, int64_t trim, int64_t L_out,
                                     ctconv_dtype dtype, void* stream) {
    if (!dtype_ok(dtype)) return CTCONV_ERR_DTYPE;
    if (rows < 0 || L_in < 0 || trim < 0 || L_out < 0) return CTCONV_ERR_SHAPE;
    if (trim > L_in || L_out > L_in - trim) return CTCONV_ERR_SHAPE;
    int64_t t;
    if (!mul_ok(rows, L_in, &t) || !mul_ok(t, (int64_t)esize(dtype), &t)) return CTCONV_ERR_SHAPE;
    if (rows == 0 || L_out == 0) return CTCONV_OK;
    if (!y || !env || !out) return CTCONV_ERR_NULL;
    if (!aligned16(y) || !aligned16(env) || !aligned16(out)) return CTCONV_ERR_ALIGN;
    return to_status(launch_istft_norm(y, env, out, rows, L_in, trim, L_out, dtype,
                                       static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// Depthwise transposed convolution (groups = C_in)
// ---------------------------------------------------------------------------

namespace {
ctconv_status depthwise_problem(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                const int64_t* in_spatial, const int64_t* kernel,
                                const int64_t* stride, const int64_t* padding,
                                const int64_t* output_padding, const int64_t* dilation,
                                ctconv_dtype dtype, Problem* p) {
    memset(p, 0, sizeof(*p));
    ctconv_status st =
        geometry(ndim, in_spatial, kernel, stride, padding, output_padding, dilation, p);
    if (st != CTCONV_OK) return st;
    if (!dtype_ok(dtype)) return CTCONV_ERR_DTYPE;
    if (N < 0 || C_in < 1 || C_out < 1 || C_out % C_in != 0) return CTCONV_ERR_SHAPE;
    p->N = N;
    p->C_in = C_in;
    p->C_out = C_out;
    p->dtype = dtype;
    int64_t t;
    // x, w and y byte counts must fit int64
    if (!mul_ok(N, C_in, &t) || !mul_ok(t, p->H, &t) || !mul_ok(t, p->W, &t) ||
        !mul_ok(t, (int64_t)esize(dtype), &t))
        return CTCONV_ERR_SHAPE;
    if (!mul_ok(C_out, p->kH, &t) || !mul_ok(t, p->kW, &t) ||
        !mul_ok(t, (int64_t)esize(dtype), &t))
        return CTCONV_ERR_SHAPE;
    if (!mul_ok(N, C_out, &t) || !mul_ok(t, p->Ho, &t) || !mul_ok(t, p->Wo, &t) ||
        !mul_ok(t, (int64_t)esize(dtype), &t))
        return CTCONV_ERR_SHAPE;
    if (!depthwise_element_ok(*p)) return CTCONV_ERR_SHAPE;
    return CTCONV_OK;
}
}  // namespace

ctconv_status ctconv_depthwise_query_kernel(int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                            const int64_t* in_spatial, const int64_t* kernel,
                                            const int64_t* stride, const int64_t* padding,
                                            const int64_t* output_padding,
                                            const int64_t* dilation, ctconv_dtype dtype,
                                            ctconv_dw_kernel* which) {
    if (!which) return CTCONV_ERR_NULL;
    Problem p;
    const ctconv_status st = depthwise_problem(N, C_in, C_out, ndim, in_spatial, kernel, stride,
                                               padding, output_padding, dilation, dtype, &p);
    if (st != CTCONV_OK) return st;
    *which = depthwise_row_ok(p) ? CTCONV_DW_ROW : CTCONV_DW_ELEMENT;
    return CTCONV_OK;
}

ctconv_status ctconv_depthwise_forward_kernel(const void* x, const void* w, const void* bias,
                                              void* y, int64_t N, int64_t C_in, int64_t C_out,
                                              int ndim, const int64_t* in_spatial,
                                              const int64_t* kernel, const int64_t* stride,
                                              const int64_t* padding,
                                              const int64_t* output_padding,
                                              const int64_t* dilation, ctconv_dtype dtype,
                                              ctconv_activation act, ctconv_dw_kernel which,
                                              void* stream) {
    if (which != CTCONV_DW_AUTO && which != CTCONV_DW_ROW && which != CTCONV_DW_ELEMENT)
        return CTCONV_ERR_PARAM;
    if (act != CTCONV_ACT_NONE && act != CTCONV_ACT_ELU) return CTCONV_ERR_PARAM;
    Problem p;
    const ctconv_status st = depthwise_problem(N, C_in, C_out, ndim, in_spatial, kernel, stride,
                                               padding, output_padding, dilation, dtype, &p);
    if (st != CTCONV_OK) return st;
    p.act = (int)act;
    const bool x_empty = p.N == 0 || p.H == 0 || p.W == 0;
    if (!w || (!x && !x_empty) || (!y && p.N != 0)) return CTCONV_ERR_NULL;
    if ((x && !aligned16(x)) || !aligned16(w) || (y && !aligned16(y)) ||
        (bias && !aligned16(bias)))
        return CTCONV_ERR_ALIGN;
    const bool row_ok = depthwise_row_ok(p);
    if (which == CTCONV_DW_ROW && !row_ok && !x_empty) return CTCONV_ERR_PARAM;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.N == 0) return CTCONV_OK;
    if (x_empty) return to_status(launch_fill(p, bias, y, s));  // no tap reaches y
    const bool use_row = which == CTCONV_DW_AUTO ? row_ok : which == CTCONV_DW_ROW;
    return to_status(launch_depthwise(p, x, w, bias, y, use_row, s));
}

ctconv_status ctconv_depthwise_forward(const void* x, const void* w, const void* bias, void* y,
                                       int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                       const int64_t* in_spatial, const int64_t* kernel,
                                       const int64_t* stride, const int64_t* padding,
                                       const int64_t* output_padding, const int64_t* dilation,
                                       ctconv_dtype dtype, ctconv_activation act, void* stream) {
    return ctconv_depthwise_forward_kernel(x, w, bias, y, N, C_in, C_out, ndim, in_spatial,
                                           kernel, stride, padding, output_padding, dilation,
                                           dtype, act, CTCONV_DW_AUTO, stream);
}

ctconv_status ctconv_elu(const void* x, void* y, int64_t n, ctconv_dtype dtype, void* stream) {
    if (!x || !y) return CTCONV_ERR_NULL;
    if (!dtype_ok(dtype)) return CTCONV_ERR_DTYPE;
    if (n < 0) return CTCONV_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(y)) return CTCONV_ERR_ALIGN;
    return to_status(launch_elu(x, y, n, dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

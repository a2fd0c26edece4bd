// Depthwise transposed convolution (groups = C_in, C_out = M * C_in): output
// channel co reads input channel co / M only, through w[co / M, co % M, ...],
// which is the flat weight row co of the [C_in, M, k...] layout.
//
// ExecuTorch PR #25037 (commit "Decompose depthwise transposed convs")
// rewrites such a layer into one stride-1 depthwise convolution per output
// phase on the low-resolution input (each phase taking every s-th tap) and a
// depth-to-space.  The same phase structure drives the kernel here, but the
// phases are never materialised: every output column o belongs to phase
// j = (o + p) mod s and gathers input columns floor((o + p) / s) - r through
// taps s*r + j, so a lane that owns a run of consecutive outputs computes all
// their phases from one window of input columns and writes the interleaved
// result directly.  There is no reduction over channels, so the work is a
// stream: about one input read per s*s outputs and one output write per
// output; it is bound by HBM bandwidth, not by arithmetic, and runs on the
// vector ALUs (a matrix-core formulation would only add traffic).
//
// Kernels:
//  - strip kernel (dilation 1; 1-D shapes with a row stride of 1, 2 or 4 and
//    at most 4 taps per phase, and 2-D shapes with the same stride and taps
//    per phase in both dimensions and at most 16 weights per channel): the
//    phase split is applied along H as well, where the sH output rows with
//    one ay = floor((oy + pH) / sH) read the same input rows ay - r.  A work
//    item is such a row group over 64 lanes x 4 outputs (2-D) or a 64 x 8
//    segment of a row (1-D); a wave walks a run of consecutive items (down
//    a column strip of one plane in 2-D, sliding one new input row per
//    step; along the row in 1-D), with the channel's weights and bias loaded
//    once per plane into scalar registers and every load of a step issued
//    before its first use.  Strides and taps per phase are compile-time.
//  - row-phase kernel (the other dilation-1 shapes with at most 4 taps per
//    phase in each dimension and an H stride of at most 4): the same row
//    groups over 64 x 4 columns with the row structure at run time; a
//    resident grid (kDwWavesPerCU waves per compute unit) walks the items
//    with the grid's stride, issuing the next item's loads before it
//    computes and stores the current one.
//  - element kernel (every other shape): one output per lane, taps found from
//    the tap condition (o + p - t*d divisible by s, quotient inside the input).
// In the strip and row-phase kernels everything that depends on the rows
// alone is the same in every lane and lives in scalar registers, each lane
// keeps its window of input columns in registers, and its outputs' tap
// classes are known at compile time up to one launch constant.

#include <string.h>

#include "ctconv_internal.h"

namespace ctconv {

namespace {

constexpr int kDwOut = 4;          // outputs per lane along the row
constexpr int kDwCUs = 256;        // compute units of the chip (grid sizing)
constexpr int kDwWavesPerCU = 32;  // resident waves per compute unit (row-phase grid)
constexpr int kDwGridWavesPerCU1D = 512;  // strip kernel, 1-D: grid waves per compute unit
constexpr int kDwGridWavesPerCU2D = 24;   // strip kernel, 2-D: grid waves per compute unit
constexpr int kDwMaxRowStride = 4; // row-phase kernel: stride along H at most 4
constexpr int kDwMaxRowTaps = 4;   // and ceil(kH / sH) <= 4 input rows per group
constexpr int kDwBufferWord3 = 0x00020000;  // raw buffer: 32-bit format, range-checked

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DwArgs {
    const void* x;
    const void* w;
    const void* bias;
    void* y;
    int64_t C_in, C_out;
    int H, W, Ho, Wo;
    int kH, kW, sH, sW, pH, pW, dH, dW;
    int mH;              // ceil(kH / sH): input rows of a row group
    int ay_min, NG;      // row groups ay = floor((oy + pH) / sH): first and count
    uint32_t x_bytes4;   // x size in bytes rounded up to 4 (range of the x buffer)
    uint32_t n_items;    // planes x row groups x segments per row
    int segs;            // wave segments (64 * kDwOut outputs) per output row
    int vec;             // 1: Wo % 4 == 0, whole runs of 4 outputs are stored as one vector
    FastDiv fd_segs, fd_NG, fd_Cout, fd_M;
    int run;             // strip kernel: consecutive work items per wave
    int segs_base;       // segs for kDwOut outputs per lane (n_items = planes * NG * segs_base)
    int act;
};

__device__ inline uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline void* uni_ptr(const void* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    return reinterpret_cast<void*>(((uint64_t)uni((uint32_t)(u >> 32)) << 32) |
                                   uni((uint32_t)u));
}

template <class TR>
__device__ inline float finish(float v, int act) {
    return act == CTCONV_ACT_ELU ? elu_act<TR>(v) : v;
}

// Element e of a weight or bias tensor at a wave-uniform index, read as the
// aligned dword that holds it through the constant address space, so that
// the load is a scalar one (the tensors are 16-byte aligned; the dword of a
// last 16-bit element stays inside that 16-byte granule).
template <class TR>
__device__ inline float load_uniform(const void* base, uint32_t e) {
    typedef const __attribute__((address_space(4))) uint32_t* cptr;
    const cptr p = (cptr)base;
    if constexpr (sizeof(typename TR::storage) == 4) {
        return __uint_as_float(p[e]);
    } else {
        const uint32_t d = p[e >> 1];
        return TR::to_f32((typename TR::storage)((e & 1u) ? d >> 16 : d & 0xFFFFu));
    }
}

// Accumulate one input row into the 4 outputs of a lane.  Output g*SX + b of
// the lane's run has tap class j_b = (b + pW) mod SX and reads input column
// A + g + e_b - r through tap SX*r + j_b, where e_b = 1 when b + (pW mod SX)
// reaches SX; xv[v] holds input column A - (MX-1) + v.
template <int SX, int MX, int OUT = kDwOut>
__device__ inline void row_taps(float (&acc)[OUT], const float (&xv)[OUT / SX + MX],
                                const float (&wv)[SX][MX], int rp) {
    constexpr int G = OUT / SX;
#pragma unroll
    for (int b = 0; b < SX; ++b) {
        // e_b is uniform (rp is a launch constant); both index sets are
        // compile-time, so the choice is one scalar branch per b
        if (b + rp >= SX) {
#pragma unroll
            for (int r = 0; r < MX; ++r)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    acc[g * SX + b] = fmaf(xv[g + MX - r], wv[b][r], acc[g * SX + b]);
        } else {
#pragma unroll
            for (int r = 0; r < MX; ++r)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    acc[g * SX + b] = fmaf(xv[g + MX - 1 - r], wv[b][r], acc[g * SX + b]);
        }
    }
}

// One work item of the row-phase kernel: a row group of one plane over one
// segment of 64 * kDwOut columns, with this lane's input window loaded.
template <class TR, int SX, int MX>
struct DwItem {
    static constexpr int NV = kDwOut / SX + MX;
    uint32_t plane, co;
    int ay, o0;
    float xv[kDwMaxRowTaps][NV];

    // decode item `item` and issue the loads of its input rows ay - r
    __device__ inline void load(const DwArgs& a, const __amdgpu_buffer_rsrc_t xrs, uint32_t item,
                                int lane, int q) {
        using S = typename TR::storage;
        constexpr int ES = sizeof(S);
        // item = ((plane * NG) + group) * segs + seg
        const uint32_t t = fdiv(item, a.fd_segs);
        const uint32_t seg = item - t * (uint32_t)a.segs;
        plane = fdiv(t, a.fd_NG);
        ay = a.ay_min + (int)(t - plane * (uint32_t)a.NG);
        const uint32_t n = fdiv(plane, a.fd_Cout);
        co = plane - n * (uint32_t)a.C_out;
        const uint32_t in_plane = n * (uint32_t)a.C_in + fdiv(co, a.fd_M);
        // outputs o0 .. o0+3 (o0 a multiple of SX) read input columns
        // A - (MX-1) .. A + kDwOut/SX; a column outside the row gets an offset
        // past the buffer's range, which reads as zero
        o0 = ((int)seg * 64 + lane) * kDwOut;
        const int A = o0 / SX + q;
        uint32_t voff[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int col = A - (MX - 1) + v;
            voff[v] = (uint32_t)col < (uint32_t)a.W ? (uint32_t)col * ES : 0x80000000u;
        }
#pragma unroll
        for (int r = 0; r < kDwMaxRowTaps; ++r) {
            const int iy = ay - r;
            const bool live = r < a.mH && iy >= 0 && iy < a.H;  // uniform
            const uint32_t rowb =
                uni(((in_plane * (uint32_t)a.H + (uint32_t)(live ? iy : 0)) * (uint32_t)a.W) * ES);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                xv[r][v] = 0.f;
                if (live) {
                    if constexpr (ES == 2)
                        xv[r][v] = TR::to_f32(
                            __builtin_amdgcn_raw_buffer_load_b16(xrs, voff[v], rowb, 0));
                    else
                        xv[r][v] = __uint_as_float(
                            __builtin_amdgcn_raw_buffer_load_b32(xrs, voff[v], rowb, 0));
                }
            }
        }
    }
};

template <class TR, int SX, int MX>
__global__ __launch_bounds__(256) void dw_row_kernel(const DwArgs a) {
    using S = typename TR::storage;
    constexpr int ES = sizeof(S);
    const int lane = threadIdx.x & 63;
    const uint32_t n_waves = gridDim.x * 4u;
    uint32_t item = uni(blockIdx.x * 4u + threadIdx.x / 64u);
    if (item >= a.n_items) return;  // uniform

    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc(uni_ptr(a.x), (short)0, (int)a.x_bytes4, kDwBufferWord3);
    S* __restrict__ yg = static_cast<S*>(a.y);
    const int q = a.pW / SX, rp = a.pW % SX;

    // items item, item + n_waves, ...: the next item's input rows are loaded
    // before the current item is computed and stored, so that their latency
    // overlaps (loads and stores retire in issue order)
    DwItem<TR, SX, MX> cur;
    cur.load(a, xrs, item, lane, q);
    for (;;) {
        const uint32_t next = item + n_waves;
        const bool has_next = next < a.n_items;  // uniform
        DwItem<TR, SX, MX> nxt;
        if (has_next) nxt.load(a, xrs, next, lane, q);

        const uint32_t wrow = cur.co * (uint32_t)(a.kH * a.kW);  // first weight of channel co
        const float bv = a.bias != nullptr ? load_uniform<TR>(a.bias, cur.co) : 0.f;
        // output rows of the group: oy = sH*ay + jy - pH, taps ty = sH*r + jy
#pragma unroll 1
        for (int jy = 0; jy < a.sH; ++jy) {
            const int oy = a.sH * cur.ay + jy - a.pH;
            if (oy < 0 || oy >= a.Ho) continue;  // uniform
            float acc[kDwOut];
#pragma unroll
            for (int u = 0; u < kDwOut; ++u) acc[u] = 0.f;
#pragma unroll
            for (int r = 0; r < kDwMaxRowTaps; ++r) {
                const int ty = a.sH * r + jy;
                const int iy = cur.ay - r;
                if (r >= a.mH || ty >= a.kH || iy < 0 || iy >= a.H) continue;  // uniform
                float wv[SX][MX];
#pragma unroll
                for (int b = 0; b < SX; ++b) {
                    const int jb = b + rp >= SX ? b + rp - SX : b + rp;
#pragma unroll
                    for (int rr = 0; rr < MX; ++rr) {
                        const int tx = SX * rr + jb;
                        wv[b][rr] =
                            tx < a.kW ? load_uniform<TR>(a.w, uni(wrow + ty * a.kW + tx)) : 0.f;
                    }
                }
                row_taps<SX, MX>(acc, cur.xv[r], wv, rp);
            }
#pragma unroll
            for (int u = 0; u < kDwOut; ++u) acc[u] += bv;
            if (a.act == CTCONV_ACT_ELU) {  // uniform
#pragma unroll
                for (int u = 0; u < kDwOut; ++u) acc[u] = elu_act<TR>(acc[u]);
            }
            S* yr = yg + ((int64_t)cur.plane * a.Ho + oy) * a.Wo;
            const int o0 = cur.o0;
            if (a.vec && o0 < a.Wo) {
                if constexpr (ES == 2) {
                    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
                    u32x2v st;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        st[h] = (uint32_t)TR::from_f32(acc[2 * h]) |
                                ((uint32_t)TR::from_f32(acc[2 * h + 1]) << 16);
                    *reinterpret_cast<u32x2v*>(yr + o0) = st;
                } else {
                    f32x4 st;
#pragma unroll
                    for (int u = 0; u < 4; ++u) st[u] = acc[u];
                    *reinterpret_cast<f32x4*>(yr + o0) = st;
                }
            } else {
#pragma unroll
                for (int u = 0; u < kDwOut; ++u)
                    if (o0 + u < a.Wo) yr[o0 + u] = TR::from_f32(acc[u]);
            }
        }
        if (!has_next) break;
        item = next;
        cur = nxt;
    }
}

// Strip kernel: the row-phase computation with the strides and taps per
// phase of both dimensions fixed at compile time (SY, MY along H; 1-D has
// SY = MY = 1) and OUT outputs per lane (8 in 1-D, 4 in 2-D, where rows are
// shorter).  A wave walks `run` consecutive work items in the order
// ((plane * segs + seg) * NG + group): down a column strip of one plane in
// 2-D, along the row in 1-D.  The channel's weights (at most 16) and bias
// are loaded once per plane into scalar registers; consecutive row groups of
// a strip share MY - 1 input rows, so each step loads one new row.  All of a
// step's loads are issued before their first use.
template <class TR, int SX, int MX, int SY, int MY, int OUT>
__global__ __launch_bounds__(256) void dw_strip_kernel(const DwArgs a) {
    using S = typename TR::storage;
    constexpr int ES = sizeof(S);
    constexpr int G = OUT / SX;
    constexpr int NV = G + MX;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = uni(blockIdx.x * 4u + threadIdx.x / 64u);
    uint32_t item = wave * (uint32_t)a.run;
    if (item >= a.n_items) return;  // uniform
    const uint32_t item_end =
        item + (uint32_t)a.run < a.n_items ? item + (uint32_t)a.run : a.n_items;

    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc(uni_ptr(a.x), (short)0, (int)a.x_bytes4, kDwBufferWord3);
    S* __restrict__ yg = static_cast<S*>(a.y);
    const int q = a.pW / SX, rp = a.pW % SX;
    const uint32_t row_bytes = (uint32_t)a.W * ES;

    // position of the first item
    uint32_t g = item % (uint32_t)a.NG;
    uint32_t t = item / (uint32_t)a.NG;
    uint32_t seg = t % (uint32_t)a.segs;
    uint32_t plane = t / (uint32_t)a.segs;

    // per-plane state: weights, bias, x plane offset, y plane
    float wts[SY][MY][SX][MX];
    float bv = 0.f;
    uint32_t xplane = 0;
    auto load_plane = [&](uint32_t pl) {
        const uint32_t n = fdiv(pl, a.fd_Cout);
        const uint32_t co = pl - n * (uint32_t)a.C_out;
        xplane = uni((n * (uint32_t)a.C_in + fdiv(co, a.fd_M)) * (uint32_t)a.H * row_bytes);
        const uint32_t wrow = co * (uint32_t)(a.kH * a.kW);
#pragma unroll
        for (int jy = 0; jy < SY; ++jy)
#pragma unroll
            for (int r = 0; r < MY; ++r) {
                const int ty = SY * r + jy;
#pragma unroll
                for (int b = 0; b < SX; ++b) {
                    const int jb = b + rp >= SX ? b + rp - SX : b + rp;
#pragma unroll
                    for (int rr = 0; rr < MX; ++rr) {
                        const int tx = SX * rr + jb;
                        wts[jy][r][b][rr] = (ty < a.kH && tx < a.kW)
                                                ? load_uniform<TR>(a.w, wrow + ty * a.kW + tx)
                                                : 0.f;
                    }
                }
            }
        bv = a.bias != nullptr ? load_uniform<TR>(a.bias, co) : 0.f;
    };
    // lane window offsets of segment sg
    auto lane_offsets = [&](uint32_t sg, uint32_t (&voff)[NV]) {
        const int A = (((int)sg * 64 + lane) * OUT) / SX + q;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int col = A - (MX - 1) + v;
            voff[v] = (uint32_t)col < (uint32_t)a.W ? (uint32_t)col * ES : 0x80000000u;
        }
    };
    // one input row as raw bits (zero outside [0, H)): the loads are issued
    // unconditionally (a row outside the input gets lane offsets past the
    // buffer's range) and their values are first used at the next compute,
    // so that nothing waits for them here
    auto load_row = [&](int iy, const uint32_t (&voff)[NV], uint32_t (&dst)[NV]) {
        const bool live = iy >= 0 && iy < a.H;  // uniform
        const uint32_t rowb = uni(xplane + (uint32_t)(live ? iy : 0) * row_bytes);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint32_t o = live ? voff[v] : 0x80000000u;
            if constexpr (ES == 2)
                dst[v] = __builtin_amdgcn_raw_buffer_load_b16(xrs, o, rowb, 0);
            else
                dst[v] = __builtin_amdgcn_raw_buffer_load_b32(xrs, o, rowb, 0);
        }
    };

    load_plane(plane);
    uint32_t voff[NV];
    lane_offsets(seg, voff);
    uint32_t xv[MY][NV];  // rows ay - r of the current group (raw bits)
    bool fresh = true;    // the current item starts a strip: all MY rows to load

    for (;;) {
        // the item's input rows: all of them at the start of a strip, else
        // the one new row (the others slide down from the previous group);
        // every load is issued before the first use
        const int ay = a.ay_min + (int)g;
        if (fresh) {
#pragma unroll
            for (int r = 0; r < MY; ++r) load_row(ay - r, voff, xv[r]);
        } else {
#pragma unroll
            for (int r = MY - 1; r > 0; --r)
#pragma unroll
                for (int v = 0; v < NV; ++v) xv[r][v] = xv[r - 1][v];
            load_row(ay, voff, xv[0]);
        }
        float xf[MY][NV];
#pragma unroll
        for (int r = 0; r < MY; ++r)
#pragma unroll
            for (int v = 0; v < NV; ++v)
                xf[r][v] = ES == 2 ? TR::to_f32((S)xv[r][v]) : __uint_as_float(xv[r][v]);

        // compute and store the group's output rows
        const int o0 = ((int)seg * 64 + lane) * OUT;
#pragma unroll
        for (int jy = 0; jy < SY; ++jy) {
            const int oy = SY * ay + jy - a.pH;
            if (oy < 0 || oy >= a.Ho) continue;  // uniform
            float acc[OUT];
#pragma unroll
            for (int u = 0; u < OUT; ++u) acc[u] = 0.f;
#pragma unroll
            for (int r = 0; r < MY; ++r) row_taps<SX, MX, OUT>(acc, xf[r], wts[jy][r], rp);
#pragma unroll
            for (int u = 0; u < OUT; ++u) acc[u] += bv;
            if (a.act == CTCONV_ACT_ELU) {  // uniform
#pragma unroll
                for (int u = 0; u < OUT; ++u) acc[u] = elu_act<TR>(acc[u]);
            }
            S* yr = yg + ((int64_t)plane * a.Ho + oy) * a.Wo;
            if (a.vec && o0 < a.Wo) {
                // whole run inside the row, aligned to OUT elements
                if constexpr (ES == 2) {
#pragma unroll
                    for (int c = 0; c < OUT / 8; ++c) {
                        u32x4 st;
#pragma unroll
                        for (int h = 0; h < 4; ++h)
                            st[h] = (uint32_t)TR::from_f32(acc[8 * c + 2 * h]) |
                                    ((uint32_t)TR::from_f32(acc[8 * c + 2 * h + 1]) << 16);
                        *reinterpret_cast<u32x4*>(yr + o0 + 8 * c) = st;
                    }
                    if constexpr (OUT % 8 == 4) {
                        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
                        u32x2v st;
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            st[h] = (uint32_t)TR::from_f32(acc[OUT - 4 + 2 * h]) |
                                    ((uint32_t)TR::from_f32(acc[OUT - 3 + 2 * h]) << 16);
                        *reinterpret_cast<u32x2v*>(yr + o0 + OUT - 4) = st;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < OUT / 4; ++c) {
                        f32x4 st;
#pragma unroll
                        for (int u = 0; u < 4; ++u) st[u] = acc[4 * c + u];
                        *reinterpret_cast<f32x4*>(yr + o0 + 4 * c) = st;
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < OUT; ++u)
                    if (o0 + u < a.Wo) yr[o0 + u] = TR::from_f32(acc[u]);
            }
        }

        // next item: the following row group of the strip, or the start of
        // the next strip (next segment, or the next plane)
        if (++item >= item_end) break;  // uniform
        if (++g < (uint32_t)a.NG) {
            fresh = false;
        } else {
            g = 0;
            fresh = true;
            if (++seg == (uint32_t)a.segs) {
                seg = 0;
                ++plane;
                load_plane(plane);
            }
            lane_offsets(seg, voff);
        }
    }
}



template <class TR>
__global__ __launch_bounds__(256) void dw_element_kernel(const DwArgs a, int64_t total) {
    using S = typename TR::storage;
    const S* __restrict__ xg = static_cast<const S*>(a.x);
    const S* __restrict__ wg = static_cast<const S*>(a.w);
    const S* __restrict__ bg = static_cast<const S*>(a.bias);
    S* __restrict__ yg = static_cast<S*>(a.y);
    const int64_t M = a.C_out / a.C_in;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ox = i % a.Wo;
        const int64_t t = i / a.Wo;
        const int64_t oy = t % a.Ho;
        const int64_t plane = t / a.Ho;
        const int64_t co = plane % a.C_out;
        const int64_t n = plane / a.C_out;
        const int64_t ci = co / M;
        const S* xp = xg + (n * a.C_in + ci) * a.H * a.W;
        const S* wc = wg + co * a.kH * a.kW;
        float acc = 0.f;
        for (int ty = 0; ty < a.kH; ++ty) {
            const int64_t ny = oy + a.pH - (int64_t)ty * a.dH;
            if (ny < 0) break;
            const int64_t iy = ny / a.sH;
            if (iy * a.sH != ny || iy >= a.H) continue;
            for (int tx = 0; tx < a.kW; ++tx) {
                const int64_t nx = ox + a.pW - (int64_t)tx * a.dW;
                if (nx < 0) break;
                const int64_t ix = nx / a.sW;
                if (ix * a.sW != nx || ix >= a.W) continue;
                acc = fmaf(TR::to_f32(xp[iy * a.W + ix]), TR::to_f32(wc[ty * a.kW + tx]), acc);
            }
        }
        const float bv = bg != nullptr ? TR::to_f32(bg[co]) : 0.f;
        yg[i] = TR::from_f32(finish<TR>(acc + bv, a.act));
    }
}

// Shapes of the row-phase kernel: dilation 1; along the row SX = sW in
// {1, 2, 4} and MX = ceil(kW / SX) in 1..4 (compiled instances); along H a
// stride of at most kDwMaxRowStride and at most kDwMaxRowTaps taps per phase.
bool row_kernel_shape(const Problem& p, int* SX, int* MX) {
    if (p.dW != 1 || p.dH != 1 || (p.sW != 1 && p.sW != 2 && p.sW != 4)) return false;
    if (p.sH > kDwMaxRowStride || (p.kH + p.sH - 1) / p.sH > kDwMaxRowTaps) return false;
    const int64_t mx = (p.kW + p.sW - 1) / p.sW;
    if (mx > 4) return false;
    *SX = (int)p.sW;
    *MX = (int)mx;
    return true;
}

bool fill_args(const Problem& p, DwArgs* a) {
    memset(a, 0, sizeof(*a));
    const int64_t es = p.dtype == CTCONV_F32 ? 4 : 2;
    const int64_t x_bytes = p.N * p.C_in * p.H * p.W * es;
    // row groups: output rows with the same ay = floor((oy + pH) / sH) read
    // the same input rows ay - r, r < ceil(kH / sH)
    const int64_t ay_min = p.pH / p.sH, ay_max = (p.Ho - 1 + p.pH) / p.sH;
    const int64_t NG = ay_max - ay_min + 1;
    const int64_t segs = (p.Wo + 64 * kDwOut - 1) / (64 * kDwOut);
    // 32-bit lane arithmetic: x below 2^31 bytes (offsets past the range stay
    // below 2^32), work items and all sizes below 2^31, sH * ay below 2^30
    if (x_bytes >= (int64_t(1) << 31) || p.N * p.C_out >= (int64_t(1) << 31) ||
        p.N * p.C_out * NG * segs >= (int64_t(1) << 31) - kDwCUs * kDwGridWavesPerCU1D ||
        p.Wo >= (int64_t(1) << 29) || p.Ho + p.pH >= (int64_t(1) << 30) ||
        p.pW >= (int64_t(1) << 30) || p.kH * p.kW >= (1 << 30))
        return false;
    a->C_in = p.C_in;
    a->C_out = p.C_out;
    a->H = (int)p.H;
    a->W = (int)p.W;
    a->Ho = (int)p.Ho;
    a->Wo = (int)p.Wo;
    a->kH = (int)p.kH;
    a->kW = (int)p.kW;
    a->sH = (int)p.sH;
    a->sW = (int)p.sW;
    a->pH = (int)p.pH;
    a->pW = (int)p.pW;
    a->dH = (int)p.dH;
    a->dW = (int)p.dW;
    a->mH = (int)((p.kH + p.sH - 1) / p.sH);
    a->ay_min = (int)ay_min;
    a->NG = (int)NG;
    a->x_bytes4 = (uint32_t)((x_bytes + 3) & ~int64_t(3));
    a->n_items = (uint32_t)(p.N * p.C_out * NG * segs);
    a->segs = (int)segs;
    a->segs_base = (int)segs;
    a->vec = p.Wo % kDwOut == 0;
    a->fd_segs = make_fastdiv((uint32_t)segs);
    a->fd_NG = make_fastdiv((uint32_t)NG);
    a->fd_Cout = make_fastdiv((uint32_t)p.C_out);
    a->fd_M = make_fastdiv((uint32_t)(p.C_out / p.C_in));
    a->act = p.act;
    return true;
}

template <class TR, int SX, int MX>
hipError_t launch_row(const DwArgs& a, hipStream_t s) {
    // a resident grid: each wave walks the items with a stride of the grid's
    // wave count (kDwWavesPerCU waves per compute unit, fewer for small jobs)
    const uint32_t waves_max = (uint32_t)kDwCUs * kDwWavesPerCU;
    const uint32_t waves = a.n_items < waves_max ? a.n_items : waves_max;
    dw_row_kernel<TR, SX, MX><<<dim3((waves + 3) / 4), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

// Strip-kernel instances: 1-D (SY = MY = 1, any compiled SX, MX) and 2-D with
// the same stride and taps per phase in both dimensions and at most 16
// weights per channel.
bool strip_shape(int SX, int MX, int SY, int MY) {
    if (SY == 1 && MY == 1) return true;
    return SY == SX && MY == MX && SX * MX * SY * MY <= 16;
}

template <class TR, int SX, int MX, int SY, int MY>
hipError_t launch_strip(DwArgs a, hipStream_t s) {
    // 1-D rows are long: 8 outputs per lane; 2-D: 4 (one wave per 256 columns)
    constexpr int OUT = SY == 1 && MY == 1 ? 8 : 4;
    const int64_t segs = ((int64_t)a.Wo + 64 * OUT - 1) / (64 * OUT);
    a.segs = (int)segs;
    a.fd_segs = make_fastdiv((uint32_t)segs);
    a.n_items = (uint32_t)((int64_t)a.n_items / a.segs_base * segs);
    a.vec = a.Wo % OUT == 0;
    // grid size, measured on the k4 s2 upsamplers.  1-D: many short-lived
    // waves of about two items each, 16x the resident wave slots (as waves
    // end, new ones start issuing loads at once): 110 us, against 129 us with
    // a resident grid of 32 per CU walking ~32 items.  2-D: a resident grid
    // of 24 waves per CU walking down the strips, whose items share input
    // rows (111 us; 118 at 32; flat from 64 to 256)
    const uint32_t target =
        (uint32_t)kDwCUs * (SY == 1 && MY == 1 ? kDwGridWavesPerCU1D : kDwGridWavesPerCU2D);
    uint32_t run = a.n_items / target;
    run = run < 1 ? 1 : run > 256 ? 256 : run;
    a.run = (int)run;
    const uint32_t waves = (a.n_items + run - 1) / run;
    dw_strip_kernel<TR, SX, MX, SY, MY, OUT><<<dim3((waves + 3) / 4), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <class TR>
hipError_t launch_strip_t(const DwArgs& a, int SX, int MX, int SY, int MY, hipStream_t s) {
#define CTCONV_DW_STRIP(sx, mx, sy, my) \
    if (SX == sx && MX == mx && SY == sy && MY == my) return launch_strip<TR, sx, mx, sy, my>(a, s);
    CTCONV_DW_STRIP(1, 1, 1, 1) CTCONV_DW_STRIP(1, 2, 1, 1) CTCONV_DW_STRIP(1, 3, 1, 1)
    CTCONV_DW_STRIP(1, 4, 1, 1) CTCONV_DW_STRIP(2, 1, 1, 1) CTCONV_DW_STRIP(2, 2, 1, 1)
    CTCONV_DW_STRIP(2, 3, 1, 1) CTCONV_DW_STRIP(2, 4, 1, 1) CTCONV_DW_STRIP(4, 1, 1, 1)
    CTCONV_DW_STRIP(4, 2, 1, 1) CTCONV_DW_STRIP(4, 3, 1, 1) CTCONV_DW_STRIP(4, 4, 1, 1)
    CTCONV_DW_STRIP(1, 2, 1, 2) CTCONV_DW_STRIP(1, 3, 1, 3) CTCONV_DW_STRIP(1, 4, 1, 4)
    CTCONV_DW_STRIP(2, 1, 2, 1) CTCONV_DW_STRIP(2, 2, 2, 2) CTCONV_DW_STRIP(4, 1, 4, 1)
#undef CTCONV_DW_STRIP
    return hipErrorInvalidValue;
}

template <class TR>
hipError_t launch_row_t(const DwArgs& a, int SX, int MX, hipStream_t s) {
#define CTCONV_DW_ROW(sx, mx) \
    if (SX == sx && MX == mx) return launch_row<TR, sx, mx>(a, s);
    CTCONV_DW_ROW(1, 1) CTCONV_DW_ROW(1, 2) CTCONV_DW_ROW(1, 3) CTCONV_DW_ROW(1, 4)
    CTCONV_DW_ROW(2, 1) CTCONV_DW_ROW(2, 2) CTCONV_DW_ROW(2, 3) CTCONV_DW_ROW(2, 4)
    CTCONV_DW_ROW(4, 1) CTCONV_DW_ROW(4, 2) CTCONV_DW_ROW(4, 3) CTCONV_DW_ROW(4, 4)
#undef CTCONV_DW_ROW
    return hipErrorInvalidValue;
}

template <class TR>
hipError_t launch_element(const Problem& p, const void* x, const void* w, const void* bias,
                          void* y, hipStream_t s) {
    DwArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.C_in = p.C_in;
    a.C_out = p.C_out;
    a.H = (int)p.H;
    a.W = (int)p.W;
    a.Ho = (int)p.Ho;
    a.Wo = (int)p.Wo;
    a.kH = (int)p.kH;
    a.kW = (int)p.kW;
    a.sH = (int)p.sH;
    a.sW = (int)p.sW;
    a.pH = (int)p.pH;
    a.pW = (int)p.pW;
    a.dH = (int)p.dH;
    a.dW = (int)p.dW;
    a.act = p.act;
    const int64_t total = p.N * p.C_out * p.Ho * p.Wo;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    dw_element_kernel<TR><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a, total);
    return hipGetLastError();
}

}  // namespace

bool depthwise_element_ok(const Problem& p) {
    // 32-bit fields of the element kernel
    return p.H < (int64_t(1) << 31) && p.W < (int64_t(1) << 31) && p.Ho < (int64_t(1) << 31) &&
           p.Wo < (int64_t(1) << 31) && p.kH < (int64_t(1) << 31) && p.kW < (int64_t(1) << 31) &&
           p.sH < (int64_t(1) << 31) && p.sW < (int64_t(1) << 31) && p.pH < (int64_t(1) << 31) &&
           p.pW < (int64_t(1) << 31) && p.dH < (int64_t(1) << 31) && p.dW < (int64_t(1) << 31);
}

bool depthwise_row_ok(const Problem& p) {
    int SX, MX;
    DwArgs a;
    return row_kernel_shape(p, &SX, &MX) && fill_args(p, &a) && depthwise_element_ok(p);
}

hipError_t launch_depthwise(const Problem& p, const void* x, const void* w, const void* bias,
                            void* y, bool row_kernel, hipStream_t s) {
    if (p.N * p.C_out * p.Ho * p.Wo <= 0) return hipSuccess;
    if (row_kernel) {
        int SX = 0, MX = 0;
        DwArgs a;
        if (!row_kernel_shape(p, &SX, &MX) || !fill_args(p, &a)) return hipErrorInvalidValue;
        a.x = x;
        a.w = w;
        a.bias = bias;
        a.y = y;
        const int SY = (int)p.sH, MY = (int)((p.kH + p.sH - 1) / p.sH);
        if (strip_shape(SX, MX, SY, MY)) {
            switch (p.dtype) {
                case CTCONV_F32: return launch_strip_t<TF32>(a, SX, MX, SY, MY, s);
                case CTCONV_BF16: return launch_strip_t<TBF16>(a, SX, MX, SY, MY, s);
                case CTCONV_F16: return launch_strip_t<TF16>(a, SX, MX, SY, MY, s);
            }
            return hipErrorInvalidValue;
        }
        switch (p.dtype) {
            case CTCONV_F32: return launch_row_t<TF32>(a, SX, MX, s);
            case CTCONV_BF16: return launch_row_t<TBF16>(a, SX, MX, s);
            case CTCONV_F16: return launch_row_t<TF16>(a, SX, MX, s);
        }
        return hipErrorInvalidValue;
    }
    switch (p.dtype) {
        case CTCONV_F32: return launch_element<TF32>(p, x, w, bias, y, s);
        case CTCONV_BF16: return launch_element<TBF16>(p, x, w, bias, y, s);
        case CTCONV_F16: return launch_element<TF16>(p, x, w, bias, y, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ctconv

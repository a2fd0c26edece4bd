// Internal declarations shared by the ctconv HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ctconv.h"

namespace ctconv {

// ---------------------------------------------------------------------------
// Element types.  Storage is the raw 16/32-bit pattern; arithmetic is fp32.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct TBF16 {
    using storage = uint16_t;
    static constexpr int kVec = 8;  // elements per 16-byte fragment
    __device__ static inline float to_f32(storage v) {
        return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }
    __device__ static inline storage from_f32(float f) {
        // round to nearest even; NaN stays a quiet NaN
        __bf16 b = static_cast<__bf16>(f);
        return __builtin_bit_cast(uint16_t, b);
    }
};

struct TF16 {
    using storage = uint16_t;
    static constexpr int kVec = 8;
    __device__ static inline float to_f32(storage v) {
        return static_cast<float>(__builtin_bit_cast(_Float16, v));
    }
    __device__ static inline storage from_f32(float f) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
    }
};

struct TF32 {
    using storage = float;
    static constexpr int kVec = 4;
    __device__ static inline float to_f32(storage v) { return v; }
    __device__ static inline storage from_f32(float f) { return f; }
};

// ---------------------------------------------------------------------------
// Normalised problem description (1-D problems use H = Ho = 1, kH = sH = 1,
// pH = opH = 0, dH = 1).
// ---------------------------------------------------------------------------
struct Problem {
    int ndim;
    int64_t N, C_in, C_out;
    int64_t H, W, Ho, Wo;
    int64_t kH, kW, sH, sW, pH, pW, opH, opW, dH, dW;
    int64_t mH, mW;   // taps per phase: ceil(k / s)
    int64_t P, T;     // phases sH*sW, taps mH*mW
    int64_t C_in_pad; // C_in rounded up to 32
    ctconv_dtype dtype;
    int act;          // ctconv_activation applied to every output before rounding
};

// ELU with alpha = 1, computed in fp32 and rounded once to the storage type
// (the fused epilogues and the standalone ELU kernel share it, so a fused
// forward and a forward followed by the ELU pass agree bit for bit).  For
// v <= 0 it needs e^v - 1, branch free:
//  - fp32 storage: above -1/2 the Taylor series of e^t - 1 through t^8
//    (truncation below 2e-8 relative there), else 2^(t log2 e) - 1 from the
//    hardware exp2, whose cancellation error is at most ~2.5 ulp at -1/2 and
//    shrinks below it;
//  - 16-bit storage: 2^(t log2 e) - 1 everywhere; its absolute error (about
//    1e-7) stays below half an ulp of the bf16/fp16 result down to |v| ~ 1e-4.
// A NaN passes through.
template <class TR>
__device__ inline float elu_act(float v) {
    const float t = v > 0.f ? 0.f : v;
    const float e = __builtin_amdgcn_exp2f(t * 1.44269504088896341f) - 1.f;
    float m = e;
    if constexpr (sizeof(typename TR::storage) == 4) {
        float p = 1.f / 40320.f;
        p = fmaf(p, t, 1.f / 5040.f);
        p = fmaf(p, t, 1.f / 720.f);
        p = fmaf(p, t, 1.f / 120.f);
        p = fmaf(p, t, 1.f / 24.f);
        p = fmaf(p, t, 1.f / 6.f);
        p = fmaf(p, t, 0.5f);
        p = fmaf(p, t, 1.f) * t;
        m = t > -0.5f ? p : e;
    }
    return v > 0.f ? v : m;
}

constexpr int64_t kCinAlign = 32;

// Division by a launch-constant divisor d >= 1 as a multiply and a shift:
// q = floor(n * m / 2^s) with s = 31 + ceil(log2 d) and m = ceil(2^s / d)
// (below 2^32).  m exceeds 2^s / d by e < 1, so n * m / 2^s exceeds n / d by
// n * e / 2^s < 2^31 / 2^s <= 1 / d, which never reaches the next integer
// for 0 <= n < 2^31.
struct FastDiv {
    uint32_t m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    const uint32_t s = 31 + l;
    const uint64_t pw = 1ull << s;
    return FastDiv{(uint32_t)((pw + d - 1) / d), s};
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

// Arguments of the polyphase MFMA kernel (filled by the host planner).
struct PolyArgs {
    const void* x;
    const void* pw;
    const void* bias;
    void* y;
    int64_t N, C_in, C_out, C_in_pad;
    int64_t H, W, Ho, Wo;  // Ho, Wo: outputs of the problem the kernel runs
    int sy, sx, py, px;    // its stride and padding (padding 0 unless cmode)
    int P, T;
    int Ay, Ax;            // output rows per dimension in units of the stride
    // Class mode (cmode = 1): phase rows aligned to the output under padding
    // p; output phase b reads input rows from floor((b + p) / s) on, i.e.
    // dmin = floor(p / s) plus 0 or 1 per phase and dimension, and each column
    // block reads its own A fragments.  Without it the planner has removed
    // the padding (dmin = 0, every phase alike).
    int cmode, dminy, dminx;
    int WY, WX;            // x window per tile (rows x columns)
    int xofs;              // window start moved back by this many positions so
                           // that every x load is 8-byte aligned (0 when rows
                           // are not a multiple of 8 bytes)
    int TCO, PT;           // output channels and phases per column tile
    int phase_subset;      // 0: a column tile holds every phase; 1: a run of PT phases
    int pfast;             // column order: 0 channel-major, 1 phase-fastest, 2 row-phase-
                           // fastest (class mode, sx = 2); 1 and 2 stage the epilogue in runs
    
    int n_ph_tiles, n_col_tiles;
    int tiles_y, tiles_x;
    int64_t n_row_tiles;
    uint32_t n_tiles;      // row tiles x column tiles (below 2^31): the grid
    // divisions by launch constants (tile decomposition, window rows, column
    // tile channels, strides, staged output rows and their 16-byte chunks)
    FastDiv fd_cols, fd_ph, fd_tx, fd_ty, fd_wy, fd_tco, fd_sx, fd_sy, fd_R;
    FastDiv fd_cpr;        // 16-byte chunks per staged output row
    FastDiv fd_pt;         // blocks per cycle of the column order: PT (pfast 1), 2 TCO/16 (pfast 2)
    FastDiv fd_psy, fd_psx;  // strides of the packed weight
    int n_chunks;          // C_in_pad / KC
    int chunks_per_split;  // split over C_in: each blockIdx.y takes this many chunks
    int partial;           // 1: split over C_in; split 0 writes its fp32 partial sums
                           // (no bias, no activation) to y, split s > 0 to slab s - 1
                           // of ws, and a second kernel adds them in order
    float* ws;             // the slabs (partial = 1)
    int64_t ws_slab;       // elements per slab (the size of y)
    int xcd_remap;         // 1: gridDim.x is a multiple of 8, remap for L2 locality
    int colmajor;          // tile order: 1 all row tiles of a column tile, then the
                           // next column tile; 0 all column tiles of a row tile first
    FastDiv fd_rows;       // n_row_tiles
    uint32_t pw_bytes;     // size of the packed weight (below 2^32)
    int act;               // ctconv_activation of the epilogue
    int outf32;            // 1: y is fp32, written straight from the accumulators (1-D
                           // shapes without padding shift classes, reduction or split:
                           // the chunks of a 16-bit stream)
    // Dilation (per dimension): the kernel runs the problem reduced by
    // g = gcd(s, d) (stride s/g), whose output u' sits at o0 + g*u' of the
    // real output; the other outputs are bias only (pre-filled).  Identity
    // (g = 1, o0 = 0, real sizes = Ho, Wo) when g = 1.
    int gy, gx, o0y, o0x;
    // Remaining dilation d' = d / g: the kernel's taps are the expanded
    // kernel's, real tap e / d' where d' divides e (1 without dilation)
    int dey, dex;
    FastDiv fd_dey, fd_dex;
    int64_t HoR, WoR;      // real output sizes (addressing of y)
    // Padding as an output shift: the kernel computes the transposed
    // convolution without padding (of the dilation-reduced problem under
    // dilation) and writes its output o' as output o' - os of that problem
    // when it lies inside, i.e. below Ho - os (Wo - os)
    int oys, oxs;
    // Tap groups (fp32 shapes with more taps per phase than a compiled
    // kernel instance): launch g runs tap slots r0 .. r0 + MY/MX - 1 of every
    // phase on the input window shifted back by r0, and launches after the
    // first add their sums to y (accum = 1; the bias comes with the first,
    // the activation with the last, after its sum)
    int r0y, r0x, accum, ngy, ngx, gmy, gmx;  // gmy, gmx: tap slots per group
    // Packed-weight geometry (the real stride and taps the weight was packed
    // with): the kernel's tap e = s' r + j per dimension is real tap t = e / d',
    // stored as phase t mod ps, tap t / ps; other taps and t >= k read as zero.
    int psy, psx, pmx, pT, kH, kW;
    uint32_t pw_cblock;    // bytes of one 32-channel block of a phase (C_out * pT * 32)
};

// Launchers (each returns hipGetLastError() of its launch).
hipError_t launch_prepack(const Problem& p, const void* w, void* pw, hipStream_t s);
hipError_t launch_gather(const Problem& p, const void* x, const void* pw, const void* bias,
                         void* y, bool out_f32, hipStream_t s);
// the staged gather kernel covers p (else the general one runs)
bool gather_staged_ok(const Problem& p);
hipError_t launch_fill(const Problem& p, const void* bias, void* y, hipStream_t s);
// y = act(y + ws[0] + ... + ws[nslab-1] + bias), fp32, added in that order.
hipError_t launch_split_reduce(const Problem& p, const void* bias, void* y, const void* ws,
                               int nslab, hipStream_t s);
hipError_t launch_elu(const void* x, void* y, int64_t n, ctconv_dtype dt, hipStream_t s);
hipError_t launch_istft_norm(const void* y, const void* env, void* out, int64_t rows,
                             int64_t L_in, int64_t trim, int64_t L_out, ctconv_dtype dt,
                             hipStream_t s);

// Streaming overlap-add and flush (rows = N * C_out; Ly emitted outputs and
// Tl tail values per row).
hipError_t launch_stream_overlap(const float* z, const float* tail_in, const void* bias, void* y,
                                 float* tail_out, int64_t rows, int64_t C_out, int64_t Ly,
                                 int64_t Tl, ctconv_dtype dt, int act, hipStream_t s);
hipError_t launch_stream_flush(const float* tail_in, const void* bias, void* y, int64_t rows,
                               int64_t C_out, int64_t Tl, ctconv_dtype dt, int act,
                               hipStream_t s);

// Depthwise transposed convolution (groups = C_in, C_out a multiple of C_in;
// the weight is the unpacked [C_in, C_out / C_in, k...] tensor).
// depthwise_row_ok: the row-phase kernel covers the shape; depthwise_element_ok:
// the element kernel's 32-bit fields hold its sizes.
bool depthwise_row_ok(const Problem& p);
bool depthwise_element_ok(const Problem& p);
hipError_t launch_depthwise(const Problem& p, const void* x, const void* w, const void* bias,
                            void* y, bool row_kernel, hipStream_t s);

// Polyphase planning and launch.  polyphase_supported returns false when no
// compiled kernel instance covers the shape.  polyphase_workspace_bytes: the
// workspace the launch splits its reduction into when it may use one (0: no
// split).  launch_polyphase splits only when ws is given and holds at least
// that many bytes.
bool polyphase_supported(const Problem& p);
size_t polyphase_workspace_bytes(const Problem& p);
// The register-weight streaming kernel (16-bit 1-D, stride a multiple of 4,
// taps x padded input channels <= 256): never splits, needs no workspace.
bool polyrw_supported(const Problem& p);
hipError_t launch_polyrw(const Problem& p, const void* x, const void* pw, const void* bias,
                         void* y, bool out_f32, hipStream_t s);
hipError_t launch_polyphase(const Problem& p, const void* x, const void* pw, const void* bias,
                            void* y, void* ws, size_t ws_bytes, hipStream_t s);
// The tiled kernel with fp32 outputs and no bias or activation, for 16-bit
// 1-D shapes (the conv part of a stream step); false / hipErrorInvalidValue
// where its plan would shift padding by phase class, reduce a dilation or
// split the reduction.
bool polyphase_f32out_supported(const Problem& p);
hipError_t launch_polyphase_f32out(const Problem& p, const void* x, const void* pw, float* y,
                                   hipStream_t s);

}  // namespace ctconv

// Gather-form transposed convolution: the route for the shapes the polyphase
// kernels do not take (more taps per phase than any compiled instance, 2-D
// tiles that cannot hold every phase, rows shorter than one 8-byte load).
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
// Staged kernel (every shape within its staging limits).  Which taps reach an
// output depends only on its row oy and on ox mod sW: the outputs
// ox = sW*ax + bx of one row and one column phase bx share the tap set, and
// tap tx reads input column ax + c_tx with c_tx = (bx + pW - tx*dW) / sW.  A
// workgroup takes 64 such outputs (consecutive ax) for 32 output channels,
// for each column phase in turn.
// Per 32-channel chunk of C_in and per valid tap row it stages in LDS, as
// fp32, the x row segment all its taps read (zeros outside the input) and
// the weights of its valid taps, then every lane accumulates 32 output
// channels for one output over a quarter of the chunk's channels; the four
// quarters (lanes 16 apart) are summed with cross-lane shuffles at the end --
// the reduction over C_in is spread over the wavefront.  The epilogue adds
// the bias, applies the activation and rounds once (or writes fp32 when
// asked).
//
// General kernel (shapes past the staging limits: more than 8 valid taps
// per row or a tap reach wider than 64 input columns): one output per lane,
// 8 output channels in registers, the whole reduction in the lane.

#include "ctconv_internal.h"

namespace ctconv {

namespace {

// ---------------------------------------------------------------------------
// staged kernel
// ---------------------------------------------------------------------------

constexpr int kGAx = 64;     // outputs (consecutive ax) per workgroup
constexpr int kGCo = 32;     // output channels per workgroup (in registers)
constexpr int kGKc = 32;     // input channels per staged chunk
constexpr int kGTx = 8;      // valid column taps per row, at most
constexpr int kGMinTiles = 64;   // tiles below which the per-lane kernel runs instead
constexpr int kGXw = 128;    // staged x columns: kGAx + the taps' reach
constexpr int kGQ = 4;       // lanes sharing one output (quarters of a chunk)

struct GArgs {
    const void* x;
    const void* pw;
    const void* bias;
    void* y;
    int64_t N, C_in, C_out, C_in_pad, H, W, Ho, Wo;
    int kH, kW, sH, sW, pH, pW, dH, dW, mW, T;  // T: packed taps per phase
    int n_axb, n_cob;                           // ax blocks, channel blocks
    int64_t tiles;
    int act;
};

__device__ inline int floor_div(int a, int b) {
    const int q = a / b;
    return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

template <class TR, bool OUTF>
__global__ __launch_bounds__(256) void gather_staged_kernel(const GArgs a) {
    using S = typename TR::storage;
    __shared__ __attribute__((aligned(16))) float xs[kGKc * kGXw];
    __shared__ __attribute__((aligned(16))) float ws[kGTx * kGKc * kGCo];
    __shared__ int tcs[kGTx];   // c_tx of the valid column taps
    __shared__ int tws[kGTx];   // packed (phase, tap) weight offset base of each

    const S* __restrict__ xg = static_cast<const S*>(a.x);
    const S* __restrict__ pwg = static_cast<const S*>(a.pw);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int pos = wave * 16 + (lane & 15);  // output within the tile
    const int kq = lane >> 4;                 // quarter of the chunk's channels

    // Tiles of consecutive workgroups of one XCD (dispatched round robin over
    // the 8 XCDs) are consecutive, and a tile runs every column phase of its
    // outputs itself: the sW interleaved phases of an output row segment are
    // written by one workgroup close together in time, so its cache lines
    // are completed in one L2 before they go to memory.
    const int64_t wgid = (gridDim.x % 8u == 0)
                             ? (int64_t)(blockIdx.x % 8u) * (gridDim.x / 8u) + blockIdx.x / 8u
                             : (int64_t)blockIdx.x;
    for (int64_t tile = wgid; tile < a.tiles; tile += gridDim.x)
    for (int bx = 0; bx < a.sW; ++bx) {
        __syncthreads();  // the previous step's reads of tcs, xs and ws are done
        // tile = ((n * n_cob + cob) * Ho + oy) * n_axb + axb
        int64_t r = tile;
        const int axb = (int)(r % a.n_axb);
        r /= a.n_axb;
        const int oy = (int)(r % a.Ho);
        r /= a.Ho;
        const int cob = (int)(r % a.n_cob);
        const int64_t n = r / a.n_cob;
        const int ax0 = axb * kGAx, co0 = cob * kGCo;

        // valid column taps of this column phase and their input offsets
        int nvt = 0, cmin = 0, xw = 0;
        {
            int cm = 1 << 30, cx = -(1 << 30);
            for (int tx = 0; tx < a.kW; ++tx) {
                const int nx = bx + a.pW - tx * a.dW;
                if (((nx % a.sW) + a.sW) % a.sW != 0) continue;
                const int c = floor_div(nx, a.sW);
                if (tid == 0 && nvt < kGTx) tcs[nvt] = c;  // (the planner bounds nvt)
                cm = c < cm ? c : cm;
                cx = c > cx ? c : cx;
                ++nvt;
            }
            cmin = nvt > 0 ? cm : 0;
            xw = nvt > 0 ? kGAx + cx - cm : 0;  // staged columns actually read
        }

        float acc[kGCo];
#pragma unroll
        for (int c = 0; c < kGCo; ++c) acc[c] = 0.f;

        for (int ty = 0; ty < a.kH && nvt > 0; ++ty) {
            const int ny = oy + a.pH - ty * a.dH;
            if (ny < 0 || ny % a.sH != 0 || ny / a.sH >= a.H) continue;
            const int iy = ny / a.sH;
            for (int64_t c0 = 0; c0 < a.C_in; c0 += kGKc) {
                __syncthreads();  // the previous step's LDS reads are done
                if (tid < kGTx) {
                    // packed weight offset of (tap ty, valid column tap tid) at
                    // channel block 0, channel 0 of output channel 0
                    int t = 0, k = 0;
                    for (int tx = 0; tx < a.kW; ++tx) {
                        const int nx = bx + a.pW - tx * a.dW;
                        if (((nx % a.sW) + a.sW) % a.sW != 0) continue;
                        if (k == tid) {
                            const int j = (ty % a.sH) * a.sW + (tx % a.sW);
                            const int rr = (ty / a.sH) * a.mW + (tx / a.sW);
                            t = (int)((int64_t)j * (a.C_in_pad / kCinAlign) * a.C_out * a.T + rr) *
                                kCinAlign;
                        }
                        ++k;
                    }
                    tws[tid] = t;
                }
                // x segment: channels c0 .. c0+31, columns ax0 + cmin + [0, kGXw)
                const S* xrow = xg + (n * a.C_in * a.H + iy) * a.W;
                for (int e = tid; e < kGKc * xw; e += 256) {
                    const int ci = e / xw, xc = e - ci * xw;
                    const int64_t cg = c0 + ci;
                    const int64_t ix = (int64_t)ax0 + cmin + xc;
                    float v = 0.f;
                    if (cg < a.C_in && ix >= 0 && ix < a.W) v = TR::to_f32(xrow[cg * a.H * a.W + ix]);
                    xs[ci * kGXw + xc] = v;
                }
                __syncthreads();  // tws ready
                // weights [valid tap][ci][co] of this chunk
                const int64_t cblk = (c0 / kCinAlign) * a.C_out * a.T * kCinAlign;
                for (int e = tid; e < nvt * kGKc * kGCo; e += 256) {
                    const int ci = e % kGKc, co = (e / kGKc) % kGCo, vt = e / (kGKc * kGCo);
                    const int64_t cg = c0 + ci, cog = co0 + co;
                    float v = 0.f;
                    if (cg < a.C_in && cog < a.C_out)
                        v = TR::to_f32(pwg[tws[vt] + cblk + cog * a.T * kCinAlign + (cg % kCinAlign)]);
                    ws[(vt * kGKc + ci) * kGCo + co] = v;
                }
                __syncthreads();
                for (int vt = 0; vt < nvt; ++vt) {
                    const float* xr = xs + (tcs[vt] - cmin) + pos;
                    const float* wr = ws + vt * kGKc * kGCo;
#pragma unroll
                    for (int i = 0; i < kGKc / kGQ; ++i) {
                        const int ci = kq + kGQ * i;
                        const float xv = xr[ci * kGXw];
                        const float4* w4 = reinterpret_cast<const float4*>(wr + ci * kGCo);
#pragma unroll
                        for (int q = 0; q < kGCo / 4; ++q) {
                            const float4 w = w4[q];
                            acc[4 * q + 0] = fmaf(xv, w.x, acc[4 * q + 0]);
                            acc[4 * q + 1] = fmaf(xv, w.y, acc[4 * q + 1]);
                            acc[4 * q + 2] = fmaf(xv, w.z, acc[4 * q + 2]);
                            acc[4 * q + 3] = fmaf(xv, w.w, acc[4 * q + 3]);
                        }
                    }
                }
            }
        }
        // sum the four quarters (lanes 16 and 32 apart); each then holds the
        // total and writes a quarter of the channels
#pragma unroll
        for (int c = 0; c < kGCo; ++c) {
            acc[c] += __shfl_xor(acc[c], 16, 64);
            acc[c] += __shfl_xor(acc[c], 32, 64);
        }
        const int64_t ox = (int64_t)a.sW * (ax0 + pos) + bx;
        if (ax0 + pos < (a.Wo + a.sW - 1) / a.sW && ox < a.Wo) {
#pragma unroll
            for (int c = 0; c < kGCo; ++c) {
                if (c / (kGCo / kGQ) != kq) continue;
                const int64_t co = co0 + c;
                if (co >= a.C_out) continue;
                float v = acc[c];
                if (a.bias) v += TR::to_f32(static_cast<const S*>(a.bias)[co]);
                if (a.act == CTCONV_ACT_ELU) v = elu_act<TR>(v);
                const int64_t o = ((n * a.C_out + co) * a.Ho + oy) * a.Wo + ox;
                if constexpr (OUTF)
                    static_cast<float*>(a.y)[o] = v;
                else
                    static_cast<S*>(a.y)[o] = TR::from_f32(v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// general kernel
// ---------------------------------------------------------------------------

constexpr int kCoT = 8;

template <class TR, bool OUTF>
__global__ __launch_bounds__(256) void gather_kernel(
    const typename TR::storage* __restrict__ x, const typename TR::storage* __restrict__ pw,
    const typename TR::storage* __restrict__ bias, void* __restrict__ y, int64_t total,
    int64_t C_in, int64_t C_out, int64_t C_in_pad, int64_t H, int64_t W, int64_t Ho, int64_t Wo,
    int64_t Wq, int64_t n_cot, int64_t kH, int64_t kW, int64_t sH, int64_t sW, int64_t pH,
    int64_t pW, int64_t dH, int64_t dW, int64_t mW, int64_t T, int act) {
    for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < total;
         id += (int64_t)gridDim.x * blockDim.x) {
        // consecutive lanes: consecutive outputs of one column phase of a row
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
                const int64_t o = ((n * C_out + co) * Ho + oy) * Wo + ox;
                if constexpr (OUTF)
                    static_cast<float*>(y)[o] = v;
                else
                    static_cast<typename TR::storage*>(y)[o] = TR::from_f32(v);
            }
        }
    }
}

int64_t gcd_i(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

template <class TR, bool OUTF>
hipError_t launch_gather_t(const Problem& p, const void* x, const void* pw, const void* bias,
                           void* y, hipStream_t s) {
    using S = typename TR::storage;
    // The staged kernel keeps a workgroup on one tile through every phase,
    // tap and channel chunk: with very few tiles (small problems, such as
    // the frames of a stream: eight tiles per layer) that chain runs on a
    // few workgroups, and the per-lane kernel's spread over many lanes wins.
    const int64_t n_tiles = p.N * ((p.C_out + kGCo - 1) / kGCo) * p.Ho *
                            (((p.Wo + p.sW - 1) / p.sW + kGAx - 1) / kGAx);
    if (gather_staged_ok(p) && n_tiles >= kGMinTiles) {
        GArgs a{};
        a.x = x;
        a.pw = pw;
        a.bias = bias;
        a.y = y;
        a.N = p.N;
        a.C_in = p.C_in;
        a.C_out = p.C_out;
        a.C_in_pad = p.C_in_pad;
        a.H = p.H;
        a.W = p.W;
        a.Ho = p.Ho;
        a.Wo = p.Wo;
        a.kH = (int)p.kH;
        a.kW = (int)p.kW;
        a.sH = (int)p.sH;
        a.sW = (int)p.sW;
        a.pH = (int)p.pH;
        a.pW = (int)p.pW;
        a.dH = (int)p.dH;
        a.dW = (int)p.dW;
        a.mW = (int)p.mW;
        a.T = (int)p.T;
        const int64_t Aq = (p.Wo + p.sW - 1) / p.sW;
        a.n_axb = (int)((Aq + kGAx - 1) / kGAx);
        a.n_cob = (int)((p.C_out + kGCo - 1) / kGCo);
        a.tiles = p.N * a.n_cob * p.Ho * a.n_axb;
        a.act = p.act;
        int64_t blocks = a.tiles;
        if (blocks > 256 * 64) blocks = 256 * 64;
        if (blocks >= 64) blocks = blocks / 8 * 8;  // (the XCD-contiguous tile order)
        gather_staged_kernel<TR, OUTF><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
        return hipGetLastError();
    }
    const int64_t Wq = (p.Wo + p.sW - 1) / p.sW;
    const int64_t n_cot = (p.C_out + kCoT - 1) / kCoT;
    const int64_t total = p.N * n_cot * p.Ho * p.sW * Wq;
    int64_t blocks = (total + 255) / 256;
    if (blocks > (int64_t)1 << 20) blocks = (int64_t)1 << 20;
    if (blocks < 1) blocks = 1;
    gather_kernel<TR, OUTF><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<const S*>(x), static_cast<const S*>(pw), static_cast<const S*>(bias), y, total,
        p.C_in, p.C_out, p.C_in_pad, p.H, p.W, p.Ho, p.Wo, Wq, n_cot, p.kH, p.kW, p.sH, p.sW, p.pH,
        p.pW, p.dH, p.dW, p.mW, p.T, p.act);
    return hipGetLastError();
}

}  // namespace

// The staged kernel's limits: at most kGTx valid column taps per column
// phase (ceil(kW / (sW / gcd(sW, dW)))), their input columns within
// kGXw - kGAx of each other, and int-sized indices.
bool gather_staged_ok(const Problem& p) {
    const int64_t sx = p.sW / gcd_i(p.sW, p.dW);
    const int64_t nvt = (p.kW + sx - 1) / sx;
    const int64_t reach = ((p.kW - 1) * p.dW) / p.sW + 1;
    return nvt <= kGTx && reach <= kGXw - kGAx && p.Ho < ((int64_t)1 << 30) &&
           p.Wo < ((int64_t)1 << 30) && p.kH < 65536 && p.kW < 65536 && p.sH < 65536 &&
           p.sW < 65536 && p.pH < ((int64_t)1 << 30) && p.pW < ((int64_t)1 << 30) &&
           p.dH < 65536 && p.dW < 65536 &&
           p.P * (p.C_in_pad / kCinAlign) * p.C_out * p.T * kCinAlign < ((int64_t)1 << 31);
}

hipError_t launch_gather(const Problem& p, const void* x, const void* pw, const void* bias,
                         void* y, bool out_f32, hipStream_t s) {
    switch (p.dtype) {
        case CTCONV_F32:
            return launch_gather_t<TF32, false>(p, x, pw, bias, y, s);
        case CTCONV_BF16:
            return out_f32 ? launch_gather_t<TBF16, true>(p, x, pw, bias, y, s)
                           : launch_gather_t<TBF16, false>(p, x, pw, bias, y, s);
        case CTCONV_F16:
            return out_f32 ? launch_gather_t<TF16, true>(p, x, pw, bias, y, s)
                           : launch_gather_t<TF16, false>(p, x, pw, bias, y, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ctconv

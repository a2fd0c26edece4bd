// Polyphase transposed convolution as an implicit GEMM on the gfx950 MFMA
// matrix cores.
//
// Method.  For k = m*s (per dimension), d = 1 and output_padding 0, a
// transposed convolution is one stride-1 convolution with m taps that yields
// every output phase, followed by an interleave of the phases and a slice of
// the padding (ExecuTorch PR #25037, "[XNNPACK] Lower dense transposed convs
// as one polyphase conv + depth to space", Summary formula
// y[s*q + j] = sum_{u<m} x[q + u - (m-1)] * w[s*(m-1-u) + j]).
//
// Output-aligned phases.  Writing each output index as o = s*a + b (b the
// output phase) and j_b = (b + p) mod s, delta_b = floor((b + p) / s), the
// same identity reads
//     y[s*a + b] = sum_{r<m} sum_ci x[ci, a + delta_b - r] * w[ci, co, s*r + j_b]
// (r = m-1-u).  Indexing GEMM rows by a instead of q folds the padding slice
// into the row range: every GEMM row lands inside the output and nothing is
// computed to be discarded.  The per-phase shift delta_b generalises the
// page's asymmetric per-phase zero pad (same PR, commit "Decompose depthwise
// transposed convs").  In 2-D everything holds per dimension and phases are
// b = by*sx + bx (block-major depth-to-space order of the same page).
//
// GEMM.  Rows (n, ay, ax), columns (b, co), reduction (r, ci):
//     C[(n,ay,ax)][(b,co)] += X[ci][ay + dy_b - ry][ax + dx_b - rx] * B[(j_b,co)][(ry,rx,ci)]
// with B the phase-major packed weight.  One workgroup computes a BM x BN tile
// (4 waves, each RB x CB blocks of 16x16).  Per chunk of KC input channels:
//   * x window: the tile's output rows plus an (m-1) halo (plus one row when
//     delta_b differs between phases), staged in LDS as rows of KC contiguous
//     channels.  Global x is NCL/NCHW (contiguous along the spatial axis), so
//     each thread loads VEC channels of one spatial position (coalesced across
//     lanes along the spatial axis) and writes them as one 16-byte LDS vector:
//     the transpose to the MFMA operand order (channels contiguous per lane)
//     happens on the way into LDS and activations are never transposed in HBM.
//     All m taps reuse the same window at different row offsets.
//   * B: for every column, the m taps' KC-channel runs (16-byte loads from the
//     packed weight, contiguous in ci).
//   * MFMA: bf16/fp16 use v_mfma_f32_16x16x32 (8 channels per lane), fp32
//     uses v_mfma_f32_16x16x4_f32 (true fp32 products) four times per 16-byte
//     fragment.  A fragments are loaded once per distinct window offset and
//     reused by every column block and tap that needs that offset.
//   * two LDS stages; the next chunk's global loads are issued before the
//     current chunk's MFMAs.
// Epilogue: + bias, one rounding to the output type, staged in LDS in output
// order so that each tile writes contiguous runs of y (the phase interleave
// and the padding slice cost nothing beyond address arithmetic).  Shapes with
// few tiles split the C_in reduction across workgroups (fp32 output only) and
// accumulate with fp32 atomics into a bias-filled y.

#include "ctconv_internal.h"

namespace ctconv {

namespace {

template <class TR>
struct Mma;

template <>
struct Mma<TBF16> {
    __device__ static inline void step(f32x4& acc, const uint4& a, const uint4& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

template <>
struct Mma<TF16> {
    __device__ static inline void step(f32x4& acc, const uint4& a, const uint4& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    }
};

template <>
struct Mma<TF32> {
    // Lane group g holds channels 4g..4g+3 of the 16-channel step in one
    // 16-byte fragment; MFMA number e consumes element e of every group, so
    // the four MFMAs together reduce over all 16 channels.
    __device__ static inline void step(f32x4& acc, const uint4& a, const uint4& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x),
                                                   acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y),
                                                   acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z),
                                                   acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w),
                                                   acc, 0, 0, 0);
    }
};

template <class TR, int MY, int MX, int TAX, int RB, int CB, int WM, int WN, int KS>
struct Cfg {
    using S = typename TR::storage;
    static constexpr int ES = sizeof(S);
    static constexpr int VEC = 16 / ES;     // elements per 16-byte fragment
    static constexpr int KSTEP = 4 * VEC;   // channels per MFMA k-step
    static constexpr int KC = KSTEP * KS;   // channels per LDS stage
    static constexpr int RSA = KC + VEC;    // LDS row stride (16-byte pad: odd multiple of 16 B)
    static constexpr int BM = WM * RB * 16;
    static constexpr int BN = WN * CB * 16;
    static constexpr int TAY = BM / TAX;
    static constexpr int T = MY * MX;
    static constexpr int WYM = TAY + MY - 1 + (TAY > 1 ? 1 : 0);
    static constexpr int WXM = TAX + MX;
    static constexpr int XROWS = WYM * WXM;
    static constexpr int BROWS = T * BN;
    static constexpr int STAGE = (XROWS + BROWS) * RSA;
    static constexpr int NG = KC / VEC;
    static constexpr int XITEMS = (XROWS * NG + 255) / 256;
    static constexpr int BITEMS = (BROWS * NG + 255) / 256;
    static constexpr int SMEM = (2 * STAGE > BM * BN ? 2 * STAGE : BM * BN);
    static_assert(BM % TAX == 0 && TAX % 16 == 0, "tile rows");
    static_assert(WM * WN == 4, "four waves");
    static_assert(SMEM * ES <= 160 * 1024, "LDS");
};

template <class TR, int MY, int MX, int TAX, int RB, int CB, int WM, int WN, int KS>
__global__ __launch_bounds__(256) void poly_kernel(const PolyArgs a) {
    using C = Cfg<TR, MY, MX, TAX, RB, CB, WM, WN, KS>;
    using S = typename TR::storage;
    constexpr int VEC = C::VEC, KC = C::KC, RSA = C::RSA, BN = C::BN, T = C::T;
    constexpr int NG = C::NG;

    __shared__ __attribute__((aligned(16))) S smem[C::SMEM];

    const S* __restrict__ xg = static_cast<const S*>(a.x);
    const S* __restrict__ pwg = static_cast<const S*>(a.pw);

    // ---- tile coordinates -------------------------------------------------
    int64_t bid = blockIdx.x;
    if (a.xcd_remap) {
        const int64_t per = gridDim.x / 8;
        bid = (bid % 8) * per + bid / 8;
    }
    const int col_tile = (int)(bid % a.n_col_tiles);
    const int64_t row_tile = bid / a.n_col_tiles;
    const int tx_t = (int)(row_tile % a.tiles_x);
    const int64_t rt2 = row_tile / a.tiles_x;
    const int ty_t = (int)(rt2 % a.tiles_y);
    const int64_t n = rt2 / a.tiles_y;
    const int co0 = (col_tile / a.n_ph_tiles) * a.TCO;
    const int b0 = (col_tile % a.n_ph_tiles) * a.PT;
    const int ay0 = ty_t * C::TAY, ax0 = tx_t * TAX;
    const int64_t wy0 = (int64_t)ay0 + a.dminy - (MY - 1);
    const int64_t wx0 = (int64_t)ax0 + a.dminx - (MX - 1);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 15, lg = lane >> 4;

    // ---- per-thread load descriptors (fixed across chunks) ----------------
    const int64_t HW = a.H * a.W;
    const int npos = a.WY * a.WX;
    const int xitems = npos * NG;
    int64_t xsp[C::XITEMS];   // spatial offset, -1 when outside the input
    int xch[C::XITEMS];       // channel offset of the group within a chunk
    int xlds[C::XITEMS];      // LDS element offset (-1: no item)
#pragma unroll
    for (int it = 0; it < C::XITEMS; ++it) {
        const int q = tid + 256 * it;
        xlds[it] = -1;
        xsp[it] = -1;
        xch[it] = 0;
        if (q < xitems) {
            const int pos = q % npos, g = q / npos;
            const int64_t iy = wy0 + pos / a.WX, ix = wx0 + pos % a.WX;
            if (iy >= 0 && iy < a.H && ix >= 0 && ix < a.W) xsp[it] = iy * a.W + ix;
            xch[it] = g * VEC;
            xlds[it] = pos * RSA + g * VEC;
        }
    }
    const S* xn = xg + n * a.C_in * HW;

    int64_t boff[C::BITEMS];  // packed-weight element offset, -1 for a zero row
    int blds[C::BITEMS];
#pragma unroll
    for (int it = 0; it < C::BITEMS; ++it) {
        const int q = tid + 256 * it;
        boff[it] = -1;
        blds[it] = -1;
        if (q < C::BROWS * NG) {
            const int row = q / NG, piece = q % NG;
            const int r = row / BN, tc = row % BN;
            const int pb = tc / a.TCO, co = co0 + tc % a.TCO, b = b0 + pb;
            if (pb < a.PT && b < a.P && co < a.C_out) {
                const int by = b / a.sx, bx = b % a.sx;
                const int j = ((by + a.py) % a.sy) * a.sx + (bx + a.px) % a.sx;
                boff[it] = (((int64_t)j * a.C_out + co) * T + r) * a.C_in_pad + piece * VEC;
            }
            blds[it] = (r * BN + tc) * RSA + piece * VEC;
        }
    }

    // ---- per-wave column-block phase shifts -------------------------------
    int ddy[CB], ddx[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int tc0 = (wn * CB + cb) * 16;
        const int pb = tc0 / a.TCO, b = b0 + pb;
        ddy[cb] = 0;
        ddx[cb] = 0;
        if (pb < a.PT && b < a.P) {
            const int by = b / a.sx, bx = b % a.sx;
            ddy[cb] = (by + a.py) / a.sy - a.dminy;
            ddx[cb] = (bx + a.px) / a.sx - a.dminx;
        }
    }

    uint4 xr[C::XITEMS];
    uint4 br[C::BITEMS];

    auto gload = [&](int c) {
        const int cbase = c * KC;
#pragma unroll
        for (int it = 0; it < C::XITEMS; ++it) {
            S v[VEC];
            const int ch = cbase + xch[it];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                v[e] = S(0);
                if (xsp[it] >= 0 && ch + e < a.C_in) v[e] = xn[(int64_t)(ch + e) * HW + xsp[it]];
            }
            xr[it] = *reinterpret_cast<const uint4*>(v);
        }
#pragma unroll
        for (int it = 0; it < C::BITEMS; ++it) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (boff[it] >= 0) v = *reinterpret_cast<const uint4*>(pwg + boff[it] + cbase);
            br[it] = v;
        }
    };

    auto lstore = [&](int st) {
        S* xs = smem + st * C::STAGE;
        S* bs = xs + C::XROWS * RSA;
#pragma unroll
        for (int it = 0; it < C::XITEMS; ++it)
            if (xlds[it] >= 0) *reinterpret_cast<uint4*>(xs + xlds[it]) = xr[it];
#pragma unroll
        for (int it = 0; it < C::BITEMS; ++it)
            if (blds[it] >= 0) *reinterpret_cast<uint4*>(bs + blds[it]) = br[it];
    };

    f32x4 acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A-fragment window rows of this wave's row blocks (without the shift)
    int arow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int tr0 = (wm * RB + rb) * 16;
        arow[rb] = (tr0 / TAX) * a.WX + (tr0 % TAX) + li;
    }

    auto compute = [&](int st) {
        const S* xs = smem + st * C::STAGE;
        const S* bs = xs + C::XROWS * RSA;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kofs = ks * C::KSTEP + lg * VEC;
            uint4 bfr[CB][T];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < T; ++r)
                    bfr[cb][r] = *reinterpret_cast<const uint4*>(
                        bs + (r * BN + (wn * CB + cb) * 16 + li) * RSA + kofs);
#pragma unroll
            for (int ey = 0; ey <= MY; ++ey) {
                if (ey == MY && !a.spready) continue;
#pragma unroll
                for (int ex = 0; ex <= MX; ++ex) {
                    if (ex == MX && !a.spreadx) continue;
                    uint4 afr[RB];
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        afr[rb] = *reinterpret_cast<const uint4*>(
                            xs + (arow[rb] + ey * a.WX + ex) * RSA + kofs);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const int ry = ddy[cb] + MY - 1 - ey;
                        const int rx = ddx[cb] + MX - 1 - ex;
#pragma unroll
                        for (int ryc = 0; ryc < MY; ++ryc)
#pragma unroll
                            for (int rxc = 0; rxc < MX; ++rxc)
                                if (ryc == ry && rxc == rx) {
#pragma unroll
                                    for (int rb = 0; rb < RB; ++rb)
                                        Mma<TR>::step(acc[rb][cb], afr[rb], bfr[cb][ryc * MX + rxc]);
                                }
                    }
                }
            }
        }
    };

    // ---- main loop over input-channel chunks -------------------------------
    const int c_begin = blockIdx.y * a.chunks_per_split;
    const int c_end = min(c_begin + a.chunks_per_split, a.n_chunks);
    if (c_begin < c_end) {
        gload(c_begin);
        lstore(0);
        __syncthreads();
        for (int c = c_begin; c < c_end; ++c) {
            const int st = (c - c_begin) & 1;
            if (c + 1 < c_end) gload(c + 1);
            compute(st);
            if (c + 1 < c_end) lstore(st ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: bias, round, stage in output order, store ---------------
    const S* __restrict__ biasg = static_cast<const S*>(a.bias);
    const int R = a.phase_subset ? TAX : C::TAY * a.sy;
    const int SS = a.phase_subset ? a.PT : TAX * a.sx;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int tc = (wn * CB + cb) * 16 + li;
            const int pb = tc / a.TCO, co_l = tc % a.TCO;
            if (pb >= a.PT) continue;
            const int co = co0 + co_l;
            float bv = 0.f;
            if (!a.atomic_out && biasg != nullptr && co < a.C_out) bv = TR::to_f32(biasg[co]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = (wm * RB + rb) * 16 + lg * 4 + i;
                const int ayl = tr / TAX, axl = tr % TAX;
                int rr, ss;
                if (a.phase_subset) {
                    rr = axl;
                    ss = pb;
                } else {
                    rr = ayl * a.sy + pb / a.sx;
                    ss = axl * a.sx + pb % a.sx;
                }
                smem[(co_l * R + rr) * SS + ss] = TR::from_f32(acc[rb][cb][i] + bv);
            }
        }
    __syncthreads();

    S* __restrict__ yg = static_cast<S*>(a.y);
    const int total = a.TCO * R * SS;
    for (int e = tid; e < total; e += 256) {
        const int ss = e % SS;
        const int rr = (e / SS) % R;
        const int co = co0 + e / (SS * R);
        if (co >= a.C_out) continue;
        int64_t oy, ox;
        if (a.phase_subset) {
            const int b = b0 + ss;
            if (b >= a.P) continue;
            oy = 0;
            ox = (int64_t)(ax0 + rr) * a.sx + b;
        } else {
            oy = (int64_t)ay0 * a.sy + rr;
            ox = (int64_t)ax0 * a.sx + ss;
        }
        if (oy >= a.Ho || ox >= a.Wo) continue;
        const int64_t idx = ((n * a.C_out + co) * a.Ho + oy) * a.Wo + ox;
        if (a.atomic_out)
            atomicAdd(reinterpret_cast<float*>(yg) + idx, TR::to_f32(smem[e]));
        else
            yg[idx] = smem[e];
    }
}

// ---------------------------------------------------------------------------
// Host-side planning
// ---------------------------------------------------------------------------

using KernelFn = void (*)(const PolyArgs);

struct Inst {
    KernelFn fn;
    int BM, BN, TAX, TAY, KC, lds_bytes;
};

template <class TR, int MY, int MX, int TAX, int CB>
Inst make_inst() {
    using C = Cfg<TR, MY, MX, TAX, 4, CB, 2, 2, 1>;
    return Inst{&poly_kernel<TR, MY, MX, TAX, 4, CB, 2, 2, 1>, C::BM, C::BN, TAX, C::TAY, C::KC,
                (int)(C::SMEM * C::ES)};
}

template <class TR>
bool pick_inst(const Problem& p, int CB, Inst* out) {
    if (p.ndim == 1) {
        if (CB == 5) {
            switch (p.mW) {
                case 1: *out = make_inst<TR, 1, 1, 128, 5>(); return true;
                case 2: *out = make_inst<TR, 1, 2, 128, 5>(); return true;
                case 3: *out = make_inst<TR, 1, 3, 128, 5>(); return true;
                case 4: *out = make_inst<TR, 1, 4, 128, 5>(); return true;
            }
            return false;
        }
        switch (p.mW) {
            case 1: *out = make_inst<TR, 1, 1, 128, 4>(); return true;
            case 2: *out = make_inst<TR, 1, 2, 128, 4>(); return true;
            case 3: *out = make_inst<TR, 1, 3, 128, 4>(); return true;
            case 4: *out = make_inst<TR, 1, 4, 128, 4>(); return true;
        }
        return false;
    }
    if (CB != 4) return false;
    if (p.mH == 1 && p.mW == 1) { *out = make_inst<TR, 1, 1, 32, 4>(); return true; }
    if (p.mH == 1 && p.mW == 2) { *out = make_inst<TR, 1, 2, 32, 4>(); return true; }
    if (p.mH == 2 && p.mW == 1) { *out = make_inst<TR, 2, 1, 32, 4>(); return true; }
    if (p.mH == 2 && p.mW == 2) { *out = make_inst<TR, 2, 2, 32, 4>(); return true; }
    return false;
}

bool get_inst(const Problem& p, int CB, Inst* out) {
    switch (p.dtype) {
        case CTCONV_F32: return pick_inst<TF32>(p, CB, out);
        case CTCONV_BF16: return pick_inst<TBF16>(p, CB, out);
        case CTCONV_F16: return pick_inst<TF16>(p, CB, out);
    }
    return false;
}

constexpr int64_t kInt32Max = 2147483647;

// Fill PolyArgs for problem p; false when no kernel instance covers it.
bool plan(const Problem& p, PolyArgs* a, Inst* inst, int* splits) {
    if (p.kH % p.sH || p.kW % p.sW || p.dH != 1 || p.dW != 1 || p.opH || p.opW) return false;
    if (p.H == 0 || p.W == 0 || p.N == 0) return false;
    const int64_t P = p.P;
    const bool spread_y = (p.pH % p.sH) != 0, spread_x = (p.pW % p.sW) != 0;
    const bool mixed_ok = !spread_y && !spread_x;  // delta_b is the same for every phase

    // Column tiling: TCO output channels x PT phases per tile.
    int CB = (P % 5 == 0 && P * 16 <= 160) ? 5 : 4;
    Inst in;
    if (!get_inst(p, CB, &in)) return false;
    const int64_t BN = in.BN;
    int64_t TCO, PT;
    int subset = 0;
    const bool narrow = (p.C_out < 16) && mixed_ok;  // blocks may span phases
    const int64_t tco_min = narrow ? p.C_out : 16;
    if (P * tco_min <= BN) {
        PT = P;
        if (narrow) {
            TCO = p.C_out;
        } else {
            TCO = (BN / P) / 16 * 16;
            const int64_t cpad = (p.C_out + 15) / 16 * 16;
            if (TCO > cpad) TCO = cpad;
        }
    } else {
        if (p.ndim != 1) return false;
        subset = 1;
        TCO = tco_min;
        PT = BN / TCO;
        if (!narrow) PT = PT / 1;  // 16-channel blocks, one phase each
    }
    if (TCO < 1 || PT < 1) return false;
    const int64_t n_co_tiles = (p.C_out + TCO - 1) / TCO;
    const int64_t n_ph_tiles = (P + PT - 1) / PT;
    const int64_t Ay = (p.Ho + p.sH - 1) / p.sH, Ax = (p.Wo + p.sW - 1) / p.sW;
    const int64_t tiles_y = (Ay + in.TAY - 1) / in.TAY, tiles_x = (Ax + in.TAX - 1) / in.TAX;
    const int64_t n_row_tiles = p.N * tiles_y * tiles_x;
    const int64_t n_col_tiles = n_co_tiles * n_ph_tiles;
    const int64_t n_chunks = p.C_in_pad / in.KC;
    if (n_row_tiles * n_col_tiles > kInt32Max || P > kInt32Max / 2 || p.C_out > kInt32Max / 2 ||
        Ax > kInt32Max / 2 || Ay > kInt32Max / 2 || n_chunks > kInt32Max)
        return false;

    a->N = p.N;
    a->C_in = p.C_in;
    a->C_out = p.C_out;
    a->C_in_pad = p.C_in_pad;
    a->H = p.H;
    a->W = p.W;
    a->Ho = p.Ho;
    a->Wo = p.Wo;
    a->sy = (int)p.sH;
    a->sx = (int)p.sW;
    a->py = (int)p.pH;
    a->px = (int)p.pW;
    a->P = (int)P;
    a->T = (int)p.T;
    a->Ay = (int)Ay;
    a->Ax = (int)Ax;
    a->dminy = (int)(p.pH / p.sH);
    a->dminx = (int)(p.pW / p.sW);
    a->spready = spread_y ? 1 : 0;
    a->spreadx = spread_x ? 1 : 0;
    a->WY = in.TAY + (int)p.mH - 1 + a->spready;
    a->WX = in.TAX + (int)p.mW - 1 + a->spreadx;
    a->TCO = (int)TCO;
    a->PT = (int)PT;
    a->phase_subset = subset;
    a->n_ph_tiles = (int)n_ph_tiles;
    a->n_col_tiles = (int)n_col_tiles;
    a->tiles_y = (int)tiles_y;
    a->tiles_x = (int)tiles_x;
    a->n_row_tiles = n_row_tiles;
    a->n_chunks = (int)n_chunks;

    // Split the C_in reduction when the tile grid leaves CUs idle (fp32 output
    // only: partial sums meet through fp32 atomics).  Choose the split that
    // minimises (rounds of workgroups) x (chunks per workgroup).
    const int64_t tiles = n_row_tiles * n_col_tiles;
    const int64_t per_cu = in.lds_bytes <= 80 * 1024 ? 2 : 1;
    const int64_t slots = 256 * per_cu;
    int best = 1;
    if (p.dtype == CTCONV_F32 && tiles < 2 * slots && n_chunks >= 8) {
        double best_cost = 1e300;
        for (int sp = 1; sp <= 64 && sp <= n_chunks; ++sp) {
            const int64_t cps = (n_chunks + sp - 1) / sp;
            const int64_t used = (n_chunks + cps - 1) / cps;
            const int64_t rounds = (tiles * used + slots - 1) / slots;
            const double cost = (double)rounds * (double)cps + 0.5 * used;  // mild split penalty
            if (cost < best_cost) {
                best_cost = cost;
                best = (int)used;
            }
        }
    }
    a->chunks_per_split = (int)((n_chunks + best - 1) / best);
    a->atomic_out = best > 1 ? 1 : 0;
    a->xcd_remap = (tiles % 8 == 0) ? 1 : 0;
    *inst = in;
    *splits = best;
    return true;
}

}  // namespace

bool polyphase_supported(const Problem& p) {
    PolyArgs a{};
    Inst in{};
    int sp = 1;
    return plan(p, &a, &in, &sp);
}

hipError_t launch_polyphase(const Problem& p, const void* x, const void* pw, const void* bias,
                            void* y, hipStream_t s) {
    PolyArgs a{};
    Inst in{};
    int splits = 1;
    if (!plan(p, &a, &in, &splits)) return hipErrorInvalidValue;
    a.x = x;
    a.pw = pw;
    a.bias = bias;
    a.y = y;
    if (a.atomic_out) {
        const hipError_t e = launch_fill(p, bias, y, s);
        if (e != hipSuccess) return e;
    }
    const int64_t tiles = a.n_row_tiles * a.n_col_tiles;
    hipLaunchKernelGGL(in.fn, dim3((unsigned)tiles, (unsigned)splits), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ctconv

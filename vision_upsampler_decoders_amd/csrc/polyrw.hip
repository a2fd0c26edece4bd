// Polyphase transposed convolution with the weights held in registers: a
// streaming form of the polyphase implicit GEMM for 16-bit 1-D shapes whose
// reduction is short (taps per phase x input channels <= 256), such as the
// last layers of an audio upsampler stack (128 -> 64 channels, k = 2s).
//
// Method (ExecuTorch PR #25037, "[XNNPACK] Lower dense transposed convs as
// one polyphase conv + depth to space", Summary formula): with input-aligned
// phase positions q,
//     y[n, co, s*q + j - p] = sum_{r < m} sum_ci x[n, ci, q - r] * w[ci, co, s*r + j]
// for m = ceil(k / s) taps per phase (taps s*r + j >= k are zero in the
// packed weight) and x = 0 outside [0, L).  Outputs s*q + j - p outside
// [0, L_out) are not written: that is the padding slice.
//
// GEMM view (rows are the matrix cores' M dimension): rows (co, j) with the
// phase j fastest, columns q, reduction (r, ci).  Each wave owns 32 rows for
// the whole launch and keeps their weights -- every tap and input channel,
// at most 8 k-steps of 32 channels, 64 registers -- loaded once.  A
// persistent workgroup of 8 waves (256 rows) walks a contiguous run of
// 64-position column tiles: per tile it stages x's window (64 + m - 1
// positions, every input channel) in LDS as rows of channels (the transpose
// to the MFMA operand order happens on the way into LDS), and each wave runs
// v_mfma_f32_16x16x32 with A = its weights and B = x fragments read from
// LDS at the tap's row offset.
//
// Epilogue from registers: a lane of a 16x16 block holds rows 4*lg .. 4*lg+3
// of column li, i.e. (when s is a multiple of 4) phases j0 .. j0+3 of one
// output channel at one q -- four consecutive outputs s*q + j0 - p .. +3 --
// so every lane writes one 8-byte run and a wave's four stores of a row
// block cover 512 consecutive bytes of four output rows: no LDS staging.
//
// Pipeline per tile: the x loads of the tile after next are issued first
// (a scheduling barrier keeps the compiler from sinking them toward their
// use), then the MFMAs, then the next tile's x is moved from registers to
// the other LDS stage (its wait for those loads comes before this tile's
// stores: a wait for a load also waits for every memory operation issued
// before it), then the stores, then one barrier.

#include "ctconv_internal.h"
#include "mfma_common.h"

namespace ctconv {

namespace {

using namespace mfma;

constexpr int RW_BQ = 64;                       // q positions per tile
constexpr int RW_CB = RW_BQ / 16;               // column blocks per wave
constexpr int RW_KMAX = 8;                      // k-steps of 32 channels held per row block
constexpr int RW_NPMAX = 8;                     // positions per x load item (at most)
constexpr int RW_WPMAX = RW_BQ + RW_NPMAX;      // window positions

// Launch shape (measured on the 128 -> 64, k8 s4 vocoder layer against the
// other combinations): WAVES waves per workgroup, 32 rows each (8: one
// workgroup of 256 rows per CU, two waves per SIMD), NP positions per x load
// item (4: 8-byte loads), NBUF register buffers of x (2: the next tile's x
// waits in one while the tile after is loaded into the other).
constexpr int RW_WAVES = 8;
constexpr int RW_NP = 4;
constexpr int RW_ROWS = 32 * RW_WAVES;          // (co, j) rows per row group
constexpr int RW_LDS_MAX = 65536;               // dynamic LDS per workgroup (bytes, the default limit)
constexpr int RW_NBUF = 2;
constexpr int RW_THREADS = 64 * RW_WAVES;


struct RWArgs {
    const void* x;
    const void* pw;
    const void* bias;
    void* y;
    int Lo;             // output length
    int64_t n_tiles;    // N * tiles per image
    int L;              // input length
    int C_in, C_out, C_in_pad, ncb;  // ncb = C_in_pad / 32
    int s, p, T;        // stride, padding, taps per phase
    int KS;             // k-steps T * ncb (<= RW_KMAX)
    int tpi;            // tiles per image
    int rg, wg_per_rg;  // row groups (ceil(C_out * s / 256)), workgroups per row group
    int xofs, WP;       // window: start shift (positions) and length (multiple of 8)
    int RS;             // LDS row stride in elements (C_in_pad + 8)
    int stage;          // elements of one LDS x stage (WP * RS, a multiple of 8)
    uint32_t plane;     // bytes of one input channel (2 L)
    uint32_t img;       // bytes of one image (C_in * plane)
    uint32_t pw_bytes;
    FastDiv fd_tpi;     // division by tpi (tile indices < 2^31)
};

// Epilogue modes (compile time, so that neither the activation nor the
// output type costs a select per element): the storage type with no
// activation, the storage type after ELU, fp32 with no activation (a chunk
// of a stream, rounded later).
enum RWEpi { RW_PLAIN = 0, RW_ELU = 1, RW_F32 = 2 };

// KS: k-steps of 32 channels (taps x channel blocks), at most RW_KMAX
template <class TR, bool XODD, int KS, int WAVES, int NP, int NBUF, int EPI>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void polyrw_kernel(const RWArgs a) {
    constexpr int THREADS = 64 * WAVES;
    constexpr int RW_ROWS = 32 * WAVES;            // rows of a workgroup
    constexpr int RW_RB = 2;                       // 16-row blocks per wave
    // x load items per thread: the planner admits only windows whose
    // (WP / NP) position groups x (C_in_pad / 8) channel groups fit one each
    constexpr int RW_XI = 1;
    constexpr int RW_NP = NP;
    using S = typename TR::storage;
    static_assert(sizeof(S) == 2, "16-bit storage");
    // LDS (sized at launch): two x stages of a.stage elements
    extern __shared__ __attribute__((aligned(16))) S smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // workgroup -> (row group g, tile run kw).  Workgroups are dispatched
    // round robin over the 8 XCDs; with wg_per_rg a multiple of 8 the row
    // groups of one tile run share an XCD (blockIdx b and b + 8k), so x's
    // tile is fetched into that XCD's L2 once for all of them.
    int g, kw;
    if (a.wg_per_rg % 8 == 0) {
        const uint32_t b = blockIdx.x, slot = b / 8u;
        g = (int)(slot % (uint32_t)a.rg);
        kw = (int)(b % 8u + 8u * (slot / (uint32_t)a.rg));
    } else {
        g = (int)(blockIdx.x % (uint32_t)a.rg);
        kw = (int)(blockIdx.x / (uint32_t)a.rg);
    }
    // a contiguous run of tiles: consecutive tiles write adjacent output runs
    // (their shared cache lines meet in this CU's L2) and share x's halo
    const int64_t t_begin = (int64_t)kw * a.n_tiles / a.wg_per_rg;
    const int64_t t_end = (int64_t)(kw + 1) * a.n_tiles / a.wg_per_rg;
    if (t_begin >= t_end) return;  // whole workgroup

    // ---- weights of this wave's rows, every k-step, into registers --------
    // packed layout [j][ci / 32][co][r][ci % 32]; rows past C_out read zero
    // (an offset past the resource), as do taps past k (zero in the packing)
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(a.pw), (short)0, (int)uniform(a.pw_bytes), kBufferWord3);
    u32x4 wf[RW_RB][KS];
    float bv[RW_RB];
    int co_e[RW_RB], j0_e[RW_RB];
    {
        const bool has_bias = a.bias != nullptr;
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(has_bias ? a.bias : a.pw), (short)0,
            (int)uniform(has_bias ? (uint32_t)(a.C_out * 2) : 0u), kBufferWord3);
#pragma unroll
        for (int rb = 0; rb < RW_RB; ++rb) {
            const int r0 = g * RW_ROWS + wave * (RW_RB * 16) + rb * 16;
            // A-fragment row of this lane
            const int R = r0 + li;
            const int co = R / a.s, j = R - co * a.s;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int r = ks / a.ncb, cb = ks - r * a.ncb;
                const bool ok = co < a.C_out;
                const uint32_t off =
                    ok ? (uint32_t)(((((int64_t)j * a.ncb + cb) * a.C_out + co) * a.T + r) * 32 +
                                    lg * 8) * 2u
                       : 0x80000000u;
                wf[rb][ks] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
            }
            // output rows of this lane in the MFMA result: r0 + 4 lg + i, one
            // output channel (s is a multiple of 4), phases j0 .. j0 + 3
            const int Re = r0 + 4 * lg;
            co_e[rb] = Re / a.s;
            j0_e[rb] = Re - co_e[rb] * a.s;
            const uint32_t boff = co_e[rb] < a.C_out ? (uint32_t)co_e[rb] * 2u : 0x7FFFFFF0u;
            bv[rb] = TR::to_f32(__builtin_amdgcn_raw_buffer_load_b16(brs, boff, 0, 0));
        }
    }

    // ---- x staging items: (8 positions, 8 channels), positions fastest ----
    const int npg = a.WP / RW_NP;
    const int nitems = npg * (a.C_in_pad / 8);
    int ipg[RW_XI], icg[RW_XI];
    bool ion[RW_XI];
#pragma unroll
    for (int it = 0; it < RW_XI; ++it) {
        const int q = tid + THREADS * it;
        ion[it] = q < nitems;
        const int qq = ion[it] ? q : 0;
        icg[it] = qq / npg;
        ipg[it] = qq - icg[it] * npg;
    }
    // One tile's x in registers with its per-item descriptors: realignment
    // shift (positions), valid-position mask, byte offset of channel 0 of
    // the item's group at its (clamped) start.  Two of them: the tile after
    // next is loaded while the next one waits to be stored to LDS.
    // an item's channel: NP positions (odd rows: the dword-aligned bytes that
    // hold them, 4 more)
    using XRaw = std::conditional_t<NP == 8, u32x4, u32x2>;
    struct XOdd {
        XRaw lo;
        uint32_t hi;
    };
    using XEl = std::conditional_t<XODD, XOdd, XRaw>;
    struct XBuf {
        XEl v[RW_XI][8];
        int sh[RW_XI];
        uint32_t pm[RW_XI];
        uint32_t o0[RW_XI];
    };
    XBuf bufA;
    std::conditional_t<NBUF == 2, XBuf, char> bufB;

    auto tile_of = [&](int64_t tl, int& n, int& q0) __attribute__((always_inline)) {
        const uint32_t t = (uint32_t)tl, nn = fdiv(t, a.fd_tpi);
        n = (int)nn;
        q0 = (int)(t - nn * (uint32_t)a.tpi) * RW_BQ;
    };

    // Global -> registers for tile tl (loads only; the values are consumed
    // by lstore).  Positions outside the row and channels past C_in are
    // zeroed there; the loads themselves stay inside the image (clamped
    // starts; the resource covers one image, rounded to a whole dword).
    auto gload = [&](int64_t tl, XBuf& b) __attribute__((always_inline)) {
        int n, q0;
        tile_of(tl, n, q0);
        const int w0 = q0 - (a.T - 1) - a.xofs;
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(static_cast<const S*>(a.x) + (int64_t)n * a.C_in * a.L), (short)0,
            (int)uniform((a.img + 3u) & ~3u), kBufferWord3);
#pragma unroll
        for (int it = 0; it < RW_XI; ++it) {
            const int p0 = w0 + RW_NP * ipg[it];
            int p0c = p0 < 0 ? 0 : p0;
            if (p0c > a.L - RW_NP) p0c = a.L - RW_NP;
            uint32_t pm = 0;
#pragma unroll
            for (int pp = 0; pp < RW_NP; ++pp)
                pm |= (p0 + pp >= 0 && p0 + pp < a.L) ? (1u << pp) : 0u;
            const int sh = p0 - p0c;
            b.sh[it] = (sh > -RW_NP && sh < RW_NP) ? sh : 0;
            b.pm[it] = ion[it] ? pm : 0u;
            b.o0[it] = (uint32_t)icg[it] * 8u * a.plane + (uint32_t)p0c * 2u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t off = b.o0[it] + (uint32_t)e * a.plane;
                if constexpr (NP == 8) {
                    if constexpr (XODD) {
                        b.v[it][e].lo = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, off & ~3u, 0, 0));
                        b.v[it][e].hi =
                            __builtin_amdgcn_raw_buffer_load_b32(xrs, (off & ~3u) + 16u, 0, 0);
                    } else {
                        b.v[it][e] = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
                    }
                } else {
                    if constexpr (XODD) {
                        b.v[it][e].lo = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_raw_buffer_load_b64(xrs, off & ~3u, 0, 0));
                        b.v[it][e].hi =
                            __builtin_amdgcn_raw_buffer_load_b32(xrs, (off & ~3u) + 8u, 0, 0);
                    } else {
                        b.v[it][e] = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_raw_buffer_load_b64(xrs, off, 0, 0));
                    }
                }
            }
        }
    };

    // Registers -> LDS stage st: each item's 8 channels x 8 positions are
    // realigned, masked and transposed into 8 rows of 8 channels.
    auto lstore = [&](int st, const XBuf& b) __attribute__((always_inline)) {
        S* xs = smem + st * a.stage;
#pragma unroll
        for (int it = 0; it < RW_XI; ++it) {
            if (!ion[it]) continue;
            XRaw in[8];
            const int nval = a.C_in - icg[it] * 8;  // valid channels of the group
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (XODD) {
                    const uint32_t off = b.o0[it] + (uint32_t)e * a.plane;
                    const uint32_t bsh = (off & 2u) * 8u;
                    const XRaw w = b.v[it][e].lo;
                    XRaw o;
#pragma unroll
                    for (int d = 0; d + 1 < NP / 2; ++d)
                        o[d] = __builtin_amdgcn_alignbit(w[d + 1], w[d], bsh);
                    o[NP / 2 - 1] = __builtin_amdgcn_alignbit(b.v[it][e].hi, w[NP / 2 - 1], bsh);
                    in[e] = o;
                } else {
                    in[e] = b.v[it][e];
                }
                if (e >= nval) in[e] = XRaw{};
            }
            const uint32_t m = b.pm[it];
            if (m != (1u << NP) - 1u || b.sh[it] != 0) {
                // row edge: element pp takes loaded element pp + sh
                const int sh = b.sh[it] * 16;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (NP == 8) {
                        unsigned __int128 v = __builtin_bit_cast(unsigned __int128, in[e]);
                        v = sh >= 0 ? (v >> sh) : (v << -sh);
                        in[e] = __builtin_bit_cast(XRaw, v);
                    } else {
                        uint64_t v = __builtin_bit_cast(uint64_t, in[e]);
                        v = sh >= 0 ? (v >> sh) : (v << -sh);
                        in[e] = __builtin_bit_cast(XRaw, v);
                    }
                }
            }
            const u32x4 z = {0u, 0u, 0u, 0u};
            // positions pp = 0..7: dword c of row pp holds channels 2c, 2c + 1
#pragma unroll
            for (int pp = 0; pp < RW_NP; ++pp) {
                const unsigned sel = (pp & 1) ? 0x07060302u : 0x05040100u;
                u32x4 row;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    row[c] = __builtin_amdgcn_perm(in[2 * c + 1][pp >> 1], in[2 * c][pp >> 1], sel);
                *reinterpret_cast<u32x4*>(xs + (RW_NP * ipg[it] + pp) * a.RS + icg[it] * 8) =
                    (m & (1u << pp)) ? row : z;
            }
        }
    };

    S* __restrict__ yg = static_cast<S*>(a.y);
    const int arow = li + (a.T - 1) + a.xofs;  // window row of q = q0 + li at tap 0
    // LDS element offset of a B fragment: this lane's part (window row of
    // q = q0 + li at tap 0, its 8 channels) plus the k-step's wave-uniform part
    // (tap r one row back per tap, 32-channel block cb)
    const int lofs = arow * a.RS + lg * 8;
    auto kofs = [&](int ks) __attribute__((always_inline)) {
        const int r = ks / a.ncb, cb = ks - r * a.ncb;
        return (int)uniform((uint32_t)(cb * 32 - r * a.RS));
    };

    // One tile: the MFMAs (B fragments double-buffered in registers, the next
    // k-step's LDS reads issued ahead of the current k-step's MFMAs), then
    // the epilogue straight from the accumulators.
    // `mid` runs between the MFMAs and the epilogue: the next tile's LDS
    // staging, whose wait for its loads then precedes this tile's stores (a
    // wait for a load also waits for every memory operation issued before
    // it, and the stores' count is not known to the compiler)
    auto tile = [&](int64_t cur, int st, auto&& mid) __attribute__((always_inline)) {
        f32x4 acc[RW_RB][RW_CB];
#pragma unroll
        for (int rb = 0; rb < RW_RB; ++rb)
#pragma unroll
            for (int c = 0; c < RW_CB; ++c) acc[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        const S* xs = smem + st * a.stage;
        u32x4 bfr[2][RW_CB];
#pragma unroll
        for (int c = 0; c < RW_CB; ++c)
            bfr[0][c] = *reinterpret_cast<const u32x4*>(xs + lofs + kofs(0) + c * 16 * a.RS);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) {
#pragma unroll
                for (int c = 0; c < RW_CB; ++c)
                    bfr[(ks + 1) & 1][c] = *reinterpret_cast<const u32x4*>(
                        xs + lofs + kofs(ks + 1) + c * 16 * a.RS);
            }
#pragma unroll
            for (int c = 0; c < RW_CB; ++c)
#pragma unroll
                for (int rb = 0; rb < RW_RB; ++rb)
                    Mma<TR>::step(acc[rb][c], wf[rb][ks], bfr[ks & 1][c]);
            // keep the next k-step's reads ahead of this k-step's MFMAs
            if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, RW_CB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, RW_CB * RW_RB, 0);
        }
        mid();

        int n, q0;
        tile_of(cur, n, q0);
        // outputs s*q + j - p of this tile's positions q0 .. q0 + 63: when
        // all of them lie inside the row no lane needs a bounds check
        const int olo = a.s * q0 - a.p, ohi = a.s * (q0 + RW_BQ) - a.p;
        const bool inside = olo >= 0 && ohi <= a.Lo;
        // each lane writes its four consecutive outputs as one run; a wave's
        // four stores per row block cover 512 (fp32: 1024) consecutive bytes
        // of four output rows
#pragma unroll
        for (int rb = 0; rb < RW_RB; ++rb) {
            const int co = co_e[rb];
            if (co >= a.C_out) continue;
            const int64_t row = ((int64_t)n * a.C_out + co) * a.Lo;
#pragma unroll
            for (int c = 0; c < RW_CB; ++c) {
                const int o0 = a.s * (q0 + c * 16 + li) + j0_e[rb] - a.p;
                float f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = acc[rb][c][i] + bv[rb];
                    f[i] = EPI == RW_ELU ? elu_act<TR>(v) : v;
                }
                if constexpr (EPI == RW_F32) {
                    float* frow = static_cast<float*>(a.y) + row;
                    if (inside || (o0 >= 0 && o0 + 3 < a.Lo)) {
                        store16_unaligned(frow + o0, u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]),
                                                           __float_as_uint(f[2]), __float_as_uint(f[3])});
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (o0 + i >= 0 && o0 + i < a.Lo) frow[o0 + i] = f[i];
                    }
                } else {
                    S* yrow = yg + row;
                    if (inside || (o0 >= 0 && o0 + 3 < a.Lo)) {
                        *reinterpret_cast<u32x2_u*>(yrow + o0) =
                            u32x2{pack2<TR>(f[0], f[1]), pack2<TR>(f[2], f[3])};
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (o0 + i >= 0 && o0 + i < a.Lo) yrow[o0 + i] = TR::from_f32(f[i]);
                    }
                }
            }
        }
    };

    const int64_t last = t_end - 1;
    if constexpr (NBUF == 1) {
        // tile cur computes from LDS stage st while the x of tile cur + 1 is
        // loaded into registers (stored to the other stage after the MFMAs);
        // the last iteration re-reads its own tile (an unconditional load
        // whose values are never stored)
        gload(t_begin, bufA);
        lstore(0, bufA);
        __syncthreads();
        int st = 0;
        for (int64_t cur = t_begin;; ++cur) {
            gload(cur + 1 <= last ? cur + 1 : last, bufA);
            // the loads go out now, not sunk toward their use after the MFMAs
            __builtin_amdgcn_sched_barrier(0);
            const bool more = cur < last;
            tile(cur, st, [&]() __attribute__((always_inline)) {
                if (more) lstore(st ^ 1, bufA);
            });
            if (!more) break;
            __syncthreads();
            st ^= 1;
        }
    } else {
        // as above, one tile deeper: the x of tile cur + 1 waits in one
        // register buffer while that of cur + 2 is loaded into the other
        gload(t_begin, bufA);
        lstore(0, bufA);
        gload(t_begin + 1 < t_end ? t_begin + 1 : last, bufB);
        __syncthreads();
        int64_t cur = t_begin;
        while (true) {
            // stage 0 holds cur, bufB holds cur + 1
            gload(cur + 2 <= last ? cur + 2 : last, bufA);
            // the loads go out now, not sunk toward their use after the MFMAs
            __builtin_amdgcn_sched_barrier(0);
            const bool more0 = cur + 1 <= last;
            tile(cur, 0, [&]() __attribute__((always_inline)) {
                if (more0) lstore(1, bufB);
            });
            if (!more0) break;
            __syncthreads();
            ++cur;
            // stage 1 holds cur, bufA holds cur + 1
            gload(cur + 2 <= last ? cur + 2 : last, bufB);
            // the loads go out now, not sunk toward their use after the MFMAs
            __builtin_amdgcn_sched_barrier(0);
            const bool more1 = cur + 1 <= last;
            tile(cur, 1, [&]() __attribute__((always_inline)) {
                if (more1) lstore(0, bufA);
            });
            if (!more1) break;
            __syncthreads();
            ++cur;
        }
    }
}

using RWFn = void (*)(const RWArgs);

template <class TR, int KS, int EPI>
RWFn pick_ks(bool xodd) {
    return xodd ? &polyrw_kernel<TR, true, KS, RW_WAVES, RW_NP, RW_NBUF, EPI>
                : &polyrw_kernel<TR, false, KS, RW_WAVES, RW_NP, RW_NBUF, EPI>;
}

template <class TR, int EPI>
RWFn pick_e(bool xodd, int ks) {
    switch (ks) {
        case 1: return pick_ks<TR, 1, EPI>(xodd);
        case 2: return pick_ks<TR, 2, EPI>(xodd);
        case 3: return pick_ks<TR, 3, EPI>(xodd);
        case 4: return pick_ks<TR, 4, EPI>(xodd);
        case 5: return pick_ks<TR, 5, EPI>(xodd);
        case 6: return pick_ks<TR, 6, EPI>(xodd);
        case 7: return pick_ks<TR, 7, EPI>(xodd);
        case 8: return pick_ks<TR, 8, EPI>(xodd);
    }
    return nullptr;
}

template <class TR>
RWFn pick(bool xodd, int ks, int epi) {
    switch (epi) {
        case RW_PLAIN: return pick_e<TR, RW_PLAIN>(xodd, ks);
        case RW_ELU: return pick_e<TR, RW_ELU>(xodd, ks);
        case RW_F32: return pick_e<TR, RW_F32>(xodd, ks);
    }
    return nullptr;
}

bool plan_rw(const Problem& p, RWArgs* a) {
    if (p.ndim != 1 || p.dtype == CTCONV_F32) return false;
    // s a multiple of 4 (a lane's four MFMA rows are four phases of one
    // channel) dividing 32 (a wave's rows are whole channels)
    if (p.dW != 1 || p.sW % 4 != 0 || 32 % p.sW != 0) return false;
    if (p.N < 1 || p.W < RW_NP) return false;
    if (p.mW < 1 || p.mW > 4 || p.mW * p.C_in_pad > 256) return false;
    // 32-bit byte offsets: one image of x, the packed weight; int positions
    const int64_t img = p.C_in * p.W * 2;
    if (img + 4 > 0x7FFFFFFFLL) return false;
    const int64_t pw_bytes = p.sW * p.C_out * p.mW * p.C_in_pad * 2;
    if (pw_bytes >= 0x7FFFFFF0LL) return false;
    const int64_t Q = (p.Wo - 1 + p.pW) / p.sW + 1;  // q positions reaching an output
    // int positions and output indices (s * (q + 64) stays below 2^31)
    if (Q + RW_BQ > 0x3FFFFFFFLL || p.Wo > 0x3FFFFFFFLL || (Q + RW_BQ) * p.sW > 0x7FFFFFFFLL)
        return false;
    if (p.C_out * p.sW > 0x3FFFFFFFLL) return false;
    const int64_t tpi = (Q + RW_BQ - 1) / RW_BQ;
    a->Lo = (int)p.Wo;
    a->n_tiles = p.N * tpi;
    a->L = (int)p.W;
    a->C_in = (int)p.C_in;
    a->C_out = (int)p.C_out;
    a->C_in_pad = (int)p.C_in_pad;
    a->ncb = (int)(p.C_in_pad / 32);
    a->s = (int)p.sW;
    a->p = (int)p.pW;
    a->T = (int)p.mW;
    a->KS = a->T * a->ncb;
    a->tpi = (int)tpi;
    a->fd_tpi = make_fastdiv((uint32_t)tpi);
    if (a->n_tiles > 0x7FFFFFFFLL) return false;  // 32-bit tile indices
    a->rg = (int)((p.C_out * p.sW + RW_ROWS - 1) / RW_ROWS);
    // (8 / WAVES) workgroups per CU; at least four tiles per workgroup
    int64_t per = 256 * (8 / RW_WAVES) / a->rg;
    if (per < 1) per = 1;
    int64_t want = (a->n_tiles + 3) / 4;
    if (want < 1) want = 1;
    int64_t wpr = per < want ? per : want;
    if (wpr >= 16) wpr -= wpr % 8;  // a multiple of 8: row groups of a run share an XCD
    a->wg_per_rg = (int)wpr;
    // window start a multiple of NP positions (q0 is a multiple of 64)
    a->xofs = (RW_NP - (a->T - 1) % RW_NP) % RW_NP;
    a->WP = RW_BQ + a->T - 1 + a->xofs;  // a multiple of RW_NP, at most RW_WPMAX
    a->RS = a->C_in_pad + 8;
    a->stage = a->WP * a->RS;
    a->plane = (uint32_t)(p.W * 2);
    a->img = (uint32_t)img;
    a->pw_bytes = (uint32_t)pw_bytes;
    // (with m * C_in_pad <= 256 the window's load items fit one per thread)
    // the two x stages within RW_LDS_MAX bytes of dynamic LDS
    if (2 * (int64_t)a->stage * 2 > RW_LDS_MAX) return false;
    return a->KS <= RW_KMAX && a->WP <= RW_WPMAX && (a->WP / RW_NP) * (a->C_in_pad / 8) <= RW_THREADS &&
           (int64_t)a->rg * a->wg_per_rg <= 0x7FFFFFFF;
}

}  // namespace

bool polyrw_supported(const Problem& p) {
    RWArgs a{};
    return plan_rw(p, &a);
}

hipError_t launch_polyrw(const Problem& p, const void* x, const void* pw, const void* bias,
                         void* y, bool out_f32, hipStream_t s) {
    RWArgs a{};
    if (!plan_rw(p, &a)) return hipErrorInvalidValue;
    // the fp32 output of a stream chunk takes no activation
    if (out_f32 && p.act != CTCONV_ACT_NONE) return hipErrorInvalidValue;
    const int epi = out_f32 ? RW_F32 : (p.act == CTCONV_ACT_ELU ? RW_ELU : RW_PLAIN);
    a.x = x;
    a.pw = pw;
    a.bias = bias;
    a.y = y;
    const bool xodd = (p.W % 2) == 1;
    RWFn fn = p.dtype == CTCONV_BF16 ? pick<TBF16>(xodd, a.KS, epi) : pick<TF16>(xodd, a.KS, epi);
    if (fn == nullptr) return hipErrorInvalidValue;
    const size_t lds = (size_t)(2 * a.stage) * 2;  // at most RW_LDS_MAX
    hipLaunchKernelGGL(fn, dim3((unsigned)(a.rg * a.wg_per_rg)), dim3(RW_THREADS), lds, s, a);
    return hipGetLastError();
}

}  // namespace ctconv

// Polyphase transposed convolution as an implicit GEMM on the gfx950 MFMA
// matrix cores.
//
// Method.  For k = m*s (per dimension) and d = 1, a transposed convolution is
// one stride-1 convolution with m taps that yields every output phase,
// followed by an interleave of the phases and a slice of the padding
// (ExecuTorch PR #25037, "[XNNPACK] Lower dense transposed convs as one
// polyphase conv + depth to space", Summary formula
// y[s*q + j] = sum_{u<m} x[q + u - (m-1)] * w[s*(m-1-u) + j]).  The identity
// below holds for any k with m = ceil(k / s) when the taps s*r + j >= k are
// zero (the packed weight is zero there), and output_padding only extends the
// range of output rows, so every shape with d = 1 takes this kernel.
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
// few tiles may split the C_in reduction across workgroups (fp32 only, when
// the caller gives a workspace): each split writes its fp32 partial sums to y
// or to a workspace slab with plain stores, and a second kernel adds them in
// a fixed order, so results are the same bits on every run.
// More phases than a column tile holds: each column tile takes a subset of
// whole phases.  More taps per phase than an instance (fp32): launches over
// groups of tap slots, each on the input window shifted back by its first
// slot, the later ones adding to y in launch order.

#include <type_traits>

#include "ctconv_internal.h"
#include "mfma_common.h"

namespace ctconv {

namespace {

using namespace mfma;

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
    // window rows: the tile, the halo and (2-D, output-aligned phase rows
    // under padding) one more row for the phases whose inputs start a row
    // later
    static constexpr int WYM = TAY + MY - 1 + (TAY > 1 ? 1 : 0);
    static constexpr int NP = 8 / ES;                             // positions per load item
    // window columns: the tile, the halo, one more column for output-aligned
    // phase rows under padding and up to NP-1 positions of alignment shift,
    // padded to whole fragments
    static constexpr int WXP = (TAX + MX + NP - 1 + VEC - 1) / VEC * VEC;
    static constexpr int XROWS = WYM * WXP;
    static constexpr int BROWS = T * BN;
    static constexpr int STAGE = (XROWS + BROWS) * RSA;
    static constexpr int NG = KC / VEC;                           // channel groups per chunk
    static constexpr int NW = WM * WN;                            // waves per workgroup
    static constexpr int NT = 64 * NW;                            // threads per workgroup
    // load items are split into NW contiguous per-wave ranges (coalesced lanes)
    static constexpr int XMAX = WYM * (WXP / NP) * NG;
    static constexpr int XITEMS = ((XMAX + NW - 1) / NW + 63) / 64;
    static constexpr int BMAX = BROWS * NG;
    static constexpr int BITEMS = ((BMAX + NW - 1) / NW + 63) / 64;
    static constexpr int EPI = BM * BN + BN * VEC;  // staged output tile, padded
    static constexpr int SMEM = (2 * STAGE > EPI ? 2 * STAGE : EPI);
    // global -> register prefetch depth in chunks: one wave per SIMD with a
    // 128 x 128-class wave tile has long MFMA phases but no registers for a
    // second buffer
    static constexpr int PF = (RB * CB >= 32 || KS >= 2) ? 1 : 2;
    static_assert(BM % TAX == 0 && TAX % 16 == 0, "tile rows");
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(SMEM * ES <= 160 * 1024, "LDS");
};

// XODD: 16-bit input rows of odd length.  Row pieces then start at 2-byte
// offsets in every other channel plane or row; each piece is loaded as the 12
// dword-aligned bytes that contain it and extracted at LDS-store time (a
// 2-byte-misaligned 8-byte load costs the texture path per lane).
// At least two waves per SIMD (256 registers per wave): an 8-wave workgroup
// per CU, or two 4-wave ones; only 128 x 128 wave tiles need the whole file.
template <class TR, int MY, int MX, int TAX, int RB, int CB, int WM, int WN, int KS, bool XODD>
__global__ __launch_bounds__(64 * WM * WN, (RB * CB >= 64 ? 1 : 2)) void poly_kernel(
    const PolyArgs a) {
    using C = Cfg<TR, MY, MX, TAX, RB, CB, WM, WN, KS>;
    using S = typename TR::storage;
    constexpr int VEC = C::VEC, KC = C::KC, RSA = C::RSA, BN = C::BN, T = C::T;
    constexpr int NG = C::NG, WXP = C::WXP;

    __shared__ __attribute__((aligned(16))) S smem[C::SMEM];

    const S* __restrict__ xg = static_cast<const S*>(a.x);
    const S* __restrict__ pwg = static_cast<const S*>(a.pw);

    // ---- tile coordinates -------------------------------------------------
    // linear tile = row_tile * n_col_tiles + col (row-major order) or
    // col * n_row_tiles + row_tile (column-major order, for fp32 shapes whose
    // packed weight outweighs their input), row_tile = (n * tiles_y + ty) *
    // tiles_x + tx; with the XCD remap the gridDim.x / 8 workgroups of one
    // XCD (dispatched round robin) take a contiguous run of tiles, so that
    // the tiles that read the same input rows (row-major) or the same weight
    // rows (column-major) meet in one L2
    uint32_t bid = blockIdx.x;
    if (a.xcd_remap) bid = (bid % 8u) * (gridDim.x / 8u) + bid / 8u;
    // (fp32 instances only: in the 16-bit ones the remap's extra uniform
    // values tip the scalar registers into spills that cost the vocoder
    // layers 5 % and the 2-D upsampler 8 %)
    if constexpr (C::ES == 4) {
        if (a.colmajor) {
            // the column-major position of bid as its row-major tile index
            const uint32_t cq = fdiv(bid, a.fd_rows);
            bid = (bid - cq * (uint32_t)a.n_row_tiles) * (uint32_t)a.n_col_tiles + cq;
        }
    }
    const uint32_t row_tile = fdiv(bid, a.fd_cols);
    const int col_tile = (int)(bid - row_tile * (uint32_t)a.n_col_tiles);
    const uint32_t rt2 = fdiv(row_tile, a.fd_tx);
    const int tx_t = (int)(row_tile - rt2 * (uint32_t)a.tiles_x);
    const uint32_t nq = fdiv(rt2, a.fd_ty);
    const int ty_t = (int)(rt2 - nq * (uint32_t)a.tiles_y);
    const int64_t n = nq;
    const int cq = (int)fdiv((uint32_t)col_tile, a.fd_ph);
    const int co0 = cq * a.TCO;
    const int b0 = (col_tile - cq * a.n_ph_tiles) * a.PT;
    const int ay0 = ty_t * C::TAY, ax0 = tx_t * TAX;
    // output phase row q takes input rows q + delta_b - r, r < m (delta_b = 0
    // for every phase unless the phase rows are output-aligned under
    // padding): the window starts m - 1 rows before the tile's smallest
    // delta
    // (a tap group starting at slot r0 reads r0 rows and columns further back)
    const int wy0 = ay0 + a.dminy - (MY - 1) - a.r0y;
    const int wx0 = ax0 + a.dminx - (MX - 1) - a.r0x - a.xofs;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 15, lg = lane >> 4;

    // Column tc of the tile -> (phase pb within the tile, output channel
    // co_l within the tile).  Channel-major: TCO channels of phase 0, then of
    // phase 1, ...  Phase-fastest (pfast): 16-column blocks cycle through the
    // PT phases of one 16-channel group before the next group, so that a wave
    // holds whole runs of consecutive phases of its channels (stored straight
    // from registers).  co_l >= TCO marks a padding block.
    // Row-phase-fastest (pfast = 2, class mode with two phases per output
    // row): blocks cycle through the 2 phases b_x of one output row b_y, then
    // the next 16-channel group, then the next row, so that block cb's phase
    // b_x is cb mod 2 and a wave's blocks share b_y.
    auto col_map = [&](int tc, int& pb, int& co_l) __attribute__((always_inline)) {
        if (a.pfast == 1) {
            const int blk = tc >> 4;
            const int g = (int)fdiv((uint32_t)blk, a.fd_pt);
            pb = blk - g * a.PT;
            co_l = g * 16 + (tc & 15);
        } else if (a.pfast == 2) {
            const int blk = tc >> 4;
            const int by = (int)fdiv((uint32_t)blk, a.fd_pt);  // fd_pt: 2 TCO / 16
            const int rem = blk - by * (2 * (a.TCO >> 4));
            pb = by * 2 + (rem & 1);
            co_l = (rem >> 1) * 16 + (tc & 15);
        } else {
            pb = (int)fdiv((uint32_t)tc, a.fd_tco);
            co_l = tc - pb * a.TCO;
        }
    };

    // ---- x staging descriptors: item = (window row, NP positions, VEC channels)
    // Each channel of an item is one 8-byte global load (NP positions); the
    // VEC x NP block is transposed in registers into NP LDS rows of VEC
    // channels.  Positions fastest across lanes: one load instruction of a
    // wave reads a contiguous run of one channel plane (whole cache lines),
    // which keeps the vector L1 to a few line accesses per instruction.
    constexpr int NP = C::NP;
    const int64_t HW = a.H * a.W;
    const int ngx = WXP / NP;
    const int xitems = a.WY * ngx * NG;
    const int xper = (xitems + C::NW - 1) / C::NW;  // items per wave
    // Per item: the lane's byte offset within the image (channel 0 of its
    // group, clamped in-row start position), the realignment shift
    // (positions), the valid-position mask and its LDS slot.
    uint32_t xlo[C::XITEMS];
    uint32_t xv0[XODD ? C::XITEMS : 1], xs0[XODD ? C::XITEMS : 1];
    uint32_t xv1[XODD ? C::XITEMS : 1], xs1[XODD ? C::XITEMS : 1];
    int xsh[C::XITEMS];
    uint32_t xpm[C::XITEMS];
    int xgv[C::XITEMS];  // first channel of the item's group (odd rows: ragged mask)
    // LDS element offset of the first position row.  Lanes without an item
    // get the 16-byte padding at the end of NP rows (never read by the
    // MFMA operand loads), spread over rows, so that every store is
    // unconditional.
    int xlds[C::XITEMS];
    bool inside = true;  // the lane's items need no realignment or masks
    // Bank spreading of the transposed stores (16-bit: four positions per
    // item).  Consecutive lanes own items four position rows apart, i.e. 4 x
    // 80 bytes, which is 64 bytes modulo the 256 bytes of the 64 banks: in
    // lane order the same position of 16 consecutive lanes falls into four
    // bank groups only, and a probe of that store pattern alone measured it
    // 4-way conflicted on gfx950.  So lane l first rotates its item's
    // positions by rho(l) and store j writes position (j + rho) mod 4:
    // within every 8-lane group (bits 1-2 of l) and every 16-lane group
    // (bits 2-3 of l) with the other bits fixed, rho takes all four values
    // (bit 2 of l as its high bit, bit 1 xor bit 3 of l as its low bit); the
    // same probe measured the rotated pattern free of conflicts.  The
    // rotation is two byte permutes per channel.
    constexpr bool ROT = C::ES == 2;
    const int rho = ROT ? ((((lane >> 1) ^ (lane >> 3)) & 1) | ((lane >> 1) & 2)) : 0;
    // v_perm selectors: the dword of positions (r, r + 1) mod 4 of a channel
    // held as positions 0-3 in two dwords (bytes 2 p, 2 p + 1 of the pair)
    auto rot_sel = [](int r) -> uint32_t {
        const uint32_t b0 = 2u * (uint32_t)(r & 3), b1 = 2u * (uint32_t)((r + 1) & 3);
        return b0 | (b0 + 1u) << 8 | b1 << 16 | (b1 + 1u) << 24;
    };
    const uint32_t rsel_lo = rot_sel(rho), rsel_hi = rot_sel(rho + 2);
#pragma unroll
    for (int it = 0; it < C::XITEMS; ++it) {
        const int qw = lane + 64 * it;
        const int q = wave * xper + qw;
        xlds[it] = (lane % (C::XROWS / NP)) * NP * RSA + KC;
        xlo[it] = 0;
        if constexpr (XODD) {
            xv0[it] = 0;
            xs0[it] = 0;
            xv1[it] = 0;
            xs1[it] = 0;
        }
        xsh[it] = 0;
        xpm[it] = 0;
        xgv[it] = 0;
        if (qw < xper && q < xitems) {
            const int gx = q % ngx;
            const int r2 = q / ngx;
            const int g = (int)fdiv((uint32_t)r2, a.fd_wy);
            const int wy = r2 - g * a.WY;
            const int iy = wy0 + wy;
            const bool rowok = iy >= 0 && iy < a.H;
            const int p0 = wx0 + gx * NP;
            // one NP-element load from an in-row start (the planner admits
            // only rows of at least NP elements, so one always exists)
            int p0c = p0 < 0 ? 0 : p0;
            if (p0c > (int)a.W - NP) p0c = (int)a.W - NP;
            if (p0c < 0) p0c = 0;
            uint32_t pm = 0;
#pragma unroll
            for (int p = 0; p < NP; ++p)
                pm |= (rowok && p0 + p >= 0 && p0 + p < a.W) ? (1u << p) : 0u;
            xpm[it] = pm;
            // data for position p sits at loaded index p + shift; an item with
            // no valid position is masked entirely, so its shift is irrelevant
            const int shft = p0 - p0c;
            xsh[it] = (shft > -NP && shft < NP) ? shft : 0;
            xlo[it] = (uint32_t)(((int64_t)g * VEC * HW + (int64_t)(rowok ? iy : 0) * a.W + p0c) *
                                 C::ES);
            if constexpr (XODD) {
                // dword-aligned start and bit shift of the piece, for channel
                // planes at even and at odd 2-byte offsets
                xv0[it] = xlo[it] & ~3u;
                xs0[it] = (xlo[it] & 2u) * 8u;
                xv1[it] = (xlo[it] + 2u) & ~3u;
                xs1[it] = ((xlo[it] + 2u) & 2u) * 8u;
            }
            xlds[it] = (wy * WXP + gx * NP) * RSA + g * VEC;
            xgv[it] = g * VEC;
            inside = inside && pm == (1u << NP) - 1u && xsh[it] == 0;
        }
    }
    // The whole wave's items sit inside their rows with no realignment shift
    // (true for most tiles): its LDS stores need no shift and no masks.
    const bool wave_inside = __all(inside);
    // Buffer resources: x of this tile's image and the packed weight.  Loads
    // take a 32-bit lane offset plus a wave-uniform offset; the resource's
    // size bounds every access (out-of-range dwords read as zero, no fault).
    const uint32_t ch_bytes = uniform((uint32_t)(HW * C::ES));  // one channel plane
    const bool odd_plane = (ch_bytes & 2u) != 0u;
    // (the image's extent rounded up to a whole dword: with odd 16-bit rows the
    // 12-byte load of the last piece of the last channel ends in the dword
    // that holds the image's last element, and the range check zeroes every
    // dword that reaches past the size)
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(xg + n * a.C_in * HW), (short)0,
        (int)uniform((ch_bytes * (uint32_t)a.C_in + 3u) & ~3u), kBufferWord3);
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(pwg), (short)0, (int)uniform(a.pw_bytes), kBufferWord3);

    // B items: packed-weight byte offset (0 for a row past C_out or past the
    // phases: the load is made anyway so that no load sits under a branch;
    // such rows feed only columns that are never stored) and LDS slot (row
    // padding for lanes without one).
    // The 64 items of one load instruction are 16 rows of NG = 4 pieces.
    // Lanes take them in the order that puts rows 0, 4, 8, 12 (then 1, 5, 9,
    // 13, ...) into 16 consecutive lanes: those rows start 80 r bytes in,
    // i.e. 0, 64, 128 and 192 modulo 256, so their 64-byte runs fill
    // distinct bank groups (four consecutive rows span 320 bytes and meet
    // twice: 2-way conflicted in lane order, conflict-free in this order, as
    // probed on gfx950).  The instruction reads the same rows of global
    // memory as in lane order.
    uint32_t boff[C::BITEMS];
    int blds[C::BITEMS];
    constexpr int bper = (C::BMAX + C::NW - 1) / C::NW;
    const int bl = (lane & 3) | ((lane >> 4) << 2) | (((lane >> 2) & 3) << 4);
#pragma unroll
    for (int it = 0; it < C::BITEMS; ++it) {
        const int qw = bl + 64 * it;
        const int q = wave * bper + qw;
        boff[it] = 0;
        blds[it] = (lane % C::BROWS) * RSA + KC;  // row padding: no item
        if (qw < bper && q < C::BMAX) {
            const int row = q / NG, piece = q % NG;
            const int r = row / BN, tc = row % BN;
            int pb, co_l;
            col_map(tc, pb, co_l);
            const int co = co0 + co_l, b = b0 + pb;
            if (pb < a.PT && b < a.P && co_l < a.TCO && co < a.C_out) {
                const int by = (int)fdiv((uint32_t)b, a.fd_sx), bx = b - by * a.sx;
                // weight phase of output phase b: (b + p) mod s (b itself
                // without padding)
                const int jy = by + a.py - (int)fdiv((uint32_t)(by + a.py), a.fd_sy) * a.sy;
                const int jx = bx + a.px - (int)fdiv((uint32_t)(bx + a.px), a.fd_sx) * a.sx;
                // Kernel tap (ry, rx) of kernel phase (jy, jx) is tap e = s' r + j
                // of the kernel the kernel runs (per dimension: stride s' and
                // the real taps spread d' apart, d' = 1 without dilation).  A
                // real tap t = e / d' exists when d' divides e and t < k; the
                // packed weight holds it as phase t mod s, tap t / s of the
                // real stride s.  Missing taps read as zero (an offset past the
                // packed weight, which is below 2^31 bytes: the range check of
                // the load returns zeros).
                const int ey = a.sy * (r / MX + a.r0y) + jy, ex = a.sx * (r % MX + a.r0x) + jx;
                const int ty = (int)fdiv((uint32_t)ey, a.fd_dey), tx = (int)fdiv((uint32_t)ex, a.fd_dex);
                if (ty * a.dey == ey && tx * a.dex == ex && ty < a.kH && tx < a.kW) {
                    const int qy = (int)fdiv((uint32_t)ty, a.fd_psy);
                    const int qx = (int)fdiv((uint32_t)tx, a.fd_psx);
                    const int jp = (ty - qy * a.psy) * a.psx + (tx - qx * a.psx);
                    const int rp = qy * a.pmx + qx;
                    // packed layout [j][ci / 32][co][t][ci % 32]: row (co, t) of
                    // phase j in channel block 0 (the chunk adds its block)
                    boff[it] = (uint32_t)((((int64_t)jp * (a.C_in_pad / kCinAlign) * a.C_out + co) *
                                               a.pT + rp) * kCinAlign + piece * VEC) *
                               C::ES;
                } else {
                    boff[it] = 0x80000000u;
                }
            }
            blds[it] = (r * BN + tc) * RSA + piece * VEC;
        }
    }

    // Two register buffers: the loads of chunk c+2 are issued before the
    // MFMAs of chunk c and stored to LDS after those of chunk c+1.
    using XEl = std::conditional_t<XODD, u32x3, u32x2>;
    using XBuf = XEl[C::XITEMS][VEC];
    using BBuf = u32x4[C::BITEMS];
    XBuf xr0, xr1;
    BBuf br0, br1;
    int cx0 = 0, cx1 = 0;  // chunk held by each register buffer

    // Global -> registers.  Loads only: nothing here consumes a loaded value,
    // so no wait is needed before the MFMAs of the current chunk.
    auto gload = [&](int c, XBuf& xr, BBuf& br, int& cx) __attribute__((always_inline)) {
        cx = c;
        const uint32_t cbase = uniform((uint32_t)c * KC);
        // The channel term goes into the per-lane offset, which the raw-buffer
        // range check covers: channels past C_in (a ragged last chunk) start
        // at or past the end of the image's resource, so their loads return
        // zeros and never read outside x.  Every chunk uses the same load form
        // and no load sits under a branch.
#pragma unroll
        for (int it = 0; it < C::XITEMS; ++it)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t choff = (cbase + e) * ch_bytes;
                if constexpr (XODD) {
                    // odd channels sit 2 bytes off the even ones when a plane
                    // is 2 mod 4 bytes long; their offset drops by 2 so that it
                    // stays a multiple of 4
                    const bool par = (e & 1) && odd_plane;
                    xr[it][e] = __builtin_bit_cast(
                        u32x3, __builtin_amdgcn_raw_buffer_load_b96(
                                   xrs, (par ? xv1[it] : xv0[it]) + choff - (par ? 2u : 0u), 0,
                                   0));
                } else {
                    xr[it][e] = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(xrs, xlo[it] + choff, 0, 0));
                }
            }
        // the chunk's channel block (a column tile's rows of one block are
        // contiguous) and its offset inside the block
        // (blocks of the packed weight's taps, not the kernel's)
        const uint32_t bchunk =
            uniform((cbase / kCinAlign) * a.pw_cblock + (cbase % kCinAlign) * C::ES);
#pragma unroll
        for (int it = 0; it < C::BITEMS; ++it)
            br[it] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, boff[it], bchunk, 0));
    };
    // `inside`: true_type when the caller knows that no item of the wave needs
    // realignment or masks, false_type to decide from wave_inside at run time
    auto lstore = [&](int st, const XBuf& xr, const BBuf& br, auto inside, int cx)
                      __attribute__((always_inline)) {
        S* xs = smem + st * C::STAGE;
        S* bs = xs + C::XROWS * RSA;
        const u32x4 z = {0u, 0u, 0u, 0u};
        // the 8-byte pieces of item `it` (odd rows: extracted from the 12
        // loaded bytes at the piece's 2-byte offset)
        // Odd rows: the resource extends x's extent to a whole dword, so the
        // first load of the channel after the image's last one may return the
        // two bytes past it; in a ragged chunk the channels past C_in are
        // zeroed here (wave-uniform branch, taken in the last chunk only).
        const int nval = (int)a.C_in - cx * KC;  // valid channels of the chunk
        const bool ragged = XODD && nval < KC;
        auto pieces = [&](int it, u32x2 (&in)[VEC]) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if constexpr (XODD) {
                    const bool par = (e & 1) && odd_plane;
                    const uint32_t sh = par ? xs1[it] : xs0[it];
                    const u32x3 w = xr[it][e];
                    in[e] = u32x2{__builtin_amdgcn_alignbit(w[1], w[0], sh),
                                  __builtin_amdgcn_alignbit(w[2], w[1], sh)};
                    if (ragged && xgv[it] + e >= nval) in[e] = u32x2{0u, 0u};
                } else {
                    in[e] = xr[it][e];
                }
            }
        };
        // (16-bit) position j of every channel of the item <- position
        // (j + rho) mod 4, so that the transpose's row j is that position
        auto rotate = [&](u32x2 (&in)[VEC]) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                in[e] = u32x2{__builtin_amdgcn_perm(in[e][1], in[e][0], rsel_lo),
                              __builtin_amdgcn_perm(in[e][1], in[e][0], rsel_hi)};
        };
        if (decltype(inside)::value || wave_inside) {
            // no lane of the wave touches a row edge: transpose and store only
#pragma unroll
            for (int it = 0; it < C::XITEMS; ++it) {
                u32x2 in[VEC];
                u32x4 tr[NP];
                pieces(it, in);
                if constexpr (ROT) rotate(in);
                transpose_block(in, tr);
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    *reinterpret_cast<u32x4*>(xs + xlds[it] + ((p + rho) & (NP - 1)) * RSA) = tr[p];
            }
        } else {
            // every lane realigns (shift 0 away from row edges) and zeroes
            // the positions outside its row
#pragma unroll
            for (int it = 0; it < C::XITEMS; ++it) {
                const uint32_t m = xpm[it];
                const int sh = xsh[it] * (int)(8 * C::ES);
                u32x2 in[VEC];
                u32x4 tr[NP];
                pieces(it, in);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    uint64_t v = __builtin_bit_cast(uint64_t, in[e]);
                    v = sh >= 0 ? (v >> sh) : (v << -sh);
                    in[e] = __builtin_bit_cast(u32x2, v);
                }
                if constexpr (ROT) rotate(in);
                transpose_block(in, tr);
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const int pr = (p + rho) & (NP - 1);  // the position row tr[p] holds
                    *reinterpret_cast<u32x4*>(xs + xlds[it] + pr * RSA) = (m & (1u << pr)) ? tr[p] : z;
                }
            }
        }
        // B rows past C_out or past the phases feed only columns that are
        // never stored: their (finite) values need no masking
#pragma unroll
        for (int it = 0; it < C::BITEMS; ++it)
            *reinterpret_cast<u32x4*>(bs + blds[it]) = br[it];
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
        arow[rb] = (tr0 / TAX) * WXP + (tr0 % TAX) + li + a.xofs;
    }
    const int bcol = (wn * CB) * 16 + li;

    // Bias of each column block's output channel, loaded now so that the
    // epilogue never waits for it.  One unconditional load per block: a
    // column past the phases or past C_out, a split-over-C_in launch (whose
    // bias the reduction adds) and a missing bias all read past the
    // resource's range, which returns zero.
    float bvs[CB];
    {
        const bool has_bias = a.bias != nullptr && !a.partial;
        const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(has_bias ? a.bias : a.pw), (short)0,
            (int)uniform(has_bias ? (uint32_t)(a.C_out * C::ES) : 0u), kBufferWord3);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int tc = bcol + cb * 16;
            int pb, co_l;
            col_map(tc, pb, co_l);
            const int co = co0 + co_l;
            const uint32_t off =
                (pb < a.PT && co_l < a.TCO && co < a.C_out) ? (uint32_t)co * C::ES : 0x7FFFFFF0u;
            if constexpr (C::ES == 2)
                bvs[cb] = TR::to_f32(__builtin_amdgcn_raw_buffer_load_b16(bres, off, 0, 0));
            else
                bvs[cb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bres, off, 0, 0));
        }
    }

    // Per chunk and k-step, tap by tap: the tap's B fragments, its A
    // fragments (window rows shifted back by the tap index: output phase row
    // q takes input q - r) and the MFMAs of every (row block, column block)
    // pair.  A scheduling barrier between taps keeps one tap's fragments live
    // at a time.
    // Output-aligned phase rows (class mode): column block cb holds one phase
    // b whose input rows start delta_b = floor((b + p) / s) - floor(p / s)
    // (0 or 1 per dimension) later; its A fragments sit that much further in
    // the window.  Wave-uniform element offsets, 0 outside class mode.
    int cofs[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        int o = 0;
        if (C::TAY > 1 && a.cmode) {
            int pb, co_l;
            col_map(wn * CB * 16 + cb * 16, pb, co_l);
            const int b = b0 + (pb < a.PT ? pb : 0);
            const int by = (int)fdiv((uint32_t)b, a.fd_sx), bx = b - by * a.sx;
            const int dy = (int)fdiv((uint32_t)(by + a.py), a.fd_sy) - a.dminy;
            const int dx = (int)fdiv((uint32_t)(bx + a.px), a.fd_sx) - a.dminx;
            o = (dy * WXP + dx) * RSA;
        }
        cofs[cb] = (int)uniform((uint32_t)o);
    }
    // (class mode) window row of row block rb relative to row block 0: the
    // wave's rows start at a tile-row boundary or stay inside one tile row
    static_assert(C::TAY == 1 || (RB * 16) % TAX == 0 || TAX % (RB * 16) == 0, "row blocks");
    auto rb_row_offset = [](int rb) constexpr {
        return (RB * 16) % TAX == 0 ? ((rb * 16) / TAX) * WXP + (rb * 16) % TAX : rb * 16;
    };
    int abase[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) abase[cb] = arow[0] * RSA + cofs[cb];
    auto tap_step = [&](const S* xs, const S* bs, int kofs, int r) __attribute__((always_inline)) {
        const int ry = r / MX, rx = r % MX;
        u32x4 afr[RB], bfr[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            bfr[cb] = *reinterpret_cast<const u32x4*>(bs + (r * BN + bcol + cb * 16) * RSA + kofs);
        if constexpr (C::TAY > 1) {
            if (a.cmode) {
                if constexpr (CB % 2 == 0) {
                    if (a.pfast == 2) {
                        // blocks of even and odd cb are the two phases of one
                        // output row: two A fragments per row block
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            const int rofs =
                                (rb_row_offset(rb) + (MY - 1 - ry) * WXP + (MX - 1 - rx)) * RSA;
                            const u32x4 a0 = *reinterpret_cast<const u32x4*>(xs + abase[0] + rofs + kofs);
                            const u32x4 a1 = *reinterpret_cast<const u32x4*>(xs + abase[1] + rofs + kofs);
#pragma unroll
                            for (int cb = 0; cb < CB; ++cb)
                                Mma<TR>::step(acc[rb][cb], (cb & 1) ? a1 : a0, bfr[cb]);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        return;
                    }
                }
                // every (row block, column block) pair reads its own A
                // fragment: one address register per column block, the row
                // block and the tap in the instruction's offset; one row
                // block's fragments live at a time
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int rofs = (rb_row_offset(rb) + (MY - 1 - ry) * WXP + (MX - 1 - rx)) * RSA;
                    u32x4 af[CB];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        af[cb] = *reinterpret_cast<const u32x4*>(xs + abase[cb] + rofs + kofs);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) Mma<TR>::step(acc[rb][cb], af[cb], bfr[cb]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                return;
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            afr[rb] = *reinterpret_cast<const u32x4*>(
                xs + (arow[rb] + (MY - 1 - ry) * WXP + (MX - 1 - rx)) * RSA + kofs);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) Mma<TR>::step(acc[rb][cb], afr[rb], bfr[cb]);
    };
    auto compute = [&](int st) __attribute__((always_inline)) {
        const S* xs = smem + st * C::STAGE;
        const S* bs = xs + C::XROWS * RSA;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int r = 0; r < T; ++r) {
                tap_step(xs, bs, ks * C::KSTEP + lg * VEC, r);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---- main loop over input-channel chunks (two chunks per iteration) ----
    // The fused chunk step: the next chunk's global loads first, the other
    // stage's LDS stores (which wait for loads issued one step earlier) right
    // after the first tap, so that both overlap the remaining MFMAs;
    // scheduling barriers keep the compiler from moving the loads late and
    // their consumers early, which would expose the full memory latency at
    // every step.
    auto fused = [&](int st, auto&& pre, auto&& mid) __attribute__((always_inline)) {
        const S* xs = smem + st * C::STAGE;
        const S* bs = xs + C::XROWS * RSA;
        pre();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int r = 0; r < T; ++r) {
                tap_step(xs, bs, ks * C::KSTEP + lg * VEC, r);
                if (ks == 0 && r == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    mid();
                }
            }
        }
    };

    const int c_begin = blockIdx.y * a.chunks_per_split;
    const int c_end = min(c_begin + a.chunks_per_split, a.n_chunks);
    const int nck = c_end - c_begin;
    if (nck > 0) {
        // Prefetches are issued unconditionally (past the last chunk they
        // re-read it and the values are never stored): a conditional load
        // would make each buffer a merge of old and new registers, which the
        // compiler resolves with copies that wait for the loads in flight.
        const int c_last = c_end - 1;
        // (the fused step keeps both buffers and a tap's fragments live: only
        // instances with at most 8 B fragments per k-step fit without spills)
        if (C::PF == 2 && CB * T <= 8) {
            // two copies of the loop: with and without edge handling in the
            // LDS stores, so that the chunk step has no branch
            auto run = [&](auto inside) __attribute__((always_inline)) {
                gload(c_begin, xr0, br0, cx0);
                gload(min(c_begin + 1, c_last), xr1, br1, cx1);
                lstore(0, xr0, br0, inside, cx0);
                __syncthreads();
                int i = 0;
                for (; i + 2 < nck; i += 2) {
                    // chunk i in stage 0, chunk i+1 in buffer 1; buffer 0 is free
                    fused(
                        0, [&]() __attribute__((always_inline)) { gload(c_begin + i + 2, xr0, br0, cx0); },
                        [&]() __attribute__((always_inline)) { lstore(1, xr1, br1, inside, cx1); });
                    __syncthreads();
                    // chunk i+1 in stage 1, chunk i+2 in buffer 0; buffer 1 is free
                    fused(
                        1,
                        [&]() __attribute__((always_inline)) {
                            gload(min(c_begin + i + 3, c_last), xr1, br1, cx1);
                        },
                        [&]() __attribute__((always_inline)) { lstore(0, xr0, br0, inside, cx0); });
                    __syncthreads();
                }
                if (i + 1 < nck) {
                    fused(
                        0, []() {},
                        [&]() __attribute__((always_inline)) { lstore(1, xr1, br1, inside, cx1); });
                    __syncthreads();
                    fused(1, []() {}, []() {});
                } else {
                    fused(0, []() {}, []() {});
                }
            };
            if (wave_inside)
                run(std::true_type{});
            else
                run(std::false_type{});
        } else if constexpr (C::PF == 2) {
            gload(c_begin, xr0, br0, cx0);
            gload(min(c_begin + 1, c_last), xr1, br1, cx1);
            lstore(0, xr0, br0, std::false_type{}, cx0);
            __syncthreads();
            // Steady state: chunks i and i+1 with at least one more chunk after
            // them, so every store below is unconditional (a skipped store
            // would leave its loads "in flight" for the compiler at the loop
            // head, where it then waits for every load).
            int i = 0;
            for (; i + 2 < nck; i += 2) {
                // chunk i in stage 0; buffer 0 is free, buffer 1 holds chunk i+1
                gload(c_begin + i + 2, xr0, br0, cx0);
                compute(0);
                lstore(1, xr1, br1, std::false_type{}, cx1);
                __syncthreads();
                // chunk i+1 in stage 1; buffer 1 is free, buffer 0 holds chunk i+2
                gload(min(c_begin + i + 3, c_last), xr1, br1, cx1);
                compute(1);
                lstore(0, xr0, br0, std::false_type{}, cx0);
                __syncthreads();
            }
            // last one or two chunks: chunk i in stage 0, chunk i+1 in buffer 1
            compute(0);
            if (i + 1 < nck) {
                lstore(1, xr1, br1, std::false_type{}, cx1);
                __syncthreads();
                compute(1);
            }
        } else {
            // one register buffer: chunk c+1 is loaded during the MFMAs of
            // chunk c and stored to the other stage after them
            gload(c_begin, xr0, br0, cx0);
            lstore(0, xr0, br0, std::false_type{}, cx0);
            __syncthreads();
            int i = 0;
            for (; i + 2 < nck; i += 2) {
                gload(c_begin + i + 1, xr0, br0, cx0);
                compute(0);
                lstore(1, xr0, br0, std::false_type{}, cx0);
                __syncthreads();
                gload(c_begin + i + 2, xr0, br0, cx0);
                compute(1);
                lstore(0, xr0, br0, std::false_type{}, cx0);
                __syncthreads();
            }
            if (i + 1 < nck) {
                gload(c_begin + i + 1, xr0, br0, cx0);
                compute(0);
                lstore(1, xr0, br0, std::false_type{}, cx0);
                __syncthreads();
                compute(1);
            } else {
                compute(0);
            }
        }
    }
    // the output staging below reuses the operand stages: every wave must be
    // done reading them
    __syncthreads();

    // ---- fp32 outputs straight from the accumulators (1-D, no padding
    // shift classes or reduction: the chunks of a 16-bit stream, whose
    // outputs are few): one 4-byte store per element, rounded nowhere
    if (a.outf32) {
        if constexpr (C::TAY == 1) {
            float* __restrict__ yf = static_cast<float*>(a.y);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                int pb, co_l;
                col_map(bcol + cb * 16, pb, co_l);
                const int b = b0 + pb, co = co0 + co_l;
                if (pb >= a.PT || b >= a.P || co_l >= a.TCO || co >= a.C_out) continue;
                float* yrow = yf + (n * a.C_out + co) * a.WoR;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t ax = ax0 + (wm * RB + rb) * 16 + lg * 4 + i;
                        const int64_t ox = ax * a.sx + b - a.oxs;
                        if (ox >= 0 && ox < a.WoR) yrow[ox] = acc[rb][cb][i] + bvs[cb];
                    }
            }
        }
        return;
    }

    // ---- epilogue: bias, round, stage in output order, store ---------------
    // staged rows per output channel: the tile's positions (phase subsets,
    // whose phases go to the columns) or its output rows
    const int R = a.phase_subset ? C::TAY * TAX : C::TAY * a.sy;
    const int SS = a.phase_subset ? a.PT : TAX * a.sx;
    // output-channel stride padded by 16 bytes: lanes of one MFMA column block
    // hold consecutive output channels, so an unpadded power-of-two stride
    // would put all 16 of their staging writes in one LDS bank
    const int CSTR = R * SS + VEC;
    // The output staging, compiled once without and once with the fused
    // activation (applied in fp32 after the bias, before the one rounding).
    auto stage_all = [&](auto act_tag) __attribute__((always_inline)) {
        auto actf = [](float v) __attribute__((always_inline)) {
            if constexpr (decltype(act_tag)::value) return elu_act<TR>(v);
            else return v;
        };
        // Column block cb holds 16 consecutive output channels of one phase when
        // TCO is a multiple of 16 (every shape but the narrow and phase-subset
        // ones): its phase, channel base and row offsets are wave-uniform, and
        // block cb + TCO/16 holds the next phase of the same channels, i.e. the
        // next output element of a row, so the two values go out as one 4-byte
        // LDS write when both phases sit in the same output row.
        auto stage_pairs = [&](auto step_tag) __attribute__((always_inline)) {
            constexpr int STEP = decltype(step_tag)::value;  // TCO / 16 (0: no pairing)
            const int T0 = wm * RB * 16;
    #pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int blk = wn * CB + cb;
                const int pb = (int)uniform(fdiv((uint32_t)(blk * 16), a.fd_tco));
                if (pb >= a.PT) continue;
                const int co_l = blk * 16 - pb * a.TCO + li;
                const int by = (int)fdiv((uint32_t)pb, a.fd_sx), bx = pb - by * a.sx;
                // Blocks pair up as (cb, cb + STEP) for (cb / STEP) even; a pair is
                // written together when the second block exists in the wave, holds
                // a phase of the tile and that phase continues the same output row.
                constexpr bool CAN = STEP > 0 && STEP < CB;
                const bool first = CAN && ((cb / (CAN ? STEP : 1)) % 2 == 0) && cb + STEP < CB;
                const bool second = CAN && ((cb / (CAN ? STEP : 1)) % 2 == 1);
                const int cbp = first ? cb + STEP : cb;
                const bool pair = first && pb + 1 < a.PT && bx + 1 < a.sx;
                if (second && (pb - 1) - (int)fdiv((uint32_t)(pb - 1), a.fd_sx) * a.sx + 1 < a.sx)
                    continue;  // written together with the previous phase's block
                const float bv = bvs[cb];
                // element offsets: lane part + wave-uniform part
                const int lane_base = co_l * CSTR + lg * 4 * a.sx;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int t = T0 + rb * 16;
                    const int rowpart = (int)uniform(
                        (uint32_t)(((t / TAX) * a.sy + by) * SS + (t % TAX) * a.sx + bx));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ui = (int)uniform((uint32_t)(rowpart + i * a.sx));
                        const int off = lane_base + ui;
                        const float f0 = actf(acc[rb][cb][i] + bv);
                        if (pair) {
                            const float f1 = actf(acc[rb][cbp][i] + bv);
                            if constexpr (sizeof(S) == 2) {
                                // one 4-byte LDS store when the pair starts on an
                                // even element (the parity of off is that of ui:
                                // wave-uniform), else two 2-byte stores
                                const uint32_t pk = pack2<TR>(f0, f1);
                                if ((ui & 1) == 0) {
                                    *reinterpret_cast<uint32_t*>(smem + off) = pk;
                                } else {
                                    smem[off] = (S)(pk & 0xFFFFu);
                                    smem[off + 1] = (S)(pk >> 16);
                                }
                            } else {
                                smem[off] = f0;
                                smem[off + 1] = f1;
                            }
                        } else {
                            smem[off] = TR::from_f32(f0);
                        }
                    }
                }
            }
        };
        // Phase-fastest columns: the blocks of a wave are consecutive phases
        // of one 16-channel group, so for each of its row blocks a lane holds
        // runs of consecutive staged elements of one channel row:
        //  - whole rows of phases (sx phases b_x of output row b_y): the 4
        //    rows q (MFMA rows 4 lg .. 4 lg + 3) times sx phases are 4 sx
        //    consecutive elements;
        //  - CB consecutive phases of a longer row (sx > CB): CB consecutive
        //    elements per row q.
        // Each run is rounded and written with 8- or 16-byte LDS stores (the
        // run starts are 8-byte aligned: the channel stride is a multiple of
        // 16 bytes and a run starts at a multiple of 4 sx, or of CB, elements).
        auto stage_runs = [&](auto sx_tag) __attribute__((always_inline)) {
            constexpr int SXC = decltype(sx_tag)::value;  // 0: runs of CB phases per row q
            constexpr int STEP = SXC > 0 ? SXC : CB;
            constexpr int L = SXC > 0 ? 4 * SXC : CB;     // elements per run
            static_assert(sizeof(S) == 4 || L % 4 == 0 || SXC % 2 == 1, "run shape");
            auto put = [&](const float* v, int off) __attribute__((always_inline)) {
                S* d = smem + off;
                if constexpr (sizeof(S) == 2) {
                    uint32_t w[(L + 1) / 2];
#pragma unroll
                    for (int e = 0; e < L / 2; ++e) w[e] = pack2<TR>(v[2 * e], v[2 * e + 1]);
                    if constexpr (L % 2 == 1) w[L / 2] = (uint32_t)TR::from_f32(v[L - 1]);
                    if constexpr (SXC % 2 == 0 && SXC > 0) {
                        // 16-byte aligned runs of 8 or 16 elements
#pragma unroll
                        for (int e = 0; e < L / 2; e += 4)
                            *reinterpret_cast<u32x4*>(d + 2 * e) = u32x4{w[e], w[e + 1], w[e + 2], w[e + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e + 2 <= L / 2; e += 2)
                            *reinterpret_cast<u32x2*>(d + 2 * e) = u32x2{w[e], w[e + 1]};
                        if constexpr ((L / 2) % 2 == 1)
                            *reinterpret_cast<uint32_t*>(d + L - 2) = w[L / 2 - 1];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e + 2 <= L; e += 2)
                        *reinterpret_cast<u32x2*>(d + e) = u32x2{__float_as_uint(v[e]), __float_as_uint(v[e + 1])};
                    if constexpr (L % 2 == 1) d[L - 1] = v[L - 1];
                }
            };
#pragma unroll
            for (int cb0 = 0; cb0 < CB; cb0 += STEP) {
                int pb, co_b;
                col_map((wn * CB + cb0) * 16, pb, co_b);
                pb = (int)uniform((uint32_t)pb);
                co_b = (int)uniform((uint32_t)co_b);
                if (co_b >= a.TCO || pb >= a.PT) continue;  // padding blocks
                const int by = (int)uniform(fdiv((uint32_t)pb, a.fd_sx)), bx0 = pb - by * a.sx;
                const int chan = (co_b + li) * CSTR;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int t0 = (wm * RB + rb) * 16 + 4 * lg;
                    const int rr = (t0 / TAX) * a.sy + by, tx0 = t0 % TAX;
                    if constexpr (SXC > 0) {
                        float v[L];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int bx = 0; bx < SXC; ++bx)
                                v[i * SXC + bx] = actf(acc[rb][cb0 + bx][i] + bvs[cb0 + bx]);
                        put(v, chan + rr * SS + tx0 * SXC);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float v[L];
#pragma unroll
                            for (int j = 0; j < CB; ++j) v[j] = actf(acc[rb][j][i] + bvs[j]);
                            put(v, chan + rr * SS + (tx0 + i) * a.sx + bx0);
                        }
                    }
                }
            }
        };
        if (a.pfast) {
            // the planner sets pfast only for the layouts handled here
            if (a.sx > CB) {
                if constexpr (sizeof(S) == 4 || CB % 4 == 0) stage_runs(std::integral_constant<int, 0>{});
            } else if (a.sx == 1) {
                stage_runs(std::integral_constant<int, 1>{});
            } else if (a.sx == 2) {
                if constexpr (CB % 2 == 0) stage_runs(std::integral_constant<int, 2>{});
            } else if (a.sx == 4) {
                if constexpr (CB % 4 == 0) stage_runs(std::integral_constant<int, 4>{});
            } else if (a.sx == 5) {
                if constexpr (CB % 5 == 0) stage_runs(std::integral_constant<int, 5>{});
            }
        } else if (!a.phase_subset && (a.TCO & 15) == 0 && a.TCO / 16 == 1) {
            stage_pairs(std::integral_constant<int, 1>{});
        } else if (!a.phase_subset && (a.TCO & 15) == 0 && a.TCO / 16 == 2) {
            stage_pairs(std::integral_constant<int, 2>{});
        } else if (!a.phase_subset && (a.TCO & 15) == 0) {
            stage_pairs(std::integral_constant<int, 0>{});
        } else {
        #pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int tc = bcol + cb * 16;
                const int pb = (int)fdiv((uint32_t)tc, a.fd_tco), co_l = tc - pb * a.TCO;
                if (pb >= a.PT) continue;
                const float bv = bvs[cb];
                const int by = (int)fdiv((uint32_t)pb, a.fd_sx), bx = pb - by * a.sx;
        #pragma unroll
                for (int rb = 0; rb < RB; ++rb)
        #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tr = (wm * RB + rb) * 16 + lg * 4 + i;
                        const int ayl = tr / TAX, axl = tr % TAX;
                        int rr, ss;
                        if (a.phase_subset) {
                            rr = tr;  // = axl in 1-D
                            ss = pb;
                        } else {
                            rr = ayl * a.sy + by;
                            ss = axl * a.sx + bx;
                        }
                        smem[co_l * CSTR + rr * SS + ss] = TR::from_f32(actf(acc[rb][cb][i] + bv));
                    }
            }
        }
    };
    // (a launch that adds to y applies the activation after its sum, below)
    if (a.act == CTCONV_ACT_ELU && !a.accum)
        stage_all(std::true_type{});
    else
        stage_all(std::false_type{});
    __syncthreads();

    // split s > 0 of a split reduction writes its partial sums to slab s - 1
    S* __restrict__ yg = (a.partial && blockIdx.y > 0)
                             ? reinterpret_cast<S*>(a.ws + (int64_t)(blockIdx.y - 1) * a.ws_slab)
                             : static_cast<S*>(a.y);
    const int nrows = a.TCO * R;
    // (a dilation-reduced problem writes every g-th output: element stores)
    const bool vec_ok = (SS % VEC) == 0 && a.gx == 1 && a.gy == 1;
    if (vec_ok && !a.phase_subset) {
        // Flattened over the tile: chunk e (VEC elements) is row e / cpr,
        // column chunk e % cpr of the staged output, so consecutive lanes
        // take consecutive chunks (a short row does not idle a wave's other
        // lanes) and each thread reads U chunks from LDS before it stores
        // them (one LDS latency per U stores).
        const int cpr = SS / VEC;
        const int total = nrows * cpr;
        // staged columns [lo, lim) of a row are real outputs (the padding
        // shift makes the first tile's leading ones negative)
        const int64_t ox0 = (int64_t)ax0 * a.sx - a.oxs;
        const int lo = ox0 < 0 ? (int)(-ox0) : 0;
        const int lim = (int)min((int64_t)SS, a.WoR - ox0);
        constexpr int U = 4;
        for (int e0 = tid; e0 < total; e0 += U * C::NT) {
            u32x4 v[U];
            int64_t gb[U];
            int s0v[U], sof[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = e0 + u * C::NT;
                const int ec = e < total ? e : 0;
                const int row = (int)fdiv((uint32_t)ec, a.fd_cpr);
                const int s0 = (ec - row * cpr) * VEC;
                const int co_l = (int)fdiv((uint32_t)row, a.fd_R), rr = row - co_l * R;
                const int co = co0 + co_l;
                const int64_t oy = (int64_t)ay0 * a.sy + rr - a.oys;
                ok[u] = e < total && co < a.C_out && oy >= 0 && oy < a.HoR && s0 < lim &&
                        s0 + VEC > lo;
                sof[u] = co_l * CSTR + rr * SS;
                s0v[u] = s0;
                gb[u] = ((n * a.C_out + co) * a.HoR + oy) * a.WoR + ox0;
                v[u] = *reinterpret_cast<const u32x4*>(smem + sof[u] + s0);
            }
            if constexpr (sizeof(S) == 4) {
                if (a.accum) {
                    // a later tap group: y += the staged sums (then the
                    // activation, in the last group)
                    const bool elu = a.act == CTCONV_ACT_ELU;
                    auto fin = [&](float o, float t) __attribute__((always_inline)) {
                        const float r = o + t;
                        return elu ? elu_act<TR>(r) : r;
                    };
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        if (!ok[u]) continue;
                        const int s0 = s0v[u];
                        const int qb = s0 < lo ? lo : s0, qe = s0 + VEC < lim ? s0 + VEC : lim;
                        for (int q = qb; q < qe; ++q)
                            yg[gb[u] + q] = fin(yg[gb[u] + q], smem[sof[u] + q]);
                    }
                    continue;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!ok[u]) continue;
                const int s0 = s0v[u];
                if (s0 >= lo && s0 + VEC <= lim) {
                    store16_unaligned(yg + gb[u] + s0, v[u]);
                } else {
                    const int qe = s0 + VEC < lim ? s0 + VEC : lim;
                    for (int q = s0 < lo ? lo : s0; q < qe; ++q) yg[gb[u] + q] = smem[sof[u] + q];
                }
            }
        }
        return;
    }
    if (C::TAY > 1 && a.phase_subset) {
        // 2-D phase subsets: the staged row of a position holds its phases
        // b0 .. b0 + PT - 1, which lie in different output rows: element
        // stores, each thread taking consecutive staged elements
        const int64_t Hc = a.Ho - a.oys, Wc = a.Wo - a.oxs;
        const int total = nrows * SS;
        for (int idx = tid; idx < total; idx += C::NT) {
            const int row = (int)fdiv((uint32_t)idx, a.fd_pt), e = idx - row * SS;
            const int b = b0 + e;
            const int co_l = (int)fdiv((uint32_t)row, a.fd_R), rr = row - co_l * R;
            const int co = co0 + co_l;
            if (b >= a.P || co >= a.C_out) continue;
            const int by = (int)fdiv((uint32_t)b, a.fd_sx), bx = b - by * a.sx;
            const int64_t oy = (int64_t)(ay0 + rr / TAX) * a.sy + by - a.oys;
            const int64_t ox = (int64_t)(ax0 + rr % TAX) * a.sx + bx - a.oxs;
            if (oy < 0 || oy >= Hc || ox < 0 || ox >= Wc) continue;
            yg[((n * a.C_out + co) * a.HoR + (a.o0y + a.gy * oy)) * a.WoR + a.o0x + a.gx * ox] =
                smem[co_l * CSTR + rr * SS + e];
        }
        return;
    }
    for (int row = wave; row < nrows; row += C::NW) {
        const int co_l = (int)fdiv((uint32_t)row, a.fd_R), rr = row - co_l * R;
        const int co = co0 + co_l;
        if (co >= a.C_out) continue;
        // output sizes of the padded problem (the dilation-reduced one under
        // dilation); the staged indices are shifted back by the padding
        const int64_t Hc = a.Ho - a.oys, Wc = a.Wo - a.oxs;
        int64_t oy, ox0;
        int lo, lim;  // valid elements [lo, lim) of this staged row
        if (a.phase_subset) {
            oy = 0;
            ox0 = (int64_t)(ax0 + rr) * a.sx + b0 - a.oxs;
            lim = min(SS, a.P - b0);
        } else {
            oy = (int64_t)ay0 * a.sy + rr - a.oys;
            ox0 = (int64_t)ax0 * a.sx - a.oxs;
            if (oy < 0 || oy >= Hc) continue;
            lim = SS;
        }
        lo = ox0 < 0 ? (int)min((int64_t)lim, -ox0) : 0;
        if (ox0 + lim > Wc) lim = (int)max((int64_t)0, Wc - ox0);
        if (lim <= lo) continue;
        // staged (reduced) row -> real output row o0 + g * index per dimension
        const int64_t gbase =
            ((n * a.C_out + co) * a.HoR + (a.o0y + a.gy * oy)) * a.WoR + a.o0x + a.gx * ox0;
        const S* srow = smem + co_l * CSTR + rr * SS;
        if (vec_ok) {
            for (int s0 = lane * VEC; s0 < lim; s0 += 64 * VEC) {
                if (s0 >= lo && s0 + VEC <= lim) {
                    store16_unaligned(yg + gbase + s0, *reinterpret_cast<const u32x4*>(srow + s0));
                } else {
                    const int ee = s0 + VEC < lim ? s0 + VEC : lim;
                    for (int e = s0 < lo ? lo : s0; e < ee; ++e) yg[gbase + e] = srow[e];
                }
            }
        } else {
            if (a.gx == 1) {
                for (int e = lo + lane; e < lim; e += 64) yg[gbase + e] = srow[e];
            } else {
                // every gx-th output of the real row (dilation-reduced problem)
                S* yrow = yg + gbase;
                for (int e = lo + lane; e < lim; e += 64) yrow[e * a.gx] = srow[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side planning
// ---------------------------------------------------------------------------

using KernelFn = void (*)(const PolyArgs);

struct Inst {
    KernelFn fn;
    int BM, BN, TAX, TAY, KC, threads, lds_bytes;
    int cb;  // 16-column blocks per wave
};

template <class TR, int MY, int MX, int TAX, int RB, int CB, int WM, int WN, int KS,
          bool XODD = false>
Inst make_inst() {
    using C = Cfg<TR, MY, MX, TAX, RB, CB, WM, WN, KS>;
    return Inst{&poly_kernel<TR, MY, MX, TAX, RB, CB, WM, WN, KS, XODD>, C::BM, C::BN, TAX,
                C::TAY, C::KC, C::NT, (int)(C::SMEM * C::ES), CB};
}

// Tile shapes.  16-bit storage, 1-D with one or two taps: 128 output rows x
// 128 columns (x 160 for five-phase shapes), four waves of 64 x 64 (64 x 80),
// two workgroups per CU so that one's setup, first loads and epilogue overlap
// the other's chunk loop; three or four taps: 256 rows, eight waves, one
// workgroup per CU; 2-D: 4 x 64 rows x 128 columns, eight waves of 64 x 64.
// fp32: 128 x 128 with eight waves of 64 x 32.
template <class TR, int MY, int MX, int CB, bool XO>
Inst inst_1d() {
    if constexpr (sizeof(typename TR::storage) == 2) {
        if constexpr (MY * MX <= 2)
            return make_inst<TR, MY, MX, 128, 4, CB, 2, 2, 1, XO>();
        else
            // three or four taps: a 4-wave tile would stage twice the weight
            // rows per wave and drop to one wave per SIMD
            return make_inst<TR, MY, MX, 256, 4, CB, 4, 2, 1, XO>();
    } else {
        return make_inst<TR, MY, MX, 128, 4, 2, 2, 4, 1, XO>();
    }
}

template <class TR, int MY, int MX, bool XO>
Inst inst_2d() {
    if constexpr (sizeof(typename TR::storage) == 2) {
        return make_inst<TR, MY, MX, 64, 4, 4, 4, 2, 1, XO>();
    } else {
        return make_inst<TR, MY, MX, 32, 4, 2, 2, 4, 1, XO>();
    }
}

template <class TR, bool XO>
bool pick_inst_x(const Problem& p, int CB, Inst* out) {
    if (p.ndim == 1) {
        if (CB == 5 && sizeof(typename TR::storage) == 2) {
            switch (p.mW) {
                case 1: *out = inst_1d<TR, 1, 1, 5, XO>(); return true;
                case 2: *out = inst_1d<TR, 1, 2, 5, XO>(); return true;
                case 3: *out = inst_1d<TR, 1, 3, 5, XO>(); return true;
                case 4: *out = inst_1d<TR, 1, 4, 5, XO>(); return true;
            }
            return false;
        }
        switch (p.mW) {
            case 1: *out = inst_1d<TR, 1, 1, 4, XO>(); return true;
            case 2: *out = inst_1d<TR, 1, 2, 4, XO>(); return true;
            case 3: *out = inst_1d<TR, 1, 3, 4, XO>(); return true;
            case 4: *out = inst_1d<TR, 1, 4, 4, XO>(); return true;
        }
        return false;
    }
    if (p.mH == 1 && p.mW == 1) { *out = inst_2d<TR, 1, 1, XO>(); return true; }
    if (p.mH == 1 && p.mW == 2) { *out = inst_2d<TR, 1, 2, XO>(); return true; }
    if (p.mH == 2 && p.mW == 1) { *out = inst_2d<TR, 2, 1, XO>(); return true; }
    if (p.mH == 2 && p.mW == 2) { *out = inst_2d<TR, 2, 2, XO>(); return true; }
    // 3 x 3 taps (a 3 x 3 kernel at stride 1: dilation 2 at stride 2):
    // 128 x 64 tiles, eight waves of 64 x 16, so that two stages of nine
    // taps' weight rows fit in LDS
    if (p.mH == 3 && p.mW == 3) {
        *out = make_inst<TR, 3, 3, 32, 4, 1, 2, 4, 1, XO>();
        return true;
    }
    return false;
}

// 16-bit types with odd input rows take the XODD instances; fp32 pieces are
// always dword aligned
template <class TR>
bool pick_inst(const Problem& p, int CB, Inst* out) {
    if constexpr (sizeof(typename TR::storage) == 2) {
        if (p.W % 2 == 1) return pick_inst_x<TR, true>(p, CB, out);
    }
    return pick_inst_x<TR, false>(p, CB, out);
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

// Fill PolyArgs for problem p (no dilation; no padding unless cmode); false
// when no kernel instance covers it.  cmode: phase rows aligned to the
// output, each 16-column block one phase with its own input offset.
// allow_split: the reduction may be split over workgroups (a workspace holds
// the partial sums of all splits but the first).
bool plan_core(const Problem& p, PolyArgs* a, Inst* inst, int* splits, bool allow_split,
               bool cmode) {
    if (p.dH != 1 || p.dW != 1) return false;
    if (!cmode && (p.pH != 0 || p.pW != 0)) return false;
    if (p.H == 0 || p.W == 0 || p.N == 0) return false;
    // every staged x load covers 8 bytes of one input row
    if (p.W * (p.dtype == CTCONV_F32 ? 4 : 2) < 8) return false;
    const int64_t P = p.P;

    // Column tiling: TCO output channels x PT phases per tile.
    int CB = (p.ndim == 1 && P % 5 == 0 && P * 16 <= 160) ? 5 : 4;
    Inst in;
    if (!get_inst(p, CB, &in)) return false;
    const int64_t BN = in.BN;
    int64_t TCO, PT;
    int subset = 0;
    const bool narrow = p.C_out < 16;  // blocks may span phases
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
    } else if (p.ndim == 1) {
        subset = 1;
        TCO = tco_min;
        PT = BN / TCO;
    } else {
        // 2-D with more phases than a column tile holds (s = 3: 9, s = 4:
        // 16): tiles of PT whole phases x TCO channels, TCO (a multiple of
        // 16 dividing BN) chosen for the fewest column tiles
        if (narrow) return false;
        const int64_t cpad = (p.C_out + 15) / 16 * 16;
        int64_t best = -1;
        for (int64_t t = 16; t <= BN && t <= cpad; t += 16) {
            if (BN % t != 0) continue;
            const int64_t cost = ((p.C_out + t - 1) / t) * ((P + BN / t - 1) / (BN / t));
            if (best < 0 || cost < best) {
                best = cost;
                TCO = t;
            }
        }
        if (best < 0) return false;
        subset = 1;
        PT = BN / TCO;
    }
    if (TCO < 1 || PT < 1) return false;
    // class mode reads A fragments per 16-column block: one phase per block;
    // compiled into the 2-D instances only (1-D shapes lose at most one tile
    // per batch item to the padding shift)
    if (cmode && (narrow || subset || in.TAY == 1)) return false;
    const int spready = cmode && p.pH % p.sH != 0 ? 1 : 0;
    const int spreadx = cmode && p.pW % p.sW != 0 ? 1 : 0;
    if (spready && in.TAY == 1) return false;  // (1-D tiles have one window row)
    const int64_t n_co_tiles = (p.C_out + TCO - 1) / TCO;
    const int64_t n_ph_tiles = (P + PT - 1) / PT;
    const int64_t Ay = (p.Ho + p.sH - 1) / p.sH, Ax = (p.Wo + p.sW - 1) / p.sW;
    const int64_t tiles_y = (Ay + in.TAY - 1) / in.TAY, tiles_x = (Ax + in.TAX - 1) / in.TAX;
    const int64_t n_row_tiles = p.N * tiles_y * tiles_x;
    const int64_t n_col_tiles = n_co_tiles * n_ph_tiles;
    // chunks must tile the packed channel padding exactly (a chunk past it
    // would read beyond the packed weight)
    if (p.C_in_pad % in.KC != 0) return false;
    // loads address the packed weight through a 32-bit byte offset
    const int64_t pw_bytes = P * p.C_out * p.T * p.C_in_pad * (p.dtype == CTCONV_F32 ? 4 : 2);
    if (pw_bytes > (int64_t)0xFFFFFFFFLL) return false;
    const int64_t n_chunks = p.C_in_pad / in.KC;
    if (n_row_tiles * n_col_tiles > kInt32Max || P > kInt32Max / 2 || p.C_out > kInt32Max / 2 ||
        Ax > kInt32Max / 2 || Ay > kInt32Max / 2 || n_chunks > kInt32Max ||
        p.H * p.W > kInt32Max / 2 || p.Wo > kInt32Max / 2 || p.Ho > kInt32Max / 2)
        return false;
    // x staging uses 32-bit byte offsets within one image
    if (p.C_in_pad * p.H * p.W * (p.dtype == CTCONV_F32 ? 4 : 2) > (int64_t)4000000000LL) return false;

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
    a->cmode = cmode ? 1 : 0;
    a->dminy = (int)(p.pH / p.sH);
    a->dminx = (int)(p.pW / p.sW);
    a->P = (int)P;
    a->T = (int)p.T;
    a->Ay = (int)Ay;
    a->Ax = (int)Ax;
    a->WY = in.TAY + (int)p.mH - 1 + spready;
    a->WX = in.TAX + (int)p.mW - 1 + spreadx;
    {
        // Rows a multiple of 4 bytes long start dword aligned (x itself is
        // 16-byte aligned), so a window start at a multiple of NP positions
        // makes every x load dword aligned (8-byte aligned when rows are a
        // multiple of 8 bytes).  Tile starts are multiples of 16, so the
        // shift is the same for every tile.
        const int es = p.dtype == CTCONV_F32 ? 4 : 2, np = 8 / es;
        const int w0 = a->dminx - ((int)p.mW - 1);
        a->xofs = (p.W * es) % 4 == 0 ? ((w0 % np) + np) % np : 0;
    }
    a->TCO = (int)TCO;
    a->PT = (int)PT;
    a->phase_subset = subset;
    {
        // phase-fastest columns and run staging of the epilogue, for the
        // layouts it handles: every phase in the tile, 16-channel groups,
        // staged rows a whole number of 16-byte chunks
        // (the flattened stores) and per wave either whole output rows of
        // phases (sx dividing CB) or CB consecutive phases of a row
        const int cb = in.cb;
        const int64_t sx = p.sW;
        const bool es2 = p.dtype != CTCONV_F32;
        const bool rows = (sx == 1 || sx == 2 || sx == 4 || sx == 5) && sx <= cb && cb % sx == 0 &&
                          (cb % P == 0 || P % cb == 0);
        const bool part = sx > cb && sx % cb == 0 && P % cb == 0 && (!es2 || cb % 4 == 0);
        const int64_t vec = es2 ? 8 : 4;
        a->pfast = (!subset && !narrow && TCO % 16 == 0 && PT == P &&
                    (in.TAX * sx) % vec == 0 && (rows || part))
                       ? 1 : 0;
        a->fd_pt = make_fastdiv((uint32_t)PT);
    }
    a->n_ph_tiles = (int)n_ph_tiles;
    a->n_col_tiles = (int)n_col_tiles;
    a->tiles_y = (int)tiles_y;
    a->tiles_x = (int)tiles_x;
    a->n_row_tiles = n_row_tiles;
    a->n_chunks = (int)n_chunks;

    // Split the C_in reduction when the tile grid leaves CUs idle (fp32 only,
    // with a workspace for the partial sums).  Choose the split that
    // minimises (rounds of workgroups) x (chunks per workgroup).
    const int64_t tiles = n_row_tiles * n_col_tiles;
    int64_t per_cu = (160 * 1024) / in.lds_bytes;
    if (per_cu > 512 / in.threads) per_cu = 512 / in.threads;
    if (per_cu < 1) per_cu = 1;
    const int64_t slots = 256 * per_cu;
    int best = 1;
    // (the reduction kernel adds the bias and applies the activation)
    if (allow_split && p.dtype == CTCONV_F32 && tiles < 2 * slots && n_chunks >= 8) {
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
    a->partial = best > 1 ? 1 : 0;
    a->ws = nullptr;
    a->ws_slab = p.N * p.C_out * p.Ho * p.Wo;
    a->xcd_remap = (tiles % 8 == 0) ? 1 : 0;
    {
        // Tile order: every row tile reads its input rows over all of C_in,
        // every column tile its weight rows.  An XCD's resident tiles are a
        // contiguous run of the order, so they share the operand that varies
        // slowest along it: row-major shares the input rows and needs every
        // column tile's weights, column-major the reverse.  Take the order
        // that keeps the larger operand shared (the iSTFT basis, 67 MB
        // against 45 MB of frames, halves the kernel's fetched bytes that
        // way).  fp32 only: the 16-bit instances are compiled row-major.
        const int64_t w_bytes = P * p.C_out * p.T * p.C_in_pad * 4;
        const int64_t x_bytes = p.N * p.C_in_pad * p.H * p.W * 4;
        a->colmajor = p.dtype == CTCONV_F32 && w_bytes > x_bytes ? 1 : 0;
    }
    a->n_tiles = (uint32_t)tiles;
    a->fd_cols = make_fastdiv((uint32_t)n_col_tiles);
    a->fd_rows = make_fastdiv((uint32_t)n_row_tiles);
    a->fd_ph = make_fastdiv((uint32_t)n_ph_tiles);
    a->fd_tx = make_fastdiv((uint32_t)tiles_x);
    a->fd_ty = make_fastdiv((uint32_t)tiles_y);
    a->fd_wy = make_fastdiv((uint32_t)a->WY);
    a->fd_tco = make_fastdiv((uint32_t)TCO);
    a->fd_sx = make_fastdiv((uint32_t)p.sW);
    a->fd_sy = make_fastdiv((uint32_t)p.sH);
    a->fd_R = make_fastdiv((uint32_t)(subset ? in.TAY * in.TAX : in.TAY * p.sH));
    {
        // staged-row chunks of 16 bytes (flattened output stores)
        const int64_t vec = p.dtype == CTCONV_F32 ? 4 : 8;
        const int64_t cpr = (in.TAX * p.sW) / vec;
        a->fd_cpr = make_fastdiv((uint32_t)(cpr > 0 ? cpr : 1));
    }
    a->pw_bytes = (uint32_t)pw_bytes;
    a->act = p.act;
    *inst = in;
    *splits = best;
    return true;
}

// Dilation, per dimension, in two steps.
//  1. Reduction by g = gcd(s, d): output o = i s - p + t d receives a tap
//     only when g divides o + p.  Those outputs, u = (o + p) / g, form the
//     transposed convolution with stride s' = s / g and dilation d' = d / g.
//     Counting them from the first one, o0 = (g - p mod g) mod g, gives
//     u' = (o - o0) / g and left padding (o0 + p) / g; the other outputs hold
//     the bias alone.
//  2. Expansion of the remaining dilation d' (coprime to s'): the kernel runs
//     the undilated transposed convolution whose kernel has (k - 1) d' + 1
//     taps, tap e being real tap e / d' when d' divides e and zero otherwise
//     (the kernel reads the packed weight through that map).
// Without dilation the problem is returned unchanged (g = d' = 1).
struct Reduced {
    Problem q;    // the problem the kernel runs (dilation 1)
    int g[2];     // output step per dimension (y, x)
    int o0[2];    // first reached output per dimension
    int de[2];    // tap spacing d' of the expanded kernel per dimension
};

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

bool reduce_dilation(const Problem& p, Reduced* r) {
    r->q = p;
    auto one = [](int64_t d, int64_t s, int64_t pad, int64_t L, int64_t k, int64_t* s2,
                  int64_t* pad2, int64_t* L2, int64_t* k2, int64_t* m2, int* g_out, int* o0,
                  int* de) {
        *g_out = 1;
        *o0 = 0;
        *de = 1;
        if (d == 1) return true;
        if (d < 1 || s < 1 || k < 1) return false;
        const int64_t g = gcd64(s, d);
        const int64_t first = (g - pad % g) % g;
        *g_out = (int)g;
        *o0 = (int)first;
        *de = (int)(d / g);
        *s2 = s / g;
        *pad2 = (first + pad) / g;
        *L2 = L > first ? (L - first + g - 1) / g : 0;
        *k2 = (k - 1) * (d / g) + 1;
        *m2 = (*k2 + *s2 - 1) / *s2;
        return true;
    };
    Problem& q = r->q;
    if (!one(p.dH, p.sH, p.pH, p.Ho, p.kH, &q.sH, &q.pH, &q.Ho, &q.kH, &q.mH, &r->g[0], &r->o0[0],
             &r->de[0]))
        return false;
    if (!one(p.dW, p.sW, p.pW, p.Wo, p.kW, &q.sW, &q.pW, &q.Wo, &q.kW, &q.mW, &r->g[1], &r->o0[1],
             &r->de[1]))
        return false;
    q.dH = q.dW = 1;
    q.opH = q.opW = 0;  // the reduced output sizes are set directly
    q.P = q.sH * q.sW;
    q.T = q.mH * q.mW;
    return true;
}

// Fill PolyArgs for problem p (any dilation).  A problem with a reduction
// step (g > 1) is never split (its unreached outputs hold the pre-filled
// bias, which a split's partial sums would overwrite).
bool plan(const Problem& p, PolyArgs* a, Inst* inst, int* splits, bool allow_split) {
    Reduced rd;
    if (!reduce_dilation(p, &rd)) return false;
    Problem& q = rd.q;
    const bool reduced = rd.g[0] > 1 || rd.g[1] > 1;
    // Tap groups: fp32 shapes (without a dilation reduction) with more taps
    // per phase than the compiled instances (1-D: 4; 2-D: 2 x 2, or 3 x 3)
    // run as a sequence of launches of at most that many tap slots each
    int gmy = 0, gmx = 0;
    const int64_t mH0 = q.mH, mW0 = q.mW;
    if (!reduced && p.dtype == CTCONV_F32) {
        if (q.ndim == 1 && q.mW > 4) {
            gmy = 1;
            gmx = 4;
        } else if (q.ndim == 2 && (q.mH > 2 || q.mW > 2) && !(q.mH == 3 && q.mW == 3)) {
            gmy = q.mH > 2 ? 2 : (int)q.mH;
            gmx = q.mW > 2 ? 2 : (int)q.mW;
        }
    }
    const bool grouped = gmx > 0;
    if (grouped) {
        q.mH = gmy;
        q.mW = gmx;
        q.T = q.mH * q.mW;
        allow_split = false;
    }
    // Padding as an output shift: output o of the padded problem is output
    // o + p of the same transposed convolution without padding, so the kernel
    // runs that one (outputs o' in [0, L_out + p)) and writes o' - p when it
    // lies in [0, L_out).  Without padding output phase b reads inputs
    // q - r for every phase alike (no phase-dependent input offset).
    // When that adds a phase row or column that costs a whole extra tile row
    // or column (a tile dimension the phase rows fit exactly), class mode
    // keeps output-aligned phase rows instead: the phases then read inputs
    // from different offsets, each 16-column block its own.
    Problem qs = q;
    qs.Ho += qs.pH;
    qs.Wo += qs.pW;
    qs.pH = qs.pW = 0;
    if (qs.Ho == 0 || qs.Wo == 0) return false;
    bool cmode = false;
    if (!grouped && (q.pH % q.sH != 0 || q.pW % q.sW != 0)) {
        PolyArgs ac{};
        Inst ic{};
        int spc = 1;
        if (plan_core(qs, a, inst, splits, false, false) && q.Ho > 0 && q.Wo > 0 &&
            plan_core(q, &ac, &ic, &spc, false, true)) {
            const double ts = (double)a->n_tiles, tc = (double)ac.n_tiles;
            cmode = ts > 1.1 * tc;
        }
    }
    int oys = 0, oxs = 0;
    if (cmode) {
        if (!plan_core(q, a, inst, splits, allow_split && !reduced, true)) return false;
        // two phases per output row and whole rows of (2 phases x channel
        // groups) per wave: row-phase-fastest columns (blocks share A
        // fragments by phase parity; the epilogue still stages runs)
        const int64_t groups = a->TCO / 16;
        if (a->pfast == 1 && q.sW == 2 && inst->cb % 2 == 0 && (2 * groups) % inst->cb == 0) {
            a->pfast = 2;
            a->fd_pt = make_fastdiv((uint32_t)(2 * groups));
        }
    } else {
        oys = (int)q.pH;
        oxs = (int)q.pW;
        q = qs;
        if (!plan_core(q, a, inst, splits, allow_split && !reduced, false)) return false;
    }
    // the packed weight is the real one: its size, strides and taps
    const int64_t pw_bytes = p.P * p.C_out * p.T * p.C_in_pad * (p.dtype == CTCONV_F32 ? 4 : 2);
    // (an offset of 2^31 must lie past it: taps past k read as zero)
    if (pw_bytes >= (int64_t)0x80000000LL) return false;
    if (p.Ho > kInt32Max / 2 || p.Wo > kInt32Max / 2) return false;
    a->pw_bytes = (uint32_t)pw_bytes;
    a->gy = rd.g[0];
    a->gx = rd.g[1];
    a->o0y = rd.o0[0];
    a->o0x = rd.o0[1];
    a->dey = rd.de[0];
    a->dex = rd.de[1];
    a->fd_dey = make_fastdiv((uint32_t)rd.de[0]);
    a->fd_dex = make_fastdiv((uint32_t)rd.de[1]);
    a->HoR = p.Ho;
    a->WoR = p.Wo;
    a->oys = oys;
    a->oxs = oxs;
    // the run staging writes every output of its tile in order: only where
    // every output is reached (no reduction step)
    if (reduced) a->pfast = 0;
    a->ws_slab = p.N * p.C_out * p.Ho * p.Wo;  // partial sums use y's own indexing
    a->psy = (int)p.sH;
    a->psx = (int)p.sW;
    a->pmx = (int)p.mW;
    a->pT = (int)p.T;
    a->pw_cblock = (uint32_t)(p.C_out * p.T * kCinAlign * (p.dtype == CTCONV_F32 ? 4 : 2));
    a->kH = (int)p.kH;
    a->kW = (int)p.kW;
    a->fd_psy = make_fastdiv((uint32_t)p.sH);
    a->fd_psx = make_fastdiv((uint32_t)p.sW);
    a->r0y = a->r0x = a->accum = 0;
    a->ngy = a->ngx = 1;
    a->gmy = (int)q.mH;
    a->gmx = (int)q.mW;
    if (grouped) {
        // every group adds into y through the flattened stores
        if (a->phase_subset || a->partial || *splits != 1) return false;
        a->ngy = (int)((mH0 + gmy - 1) / gmy);
        a->ngx = (int)((mW0 + gmx - 1) / gmx);
    }
    return true;
}

}  // namespace

bool polyphase_supported(const Problem& p) {
    PolyArgs a{};
    Inst in{};
    int sp = 1;
    return plan(p, &a, &in, &sp, false);
}

size_t polyphase_workspace_bytes(const Problem& p) {
    PolyArgs a{};
    Inst in{};
    int sp = 1;
    if (!plan(p, &a, &in, &sp, true) || sp <= 1) return 0;
    return (size_t)(sp - 1) * (size_t)a.ws_slab * sizeof(float);
}

namespace {

bool plan_f32out(const Problem& p, PolyArgs* a, Inst* in) {
    if (p.ndim != 1 || p.dtype == CTCONV_F32 || p.act != CTCONV_ACT_NONE) return false;
    int splits = 1;
    if (!plan(p, a, in, &splits, false)) return false;
    return in->TAY == 1 && a->cmode == 0 && a->gx == 1 && a->gy == 1 && a->partial == 0 &&
           splits == 1;
}

}  // namespace

bool polyphase_f32out_supported(const Problem& p) {
    PolyArgs a{};
    Inst in{};
    return plan_f32out(p, &a, &in);
}

hipError_t launch_polyphase_f32out(const Problem& p, const void* x, const void* pw, float* y,
                                   hipStream_t s) {
    PolyArgs a{};
    Inst in{};
    if (!plan_f32out(p, &a, &in)) return hipErrorInvalidValue;
    a.x = x;
    a.pw = pw;
    a.bias = nullptr;
    a.y = y;
    a.outf32 = 1;
    hipLaunchKernelGGL(in.fn, dim3((unsigned)a.n_tiles, 1u), dim3(in.threads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_polyphase(const Problem& p, const void* x, const void* pw, const void* bias,
                            void* y, void* ws, size_t ws_bytes, hipStream_t s) {
    PolyArgs a{};
    Inst in{};
    int splits = 1;
    if (!plan(p, &a, &in, &splits, ws != nullptr)) return hipErrorInvalidValue;
    if (splits > 1 && ws_bytes < (size_t)(splits - 1) * (size_t)a.ws_slab * sizeof(float)) {
        // a workspace too small for this plan: run it unsplit
        if (!plan(p, &a, &in, &splits, false)) return hipErrorInvalidValue;
    }
    a.x = x;
    a.pw = pw;
    a.bias = bias;
    a.y = y;
    a.ws = static_cast<float*>(ws);
    const int act = a.act;
    if (a.partial) a.act = CTCONV_ACT_NONE;  // applied by the reduction
    // outputs no tap reaches (every one but each d-th under dilation)
    if (a.gy > 1 || a.gx > 1) {
        const hipError_t e = launch_fill(p, bias, y, s);
        if (e != hipSuccess) return e;
    }
    const int64_t tiles = a.n_tiles;
    if (a.ngy * a.ngx > 1) {
        // tap groups, in order on the stream: the first writes y with the
        // bias, the others add to it, the last applies the activation
        const int G = a.ngy * a.ngx;
        const int es = p.dtype == CTCONV_F32 ? 4 : 2, np = 8 / es;
        for (int gy = 0; gy < a.ngy; ++gy)
            for (int gx = 0; gx < a.ngx; ++gx) {
                const int g = gy * a.ngx + gx;
                PolyArgs ag = a;
                ag.r0y = gy * a.gmy;
                ag.r0x = gx * a.gmx;
                // x loads stay aligned: the window start moves back by r0x
                const int w0 = a.dminx - (a.gmx - 1) - ag.r0x;
                ag.xofs = (a.W * es) % 4 == 0 ? ((w0 % np) + np) % np : 0;
                ag.accum = g > 0 ? 1 : 0;
                ag.bias = g == 0 ? bias : nullptr;
                ag.act = g == G - 1 ? act : CTCONV_ACT_NONE;
                hipLaunchKernelGGL(in.fn, dim3((unsigned)tiles, 1u), dim3(in.threads), 0, s, ag);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
        return hipSuccess;
    }
    hipLaunchKernelGGL(in.fn, dim3((unsigned)tiles, (unsigned)splits), dim3(in.threads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.partial) return e;
    Problem pr = p;
    pr.act = act;
    return launch_split_reduce(pr, bias, y, ws, splits - 1, s);
}

}  // namespace ctconv

"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle on
the same seeded inputs.

Bars: relative L2 <= 1e-5 for fp32 and <= 1e-2 for bf16/fp16, against the
float64 oracle evaluated on the storage-rounded inputs, and on every output
|y - ref| <= u_out*|ref| + 2*K*2^-24*M (u_out the unit roundoff of the output
type, K the products per output, M the oracle on |x|, |w|, |bias|); bit-exact
for the prepack copy and for impulse responses.
"""

import numpy as np
import pytest

from synth import inputs as I

from gpu_util import (TOL, check_parity, ref_and_mag, say,
                      terms_per_output, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cc():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vision_upsampler_decoders_amd import ctconv

    ctconv.load()
    return ctconv


def _run(cc, x64, w64, b64, dt, s, p, op=0, d=1, route=0, N=None):
    import torch

    x = to_dev(x64, dt)
    w = to_dev(w64, dt)
    b = None if b64 is None else to_dev(b64, dt)
    k = tuple(w64.shape[2:])
    pw = cc.prepack(w, s)
    y = cc.forward(x, pw, b, w64.shape[1], k, s, p, op, d, route=route)
    torch.cuda.synchronize()
    return y


def _rand(shape, seed, dt, lo=-1.0, hi=1.0):
    return I.uniform(seed, shape, lo, hi, dt)


# ---------------------------------------------------------------------------
# prepack: bit-exact against the documented index map
# ---------------------------------------------------------------------------


def _pack_ref(w, s):
    """packed[j][cb][co][r][cc] = w[32*cb + cc, co, sy*ry + jy, sx*rx + jx], zero padded."""
    C_in, C_out = w.shape[:2]
    k = w.shape[2:]
    if len(k) == 1:
        w = w[:, :, None, :]
        k = (1,) + tuple(k)
        s = (1, s[0])
    kH, kW = k
    sH, sW = s
    mH, mW = -(-kH // sH), -(-kW // sW)
    Cp = -(-C_in // 32) * 32
    out = np.zeros((sH * sW, C_out, mH * mW, Cp), dtype=w.dtype)
    for jy in range(sH):
        for jx in range(sW):
            for ry in range(mH):
                for rx in range(mW):
                    ty, tx = sH * ry + jy, sW * rx + jx
                    if ty < kH and tx < kW:
                        out[jy * sW + jx, :, ry * mW + rx, :C_in] = w[:, :, ty, tx].T
    # [j][co][r][ci] -> [j][ci // 32][co][r][ci % 32]
    P, T = out.shape[0], out.shape[2]
    out = out.reshape(P, C_out, T, Cp // 32, 32).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(out).reshape(-1)


@pytest.mark.parametrize("C_in,C_out,k,s,dt", [
    (64, 32, (8,), (4,), "f32"), (37, 5, (7,), (3,), "bf16"), (16, 8, (3, 3), (2, 2), "f32"),
    (40, 9, (4, 6), (2, 3), "f16"), (4098, 1, (4096,), (1024,), "f32"),
])
def test_prepack_bitwise(cc, C_in, C_out, k, s, dt):
    say(f"prepack C_in={C_in} C_out={C_out} k={k} s={s} {dt}")
    import torch

    w64 = _rand((C_in, C_out) + k, 77, dt)
    w = to_dev(w64, dt)
    pw = cc.prepack(w, s)
    torch.cuda.synchronize()
    got = pw.cpu()
    ref = _pack_ref(to_host(w), s)
    assert got.numel() == ref.size
    if dt == "f32":
        np.testing.assert_array_equal(got.numpy().view(np.uint32),
                                      ref.astype(np.float32).view(np.uint32))
    else:
        ref_t = torch.from_numpy(ref).to(got.dtype)
        assert torch.equal(got.view(torch.int16), ref_t.view(torch.int16))


# ---------------------------------------------------------------------------
# full-tensor parity at sizes the oracle finishes in seconds
# (several tiles in every GEMM dimension and a ragged tail)
# ---------------------------------------------------------------------------

FULL_CASES = [
    # name, dt, N, C_in, C_out, spatial, k, s, p, op, d, bias
    ("upsampler1d_small", "f32", 1, 64, 32, (256,), (8,), (4,), (2,), (0,), (1,), True),
    ("voc_l1_short", "bf16", 2, 512, 256, (300,), (16,), (8,), (4,), (0,), (1,), False),
    ("voc_l2_short", "bf16", 2, 256, 128, (700,), (10,), (5,), (3,), (0,), (1,), True),
    ("voc_l3_short", "bf16", 2, 128, 64, (1500,), (8,), (4,), (2,), (0,), (1,), False),
    ("istft_frames", "f32", 2, 4098, 1, (23,), (4096,), (1024,), (0,), (0,), (1,), False),
    ("up2d_small", "bf16", 2, 256, 128, (20, 37), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), True),
    ("gather2d_small", "f32", 1, 128, 64, (24, 29), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), False),
    ("gather2d_dil2_small", "f32", 1, 128, 64, (24, 29), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2),
     True),
    # ragged channel counts, m = 1, 3, 4, s = 1, odd lengths, fp16, asymmetric 2-D
    ("ragged_c_m3", "f16", 3, 33, 17, (131,), (9,), (3,), (4,), (0,), (1,), True),
    ("m1_k_eq_s", "bf16", 2, 48, 40, (257,), (4,), (4,), (0,), (0,), (1,), True),
    ("m4_s2", "f32", 2, 70, 24, (150,), (8,), (2,), (3,), (0,), (1,), True),
    ("s1_k3", "f32", 2, 20, 18, (200,), (3,), (1,), (1,), (0,), (1,), False),
    ("narrow_cout3", "f32", 2, 64, 3, (300,), (12,), (6,), (0,), (0,), (1,), True),
    ("narrow_cout1_pad", "bf16", 2, 64, 1, (300,), (12,), (6,), (2,), (0,), (1,), True),
    ("s16_subset", "bf16", 1, 96, 32, (90,), (32,), (16,), (8,), (0,), (1,), True),
    ("asym2d", "f32", 2, 36, 20, (17, 45), (2, 6), (1, 3), (0, 2), (0, 0), (1, 1), True),
    ("asym2d_m1", "bf16", 1, 64, 48, (33, 18), (2, 4), (2, 2), (0, 1), (0, 0), (1, 1), False),
    ("len1", "f32", 3, 40, 16, (1,), (8,), (4,), (2,), (0,), (1,), True),
    # shortest rows the polyphase kernel takes (one 8-byte load per row)
    ("len2_f32", "f32", 3, 40, 16, (2,), (8,), (4,), (2,), (0,), (1,), True),
    ("len4_bf16", "bf16", 3, 40, 24, (4,), (8,), (4,), (3,), (0,), (1,), True),
    ("w4_2d_bf16", "bf16", 2, 32, 16, (5, 4), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), True),
    # 2-D with more phases than a column tile holds (tiles of phase subsets)
    ("s3_2d_bf16", "bf16", 2, 48, 40, (13, 17), (5, 5), (3, 3), (1, 1), (1, 1), (1, 1), True),
    ("s3_2d_f32_k3", "f32", 1, 40, 64, (21, 10), (3, 3), (3, 3), (0, 1), (2, 0), (1, 1), False),
    ("s4_2d_f16", "f16", 2, 36, 24, (9, 11), (4, 4), (4, 4), (0, 0), (0, 0), (1, 1), True),
    ("s4x3_2d_f32", "f32", 1, 24, 96, (7, 15), (8, 6), (4, 3), (2, 1), (0, 1), (1, 1), True),
    # fp32 with more taps per phase than an instance: tap groups
    ("taps8_1d_f32", "f32", 2, 40, 24, (300,), (16,), (2,), (7,), (0,), (1,), True),
    ("taps6_1d_f32", "f32", 1, 33, 17, (211,), (12,), (2,), (3,), (1,), (1,), True),
    ("taps4x4_2d_f32", "f32", 1, 24, 32, (19, 23), (7, 7), (2, 2), (3, 3), (1, 0), (1, 1), True),
    ("taps_dil3_2d_f32", "f32", 1, 20, 16, (17, 13), (3, 3), (2, 2), (1, 1), (0, 0), (3, 3), False),
    ("taps12_1d_f32_s1", "f32", 2, 16, 40, (90,), (12,), (1,), (5,), (0,), (1,), True),
    # odd input rows (2-byte-offset row pieces): odd length with ragged
    # channels, and a 2-D plane of odd size (odd channels 2 bytes off)
    ("odd_len_bf16", "bf16", 2, 40, 24, (301,), (8,), (4,), (2,), (0,), (1,), True),
    ("odd_plane_2d_bf16", "bf16", 2, 36, 16, (5, 7), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), True),
    # k not a multiple of s and output_padding on the polyphase route (zero
    # taps past k; longer output)
    ("k7_s3_op1_bf16", "bf16", 2, 48, 24, (200,), (7,), (3,), (2,), (1,), (1,), True),
    ("k5_s4_op3_f16", "f16", 2, 40, 20, (130,), (5,), (4,), (1,), (3,), (1,), False),
    ("k3_s2_op1_2d_f32", "f32", 2, 24, 12, (13, 17), (3, 3), (2, 2), (0, 1), (1, 1), (1, 1), True),
    ("k3x4_s2x3_2d_bf16", "bf16", 1, 40, 24, (12, 15), (3, 4), (2, 3), (1, 0), (0, 2), (1, 1), True),
    # three and four taps in 16-bit storage (eight-wave tiles), five phases
    # with three and four taps (256 x 160 tiles), odd and even lengths
    ("s5_m3_op2_bf16", "bf16", 2, 72, 40, (257,), (13,), (5,), (4,), (2,), (1,), True),
    ("s5_m4_f16", "f16", 1, 40, 30, (300,), (20,), (5,), (7,), (0,), (1,), False),
    ("s4_m4_bf16", "bf16", 2, 64, 48, (400,), (16,), (4,), (6,), (0,), (1,), True),
    # dilation on the polyphase route: reduction by g = gcd(s, d) (the
    # problem of stride s / g; outputs off the g-grid are the bias) and
    # expansion of the remaining d / g into zero taps; 2-D 3 x 3 reduced taps
    # in fp32 and in 16-bit with odd rows, 1-D reductions, 1-D and 2-D
    # expansions, and both at once
    ("dil2_s2_2d_f32", "f32", 1, 24, 20, (13, 17), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2), True),
    ("dil2_s2_2d_bf16_odd", "bf16", 1, 40, 24, (9, 11), (3, 3), (2, 2), (0, 1), (0, 1), (2, 2),
     True),
    ("dil2_s4_bf16", "bf16", 2, 40, 24, (101,), (8,), (4,), (3,), (1,), (2,), True),
    ("dil3_s3_k4_f16", "f16", 2, 33, 17, (90,), (4,), (3,), (2,), (2,), (3,), False),
    ("dil3_s2_k3_bf16", "bf16", 2, 48, 40, (203,), (3,), (2,), (1,), (0,), (3,), True),
    ("dil2_s3_k4_f32", "f32", 2, 40, 24, (150,), (4,), (3,), (2,), (1,), (2,), True),
    ("dil6_s4_k3_bf16", "bf16", 1, 64, 48, (120,), (3,), (4,), (5,), (2,), (6,), True),
    ("dil2_s4_2d_f32", "f32", 1, 24, 20, (13, 17), (3, 3), (4, 4), (1, 2), (0, 1), (2, 2), True),
    ("dilx3_s2_2d_bf16", "bf16", 1, 40, 24, (11, 19), (4, 2), (2, 2), (1, 2), (0, 1), (1, 3),
     True),
    ("dil2_s3x1_2d_f16", "f16", 1, 36, 20, (10, 12), (3, 2), (3, 1), (1, 0), (2, 0), (2, 1), False),
]


_ORACLE_CACHE = {}


@pytest.mark.parametrize("case", FULL_CASES, ids=[c[0] for c in FULL_CASES])
@pytest.mark.parametrize("route", [0, 2, 3], ids=["auto", "gather", "tiled"])
def test_full_parity(cc, case, route):
    """Every route on every case it takes: auto (the streaming polyphase kernel
    where it applies, else the tiled one, else gather), gather forced, and the
    tiled polyphase kernel forced."""
    name, dt, N, C_in, C_out, sp, k, s, p, op, d, has_b = case
    if route == 2 and C_in * C_out * int(np.prod(k)) * N * int(np.prod(sp)) > 4e9:
        pytest.skip("gather cross-check limited to small cases")
    if route == 3 and cc.ctconv_query_route(N, C_in, C_out, sp, k, s, p, op, d,
                                             cc.dtype_code_of(dt)) != cc.ROUTE_POLYPHASE:
        pytest.skip("not on the polyphase route")
    say(f"full_parity {name} route={route} dt={dt} N={N} C_in={C_in} C_out={C_out} sp={sp}")
    seed = 500 + len(name)
    x64 = I.normal(seed, (N, C_in) + sp, 1.0, dt)
    w64 = I.normal(seed + 1, (C_in, C_out) + k, (C_in * np.prod(k)) ** -0.5, dt)
    b64 = _rand((C_out,), seed + 2, dt, -0.1, 0.1) if has_b else None
    if name.startswith("istft"):
        w64 = I.istft_basis(4096, dt)
    y = to_host(_run(cc, x64, w64, b64, dt, s, p, op, d, route=route))
    if name not in _ORACLE_CACHE:
        _ORACLE_CACHE[name] = ref_and_mag(x64, w64, b64, s, p, op, d)
    ref, mag = _ORACLE_CACHE[name]
    check_parity(y, ref, mag, dt, terms_per_output(C_in, k, s, d), name)


# ---------------------------------------------------------------------------
# full workload sizes, in the launch configuration the benchmark times:
# every output against the oracle (run per batch item in threads)
# ---------------------------------------------------------------------------


def _vocoder_layer_input(cc, wl, li, fused):
    """The GPU's own input to layer li of the stack (earlier layers and their
    ELUs run on the GPU)."""
    import torch

    x = to_dev(I.gen_x(wl), wl.dtype)
    for lj, L in enumerate(wl.layers[:li]):
        pw = cc.prepack(to_dev(I.gen_w(wl, lj), wl.dtype), L.stride)
        if fused:
            x = cc.forward(x, pw, None, L.C_out, L.kernel, L.stride, L.padding, act=cc.ACT_ELU)
        else:
            x = cc.elu(cc.forward(x, pw, None, L.C_out, L.kernel, L.stride, L.padding))
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("li", [0, 1, 2])
def test_vocoder_stack_full_size_per_layer(cc, li):
    """Each layer of the full-size stack (N = 8, in the launch configuration the
    benchmark times) on every output, with the oracle fed the GPU's own bf16
    layer input; the ELU after it checked element by element."""
    import torch

    from oracle import elu as oelu

    wl = I.workload("vocoder_stack")
    L = wl.layers[li]
    x = _vocoder_layer_input(cc, wl, li, fused=False)
    say(f"vocoder layer {li}: {tuple(x.shape)} -> C_out {L.C_out} k{L.kernel} s{L.stride}")
    w64 = I.gen_w(wl, li)
    pw = cc.prepack(to_dev(w64, wl.dtype), L.stride)
    y = cc.forward(x, pw, None, L.C_out, L.kernel, L.stride, L.padding)
    torch.cuda.synchronize()
    xin64 = to_host(x)
    del x
    ref, mag = ref_and_mag(xin64, w64, None, L.stride, L.padding)
    yh = to_host(y)
    check_parity(yh, ref, mag, wl.dtype, terms_per_output(L.C_in, L.kernel, L.stride),
                 f"layer {li}")
    del ref, mag
    if li + 1 < len(wl.layers):
        ye = to_host(cc.elu(y))
        # one rounding of an fp32 ELU of the bf16 input (exp2 error ~1e-7)
        check_parity(ye, oelu(yh), np.zeros(1), wl.dtype, 0, f"elu after layer {li}",
                     abs_slack=1e-6)
    del y
    torch.cuda.empty_cache()


def test_vocoder_stack_end_to_end_short(cc):
    """L1 -> ELU -> L2 -> ELU -> L3 against the oracle chain in float64."""
    import torch

    from oracle import conv_transpose, elu as oelu, rel_l2

    wl = I.workload("vocoder_stack")
    x64 = I.gen_x(wl, N=1, in_spatial=(60,))
    x = to_dev(x64, wl.dtype)
    ref = x64
    for li, L in enumerate(wl.layers):
        w64 = I.gen_w(wl, li)
        pw = cc.prepack(to_dev(w64, wl.dtype), L.stride)
        x = cc.forward(x, pw, None, L.C_out, L.kernel, L.stride, L.padding)
        ref = conv_transpose(ref, w64, None, L.stride, L.padding)
        if li + 1 < len(wl.layers):
            x = cc.elu(x)
            ref = oelu(ref)
    torch.cuda.synchronize()
    err = rel_l2(to_host(x), ref)
    say(f"vocoder end-to-end short: rel_l2 = {err:.3e}")
    assert err <= 1e-2


# ---------------------------------------------------------------------------
# fused activation: y = ELU(conv + bias), one rounding
# ---------------------------------------------------------------------------

ACT_CASES = [
    # name, dt, N, C_in, C_out, spatial, k, s, p, op, d, bias
    ("act_voc_l2", "bf16", 2, 256, 128, (300,), (10,), (5,), (3,), (0,), (1,), True),
    ("act_voc_l1", "bf16", 2, 512, 64, (120,), (16,), (8,), (4,), (0,), (1,), False),
    ("act_f32_2d", "f32", 2, 24, 20, (13, 11), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), True),
    ("act_f16_gather_dil", "f16", 1, 40, 12, (37,), (5,), (3,), (2,), (1,), (2,), True),
    ("act_dil2_2d_f32", "f32", 1, 24, 20, (13, 11), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2), True),
    # tap groups: the activation after the last group's sum
    ("act_f32_taps8", "f32", 1, 24, 16, (100,), (16,), (2,), (7,), (0,), (1,), True),
    ("act_f32_2d_taps4x3", "f32", 1, 20, 24, (11, 9), (7, 5), (2, 2), (2, 1), (1, 0), (1, 1), True),
]


@pytest.mark.parametrize("case", ACT_CASES, ids=[c[0] for c in ACT_CASES])
@pytest.mark.parametrize("route", [0, 2], ids=["auto", "gather"])
def test_fused_elu_parity(cc, case, route):
    import torch

    from oracle import elu as oelu

    name, dt, N, C_in, C_out, sp, k, s, p, op, d, has_b = case
    say(f"fused elu {name} route={route}")
    seed = 700 + len(name)
    x64 = I.normal(seed, (N, C_in) + sp, 1.0, dt)
    w64 = I.normal(seed + 1, (C_in, C_out) + k, (C_in * np.prod(k)) ** -0.5, dt)
    b64 = _rand((C_out,), seed + 2, dt, -0.1, 0.1) if has_b else None
    pw = cc.prepack(to_dev(w64, dt), s)
    y = cc.forward(to_dev(x64, dt), pw, None if b64 is None else to_dev(b64, dt), C_out, k, s, p,
                   op, d, route=route, act=cc.ACT_ELU)
    torch.cuda.synchronize()
    pre, mag = ref_and_mag(x64, w64, b64, s, p, op, d)
    # ELU is 1-Lipschitz: the accumulation bound carries over; exp2 adds ~1e-7
    check_parity(to_host(y), oelu(pre), mag, dt, terms_per_output(C_in, k, s, d), name,
                 abs_slack=1e-6)


@pytest.mark.parametrize("case", ACT_CASES, ids=[c[0] for c in ACT_CASES])
@pytest.mark.parametrize("route", [0, 2], ids=["auto", "gather"])
def test_fused_elu_matches_forward_then_elu_bitwise(cc, case, route):
    """The fused activation is the same fp32 function that the standalone ELU
    pass applies.  For fp32 storage the unfused pair rounds nothing in
    between, so the two agree bit for bit.  For 16-bit storage the unfused
    pair rounds before the ELU as well as after.  For v < 0 the slope e^v of
    the ELU times |v| is at most |e^v - 1| (u e^-u <= 1 - e^-u), so the first
    rounding, relative error 2^-9 (bf16) or 2^-12 (fp16) of v, moves the
    result by at most that relative amount of it, one unit in its last place;
    with the two final roundings the results differ by at most two units."""
    import torch

    name, dt, N, C_in, C_out, sp, k, s, p, op, d, has_b = case
    say(f"fused vs unfused elu {name} route={route}")
    seed = 900 + len(name)
    x = to_dev(I.normal(seed, (N, C_in) + sp, 1.0, dt), dt)
    w = to_dev(I.normal(seed + 1, (C_in, C_out) + k, (C_in * np.prod(k)) ** -0.5, dt), dt)
    b = to_dev(_rand((C_out,), seed + 2, dt, -0.1, 0.1), dt) if has_b else None
    pw = cc.prepack(w, s)
    fused = cc.forward(x, pw, b, C_out, k, s, p, op, d, route=route, act=cc.ACT_ELU)
    plain = cc.forward(x, pw, b, C_out, k, s, p, op, d, route=route)
    sep = cc.elu(plain)
    torch.cuda.synchronize()
    if dt == "f32":
        assert torch.equal(fused, sep)
    else:
        bits = lambda t: t.view(torch.int16).to(torch.int32)
        assert int((bits(fused) - bits(sep)).abs().max()) <= 2


def test_fused_elu_empty_input_fills_act_of_bias(cc):
    import torch

    from oracle import elu as oelu

    b64 = _rand((6,), 31, "f32", -1.0, 1.0)
    x = torch.empty((2, 4, 0), dtype=torch.float32, device="cuda")
    w64 = _rand((4, 6, 8), 32, "f32")
    pw = cc.prepack(to_dev(w64, "f32"), (4,))
    y = cc.forward(x, pw, to_dev(b64, "f32"), 6, (8,), (4,), (0,), act=cc.ACT_ELU)
    torch.cuda.synchronize()
    got = to_host(y)
    assert got.shape == (2, 6, 4)
    ref = np.broadcast_to(oelu(b64.astype(np.float32).astype(np.float64))[None, :, None], got.shape)
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("li", [0, 1])
def test_vocoder_stack_fused_elu_full_size(cc, li):
    """Layers 0 and 1 of the full-size stack with the ELU fused, every output:
    the oracle (conv, then ELU in float64) fed the GPU's own layer input."""
    import torch

    from oracle import elu as oelu

    wl = I.workload("vocoder_stack")
    L = wl.layers[li]
    x = _vocoder_layer_input(cc, wl, li, fused=True)
    w64 = I.gen_w(wl, li)
    pw = cc.prepack(to_dev(w64, wl.dtype), L.stride)
    y = cc.forward(x, pw, None, L.C_out, L.kernel, L.stride, L.padding, act=cc.ACT_ELU)
    torch.cuda.synchronize()
    xin64 = to_host(x)
    del x
    pre, mag = ref_and_mag(xin64, w64, None, L.stride, L.padding)
    check_parity(to_host(y), oelu(pre), mag, wl.dtype,
                 terms_per_output(L.C_in, L.kernel, L.stride), f"fused-elu layer {li}",
                 abs_slack=1e-6)
    del y
    torch.cuda.empty_cache()


def test_istft_full_size(cc):
    """Every output against the oracle on the fp32 basis, and the whole output
    against the independent radix-2 irfft + overlap-add oracle."""
    import torch

    from oracle import istft_ola, rel_l2

    wl = I.workload("istft")
    L = wl.layers[0]
    x64 = I.gen_x(wl)
    w64 = I.gen_w(wl)
    say("istft full size [8, 4098, 345] -> [8, 1, 356352]")
    y = to_host(_run(cc, x64, w64, None, "f32", L.stride, L.padding))
    ref = istft_ola(x64, 4096, 1024)
    err = rel_l2(y[:, 0], ref)
    say(f"  rel_l2 vs irfft+OLA = {err:.3e}")
    # the fp32-rounded basis itself differs from the exact transform by ~1e-8
    assert err <= 1e-5
    ref, mag = ref_and_mag(x64, w64, None, L.stride, L.padding)
    check_parity(y, ref, mag, "f32", terms_per_output(L.C_in, L.kernel, L.stride), "istft")
    torch.cuda.empty_cache()


def test_istft_perfect_reconstruction(cc):
    """Spectra of Hann-windowed frames at hop n/4 resynthesise 1.5 z in the interior."""
    from oracle import rel_l2

    n_fft, hop, T = 4096, 1024, 40
    z = I.normal(3011, ((T - 1) * hop + n_fft,), 1.0, "f32")
    h = I.hann_periodic(n_fft)
    F = n_fft // 2 + 1
    spec = np.zeros((1, 2 * F, T))
    for l in range(T):
        X = np.fft.rfft(h * z[l * hop:l * hop + n_fft])
        spec[0, :F, l] = X.real
        spec[0, F:, l] = X.imag
    spec = I.round_to_dtype(spec, "f32")
    y = to_host(_run(cc, spec, I.istft_basis(n_fft, "f32"), None, "f32", (hop,), (0,)))[0, 0]
    lo, hi = 3 * hop, (T - 1) * hop + hop
    err = rel_l2(y[lo:hi], 1.5 * z[lo:hi])
    say(f"istft reconstruction rel_l2 = {err:.3e}")
    assert err <= 1e-5


@pytest.mark.parametrize("name,route", [
    ("upsampler2d", 0), ("gather2d", 0), ("gather2d_dil2", 0), ("upsampler1d_small", 0),
    ("gather2d_s3", 0), ("gather2d_s3", 2), ("gather1d_m8", 0),
], ids=lambda v: str(v))
def test_workload_full_size(cc, name, route):
    """The benchmark's single-layer workloads at full size, every output (the
    5x5 s3 shape also on the gather kernel, which the bench ran it on before
    the polyphase kernel took 2-D phase subsets)."""
    import torch

    wl = I.workload(name)
    L = wl.layers[0]
    x64 = I.gen_x(wl)
    w64 = I.gen_w(wl)
    b64 = I.gen_bias(wl)
    say(f"{name} full size {x64.shape} dt={wl.dtype} route={route}")
    y = _run(cc, x64, w64, b64, wl.dtype, L.stride, L.padding, L.output_padding, L.dilation,
             route=route)
    yh = to_host(y)
    key = "workload:" + name
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = ref_and_mag(x64, w64, b64, L.stride, L.padding, L.output_padding,
                                         L.dilation)
    ref, mag = _ORACLE_CACHE[key]
    check_parity(yh, ref, mag, wl.dtype,
                 terms_per_output(L.C_in, L.kernel, L.stride, L.dilation), name)
    if name == "gather2d_dil2":
        # even rows and columns receive no tap: bias or zero exactly
        assert float(np.abs(yh[:, :, 0::2, :]).max()) == 0.0
        assert float(np.abs(yh[:, :, :, 0::2]).max()) == 0.0
    del y
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# exact special cases and edge cases
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name", ["vocoder_l1", "upsampler2d", "gather2d_dil2", "istft"])
def test_impulse_response_exact(cc, name):
    """x = e_(n0, ci0, pos0): y equals the weight taps bit for bit, zero elsewhere."""
    import torch

    if name == "vocoder_l1":
        dt, N, C_in, C_out, sp, k, s, p, op, d = "bf16", 8, 512, 256, (2000,), (16,), (8,), (4,), (0,), (1,)
    elif name == "upsampler2d":
        dt, N, C_in, C_out, sp, k, s, p, op, d = "bf16", 8, 256, 128, (64, 64), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1)
    elif name == "gather2d_dil2":
        dt, N, C_in, C_out, sp, k, s, p, op, d = "f32", 4, 128, 64, (96, 96), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2)
    else:
        dt, N, C_in, C_out, sp, k, s, p, op, d = "f32", 8, 4098, 1, (345,), (4096,), (1024,), (0,), (0,), (1,)
    w64 = _rand((C_in, C_out) + k, 13, dt)
    w = to_dev(w64, dt)
    pw = cc.prepack(w, s)
    for (n0, ci0, pos) in [(0, 0, tuple(0 for _ in sp)), (N - 1, C_in - 1, tuple(v - 1 for v in sp)),
                           (N // 2, C_in // 2, tuple(v // 2 for v in sp))]:
        say(f"impulse {name} at n={n0} ci={ci0} pos={pos}")
        x = torch.zeros((N, C_in) + sp, dtype=w.dtype, device="cuda")
        x[(n0, ci0) + pos] = 1.0
        y = cc.forward(x, pw, None, C_out, k, s, p, op, d)
        torch.cuda.synchronize()
        ref = torch.zeros_like(y)
        taps = [range(kk) for kk in k]
        import itertools

        for t in itertools.product(*taps):
            o = tuple(pos[i] * s[i] - p[i] + t[i] * d[i] for i in range(len(sp)))
            if all(0 <= o[i] < y.shape[2 + i] for i in range(len(sp))):
                ref[(n0, slice(None)) + o] = w[(ci0, slice(None)) + t]
        assert torch.equal(y, ref)


def test_empty_input_and_null_bias(cc):
    import torch

    say("empty input: L_in = 0 with a non-empty output")
    w = to_dev(_rand((6, 5, 4096), 3, "f32"), "f32")
    pw = cc.prepack(w, (1024,))
    b = to_dev(_rand((5,), 4, "f32"), "f32")
    x = torch.zeros((2, 6, 0), dtype=torch.float32, device="cuda")
    y = cc.forward(x, pw, b, 5, (4096,), (1024,), (0,))
    torch.cuda.synchronize()
    assert y.shape == (2, 5, 3072)
    assert torch.equal(y, b.view(1, 5, 1).expand_as(y))
    y0 = cc.forward(x, pw, None, 5, (4096,), (1024,), (0,))
    torch.cuda.synchronize()
    assert float(y0.abs().max()) == 0.0
    say("N = 0: nothing to do")
    x = torch.zeros((0, 6, 10), dtype=torch.float32, device="cuda")
    y = cc.forward(x, pw, b, 5, (4096,), (1024,), (0,))
    assert y.shape[0] == 0


def test_fp16_cancellation(cc):
    """Partial products beyond the fp16 range that cancel: fp32 accumulation
    must return the small exact result."""
    import torch

    say("fp16 cancelling taps")
    C_in, C_out, L = 2, 16, 40
    x = torch.ones((1, C_in, L), dtype=torch.float16, device="cuda")
    w = torch.zeros((C_in, C_out, 4), dtype=torch.float16, device="cuda")
    w[0, :, :] = 40000.0
    w[1, :, :] = -40000.0
    w[1, :, 1] = -39968.0  # 40000 - 39968 = 32
    for route in (0, 2):
        pw = cc.prepack(w, (2,))
        y = cc.forward(x, pw, None, C_out, (4,), (2,), (1,), route=route)
        torch.cuda.synchronize()
        yf = y.float().cpu().numpy()
        assert np.isfinite(yf).all()
        ref = to_host(x)
        from oracle import conv_transpose

        r = conv_transpose(ref, to_host(w), None, 2, 1)
        np.testing.assert_array_equal(yf, r)


def test_routes_agree(cc):
    """Polyphase and gather kernels on the same polyphase-eligible shapes."""
    import torch

    from oracle import rel_l2

    for dt, sp, k, s, p in [("f32", (300,), (8,), (4,), (2,)), ("bf16", (40, 50), (4, 4), (2, 2), (1, 1))]:
        say(f"route cross-check {dt} {sp}")
        x64 = I.normal(21, (2, 96) + sp, 1.0, dt)
        w64 = I.normal(22, (96, 48) + k, 0.05, dt)
        a = to_host(_run(cc, x64, w64, None, dt, s, p, route=1))
        b = to_host(_run(cc, x64, w64, None, dt, s, p, route=2))
        assert rel_l2(a, b) <= TOL[dt]


def test_non_default_stream_and_determinism(cc):
    import torch

    say("non-default stream, repeated runs")
    x64 = I.normal(31, (2, 256, 500), 1.0, "bf16")
    w64 = I.normal(32, (256, 128, 10), 0.02, "bf16")
    x, w = to_dev(x64, "bf16"), to_dev(w64, "bf16")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        pw = cc.prepack(w, (5,), stream=st)
        y1 = cc.forward(x, pw, None, 128, (10,), (5,), (3,), stream=st)
        y2 = cc.forward(x, pw, None, 128, (10,), (5,), (3,), stream=st)
    st.synchronize()
    assert torch.equal(y1, y2)
    y3 = cc.forward(x, pw, None, 128, (10,), (5,), (3,))
    torch.cuda.synchronize()
    assert torch.equal(y1, y3)

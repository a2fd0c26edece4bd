"""GPU parity of the depthwise transposed convolution (groups = C_in) against
the CPU oracle's grouped scatter definition, through the C ABI.

Bars: relative L2 <= 1e-5 for fp32 and <= 1e-2 for bf16/fp16 against the
float64 oracle on the storage-rounded inputs, and every output within the
element bound of gpu_util.check_parity; impulse responses bit-exact;
the two kernels (row-phase and element) equal in value, since both add the
taps of an output in the same order.
"""

import numpy as np
import pytest

from synth import inputs as I

from gpu_util import check_parity, ref_and_mag, say, terms_per_output, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cc():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vision_upsampler_decoders_amd import ctconv

    ctconv.load()
    return ctconv


CASES = [
    # name, dt, N, C_in, M, spatial, k, s, p, op, d, bias
    ("k4s2_1d_bf16", "bf16", 2, 6, 1, (300,), (4,), (2,), (1,), (0,), (1,), True),
    ("k4s2_1d_f32_ragged", "f32", 2, 5, 1, (301,), (4,), (2,), (1,), (1,), (1,), False),
    ("k8s4_1d_f16_mult2", "f16", 1, 4, 2, (257,), (8,), (4,), (2,), (0,), (1,), True),
    ("k5s2_1d_bf16_op", "bf16", 2, 3, 1, (131,), (5,), (2,), (2,), (1,), (1,), True),
    ("k3s1_1d_f32", "f32", 1, 4, 3, (600,), (3,), (1,), (1,), (0,), (1,), True),
    ("k16s4_1d_bf16", "bf16", 1, 3, 1, (90,), (16,), (4,), (6,), (0,), (1,), False),
    ("k6s3_1d_f32_element", "f32", 2, 3, 1, (77,), (6,), (3,), (1,), (0,), (1,), True),
    ("k3s2d2_1d_f16_element", "f16", 2, 3, 2, (64,), (3,), (2,), (1,), (1,), (2,), True),
    ("k10s2_1d_bf16_element", "bf16", 1, 2, 1, (50,), (10,), (2,), (4,), (0,), (1,), True),
    ("k4s2_2d_bf16", "bf16", 2, 5, 1, (33, 70), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), True),
    ("k3s2op1_2d_f32", "f32", 2, 3, 2, (17, 19), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), False),
    ("k3s2_dilH_2d_f16_element", "f16", 1, 4, 1, (12, 40), (3, 3), (2, 2), (1, 1), (1, 1), (2, 1),
     True),
    ("k3s2_dil2_2d_f32_element", "f32", 1, 4, 1, (12, 21), (3, 3), (2, 2), (1, 1), (1, 1),
     (2, 2), True),
    ("k5x4_s3x4_2d_bf16", "bf16", 1, 3, 2, (9, 130), (5, 4), (3, 4), (2, 1), (1, 0), (1, 1),
     True),
    ("k8s4_2d_f32", "f32", 1, 3, 1, (10, 33), (8, 8), (4, 4), (2, 2), (0, 0), (1, 1), True),
    ("k3s1_2d_bf16", "bf16", 2, 3, 1, (7, 64), (3, 3), (1, 1), (1, 1), (0, 0), (1, 1), False),
    ("k10s2_2d_f16_element", "f16", 1, 2, 1, (6, 20), (10, 4), (2, 2), (4, 1), (0, 0), (1, 1),
     True),
    # enough work items that a wave walks several (across strips and planes)
    ("k4s2_2d_bf16_walk", "bf16", 4, 128, 1, (40, 64), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1),
     True),
    ("k4s2_1d_f32_walk", "f32", 4, 64, 1, (20000,), (4,), (2,), (1,), (0,), (1,), True),
]


def _inputs(case):
    name, dt, N, C_in, M, sp, k, s, p, op, d, has_b = case
    seed = 900 + 7 * len(name)
    x64 = I.normal(seed, (N, C_in) + sp, 1.0, dt)
    w64 = I.normal(seed + 1, (C_in, M) + k, float(np.prod(k)) ** -0.5, dt)
    b64 = I.uniform(seed + 2, (C_in * M,), -0.1, 0.1, dt) if has_b else None
    return x64, w64, b64


def _dev_run(cc, x64, w64, b64, dt, s, p, op, d, which, act=0):
    import torch

    y = cc.depthwise_forward(to_dev(x64, dt), to_dev(w64, dt),
                             None if b64 is None else to_dev(b64, dt), s, p, op, d,
                             act=act, which=which)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("which", [0, 2], ids=["auto", "element"])
def test_depthwise_parity(cc, case, which):
    name, dt, N, C_in, M, sp, k, s, p, op, d, has_b = case
    say(f"depthwise {name} which={which}")
    x64, w64, b64 = _inputs(case)
    y = _dev_run(cc, x64, w64, b64, dt, s, p, op, d, which)
    ref, mag = ref_and_mag(x64, w64, b64, s, p, op, d, groups=C_in)
    check_parity(to_host(y), ref, mag, dt, terms_per_output(1, k, s, d), name)


def test_depthwise_kernel_choice_matches_cases(cc):
    """The auto cases above cover both kernels: the names say which one runs."""
    for case in CASES:
        name, dt, N, C_in, M, sp, k, s, p, op, d, has_b = case
        which = cc.ctconv_depthwise_query_kernel(N, C_in, C_in * M, sp, k, s, p, op, d)
        assert which == (2 if name.endswith("_element") else 1), name


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[3], CASES[9], CASES[13]],
                         ids=lambda c: c[0])
def test_row_and_element_kernels_agree(cc, case):
    import torch

    name, dt, N, C_in, M, sp, k, s, p, op, d, has_b = case
    say(f"row vs element {name}")
    x64, w64, b64 = _inputs(case)
    y_row = _dev_run(cc, x64, w64, b64, dt, s, p, op, d, 1)
    y_el = _dev_run(cc, x64, w64, b64, dt, s, p, op, d, 2)
    assert torch.equal(y_row, y_el)


@pytest.mark.parametrize("case", [CASES[0], CASES[9], CASES[11]], ids=lambda c: c[0])
def test_depthwise_fused_elu(cc, case):
    from oracle import elu

    name, dt, N, C_in, M, sp, k, s, p, op, d, has_b = case
    say(f"depthwise elu {name}")
    x64, w64, b64 = _inputs(case)
    pre, mag = ref_and_mag(x64, w64, b64, s, p, op, d, groups=C_in)
    for which in (0, 2):
        y = _dev_run(cc, x64, w64, b64, dt, s, p, op, d, which, act=cc.ACT_ELU)
        check_parity(to_host(y), elu(pre), mag, dt, terms_per_output(1, k, s, d),
                     f"{name} which={which}", abs_slack=1e-6)


@pytest.mark.parametrize("which", [1, 2], ids=["row", "element"])
def test_depthwise_impulse_exact(cc, which):
    """One input element reaches only its own channel's outputs, with the
    weights themselves, bit for bit (every dtype)."""
    import torch

    from oracle import conv_transpose_grouped

    for dt in ("f32", "bf16", "f16"):
        C, M, H, W, k, s, p = 3, 2, 9, 70, (4, 4), (2, 2), (1, 1)
        w64 = I.uniform(77, (C, M) + k, -1, 1, dt)
        for c0, i0, j0 in [(0, 0, 0), (2, H - 1, W - 1), (1, 4, 33)]:
            x64 = np.zeros((1, C, H, W))
            x64[0, c0, i0, j0] = 1.0
            y = _dev_run(cc, x64, w64, None, dt, s, p, 0, 1, which)
            ref = conv_transpose_grouped(x64, w64, None, C, s, p)
            assert np.array_equal(to_host(y), ref), (dt, c0, i0, j0)
    torch.cuda.synchronize()


def test_depthwise_empty_input_fills_bias(cc):
    import torch

    dt = "f32"
    b64 = I.uniform(5, (6,), -0.1, 0.1, dt)
    w = to_dev(I.uniform(6, (3, 2, 4), -1, 1, dt), dt)
    x = torch.empty((2, 3, 0), dtype=torch.float32, device="cuda")
    # L_in = 0: output length (0 - 1)*2 - 2*0 + 3 + 1 = 2, every element the bias
    y = cc.depthwise_forward(x, w, to_dev(b64, dt), 2, 0)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (2, 6, 2)
    np.testing.assert_array_equal(to_host(y), np.broadcast_to(b64[None, :, None], (2, 6, 2)))
    x0 = torch.empty((0, 3, 5), dtype=torch.float32, device="cuda")
    y0 = cc.depthwise_forward(x0, w, None, 2, 1)
    assert y0.shape[0] == 0


@pytest.mark.parametrize("name", ["depthwise2d", "depthwise1d"])
def test_depthwise_workload_full_size(cc, name):
    """The benchmark's depthwise workloads at full size, every output."""
    import torch

    wl = I.workload(name)
    L = wl.layers[0]
    say(f"full size {name}: generating inputs")
    x64 = I.gen_x(wl)
    w64 = I.gen_w(wl)
    b64 = I.gen_bias(wl)
    conv = cc.DepthwiseConv(wl.N, L.C_in, L.C_out, wl.in_spatial, L.kernel, L.stride, L.padding,
                            L.output_padding, L.dilation, {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype])
    x, w = to_dev(x64, wl.dtype), to_dev(w64, wl.dtype)
    b = None if b64 is None else to_dev(b64, wl.dtype)
    y = torch.empty(conv.out_shape(), dtype=x.dtype, device="cuda")
    say(f"  launch {conv.out_shape()}")
    conv(x.data_ptr(), w.data_ptr(), None if b is None else b.data_ptr(), y.data_ptr(),
         int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    yh = to_host(y)
    del y
    ref, mag = ref_and_mag(x64, w64, b64, L.stride, L.padding, L.output_padding, L.dilation,
                           groups=L.groups)
    check_parity(yh, ref, mag, wl.dtype, terms_per_output(1, L.kernel, L.stride, L.dilation), name)


def test_depthwise_graph_replay_and_side_stream(cc):
    """Depthwise launches captured in a HIP graph (strip kernel in 2-D and
    1-D, element kernel) and replayed with new inputs copied in, eager work
    and synchronisation between replays: each replay equals the eager call
    on the same input bit for bit; launches on a non-default stream equal
    the default-stream ones and repeat identically."""
    import torch

    dt = "bf16"
    specs = [((2, 16, 20, 40), (16, 1, 4, 4), 2, 1, 1),   # 2-D strip kernel
             ((2, 16, 700), (16, 2, 4), 2, 1, 1),        # 1-D strip kernel, multiplier 2
             ((1, 8, 30), (8, 1, 6), 3, 1, 2)]           # element kernel (stride 3)
    for xs, wsh, s, p, which in specs:
        w = to_dev(I.normal(60, wsh, 0.3, dt), dt)
        b = to_dev(I.uniform(61, (wsh[0] * wsh[1],), -0.1, 0.1, dt), dt)
        xin = [to_dev(I.normal(62 + i, xs, 1.0, dt), dt) for i in range(4)]
        ref = [cc.depthwise_forward(x, w, b, s, p, which=which) for x in xin]
        torch.cuda.synchronize()
        xa = torch.empty_like(xin[0])
        ya = torch.empty_like(ref[0])
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside the capture, on a side stream
            xa.copy_(xin[0])
            cc.depthwise_forward(xa, w, b, s, p, which=which, out=ya)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(ya, ref[0])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cc.depthwise_forward(xa, w, b, s, p, which=which, out=ya)
        for j in range(4):
            xa.copy_(xin[j])
            g.replay()
            torch.cuda.synchronize()
            _ = (xa.float() * 2).sum().item()  # eager work between replays
            assert torch.equal(ya, ref[j]), (xs, j)
        say(f"depthwise graph {xs} which={which}: 4 replays equal to eager")


def _random_cases(n, seed):
    """Deterministic random depthwise shapes within the kernels' families:
    1-D and 2-D, strides 1-4 (square and not), taps per phase 1-4, padding,
    output_padding, multipliers 1-3, widths spanning several 256/512-output
    segments, and enough items that waves walk across strips and planes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    while len(cases) < n:
        nd = int(rng.integers(1, 3))
        s = [int(rng.choice([1, 2, 3, 4])) for _ in range(nd)]
        if nd == 2 and rng.random() < 0.6:
            s[1] = s[0]
        k = [int(rng.integers(1, 4 * si + 1)) for si in s]
        if nd == 2 and s[0] == s[1] and rng.random() < 0.6:
            k[1] = k[0]
        p = [int(rng.integers(0, ki)) for ki in k]
        op = [int(rng.integers(0, si)) for si in s]
        sp = [int(rng.integers(1, 7))] if nd == 2 else []
        sp += [int(rng.integers(1, 400))]
        out = [(a - 1) * b - 2 * c + e + o for a, b, c, e, o in zip(sp, s, p, k, op)]
        if min(out) < 1:
            continue
        N, C, M = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 4))
        dt = str(rng.choice(["f32", "bf16", "f16"]))
        cases.append((dt, N, C, M, tuple(sp), tuple(k), tuple(s), tuple(p), tuple(op)))
    return cases


RANDOM_CASES = _random_cases(48, 2024)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"r{i}" for i in range(len(RANDOM_CASES))])
def test_depthwise_random_shapes(cc, case):
    import torch

    dt, N, C, M, sp, k, s, p, op = case
    x64 = I.normal(1000 + N * C, (N, C) + sp, 1.0, dt)
    w64 = I.normal(2000 + M, (C, M) + k, float(np.prod(k)) ** -0.5, dt)
    b64 = I.uniform(3000 + C, (C * M,), -0.1, 0.1, dt)
    ref, mag = ref_and_mag(x64, w64, b64, s, p, op, groups=C)
    outs = []
    for which in (0, 2):
        y = _dev_run(cc, x64, w64, b64, dt, s, p, op, 1, which)
        check_parity(to_host(y), ref, mag, dt, terms_per_output(1, k, s), f"{case} which={which}")
        outs.append(y)
    assert torch.equal(outs[0], outs[1]), case

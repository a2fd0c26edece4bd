"""GPU parity of the dense transposed convolution on seeded random shapes:
every route the planner picks (polyphase, its dilation reduction, gather)
and the forced gather route, against the CPU oracle on the same rounded
inputs.  Bars: relative L2 <= 1e-5 (fp32), <= 1e-2 (bf16/fp16), and every
output within the element bound of gpu_util.check_parity."""

import numpy as np
import pytest

from synth import inputs as I

from gpu_util import check_parity, ref_and_mag, terms_per_output, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cc():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vision_upsampler_decoders_amd import ctconv

    ctconv.load()
    return ctconv


def _cases(n, seed):
    """Channel counts across 32-channel blocks, strides 1-5, kernels up to
    4 taps per phase (some beyond, for the gather route), padding,
    output_padding, dilation (often dividing the stride in 2-D), 1-D and 2-D,
    all three dtypes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        nd = int(rng.integers(1, 3))
        s = [int(rng.integers(1, 6)) for _ in range(nd)]
        d = [1] * nd
        if rng.random() < 0.25:
            d = [int(rng.choice([2, si])) if si > 1 else 2 for si in s]
        k = [int(rng.integers(1, 4 * si + 2)) for si in s]
        if nd == 2 and rng.random() < 0.6:  # mostly 1 or 2 taps per phase in 2-D
            k = [max(1, si * int(rng.integers(1, 3)) - int(rng.integers(0, si))) for si in s]
        p = [int(rng.integers(0, di * (ki - 1) + 1)) for ki, di in zip(k, d)]
        op = [int(rng.integers(0, max(si, di))) for si, di in zip(s, d)]
        sp = [int(rng.integers(1, 12))] if nd == 2 else []
        sp += [int(rng.integers(1, 90))]
        o = [(a - 1) * b - 2 * c + e * (f - 1) + g + 1 for a, b, c, e, f, g in zip(sp, s, p, d, k, op)]
        if min(o) < 1:
            continue
        N = int(rng.integers(1, 3))
        C_in, C_out = int(rng.integers(1, 72)), int(rng.integers(1, 40))
        dt = str(rng.choice(["f32", "bf16", "f16"]))
        bias = bool(rng.random() < 0.5)
        out.append((dt, N, C_in, C_out, tuple(sp), tuple(k), tuple(s), tuple(p), tuple(op),
                    tuple(d), bias))
    return out


CASES = _cases(40, 77)


@pytest.mark.parametrize("case", CASES, ids=[f"r{i}" for i in range(len(CASES))])
def test_dense_random_shapes(cc, case):
    import torch

    dt, N, C_in, C_out, sp, k, s, p, op, d, has_b = case
    x64 = I.normal(500 + C_in, (N, C_in) + sp, 1.0, dt)
    w64 = I.normal(600 + C_out, (C_in, C_out) + k, (C_in * float(np.prod(k))) ** -0.5, dt)
    b64 = I.uniform(700 + C_out, (C_out,), -0.1, 0.1, dt) if has_b else None
    ref, mag = ref_and_mag(x64, w64, b64, s, p, op, d)
    pw = cc.prepack(to_dev(w64, dt), s)
    for route in (0, 2):
        y = cc.forward(to_dev(x64, dt), pw, None if b64 is None else to_dev(b64, dt), C_out, k,
                       s, p, op, d, route=route)
        torch.cuda.synchronize()
        check_parity(to_host(y), ref, mag, dt, terms_per_output(C_in, k, s, d),
                     f"{case} route={route}")


# ---------------------------------------------------------------------------
# the polyphase route's 2-D phase subsets and fp32 tap groups on random shapes

from random_cases import PLANNER_CASES  # noqa: E402


@pytest.mark.parametrize("case", PLANNER_CASES,
                         ids=[f"{c[0]}{i}" for i, c in enumerate(PLANNER_CASES)])
def test_planner_paths_random_shapes(cc, case):
    import torch

    from oracle import elu as oelu

    kind, dt, N, C_in, C_out, sp, k, s, p, op, d, has_b, act = case
    x64 = I.normal(800 + C_in, (N, C_in) + sp, 1.0, dt)
    w64 = I.normal(900 + C_out, (C_in, C_out) + k, (C_in * float(np.prod(k))) ** -0.5, dt)
    b64 = I.uniform(1000 + C_out, (C_out,), -0.1, 0.1, dt) if has_b else None
    ref, mag = ref_and_mag(x64, w64, b64, s, p, op, d)
    if act:
        ref = oelu(ref)  # 1-Lipschitz: the element bound on the sum carries over
    pw = cc.prepack(to_dev(w64, dt), s)
    for route in (0, 2):
        y = cc.forward(to_dev(x64, dt), pw, None if b64 is None else to_dev(b64, dt), C_out, k,
                       s, p, op, d, route=route, act=cc.ACT_ELU if act else cc.ACT_NONE)
        torch.cuda.synchronize()
        check_parity(to_host(y), ref, mag, dt, terms_per_output(C_in, k, s, d),
                     f"{case} route={route}", abs_slack=1e-6 if act else 0.0)

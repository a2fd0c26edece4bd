"""Outputs no tap reaches under a dilation reduction (g = gcd(s, d) > 1:
every output but each g-th along a dimension holds act(bias) alone).  A fill
launch writes act(bias) over y before the polyphase kernel writes the reached
outputs, and the gather kernel writes every output itself, so these tests
hand the call an output pre-filled with NaN and check every element against
the oracle: an output that neither writes keeps its NaN and fails the element
bound.  The cases vary the first reached output o0 = (g - p mod g) mod g
(padding), output_padding, ragged sizes, the reduced stride (1, 2, 3), bias,
the fused ELU and the dtype; one 2-D case has more phases than a column tile
(phase subsets) and one 1-D case reaches no output at all."""

import numpy as np
import pytest

from synth import inputs as I

from gpu_util import check_parity, ref_and_mag, say, terms_per_output, to_dev, to_host

pytestmark = pytest.mark.gpu

# name, dtype, N, C_in, C_out, in_spatial, kernel, stride, padding, output_padding,
# dilation, bias, elu, expected route (1 polyphase, None: not checked)
CASES = [
    ("2d_s2d2_p1_op1", "f32", 2, 24, 20, (13, 17), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2), True, False, 1),
    ("2d_s2d2_p0_o0even", "f32", 1, 16, 24, (11, 9), (3, 3), (2, 2), (0, 0), (0, 1), (2, 2), False, False, 1),
    ("2d_s2d2_p3_bf16_elu", "bf16", 2, 40, 24, (9, 12), (3, 3), (2, 2), (3, 1), (1, 0), (2, 2), True, True, 1),
    ("2d_s4d2_f32", "f32", 1, 32, 16, (7, 10), (4, 3), (4, 4), (1, 2), (3, 0), (2, 2), True, False, 1),
    ("2d_s2d4_f16", "f16", 1, 24, 32, (10, 8), (2, 2), (2, 2), (1, 2), (1, 3), (4, 4), True, False, 1),
    ("2d_s3d3_f32_elu", "f32", 1, 20, 16, (8, 9), (3, 3), (3, 3), (2, 1), (2, 0), (3, 3), True, True, 1),
    ("2d_mixed_g_bf16", "bf16", 1, 32, 24, (9, 11), (3, 3), (2, 1), (1, 0), (1, 0), (2, 1), True, False, 1),
    ("2d_s6d4_subsets", "bf16", 1, 32, 32, (6, 7), (3, 3), (6, 6), (1, 2), (1, 0), (4, 4), True, False, None),
    ("1d_s2d2_p1", "f32", 2, 40, 24, (57,), (4,), (2,), (1,), (1,), (2,), True, False, 1),
    ("1d_s4d2_bf16_elu", "bf16", 2, 64, 48, (75,), (8,), (4,), (3,), (1,), (2,), True, True, 1),
    ("1d_s3d3_f16", "f16", 1, 33, 17, (90,), (4,), (3,), (2,), (2,), (3,), False, False, 1),
    ("1d_reaches_none", "f32", 1, 16, 8, (1,), (2,), (2,), (1,), (0,), (2,), True, True, None),
]


@pytest.fixture(scope="module")
def cc():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vision_upsampler_decoders_amd import ctconv

    ctconv.load()
    return ctconv


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_unreached_outputs_written_once(cc, case):
    import torch

    from oracle import elu as oelu

    name, dt, N, C_in, C_out, sp, k, s, p, op, d, has_b, elu, route = case
    dcode = {"f32": cc.CTCONV_F32, "bf16": cc.CTCONV_BF16, "f16": cc.CTCONV_F16}[dt]
    r = cc.ctconv_query_route(N, C_in, C_out, sp, k, s, p, op, d, dcode)
    say(f"dilation fill {name}: route {r}")
    if route is not None:
        assert r == route, (name, r)
    x64 = I.normal(1300 + C_in, (N, C_in) + sp, 1.0, dt)
    w64 = I.normal(1400 + C_out, (C_in, C_out) + k, (C_in * float(np.prod(k))) ** -0.5, dt)
    b64 = I.uniform(1500 + C_out, (C_out,), -0.5, 0.5, dt) if has_b else None
    ref, mag = ref_and_mag(x64, w64, b64, s, p, op, d)
    if elu:
        ref = oelu(ref)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    pw = cc.prepack(to_dev(w64, dt), s)
    for rt in (0, 2):
        y = torch.full(ref.shape, float("nan"), dtype=tdt, device="cuda")
        cc.forward(to_dev(x64, dt), pw, None if b64 is None else to_dev(b64, dt), C_out, k, s, p,
                   op, d, route=rt, out=y, act=cc.ACT_ELU if elu else cc.ACT_NONE)
        torch.cuda.synchronize()
        check_parity(to_host(y), ref, mag, dt, terms_per_output(C_in, k, s, d),
                     f"{name} route={rt}", abs_slack=1e-6 if elu else 0.0)

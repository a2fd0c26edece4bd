"""GPU: the deterministic split reduction (ctconv_forward_ws).

The iSTFT workload (4098 -> 1 channels, k4096 s1024, 345 frames, N = 8) has
few output tiles, so ctconv_forward_ws splits its reduction over input
channels into partial sums in the workspace and adds them in a fixed order:
repeated calls give the same bits, the result matches the oracle on every
output, and the unsplit ctconv_forward agrees within the fp32 bar."""

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


@pytest.mark.parametrize("N", [8, 1])
def test_istft_split_is_deterministic_and_exact(cc, N):
    import torch

    wl = I.workload("istft")
    L = wl.layers[0]
    x64 = I.gen_x(wl)[:N]
    w64 = I.gen_w(wl)
    need = cc.ctconv_workspace_bytes(N, L.C_in, L.C_out, wl.in_spatial, L.kernel, L.stride,
                                     L.padding, 0, 1, cc.CTCONV_F32)
    say(f"istft N={N}: workspace {need} bytes")
    assert need > 0
    x, pw = to_dev(x64, "f32"), cc.prepack(to_dev(w64, "f32"), L.stride)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for rep in range(3):
        ws.fill_(0xFF if rep == 1 else 0x7F)  # contents on entry must not matter
        outs.append(cc.forward(x, pw, None, 1, L.kernel, L.stride, L.padding, workspace=ws))
    plain = cc.forward(x, pw, None, 1, L.kernel, L.stride, L.padding)
    torch.cuda.synchronize()
    for y in outs[1:]:
        assert torch.equal(y.view(torch.int32), outs[0].view(torch.int32))
    ref, mag = ref_and_mag(x64, w64, None, L.stride, L.padding)
    K = terms_per_output(L.C_in, L.kernel, L.stride)
    check_parity(to_host(outs[0]), ref, mag, "f32", K, f"istft N={N} split")
    check_parity(to_host(plain), ref, mag, "f32", K, f"istft N={N} unsplit")
    # a workspace one slab short is refused before anything is enqueued
    with pytest.raises(ValueError, match="workspace"):
        cc.forward(x, pw, None, 1, L.kernel, L.stride, L.padding, workspace=ws[:need - 16])


def test_split_with_bias_and_elu(cc):
    """The reduction kernel adds the bias and applies the activation after
    the partial sums (an fp32 shape with few tiles and a long reduction)."""
    import torch

    from oracle import elu

    N, C_in, C_out, L_in, k, s = 1, 1024, 8, 40, 64, 16
    x64 = I.normal(61, (N, C_in, L_in), 1.0, "f32")
    w64 = I.normal(62, (C_in, C_out, k), (C_in * k) ** -0.5, "f32")
    b64 = I.uniform(63, (C_out,), -0.5, 0.5, "f32")
    need = cc.ctconv_workspace_bytes(N, C_in, C_out, (L_in,), k, s, 0, 0, 1, cc.CTCONV_F32)
    say(f"split with bias and elu: workspace {need} bytes")
    assert need > 0
    pw = cc.prepack(to_dev(w64, "f32"), (s,))
    y = cc.forward(to_dev(x64, "f32"), pw, to_dev(b64, "f32"), C_out, (k,), (s,), 0,
                   act=cc.ACT_ELU, workspace=True)
    torch.cuda.synchronize()
    pre, mag = ref_and_mag(x64, w64, b64, (s,), 0)
    check_parity(to_host(y), elu(pre), mag, "f32", terms_per_output(C_in, (k,), (s,)),
                 "split+bias+elu", abs_slack=1e-6)

"""GPU: reads stay inside the caller's buffers, and the Python helpers reject
arguments that do not match the call.

Ragged channel counts (C_in not a multiple of the kernels' channel chunk)
with x placed inside a larger buffer whose other elements are NaN: a load
that strayed past x's extent would carry a NaN into the output (the packed
weights of the padding channels are zero, but 0 * NaN is NaN).  Each route
and kernel family is exercised, and the result is checked against the oracle
on every output."""

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


def _in_nan_buffer(t, pad_elems=4096):
    """A copy of t placed inside a NaN-filled buffer, with NaNs before and after
    it (the copy's start stays 16-byte aligned)."""
    import torch

    buf = torch.full((t.numel() + 2 * pad_elems,), float("nan"), dtype=t.dtype, device=t.device)
    v = buf[pad_elems:pad_elems + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == 0
    return buf, v


NAN_CASES = [
    # name, dt, N, C_in, C_out, spatial, k, s, p, op, d, route
    ("poly1d_bf16_c37", "bf16", 3, 37, 24, (203,), (8,), (4,), (2,), (0,), (1,), 1),
    ("poly1d_f16_c45_m3", "f16", 2, 45, 40, (130,), (12,), (4,), (3,), (1,), (1,), 1),
    ("poly1d_f32_c21", "f32", 2, 21, 16, (150,), (8,), (4,), (2,), (0,), (1,), 1),
    ("poly1d_bf16_odd_len_c33", "bf16", 2, 33, 16, (211,), (8,), (4,), (2,), (0,), (1,), 1),
    ("poly2d_bf16_c35", "bf16", 2, 35, 20, (9, 24), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), 1),
    ("poly2d_bf16_oddplane_c19", "bf16", 2, 19, 16, (5, 7), (4, 4), (2, 2), (1, 1), (0, 0),
     (1, 1), 1),
    ("poly2d_f32_dil2_c13", "f32", 2, 13, 12, (11, 13), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2), 1),
    ("gather1d_dil2_c37", "bf16", 2, 37, 24, (101,), (8,), (4,), (3,), (1,), (2,), 2),
    ("gather2d_f32_c29", "f32", 2, 29, 12, (10, 13), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), 2),
]


@pytest.mark.parametrize("case", NAN_CASES, ids=[c[0] for c in NAN_CASES])
def test_ragged_channels_read_inside_x(cc, case):
    import torch

    name, dt, N, C_in, C_out, sp, k, s, p, op, d, route = case
    say(f"nan-surrounded x: {name} route={route}")
    x64 = I.normal(40 + C_in, (N, C_in) + sp, 1.0, dt)
    w64 = I.normal(41 + C_out, (C_in, C_out) + k, (C_in * np.prod(k)) ** -0.5, dt)
    b64 = I.uniform(42, (C_out,), -0.1, 0.1, dt)
    buf, x = _in_nan_buffer(to_dev(x64, dt))
    pw = cc.prepack(to_dev(w64, dt), s)
    y = cc.forward(x, pw, to_dev(b64, dt), C_out, k, s, p, op, d, route=route)
    torch.cuda.synchronize()
    yh = to_host(y)
    assert np.isfinite(yh).all(), f"{name}: a load read outside x"
    ref, mag = ref_and_mag(x64, w64, b64, s, p, op, d)
    check_parity(yh, ref, mag, dt, terms_per_output(C_in, k, s, d), name)
    del buf


def test_forward_rejects_mismatched_arguments(cc):
    import torch

    x = torch.zeros((2, 40, 50), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((40, 24, 8), dtype=torch.bfloat16, device="cuda")
    pw = cc.prepack(w, (4,))
    b = torch.zeros(24, dtype=torch.bfloat16, device="cuda")
    y = cc.forward(x, pw, b, 24, (8,), (4,), (2,))
    assert tuple(y.shape) == (2, 24, 200)
    # a prepack made with another stride (3: 3 phases x 3 taps, not 4 x 2) has
    # another size
    pw_s3 = cc.prepack(w, (3,))
    with pytest.raises(ValueError, match="packed"):
        cc.forward(x, pw_s3, b, 24, (8,), (4,), (2,))
    # another dtype
    with pytest.raises(TypeError, match="packed"):
        cc.forward(x, pw.float(), b, 24, (8,), (4,), (2,))
    with pytest.raises(TypeError, match="bias"):
        cc.forward(x, pw, b.float(), 24, (8,), (4,), (2,))
    with pytest.raises(ValueError, match="bias"):
        cc.forward(x, pw, b[:20], 24, (8,), (4,), (2,))
    # out of the wrong shape, dtype or layout
    with pytest.raises(ValueError, match="out"):
        cc.forward(x, pw, b, 24, (8,), (4,), (2,),
                   out=torch.empty((2, 24, 199), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError, match="out"):
        cc.forward(x, pw, b, 24, (8,), (4,), (2,),
                   out=torch.empty((2, 24, 200), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="contiguous"):
        cc.forward(x, pw, b, 24, (8,), (4,), (2,),
                   out=torch.empty((2, 200, 24), dtype=torch.bfloat16, device="cuda").transpose(1, 2))
    # depthwise: weight dtype and bias length
    xd = torch.zeros((2, 6, 30), dtype=torch.float32, device="cuda")
    wd = torch.zeros((6, 2, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError, match="w"):
        cc.depthwise_forward(xd, wd.half(), None, 2, 1)
    with pytest.raises(ValueError, match="bias"):
        cc.depthwise_forward(xd, wd, torch.zeros(6, device="cuda"), 2, 1)
    with pytest.raises(ValueError, match="out"):
        cc.elu(xd, out=torch.empty((2, 6, 31), device="cuda"))


def test_explicit_stream_waits_for_current(cc):
    """forward(stream=side) from another current stream: the side stream waits
    for the work queued before it, and the result equals the current-stream
    call."""
    import torch

    x64 = I.normal(51, (2, 64, 300), 1.0, "bf16")
    w64 = I.normal(52, (64, 32, 8), 0.05, "bf16")
    w = to_dev(w64, "bf16")
    pw = cc.prepack(w, (4,))
    ref = cc.forward(to_dev(x64, "bf16"), pw, None, 32, (8,), (4,), (2,))
    side = torch.cuda.Stream()
    for _ in range(3):
        x = to_dev(x64, "bf16")
        x2 = (x.float() * 1.0).to(torch.bfloat16)  # queued on the current stream
        y = cc.forward(x2, pw, None, 32, (8,), (4,), (2,), stream=side)
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


def test_clock_probe(cc):
    """The sustained-clock probe returns a clock in the chip's range and an
    MFMA rate below the published bf16 peak; a short workspace is refused."""
    import ctypes

    import torch

    say("clock probe")
    mhz, tflops = cc.sustained_clock(iters=2048)
    assert 800.0 < mhz < 2600.0, mhz
    assert 100.0 < tflops < 2516.6 * 1.05, tflops
    nb = cc.ctconv_clock_probe_bytes()
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = ctypes.c_double()
    st = cc.load().ctconv_clock_probe(ctypes.c_void_p(ws.data_ptr()), nb - 8, 16,
                                      ctypes.byref(out), None, None)
    assert st == 7

"""GPU: ctconv_forward_noalloc (the workspace is the library's fixed scratch)
against ctconv_forward_ws with a caller workspace, through the C ABI.

Two calls in a row, the second with a smaller input: the iSTFT workload,
whose reduction is split into the workspace (N = 8, then N = 2), and a bf16
vocoder-layer shape that needs no workspace.  The same plan and the same
order of additions give the same bits; both are also checked against the
oracle on every output."""

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


def _call_both(cc, x, pw, b, C_out, k, s, p, dt, act=0):
    import torch

    N, C_in = x.shape[0], x.shape[1]
    sp = tuple(x.shape[2:])
    osp = cc.ctconv_output_shape(sp, k, s, p)
    stream = int(torch.cuda.current_stream().cuda_stream)
    y_na = torch.full((N, C_out) + osp, float("nan"), dtype=x.dtype, device="cuda")
    y_ws = torch.full_like(y_na, float("nan"))
    bptr = None if b is None else b.data_ptr()
    cc.ctconv_forward_noalloc(x.data_ptr(), pw.data_ptr(), bptr, y_na.data_ptr(), N, C_in, C_out,
                              sp, k, s, p, 0, 1, dt, act, stream)
    need = cc.ctconv_workspace_bytes(N, C_in, C_out, sp, k, s, p, 0, 1, dt)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    cc.ctconv_forward_ws(x.data_ptr(), pw.data_ptr(), bptr, y_ws.data_ptr(), N, C_in, C_out, sp,
                         k, s, p, 0, 1, dt, act, ws.data_ptr() if need else None, need, stream)
    torch.cuda.synchronize()
    return y_na, y_ws, need


def test_noalloc_matches_workspace_call_split_then_smaller(cc):
    import torch

    wl = I.workload("istft")
    L = wl.layers[0]
    w64 = I.gen_w(wl)
    pw = cc.prepack(to_dev(w64, "f32"), L.stride)
    x64_all = I.gen_x(wl)
    for N in (8, 2):  # the second call is smaller and overwrites the same scratch
        x64 = x64_all[:N]
        say(f"noalloc istft N={N}")
        y_na, y_ws, need = _call_both(cc, to_dev(x64, "f32"), pw, None, 1, L.kernel, L.stride,
                                      L.padding, cc.CTCONV_F32)
        assert 0 < need <= cc.ctconv_scratch_bytes()
        assert torch.equal(y_na.view(torch.int32), y_ws.view(torch.int32))
        ref, mag = ref_and_mag(x64, w64, None, L.stride, L.padding)
        check_parity(to_host(y_na), ref, mag, "f32", terms_per_output(L.C_in, L.kernel, L.stride),
                     f"noalloc istft N={N}")


def test_noalloc_without_split_bf16(cc):
    import torch

    for N, Lin in ((2, 300), (1, 120)):
        say(f"noalloc bf16 512->256 k16 s8 N={N} L={Lin}")
        x64 = I.normal(71, (N, 512, Lin), 1.0, "bf16")
        w64 = I.normal(72, (512, 256, 16), (512 * 16) ** -0.5, "bf16")
        b64 = I.uniform(73, (256,), -0.1, 0.1, "bf16")
        pw = cc.prepack(to_dev(w64, "bf16"), (8,))
        y_na, y_ws, need = _call_both(cc, to_dev(x64, "bf16"), pw, to_dev(b64, "bf16"), 256,
                                      (16,), (8,), (4,), cc.CTCONV_BF16, act=cc.ACT_ELU)
        assert need == 0
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))
        from oracle import elu

        pre, mag = ref_and_mag(x64, w64, b64, (8,), (4,))
        check_parity(to_host(y_na), elu(pre), mag, "bf16", terms_per_output(512, (16,), (8,)),
                     f"noalloc bf16 N={N}", abs_slack=1e-6)

"""GPU: the streaming entry points (ctconv_stream_step / ctconv_stream_flush)
through the C ABI.  Concatenating the outputs of the chunk calls and of the
flush must equal the one-shot transposed convolution of all the frames with
padding 0, computed by the CPU oracle on the same storage-rounded inputs,
with the bias and the activation applied exactly once per output."""

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


def _stream(cc, x, pw, b, C_out, k, s, chunks, act):
    """Run the stream over x [N, C_in, F] in chunks of the given frame counts."""
    import torch

    N, C_in, F = x.shape
    assert sum(chunks) == F
    dt = cc.dtype_code(x)
    stream = torch.cuda.current_stream().cuda_stream
    _, Tl, _ = cc.ctconv_stream_sizes(N, C_out, 1, k, s, dt)
    tails = [torch.empty((N, C_out, max(Tl, 1)), dtype=torch.float32, device="cuda")
             for _ in range(2)]
    tail_in = None
    outs = []
    f0 = 0
    for i, L in enumerate(chunks):
        Ly, Tl, ws_bytes = cc.ctconv_stream_sizes(N, C_out, L, k, s, dt)
        xc = x[:, :, f0:f0 + L].contiguous()
        y = torch.empty((N, C_out, Ly), dtype=x.dtype, device="cuda")
        ws = torch.empty(ws_bytes // x.element_size() + 8, dtype=x.dtype, device="cuda")
        tail_out = tails[i % 2]
        cc.ctconv_stream_step(xc.data_ptr(), pw.data_ptr(), None if b is None else b.data_ptr(),
                              y.data_ptr(), None if tail_in is None else tail_in.data_ptr(),
                              tail_out.data_ptr() if Tl > 0 else None, ws.data_ptr(), N, C_in,
                              C_out, L, k, s, dt, act, stream)
        outs.append(y)
        tail_in = tail_out if Tl > 0 else None
        f0 += L
    if Tl > 0:
        y = torch.empty((N, C_out, Tl), dtype=x.dtype, device="cuda")
        cc.ctconv_stream_flush(tail_in.data_ptr(), None if b is None else b.data_ptr(),
                               y.data_ptr(), N, C_out, k, s, dt, act, stream)
        outs.append(y)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=2)


STREAM_CASES = [
    # name, dt, N, C_in, C_out, k, s, chunks, bias, act
    ("k2s_bf16", "bf16", 2, 64, 48, 10, 5, (3, 1, 4, 2), True, 0),
    # tail (12) longer than a one-frame chunk's output (4): carried over
    ("long_tail_f32_elu", "f32", 1, 40, 24, 16, 4, (1, 1, 2, 5), True, 1),
    ("k2s_f16_nobias", "f16", 2, 32, 16, 8, 4, (5, 7), False, 0),
    ("k_eq_s_bf16", "bf16", 1, 48, 32, 4, 4, (2, 3), True, 0),
    # the first vocoder layer's channels, one 8-frame chunk after another
    ("voc_l0_bf16_elu", "bf16", 1, 512, 256, 16, 8, (8, 8, 8), True, 1),
]


def _case_inputs(case):
    name, dt, N, C_in, C_out, k, s, chunks, has_b, act = case
    F = sum(chunks)
    seed = 800 + len(name)
    x64 = I.normal(seed, (N, C_in, F), 1.0, dt)
    w64 = I.normal(seed + 1, (C_in, C_out, k), (C_in * k) ** -0.5, dt)
    b64 = I.uniform(seed + 2, (C_out,), -0.5, 0.5, dt) if has_b else None
    return x64, w64, b64


@pytest.mark.parametrize("case", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_stream_equals_one_shot(cc, case):
    """Every output of the stream against the oracle's one-shot convolution:
    relative L2 and the per-element bound (one rounding of the output, the
    fp32 accumulation of C_in * ceil(k / s) products)."""
    from oracle import elu as oelu

    name, dt, N, C_in, C_out, k, s, chunks, has_b, act = case
    say(f"stream {name}: chunks {chunks}")
    x64, w64, b64 = _case_inputs(case)
    pw = cc.prepack(to_dev(w64, dt), (s,))
    y = _stream(cc, to_dev(x64, dt), pw, None if b64 is None else to_dev(b64, dt), C_out, k, s,
                chunks, act)
    ref, mag = ref_and_mag(x64, w64, b64, (s,), (0,))
    slack = 0.0
    if act == 1:
        # ELU is 1-Lipschitz: the conv's bound carries over; plus the
        # exponential's absolute error
        ref = oelu(ref)
        slack = 1e-6
    assert tuple(y.shape) == ref.shape
    check_parity(to_host(y), ref, mag, dt, terms_per_output(C_in, (k,), (s,)), name, slack)


def _ulp_distance(a, b, dt):
    """Distance in units in the last place between two 16-bit tensors (the
    bit patterns mapped to a monotone integer order)."""
    import torch

    def key(t):
        i = t.view(torch.int16).to(torch.int32)
        return torch.where(i < 0, -(i & 0x7FFF), i)
    return (key(a) - key(b)).abs()


@pytest.mark.parametrize("case", [c for c in STREAM_CASES if c[1] != "f32"],
                         ids=[c[0] for c in STREAM_CASES if c[1] != "f32"])
def test_stream_within_one_ulp_of_forward(cc, case):
    """16-bit streams round each output once, like the one-shot forward: the
    two differ only by the order of their fp32 sums.  Every output is within
    one unit in the last place of the storage type of the forward's, unless
    cancellation lets the two fp32 sums differ by more: then the difference
    stays within one ulp plus both sums' accumulation bound
    (2 * C_ACC * K * 2^-24 * the sum of the terms' magnitudes)."""
    import torch

    from gpu_util import C_ACC, U_ACC

    name, dt, N, C_in, C_out, k, s, chunks, has_b, act = case
    x64, w64, b64 = _case_inputs(case)
    x, w = to_dev(x64, dt), to_dev(w64, dt)
    b = None if b64 is None else to_dev(b64, dt)
    pw = cc.prepack(w, (s,))
    y = _stream(cc, x, pw, b, C_out, k, s, chunks, act)
    y1 = cc.forward(x, pw, b, C_out, (k,), (s,), (0,), act=act)
    torch.cuda.synchronize()
    assert y.shape == y1.shape
    d = to_host(_ulp_distance(y, y1, dt))
    ys, yf = to_host(y).astype(np.float64), to_host(y1).astype(np.float64)
    _, mag = ref_and_mag(x64, w64, b64, (s,), (0,))
    K = terms_per_output(C_in, (k,), (s,))
    ulp = np.abs(yf) * (2.0 ** -7 if dt == "bf16" else 2.0 ** -10)
    ok = (d <= 1) | (np.abs(ys - yf) <= ulp + 2 * C_ACC * K * U_ACC * mag)
    say(f"  {name}: outputs more than one ulp apart {int((d > 1).sum())} of {d.size}, "
        f"all within the accumulation bound: {bool(ok.all())}")
    assert ok.all()
    assert (d > 1).mean() < 1e-3


def test_stream_bias_applied_once(cc):
    """Zero frames: every emitted output, including those that pass through
    the held-back tail, is exactly the bias (fp32)."""
    import torch

    N, C_in, C_out, k, s = 2, 16, 8, 12, 4
    b64 = I.uniform(5, (C_out,), -1.0, 1.0, "f32")
    w64 = I.normal(6, (C_in, C_out, k), 0.2, "f32")
    x = torch.zeros((N, C_in, 7), dtype=torch.float32, device="cuda")
    pw = cc.prepack(to_dev(w64, "f32"), (s,))
    y = _stream(cc, x, pw, to_dev(b64, "f32"), C_out, k, s, (1, 2, 4), 0)
    ref = np.broadcast_to(b64.astype(np.float32)[None, :, None], tuple(y.shape))
    np.testing.assert_array_equal(to_host(y).astype(np.float32), ref)


def test_stream_steps_in_a_graph_match_eager(cc):
    """Two stream steps (the tail buffers alternate) captured as a HIP graph
    and replayed several times, with new inputs copied in and eager work and
    synchronisation between replays: every replay's outputs equal the eager
    calls' on the same inputs, bit for bit."""
    import torch

    dt, N, C_in, C_out, k, s, L = "bf16", 1, 64, 32, 10, 5, 6
    dcode = 1
    w = to_dev(I.normal(31, (C_in, C_out, k), (C_in * k) ** -0.5, dt), dt)
    b = to_dev(I.uniform(32, (C_out,), -0.5, 0.5, dt), dt)
    pw = cc.prepack(w, (s,))
    xs = [to_dev(I.normal(40 + i, (N, C_in, L), 1.0, dt), dt) for i in range(8)]
    Ly, Tl, ws_bytes = cc.ctconv_stream_sizes(N, C_out, L, k, s, dcode)
    ws = torch.empty(ws_bytes // 2 + 8, dtype=torch.bfloat16, device="cuda")

    def run(xin, y, tin, tout):
        cc.ctconv_stream_step(xin.data_ptr(), pw.data_ptr(), b.data_ptr(), y.data_ptr(),
                              tin.data_ptr(), tout.data_ptr(), ws.data_ptr(), N, C_in, C_out, L,
                              k, s, dcode, cc.ACT_ELU, torch.cuda.current_stream().cuda_stream)

    def fresh():
        return ([torch.zeros((N, C_out, Tl), dtype=torch.float32, device="cuda")
                 for _ in range(2)],
                [torch.empty((N, C_out, Ly), dtype=torch.bfloat16, device="cuda")
                 for _ in range(2)])

    # eager reference over the eight chunks
    tails, ys = fresh()
    ref = []
    for i, x in enumerate(xs):
        run(x, ys[i % 2], tails[i % 2], tails[1 - i % 2])
        ref.append(ys[i % 2].clone())
    torch.cuda.synchronize()
    # graph of two steps reading fixed input buffers
    tails, ys = fresh()
    xa, xb = torch.empty_like(xs[0]), torch.empty_like(xs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, then reset the state
        run(xa.copy_(xs[0]), ys[0], tails[0], tails[1])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for t in tails:
        t.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(xa, ys[0], tails[0], tails[1])
        run(xb, ys[1], tails[1], tails[0])
    for j in range(4):
        xa.copy_(xs[2 * j])
        xb.copy_(xs[2 * j + 1])
        g.replay()
        torch.cuda.synchronize()
        _ = (xa.float() * 2).sum().item()  # eager work between replays
        for q in range(2):
            assert torch.equal(ys[q], ref[2 * j + q]), (j, q)
        say(f"graph replay {j}: equal to eager")


@pytest.mark.parametrize("n_fft,hop,T", [(256, 64, 20), (512, 128, 9)])
def test_istft_pipeline_matches_torch_istft(cc, n_fft, hop, T):
    """Inverse DFT + overlap-add as ctconv_forward with the Hann-windowed
    basis, the window-square envelope as ctconv_forward of ones with h^2,
    then ctconv_istft_normalize (trim n_fft/2, hop*(T-1) samples): equal to
    torch.istft (centred, periodic Hann, float64 on the CPU, an independent
    library routine) within the fp32 bar."""
    import torch

    from oracle import rel_l2

    N, F = 2, n_fft // 2 + 1
    rng = np.random.default_rng(n_fft + T)
    X = rng.standard_normal((N, F, T)) + 1j * rng.standard_normal((N, F, T))
    x64 = I.round_to_dtype(np.concatenate([X.real, X.imag], axis=1), "f32")
    Xr = x64[:, :F] + 1j * x64[:, F:]
    w = to_dev(I.istft_basis(n_fft, "f32"), "f32")
    pw = cc.prepack(w, (hop,))
    y = cc.forward(to_dev(x64, "f32"), pw, None, 1, (n_fft,), (hop,))
    h = I.hann_periodic(n_fft)
    wsq = to_dev(I.round_to_dtype((h * h).reshape(1, 1, n_fft), "f32"), "f32")
    env = cc.forward(torch.ones((1, 1, T), dtype=torch.float32, device="cuda"),
                     cc.prepack(wsq, (hop,)), None, 1, (n_fft,), (hop,))
    L_in = y.shape[2]
    trim, L_out = n_fft // 2, hop * (T - 1)
    out = torch.empty((N, L_out), dtype=torch.float32, device="cuda")
    cc.ctconv_istft_normalize(y.data_ptr(), env.data_ptr(), out.data_ptr(), N, L_in, trim, L_out,
                              0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = torch.istft(torch.from_numpy(Xr), n_fft, hop_length=hop,
                      window=torch.hann_window(n_fft, periodic=True, dtype=torch.float64),
                      center=True, normalized=False, onesided=True).numpy()
    assert ref.shape == (N, L_out)
    err = rel_l2(to_host(out), ref)
    say(f"istft n_fft={n_fft} hop={hop} T={T}: rel_l2 = {err:.3e}")
    assert err <= 1e-5, err

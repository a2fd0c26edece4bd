"""Pins of the CPU reference (oracle/) to facts other than itself.

Each check below is independent of the oracle's own loops:
  * torch.nn.functional.conv_transpose{1,2}d in float64 on the CPU (a library
    routine computing the same operation);
  * the adjoint identity <convT(x), g> = <x, conv(g)> with torch's *direct*
    convolution, a different operation;
  * the polyphase identity of ExecuTorch PR #25037 ("[XNNPACK] Lower dense
    transposed convs as one polyphase conv + depth to space", Summary formula):
    one stride-1 conv with m taps and padding m-1 giving every output phase,
    then interleave and slice;
  * impulse responses, the k = s no-overlap matmul, hand-worked examples
    (tests/golden/hand_worked.json);
  * the inverse-STFT closed forms: numpy's irfft + Hann + overlap-add, and
    perfect reconstruction (periodic Hann squared at hop n/4 sums to 3/2);
  * the grouped (depthwise) case: torch's grouped conv_transpose in float64,
    the dense oracle on the block-diagonal expansion of the grouped weight, and
    impulse responses that stay inside their channel group;
  * planted-mistake runs: copies of the oracle with one plausible bug each must
    fail these pins.
"""

import json
import os
import subprocess

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from synth import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).uniform(-1, 1, size=shape)


CASES_1D = [
    # (C_in, C_out, L, k, s, p, op, d, bias)
    (3, 2, 7, 4, 2, 1, 0, 1, True),
    (2, 3, 5, 8, 4, 2, 0, 1, False),
    (4, 2, 6, 10, 5, 3, 0, 1, True),
    (1, 1, 9, 3, 2, 1, 1, 1, True),
    (2, 2, 4, 3, 2, 0, 1, 2, False),
    (3, 1, 5, 5, 3, 2, 2, 1, True),
    (2, 2, 1, 6, 3, 1, 0, 1, True),
    (2, 3, 6, 1, 1, 0, 0, 1, False),
    (1, 2, 3, 7, 1, 3, 0, 1, False),
    (2, 2, 5, 2, 3, 0, 2, 1, True),
    (2, 1, 4, 4, 2, 2, 1, 3, True),
]

CASES_2D = [
    # (C_in, C_out, (H, W), k, s, p, op, d, bias)
    (2, 3, (4, 5), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), True),
    (3, 2, (3, 4), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), False),
    (2, 2, (4, 3), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2), True),
    (1, 2, (3, 3), (2, 6), (1, 3), (0, 2), (0, 0), (1, 1), True),
    (2, 1, (2, 5), (4, 2), (2, 2), (0, 1), (1, 0), (1, 1), False),
    (2, 2, (5, 2), (3, 1), (3, 1), (2, 0), (2, 0), (1, 1), False),
]


def _torch_ref(x, w, b, s, p, op, d):
    xt, wt = torch.from_numpy(x), torch.from_numpy(w)
    bt = None if b is None else torch.from_numpy(b)
    fn = F.conv_transpose1d if x.ndim == 3 else F.conv_transpose2d
    return fn(xt, wt, bt, stride=s, padding=p, output_padding=op, dilation=d).numpy()


def _make(case, nd, seed):
    C_in, C_out, L, k, s, p, op, d, has_b = case
    L = (L,) if nd == 1 else tuple(L)
    k = (k,) if nd == 1 else tuple(k)
    x = _rand((2, C_in) + L, seed)
    w = _rand((C_in, C_out) + k, seed + 1)
    b = _rand((C_out,), seed + 2) if has_b else None
    return x, w, b, s, p, op, d


@pytest.mark.parametrize("case", CASES_1D + CASES_2D)
def test_vs_torch_float64(oracle_mod, case):
    nd = 1 if isinstance(case[2], int) else 2
    x, w, b, s, p, op, d = _make(case, nd, 11)
    y = oracle_mod.conv_transpose(x, w, b, s, p, op, d)
    ref = _torch_ref(x, w, b, s, p, op, d)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES_1D + CASES_2D)
def test_adjoint_identity(oracle_mod, case):
    """<convT(x), g> == <x, conv(g)>: torch's direct convolution reads the same
    weight [C_in, C_out, k...] as a [out=C_in, in=C_out, k...] filter."""
    nd = 1 if isinstance(case[2], int) else 2
    x, w, _, s, p, op, d = _make(case, nd, 23)
    y = oracle_mod.conv_transpose(x, w, None, s, p, op, d)
    g = _rand(y.shape, 99)
    conv = F.conv1d if nd == 1 else F.conv2d
    cg = conv(torch.from_numpy(g), torch.from_numpy(w), None, stride=s, padding=p,
              dilation=d).numpy()
    # output_padding can leave trailing rows of conv(g) with no input behind them
    cg = cg[(slice(None), slice(None)) + tuple(slice(0, n) for n in x.shape[2:])]
    lhs = float(np.sum(y * g))
    rhs = float(np.sum(x * cg))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def _polyphase_1d(x, w, bias, s, p, op):
    """ExecuTorch PR #25037 (Summary): for k = m*s, one stride-1 conv with m taps
    and padding m-1 yields every phase, y[s*q + j] = sum_{u<m} x[q+u-(m-1)] *
    w[s*(m-1-u) + j]; the phases are interleaved (view, permute, view) and the
    padding sliced off.  Written directly with numpy."""
    N, C_in, L = x.shape
    C_out, k = w.shape[1], w.shape[2]
    m = k // s
    xp = np.concatenate([np.zeros((N, C_in, m - 1)), x, np.zeros((N, C_in, m - 1))], axis=2)
    Q = L + m - 1
    z = np.zeros((N, C_out, Q, s))  # phase outputs
    for q in range(Q):
        for j in range(s):
            for u in range(m):
                # xp index q+u corresponds to x index q+u-(m-1)
                z[:, :, q, j] += np.einsum("nc,co->no", xp[:, :, q + u], w[:, :, s * (m - 1 - u) + j])
    full = z.reshape(N, C_out, Q * s)
    L_out = (L - 1) * s - 2 * p + k + op
    y = full[:, :, p:p + L_out]
    if bias is not None:
        y = y + bias[None, :, None]
    return y


@pytest.mark.parametrize("s,m,p,op,L", [(4, 2, 2, 0, 7), (5, 2, 3, 0, 6), (2, 3, 1, 1, 5),
                                        (3, 1, 0, 0, 4), (8, 2, 4, 3, 3), (2, 2, 0, 0, 1),
                                        (6, 2, 5, 2, 5)])
def test_polyphase_identity(oracle_mod, s, m, p, op, L):
    assert op <= p or (p == 0 and op == 0)
    x = _rand((2, 3, L), 5)
    w = _rand((3, 2, m * s), 6)
    b = _rand((2,), 7)
    y = oracle_mod.conv_transpose(x, w, b, s, p, op)
    ref = _polyphase_1d(x, w, b, s, p, op)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_impulse_response(oracle_mod):
    """x = e_(n0, ci0, i0)  =>  y[n0, co, i0*s - p + t*d] = w[ci0, co, t], else 0."""
    N, C_in, C_out, L, k, s, p, op, d = 2, 3, 4, 6, 5, 2, 1, 1, 2
    w = _rand((C_in, C_out, k), 3)
    for n0, ci0, i0 in [(0, 0, 0), (1, 2, 5), (0, 1, 3)]:
        x = np.zeros((N, C_in, L))
        x[n0, ci0, i0] = 1.0
        y = oracle_mod.conv_transpose(x, w, None, s, p, op, d)
        ref = np.zeros_like(y)
        for t in range(k):
            o = i0 * s - p + t * d
            if 0 <= o < y.shape[2]:
                ref[n0, :, o] = w[ci0, :, t]
        np.testing.assert_array_equal(y, ref)


def test_k_equals_s_is_matmul(oracle_mod):
    """k = s, p = 0: windows do not overlap, y[n, co, s*i + t] = sum_ci x[n,ci,i] w[ci,co,t]."""
    x = _rand((2, 5, 7), 1)
    w = _rand((5, 3, 4), 2)
    y = oracle_mod.conv_transpose(x, w, None, 4, 0)
    mm = np.matmul(x.transpose(0, 2, 1), w.reshape(5, 12))  # [N, L, C_out*k]
    ref = mm.reshape(2, 7, 3, 4).transpose(0, 2, 1, 3).reshape(2, 3, 28)
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-14)


def test_zero_input_gives_bias(oracle_mod):
    x = np.zeros((1, 3, 4, 5))
    w = _rand((3, 2, 3, 3), 4)
    b = np.array([0.25, -2.0])
    y = oracle_mod.conv_transpose(x, w, b, 2, 1, 1)
    assert np.all(y[0, 0] == 0.25) and np.all(y[0, 1] == -2.0)


def test_empty_input_with_nonempty_output(oracle_mod):
    """L_in = 0 still has L_out = -s - 2p + d(k-1) + op + 1 outputs: all bias."""
    x = np.zeros((2, 3, 0))
    w = _rand((3, 2, 8), 4)
    b = np.array([1.5, -0.5])
    y = oracle_mod.conv_transpose(x, w, b, 2, 1)
    assert y.shape == (2, 2, -2 - 2 + 7 + 1)
    assert np.all(y[:, 0] == 1.5) and np.all(y[:, 1] == -0.5)


def test_hand_worked_examples(oracle_mod):
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        x = np.array(c["x"], dtype=np.float64)
        w = np.array(c["w"], dtype=np.float64)
        b = None if c["bias"] is None else np.array(c["bias"], dtype=np.float64)
        y = oracle_mod.conv_transpose(x, w, b, c["stride"], c["padding"],
                                      c["output_padding"], c["dilation"])
        np.testing.assert_array_equal(y, np.array(c["y"], dtype=np.float64), err_msg=c["name"])


@pytest.mark.parametrize("case", [CASES_1D[2], CASES_1D[4], CASES_2D[0], CASES_2D[2]])
def test_points_match_full(oracle_mod, case):
    nd = 1 if isinstance(case[2], int) else 2
    x, w, b, s, p, op, d = _make(case, nd, 31)
    y = oracle_mod.conv_transpose(x, w, b, s, p, op, d)
    if nd == 1:
        idx = [(n, co, 0, o) for n in range(y.shape[0]) for co in range(y.shape[1])
               for o in range(y.shape[2])]
        ref = y.reshape(-1)
    else:
        idx = [(n, co, oy, ox) for n in range(y.shape[0]) for co in range(y.shape[1])
               for oy in range(y.shape[2]) for ox in range(y.shape[3])]
        ref = y.reshape(-1)
    pts = oracle_mod.conv_transpose_points(x, w, b, idx, s, p, op, d)
    np.testing.assert_allclose(pts, ref, rtol=1e-13, atol=1e-13)


def test_output_shape_rule(oracle_mod):
    assert oracle_mod.output_shape((2000,), 16, 8, 4) == (16000,)
    assert oracle_mod.output_shape((16000,), 10, 5, 3) == (79999,)
    assert oracle_mod.output_shape((79999,), 8, 4, 2) == (319996,)
    assert oracle_mod.output_shape((345,), 4096, 1024, 0) == (356352,)
    assert oracle_mod.output_shape((64, 64), 4, 2, 1) == (128, 128)
    assert oracle_mod.output_shape((96, 96), 3, 2, 1, 1) == (192, 192)
    assert oracle_mod.output_shape((96, 96), 3, 2, 1, 1, 2) == (194, 194)
    with pytest.raises(ValueError):
        oracle_mod.output_shape((1,), 2, 4, 3)


# --------------------------------------------------------------------------
# inverse STFT
# --------------------------------------------------------------------------


def _numpy_istft(spec, n_fft, hop):
    N, C, T = spec.shape
    Fb = n_fft // 2 + 1
    h = I.hann_periodic(n_fft)
    y = np.zeros((N, (T - 1) * hop + n_fft))
    for n in range(N):
        for l in range(T):
            X = spec[n, :Fb, l] + 1j * spec[n, Fb:, l]
            X[0] = X[0].real
            X[-1] = X[-1].real
            y[n, l * hop:l * hop + n_fft] += np.fft.irfft(X, n_fft) * h
    return y


def test_istft_ola_matches_numpy(oracle_mod):
    n_fft, hop, T = 64, 16, 9
    spec = _rand((2, n_fft + 2, T), 41)
    np.testing.assert_allclose(oracle_mod.istft_ola(spec, n_fft, hop),
                               _numpy_istft(spec, n_fft, hop), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("n_fft,hop,T", [(16, 4, 7), (64, 16, 9), (128, 32, 5)])
def test_istft_basis_convT_equals_overlap_add(oracle_mod, n_fft, hop, T):
    spec = _rand((2, n_fft + 2, T), 43)
    w = I.istft_basis(n_fft, "f32")  # rounded to fp32 like the GPU operand
    y = oracle_mod.conv_transpose(spec, w, None, hop, 0)[:, 0]
    # the fp32-rounded basis differs from the exact one by ~1e-8 relative
    ref = oracle_mod.istft_ola(spec, n_fft, hop)
    assert y.shape == ref.shape
    assert oracle_mod.rel_l2(y, ref) < 1e-6
    w64 = np.empty_like(w)
    Fb = n_fft // 2 + 1
    h = I.hann_periodic(n_fft)
    t = np.arange(n_fft)
    for f in range(Fb):
        c = 1.0 if f in (0, n_fft // 2) else 2.0
        w64[f, 0] = c * np.cos(2 * np.pi * f * t / n_fft) * h / n_fft
        w64[Fb + f, 0] = -c * np.sin(2 * np.pi * f * t / n_fft) * h / n_fft
    y64 = oracle_mod.conv_transpose(spec, w64, None, hop, 0)[:, 0]
    assert oracle_mod.rel_l2(y64, ref) < 1e-12


def test_istft_perfect_reconstruction(oracle_mod):
    """Spectra of Hann-windowed frames of z at hop n/4, resynthesised through the
    basis: y = sum_l h^2(t - l*hop) z(t) = 1.5 z(t) where four frames overlap."""
    n_fft, hop, T = 64, 16, 12
    z = _rand(((T - 1) * hop + n_fft,), 47)
    h = I.hann_periodic(n_fft)
    Fb = n_fft // 2 + 1
    spec = np.zeros((1, 2 * Fb, T))
    for l in range(T):
        re, im = oracle_mod.rfft(h * z[l * hop:l * hop + n_fft])
        np.testing.assert_allclose(re + 1j * im, np.fft.rfft(h * z[l * hop:l * hop + n_fft]),
                                   rtol=1e-12, atol=1e-12)
        spec[0, :Fb, l] = re
        spec[0, Fb:, l] = im
    w = I.istft_basis(n_fft, "f32")
    y = oracle_mod.conv_transpose(spec, w, None, hop, 0)[0, 0]
    lo, hi = 3 * hop, (T - 1) * hop + hop
    assert oracle_mod.rel_l2(y[lo:hi], 1.5 * z[lo:hi]) < 1e-6


def test_elu(oracle_mod):
    x = np.array([-3.0, -1e-9, 0.0, 2.5])
    np.testing.assert_allclose(oracle_mod.elu(x), [np.expm1(-3.0), np.expm1(-1e-9), 0.0, 2.5],
                               rtol=1e-15)


# --------------------------------------------------------------------------
# planted mistakes: each mutated copy of the oracle must fail a pin above
# --------------------------------------------------------------------------

MUTATIONS = {
    "sign_of_padding": ("const int64_t oy = iy * s2[0] - p2[0] + ty * d2[0];",
                        "const int64_t oy = iy * s2[0] + p2[0] + ty * d2[0];"),
    "dropped_bias": ("double b = bias ? bias[co] : 0.0;", "double b = 0.0;"),
    "transposed_weight": ("const double wv = w[((ci * C_out + co) * kH + ty) * kW + tx];",
                          "const double wv = w[((co * C_in + ci) * kH + ty) * kW + tx];"),
    "flipped_taps": ("const double wv = w[((ci * C_out + co) * kH + ty) * kW + tx];",
                     "const double wv = w[((ci * C_out + co) * kH + (kH - 1 - ty)) * kW + (kW - 1 - tx)];"),
    "output_length_off_by_one": ("return (L - 1) * s - 2 * p + d * (k - 1) + op + 1;",
                                 "return (L - 1) * s - 2 * p + d * (k - 1) + op;"),
    "dilation_ignored": ("const int64_t ox = ix * s2[1] - p2[1] + tx * d2[1];",
                         "const int64_t ox = ix * s2[1] - p2[1] + tx;"),
}


def _build_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "ctconv_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert old in src, name
    src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-D_GNU_SOURCE", str(c), "-o",
                           str(so), "-lm"])
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(oracle_mod, tmp_path, name, monkeypatch):
    so = _build_mutant(tmp_path, name)
    monkeypatch.setattr(oracle_mod, "_lib", None)
    monkeypatch.setattr(oracle_mod, "_LIB", so)
    monkeypatch.setattr(oracle_mod, "build", lambda force=False: so)
    caught = False
    for case in CASES_1D + CASES_2D:
        nd = 1 if isinstance(case[2], int) else 2
        x, w, b, s, p, op, d = _make(case, nd, 11)
        try:
            y = oracle_mod.conv_transpose(x, w, b, s, p, op, d)
        except ValueError:
            caught = True
            break
        ref = _torch_ref(x, w, b, s, p, op, d)
        if y.shape != ref.shape or not np.allclose(y, ref, rtol=1e-12, atol=1e-12):
            caught = True
            break
    assert caught, f"mutation {name} was not detected"


# --------------------------------------------------------------------------
# grouped / depthwise transposed convolution (groups = C_in is depthwise)
# --------------------------------------------------------------------------

GROUPED_CASES = [
    # (C_in, C_out, groups, spatial, k, s, p, op, d, bias)
    (4, 4, 4, (9,), (4,), (2,), (1,), (0,), (1,), True),       # depthwise, k = 2s
    (3, 6, 3, (7,), (6,), (3,), (2,), (1,), (1,), False),      # depthwise, multiplier 2
    (4, 4, 4, (5,), (3,), (2,), (1,), (1,), (2,), True),       # dilation
    (4, 6, 2, (6,), (5,), (2,), (1,), (0,), (1,), True),       # two groups
    (3, 3, 3, (4, 5), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), True),
    (2, 4, 2, (3, 4), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), False),
    (2, 2, 2, (4, 3), (3, 3), (2, 2), (1, 1), (1, 1), (2, 2), True),
    (2, 2, 2, (3, 5), (5, 2), (3, 1), (2, 0), (2, 0), (1, 1), True),
]


def _make_grouped(case, seed):
    C_in, C_out, g, sp, k, s, p, op, d, has_b = case
    x = _rand((2, C_in) + sp, seed)
    w = _rand((C_in, C_out // g) + k, seed + 1)
    b = _rand((C_out,), seed + 2) if has_b else None
    return x, w, b, g, s, p, op, d


def _torch_grouped(x, w, b, g, s, p, op, d):
    fn = F.conv_transpose1d if x.ndim == 3 else F.conv_transpose2d
    return fn(torch.from_numpy(x), torch.from_numpy(w),
              None if b is None else torch.from_numpy(b), stride=s, padding=p,
              output_padding=op, groups=g, dilation=d).numpy()


@pytest.mark.parametrize("case", GROUPED_CASES)
def test_grouped_vs_torch_float64(oracle_mod, case):
    x, w, b, g, s, p, op, d = _make_grouped(case, 31)
    y = oracle_mod.conv_transpose_grouped(x, w, b, g, s, p, op, d)
    ref = _torch_grouped(x, w, b, g, s, p, op, d)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", GROUPED_CASES)
def test_grouped_equals_dense_with_block_diagonal_weight(oracle_mod, case):
    """A grouped weight is the dense weight that is zero between groups."""
    x, w, b, g, s, p, op, d = _make_grouped(case, 41)
    C_in, cog = w.shape[:2]
    cig = C_in // g
    dense = np.zeros((C_in, cog * g) + w.shape[2:])
    for ci in range(C_in):
        grp = ci // cig
        dense[ci, grp * cog:(grp + 1) * cog] = w[ci]
    y = oracle_mod.conv_transpose_grouped(x, w, b, g, s, p, op, d)
    yd = oracle_mod.conv_transpose(x, dense, b, s, p, op, d)
    np.testing.assert_allclose(y, yd, rtol=1e-13, atol=1e-13)


def test_depthwise_impulse_response(oracle_mod):
    """One input element of channel c reaches only channels c*M .. c*M + M-1,
    at o = i*s - p + t*d, with the weights themselves."""
    C, M, L, k, s, p = 3, 2, 6, 5, 2, 1
    w = _rand((C, M, k), 7)
    for c0, i0 in [(0, 0), (2, 5), (1, 3)]:
        x = np.zeros((1, C, L))
        x[0, c0, i0] = 1.0
        y = oracle_mod.conv_transpose_grouped(x, w, None, C, s, p)
        expect = np.zeros_like(y)
        for j in range(M):
            for t in range(k):
                o = i0 * s - p + t
                if 0 <= o < y.shape[2]:
                    expect[0, c0 * M + j, o] = w[c0, j, t]
        np.testing.assert_array_equal(y, expect)


@pytest.mark.parametrize("case", [GROUPED_CASES[1], GROUPED_CASES[2], GROUPED_CASES[5],
                                  GROUPED_CASES[7]])
def test_grouped_points_match_full(oracle_mod, case):
    x, w, b, g, s, p, op, d = _make_grouped(case, 51)
    y = oracle_mod.conv_transpose_grouped(x, w, b, g, s, p, op, d)
    rng = np.random.default_rng(3)
    n = rng.integers(0, y.shape[0], 40)
    co = rng.integers(0, y.shape[1], 40)
    if y.ndim == 3:
        oy = np.zeros(40, dtype=np.int64)
        ox = rng.integers(0, y.shape[2], 40)
        want = y[n, co, ox]
    else:
        oy = rng.integers(0, y.shape[2], 40)
        ox = rng.integers(0, y.shape[3], 40)
        want = y[n, co, oy, ox]
    got = oracle_mod.conv_transpose_grouped_points(x, w, b, np.stack([n, co, oy, ox], 1), g,
                                                   s, p, op, d)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


GROUPED_MUTATIONS = {
    "group_of_channel": ("const int64_t g = ci / cig;", "const int64_t g = ci % groups;"),
    "grouped_weight_index": ("const double wv = w[((ci * cog + j) * kH + ty) * kW + tx];",
                             "const double wv = w[((j * C_in + ci) * kH + ty) * kW + tx];"),
}


@pytest.mark.parametrize("name", sorted(GROUPED_MUTATIONS))
def test_grouped_planted_mistakes_are_caught(oracle_mod, tmp_path, name, monkeypatch):
    MUTATIONS_ALL = dict(MUTATIONS, **GROUPED_MUTATIONS)
    monkeypatch.setitem(MUTATIONS, name, MUTATIONS_ALL[name])
    so = _build_mutant(tmp_path, name)
    monkeypatch.setattr(oracle_mod, "_lib", None)
    monkeypatch.setattr(oracle_mod, "_LIB", so)
    monkeypatch.setattr(oracle_mod, "build", lambda force=False: so)
    caught = False
    for case in GROUPED_CASES:
        x, w, b, g, s, p, op, d = _make_grouped(case, 61)
        y = oracle_mod.conv_transpose_grouped(x, w, b, g, s, p, op, d)
        ref = _torch_grouped(x, w, b, g, s, p, op, d)
        if y.shape != ref.shape or not np.allclose(y, ref, rtol=1e-12, atol=1e-12):
            caught = True
            break
    assert caught, f"mutation {name} was not detected"


def test_grouped_hand_worked_examples(oracle_mod):
    with open(os.path.join(HERE, "golden", "hand_worked_grouped.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        x = np.array(c["x"], dtype=np.float64)
        w = np.array(c["w"], dtype=np.float64)
        b = None if c["bias"] is None else np.array(c["bias"], dtype=np.float64)
        y = oracle_mod.conv_transpose_grouped(x, w, b, c["groups"], c["stride"], c["padding"],
                                              c["output_padding"], c["dilation"])
        np.testing.assert_array_equal(y, np.array(c["y"], dtype=np.float64), err_msg=c["name"])

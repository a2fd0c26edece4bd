"""Helpers for the GPU parity tests: device tensors from seeded float64 arrays,
sampled output indices, the oracle run per batch item in threads, and the
comparison (relative L2 over the tensor plus a bound on every element)."""

from __future__ import annotations

import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from synth import inputs as I

TOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 1e-2}

# Unit roundoff of the output type (relative error bound of one
# round-to-nearest-even): 2^-p for p bits of precision.
U_OUT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
# Accumulation: a sum of K products in fp32 (each product exact for 16-bit
# inputs, rounded once for fp32 inputs) is off by at most about K * 2^-24 times
# the sum of the magnitudes of its terms, whatever the order of the additions.
# C_ACC = 2 leaves room for the rounded products and the bias term.
C_ACC = 2.0
U_ACC = 2.0 ** -24


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dt: str):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]


def to_dev(a: np.ndarray, dt: str):
    """float64 array holding `dt`-representable values -> device tensor of dtype dt."""
    import torch

    a = np.ascontiguousarray(a)
    if dt == "f32":
        t = torch.from_numpy(a.astype(np.float32))
    elif dt == "bf16":
        t = torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16)
    elif dt == "f16":
        t = torch.from_numpy(a.astype(np.float16))
    else:
        raise ValueError(dt)
    return t.to("cuda")


def to_host(t) -> np.ndarray:
    import torch

    return t.detach().to("cpu").to(torch.float64).numpy()


def terms_per_output(c_in_per_group: int, k, s, d=None) -> int:
    """Upper bound on the products summed into one output: the input channels
    of its group times, per dimension, the taps t with t*d = o + p (mod s),
    an arithmetic progression of step s / gcd(s, d) over [0, k)."""
    d = d if d is not None else (1,) * len(k)
    t = int(c_in_per_group)
    for kk, ss, dd in zip(k, s, d):
        step = ss // math.gcd(ss, dd)
        t *= -(-int(kk) // step)
    return t


def n_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def oracle_items(fn, x64: np.ndarray, *args, items=None, **kw) -> np.ndarray:
    """fn(x64[n:n+1], *args, **kw) for each batch item n (default: all), in
    parallel threads (the oracle is single-threaded C called through ctypes,
    which releases the interpreter lock), stacked along the batch axis."""
    items = list(range(x64.shape[0])) if items is None else list(items)
    with ThreadPoolExecutor(max_workers=n_threads()) as ex:
        parts = list(ex.map(lambda n: fn(x64[n:n + 1], *args, **kw), items))
    return np.concatenate(parts, axis=0)


def ref_and_mag(x64, w64, b64, s, p=0, op=0, d=1, groups=1, items=None):
    """The oracle's result and the same computation on |x|, |w|, |bias| (the
    sum of the magnitudes of each output's terms, for the element bound)."""
    import oracle

    if groups == 1:
        fn = oracle.conv_transpose
        args = lambda x, w, b: (x, w, b, s, p, op, d)  # noqa: E731
    else:
        fn = lambda x, w, b, *a: oracle.conv_transpose_grouped(x, w, b, groups, *a)  # noqa: E731
        args = lambda x, w, b: (x, w, b, s, p, op, d)  # noqa: E731
    ab = None if b64 is None else np.abs(b64)
    ref = oracle_items(lambda xs: fn(*args(xs, w64, b64)), x64, items=items)
    mag = oracle_items(lambda xs: fn(*args(np.abs(xs), np.abs(w64), ab)), x64, items=items)
    return ref, mag


def check_parity(got, ref, mag, dt: str, K: int, what: str = "", abs_slack: float = 0.0):
    """Relative L2 over the whole tensor <= TOL[dt], and every element within
        |got - ref| <= U_OUT[dt] * |ref| + C_ACC * K * 2^-24 * mag + abs_slack
    (K products per output, mag the oracle on the magnitudes).  A wrong output
    cannot hide behind the norm of the correct ones."""
    from oracle import rel_l2

    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = rel_l2(got, ref)
    diff = np.abs(got - ref)
    bound = U_OUT[dt] * np.abs(ref) + C_ACC * K * U_ACC * np.asarray(mag) + abs_slack
    bad = ~(diff <= bound)  # NaN counts as bad
    nbad = int(np.count_nonzero(bad))
    worst = float(np.max(diff / np.maximum(bound, 1e-300))) if got.size else 0.0
    say(f"  {what} rel_l2 = {err:.3e}, max |err| / bound = {worst:.3f} over {got.size} outputs")
    if nbad:
        i = np.unravel_index(int(np.argmax(bad)), got.shape)
        raise AssertionError(f"{what}: {nbad} outputs outside the element bound; first at "
                             f"{tuple(int(v) for v in i)}: got {got[i]!r} ref {ref[i]!r} "
                             f"bound {bound[i]!r}")
    assert err <= TOL[dt], (what, err)
    return err


def sample_indices(shape, n_random: int, seed: int, extra_rows=()):
    """(n, co, oy, ox) indices over y[N, C_out, (Ho,) Wo]: random picks plus every
    corner and the first/last elements of each tile-sized run along the
    contiguous axis (boundary-crossing outputs)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    N, C_out = shape[0], shape[1]
    Ho = shape[2] if len(shape) == 4 else 1
    Wo = shape[-1]
    pts = set()
    for _ in range(n_random):
        pts.add((int(rng.integers(N)), int(rng.integers(C_out)), int(rng.integers(Ho)),
                 int(rng.integers(Wo))))
    for n in {0, N - 1}:
        for co in {0, C_out - 1, C_out // 2}:
            for oy in {0, Ho - 1, Ho // 2}:
                for ox in {0, 1, Wo - 2, Wo - 1, Wo // 2}:
                    if 0 <= ox < Wo:
                        pts.add((n, co, oy, ox))
    for ox in extra_rows:
        if 0 <= ox < Wo:
            pts.add((int(rng.integers(N)), int(rng.integers(C_out)), int(rng.integers(Ho)), int(ox)))
    return np.array(sorted(pts), dtype=np.int64)


def gather_points(y: np.ndarray, idx: np.ndarray) -> np.ndarray:
    if y.ndim == 3:
        return y[idx[:, 0], idx[:, 1], idx[:, 3]]
    return y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]]

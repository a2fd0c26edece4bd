"""Helpers for the GPU parity tests: device tensors from seeded float64 arrays,
sampled output indices, and the comparison metric."""

from __future__ import annotations

import sys

import numpy as np

from synth import inputs as I

TOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 1e-2}


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

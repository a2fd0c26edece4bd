"""Seeded input generators and the workload catalogue.

Every tensor is drawn with numpy's PCG64 generator from an integer seed, in
float64, then rounded to its storage dtype: float64 -> float32 (round to
nearest even), and for 16-bit workloads float32 -> bfloat16 or float16 (round
to nearest even).  The float64 arrays returned here hold exactly the rounded
values, so the CPU reference and the GPU see identical operands.

Seed convention: seed = 1000 * workload_id + 10 * tensor + layer, with
tensor 1 = x, 2 = weight, 3 = bias.

The only structured operand is the inverse-STFT basis used by the
inverse-STFT-as-ConvTranspose1d workload (onnxruntime PR #33978, commit
"ConvTranspose ... GEMM + col2im", which serves iSTFT as overlap-add): a
Hann-windowed inverse real DFT, one input channel per real and imaginary
spectral bin.  It is an operand of the transposed convolution, built here so
that both sides get the same one.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

DTYPES = ("f32", "bf16", "f16")


def SEED(workload_id: int, tensor: int, layer: int = 0) -> int:
    """Seed of one tensor: 1000 * workload + 10 * tensor (x=1, w=2, bias=3) + layer."""
    return 1000 * workload_id + 10 * tensor + layer


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, rounding to nearest even."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float16)).view(np.uint16)


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 array -> float64 array of the nearest values of `dtype` (RNE)."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return a32.astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(bf16_bits(a32))
    if dtype == "f16":
        return a32.astype(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def uniform(seed: int, shape, lo: float, hi: float, dtype: str = "f32") -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return round_to_dtype(rng.uniform(lo, hi, size=shape), dtype)


def normal(seed: int, shape, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return round_to_dtype(rng.standard_normal(size=shape) * std, dtype)


def hann_periodic(n: int) -> np.ndarray:
    t = np.arange(n, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * math.pi * t / n)


def istft_basis(n_fft: int, dtype: str = "f32") -> np.ndarray:
    """ConvTranspose1d weight [n_fft + 2, 1, n_fft] whose transposed convolution
    with stride hop is the windowed inverse real DFT followed by overlap-add.

    Channel f (0 <= f <= n_fft/2) carries the real part of bin f and channel
    n_fft/2 + 1 + f its imaginary part:
        w[f, 0, t]         =  c_f cos(2 pi f t / n) h[t] / n
        w[F + f, 0, t]     = -c_f sin(2 pi f t / n) h[t] / n
    with c_0 = c_{n/2} = 1, c_f = 2 otherwise, h the periodic Hann window and
    F = n/2 + 1.  Built in float64 (angles reduced exactly modulo n), then
    rounded to `dtype`.
    """
    n = n_fft
    F = n // 2 + 1
    h = hann_periodic(n)
    t = np.arange(n, dtype=np.int64)
    out = np.empty((2 * F, 1, n), dtype=np.float64)
    for f in range(F):
        c = 1.0 if (f == 0 or f == n // 2) else 2.0
        ang = 2.0 * math.pi * ((f * t) % n) / n
        out[f, 0, :] = c * np.cos(ang) * h / n
        out[F + f, 0, :] = -c * np.sin(ang) * h / n
    return round_to_dtype(out, dtype)


# ---------------------------------------------------------------------------
# Workload catalogue
# ---------------------------------------------------------------------------


@dataclass
class Layer:
    C_in: int
    C_out: int
    kernel: Tuple[int, ...]
    stride: Tuple[int, ...]
    padding: Tuple[int, ...]
    output_padding: Tuple[int, ...]
    dilation: Tuple[int, ...]
    bias: bool
    groups: int = 1  # C_in for a depthwise layer (weight [C_in, C_out / groups, k...])

    @property
    def ndim(self) -> int:
        return len(self.kernel)


@dataclass
class Workload:
    wid: int
    name: str
    dtype: str
    N: int
    in_spatial: Tuple[int, ...]
    layers: List[Layer]
    x_dist: Tuple  # ("uniform", lo, hi) | ("normal", std)
    w_dist: str  # "uniform" | "fan_in_normal" | "istft"
    elu_between: bool = False
    note: str = ""
    extra: Dict = field(default_factory=dict)


def _L(C_in, C_out, k, s, p, op=0, d=1, bias=False, ndim=1, groups=1):
    t = lambda v: tuple(v) if isinstance(v, (tuple, list)) else (v,) * ndim  # noqa: E731
    return Layer(C_in, C_out, t(k), t(s), t(p), t(op), t(d), bias, groups)


WORKLOADS: Dict[str, Workload] = {
    # k = 2s audio-decoder upsampler, small enough for the CPU reference in well
    # under a second.
    "upsampler1d_small": Workload(
        1, "upsampler1d_small", "f32", 1, (256,),
        [_L(64, 32, 8, 4, 2, bias=True)],
        ("uniform", -1.0, 1.0), "uniform",
        note="ConvTranspose1d fp32 64->32 k8 s4 p2, L_in=256, N=1, bias"),
    # Vocoder-style three-layer upsampler stack with ELU between layers.
    "vocoder_stack": Workload(
        2, "vocoder_stack", "bf16", 8, (2000,),
        [_L(512, 256, 16, 8, 4), _L(256, 128, 10, 5, 3), _L(128, 64, 8, 4, 2)],
        ("normal", 1.0), "fan_in_normal", elu_between=True,
        note="ConvTranspose1d bf16 stack 512->256 (k16 s8 p4), 256->128 (k10 s5 p3), "
             "128->64 (k8 s4 p2), L_in=2000, N=8, ELU between layers"),
    # Inverse STFT as a transposed convolution: n_fft 4096, hop 1024, 345 frames,
    # 2049 complex bins as 4098 real channels, batch 2 x 4 sources.
    "istft": Workload(
        3, "istft", "f32", 8, (345,),
        [_L(4098, 1, 4096, 1024, 0)],
        ("normal", 1.0), "istft",
        note="iSTFT as ConvTranspose1d fp32 4098->1 k4096 s1024 p0, 345 frames, N=8",
        extra={"n_fft": 4096, "hop": 1024}),
    # 2-D 4x4 stride-2 upsampler.
    "upsampler2d": Workload(
        4, "upsampler2d", "bf16", 8, (64, 64),
        [_L(256, 128, 4, 2, 1, bias=True, ndim=2)],
        ("normal", 1.0), "fan_in_normal",
        note="ConvTranspose2d bf16 256->128 4x4 s2 p1, 64x64, N=8, bias"),
    # Shapes the polyphase form does not cover: k = 3 is not a multiple of s = 2,
    # output_padding 1, and a dilation-2 variant.
    "gather2d": Workload(
        5, "gather2d", "f32", 4, (96, 96),
        [_L(128, 64, 3, 2, 1, op=1, ndim=2)],
        ("uniform", -1.0, 1.0), "uniform",
        note="ConvTranspose2d fp32 128->64 3x3 s2 p1 op1, 96x96, N=4"),
    "gather2d_dil2": Workload(
        5, "gather2d_dil2", "f32", 4, (96, 96),
        [_L(128, 64, 3, 2, 1, op=1, d=2, ndim=2)],
        ("uniform", -1.0, 1.0), "uniform",
        note="ConvTranspose2d fp32 128->64 3x3 s2 p1 op1 dilation 2, 96x96, N=4"),
    # Stride 3 in 2-D (nine phases, more than a 2-D column tile holds: the
    # polyphase kernel's column tiles take subsets of them) with k not a
    # multiple of s, and a shape only the gather kernel takes: a 1-D kernel
    # of eight taps per phase (more than any compiled polyphase instance),
    # both fp32 in the family of the 3x3 stride-2 shapes above.
    "gather2d_s3": Workload(
        8, "gather2d_s3", "f32", 4, (64, 64),
        [_L(128, 64, 5, 3, 1, op=1, ndim=2)],
        ("uniform", -1.0, 1.0), "uniform",
        note="ConvTranspose2d fp32 128->64 5x5 s3 p1 op1, 64x64, N=4"),
    "gather1d_m8": Workload(
        9, "gather1d_m8", "f32", 4, (4096,),
        [_L(128, 64, 16, 2, 7)],
        ("uniform", -1.0, 1.0), "uniform",
        note="ConvTranspose1d fp32 128->64 k16 s2 p7, L_in=4096, N=4"),
    # Depthwise (groups = C) 4x4 stride-2 upsampling filter per channel, the
    # layer type of a StyleGAN-style x2 upsampler (MI-GAN has twelve of them).
    "depthwise2d": Workload(
        6, "depthwise2d", "bf16", 8, (128, 128),
        [_L(256, 256, 4, 2, 1, bias=True, ndim=2, groups=256)],
        ("normal", 1.0), "fan_in_normal",
        note="depthwise ConvTranspose2d bf16 256 channels 4x4 s2 p1, 128x128, N=8, bias"),
    # Depthwise k = 2s stride-2 upsampler along time (an audio decoder's
    # frame-rate upsampler), long enough to stream well past the caches.
    "depthwise1d": Workload(
        7, "depthwise1d", "bf16", 8, (16384,),
        [_L(512, 512, 4, 2, 1, groups=512)],
        ("normal", 1.0), "fan_in_normal",
        note="depthwise ConvTranspose1d bf16 512 channels k4 s2 p1, L_in=16384, N=8"),
}


def gen_x(wl: Workload, N: Optional[int] = None, in_spatial=None) -> np.ndarray:
    N = wl.N if N is None else N
    sp = wl.in_spatial if in_spatial is None else tuple(in_spatial)
    shape = (N, wl.layers[0].C_in) + sp
    seed = SEED(wl.wid, 1)
    if wl.x_dist[0] == "uniform":
        return uniform(seed, shape, wl.x_dist[1], wl.x_dist[2], wl.dtype)
    return normal(seed, shape, wl.x_dist[1], wl.dtype)


def gen_w(wl: Workload, li: int = 0) -> np.ndarray:
    L = wl.layers[li]
    shape = (L.C_in, L.C_out // L.groups) + L.kernel
    seed = SEED(wl.wid, 2, li + 1 if len(wl.layers) > 1 else 0)
    if wl.w_dist == "uniform":
        return uniform(seed, shape, -1.0, 1.0, wl.dtype)
    if wl.w_dist == "fan_in_normal":
        # N(0, v) with v = 1 / (fan-in * prod(kernel)): the second parameter is the
        # variance; an output of a grouped layer sums C_in / groups input channels.
        v = 1.0 / ((L.C_in // L.groups) * int(np.prod(L.kernel)))
        return normal(seed, shape, math.sqrt(v), wl.dtype)
    if wl.w_dist == "istft":
        return istft_basis(wl.extra["n_fft"], wl.dtype)
    raise ValueError(wl.w_dist)


def gen_bias(wl: Workload, li: int = 0) -> Optional[np.ndarray]:
    L = wl.layers[li]
    if not L.bias:
        return None
    return uniform(SEED(wl.wid, 3, li + 1 if len(wl.layers) > 1 else 0), (L.C_out,),
                   -0.1, 0.1, wl.dtype)


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def flops(N: int, L: Layer, in_sp) -> int:
    """2 * N * C_in * (C_out / groups) * prod(kernel) * prod(in_spatial)."""
    return 2 * N * L.C_in * (L.C_out // L.groups) * int(np.prod(L.kernel)) * int(np.prod(in_sp))

"""Seeded random shapes aimed at two planner paths of the polyphase route
(shared by the GPU parity test and the CPU check that the planner still
sends most of them there):

- 2-D phase subsets: strides 3-5 in both dimensions (9-25 phases, more than
  one column tile holds at 16 channels each), 1-2 taps per phase, C_out
  from 16 up;
- fp32 tap groups: 1-D with 5-12 taps per phase, 2-D with up to 5 x 5 (at
  least one dimension above 2, not 3 x 3), run as several launches that
  add into y.

Padding, output_padding, bias and the fused ELU vary; dilation is 1 (the
dilated shapes are in the general random set).  Each case:
(kind, dtype, N, C_in, C_out, in_spatial, kernel, stride, padding,
 output_padding, dilation, has_bias, fused_elu)."""

import numpy as np


def planner_cases(n: int, seed: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        kind = "subset" if len(out) % 2 == 0 else "groups"
        if kind == "subset":
            nd = 2
            s = [int(rng.integers(3, 6)), int(rng.integers(3, 6))]
            if rng.random() < 0.25:  # one dimension with few phases
                s[int(rng.integers(0, 2))] = int(rng.integers(1, 3))
            k = [max(1, si * int(rng.integers(1, 3)) - int(rng.integers(0, si))) for si in s]
            dt = str(rng.choice(["f32", "bf16", "f16"]))
            C_out = int(rng.integers(16, 97))
        else:
            nd = int(rng.integers(1, 3))
            s = [int(rng.integers(1, 5)) for _ in range(nd)]
            if nd == 1:
                taps = [int(rng.integers(5, 13))]
            else:
                while True:
                    taps = [int(rng.integers(1, 6)) for _ in range(2)]
                    if max(taps) > 2 and taps != [3, 3]:
                        break
            k = [si * t - int(rng.integers(0, si)) for si, t in zip(s, taps)]
            dt = "f32"
            C_out = int(rng.integers(1, 49))
        p = [int(rng.integers(0, ki)) for ki in k]
        op = [int(rng.integers(0, si)) for si in s]
        sp = [int(rng.integers(2, 10))] if nd == 2 else []
        sp += [int(rng.integers(2, 40 if nd == 2 else 120))]
        o = [(a - 1) * b - 2 * c + (f - 1) + g + 1 for a, b, c, f, g in zip(sp, s, p, k, op)]
        if min(o) < 1:
            continue
        N = int(rng.integers(1, 3))
        C_in = int(rng.integers(1, 72))
        bias = bool(rng.random() < 0.5)
        act = bool(rng.random() < 0.3)
        out.append((kind, dt, N, C_in, C_out, tuple(sp), tuple(k), tuple(s), tuple(p), tuple(op),
                    (1,) * nd, bias, act))
    return out


PLANNER_CASES = planner_cases(32, 91)

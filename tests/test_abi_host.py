"""Host-only checks of the C ABI (no device call is made by any of these).

* the library loads and exports every function include/ctconv.h declares;
* ctconv_output_shape agrees with the oracle's output length and rejects
  invalid parameters;
* ctconv_packed_bytes follows the documented packed layout size;
* argument validation returns the documented status before any launch;
* routing: shapes whose dilation divides the stride take the polyphase
  kernel (within its compiled tap counts and row widths), the rest the
  gather kernel.
"""

import ctypes
import os
import re

import pytest

from vision_upsampler_decoders_amd import ctconv as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(C.LIB_PATH):
        from vision_upsampler_decoders_amd import build

        build.build()
    return C.load()


def _declared():
    src = open(os.path.join(ROOT, "include", "ctconv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ctconv_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(C.EXPORTED)
    assert C.ctconv_abi_version() == 1
    assert "aligned" in C.ctconv_status_string(5)


@pytest.mark.parametrize("args", [
    ((2000,), 16, 8, 4, 0, 1), ((16000,), 10, 5, 3, 0, 1), ((79999,), 8, 4, 2, 0, 1),
    ((345,), 4096, 1024, 0, 0, 1), ((64, 64), 4, 2, 1, 0, 1), ((96, 96), 3, 2, 1, 1, 1),
    ((96, 96), 3, 2, 1, 1, 2), ((7, 5), (3, 2), (2, 1), (1, 0), (1, 0), (1, 3)),
    ((0,), 4096, 1024, 0, 0, 1), ((1,), 1, 1, 0, 0, 1), ((3,), 5, 2, 2, 3, 4),
])
def test_output_shape_matches_oracle(lib, oracle_mod, args):
    sp, k, s, p, op, d = args
    assert C.ctconv_output_shape(sp, k, s, p, op, d) == oracle_mod.output_shape(sp, k, s, p, op, d)


@pytest.mark.parametrize("args,status", [
    (((8,), 4, 2, 9, 0, 1), 2),    # output length below 1
    (((8,), 0, 2, 0, 0, 1), 3),    # kernel 0
    (((8,), 4, 0, 0, 0, 1), 3),    # stride 0
    (((8,), 4, 2, -1, 0, 1), 3),   # negative padding
    (((8,), 4, 2, 0, 2, 1), 3),    # output_padding >= max(stride, dilation)
    (((8,), 4, 2, 0, 0, 0), 3),    # dilation 0
    (((-1,), 4, 2, 0, 0, 1), 2),   # negative length
    (((1 << 62,), 4, 8, 0, 0, 1), 2),  # overflow
])
def test_output_shape_rejects(lib, args, status):
    with pytest.raises(C.CtconvError) as e:
        C.ctconv_output_shape(*args)
    assert e.value.status == status


def test_output_shape_rejects_bad_ndim_and_null(lib):
    a = (ctypes.c_int64 * 1)(4)
    out = (ctypes.c_int64 * 1)()
    assert lib.ctconv_output_shape(3, a, a, a, a, a, a, out) == 3
    assert lib.ctconv_output_shape(1, None, a, a, a, a, a, out) == 1
    assert lib.ctconv_output_shape(1, a, a, a, a, a, a, None) == 1


@pytest.mark.parametrize("ndim,C_in,C_out,k,s,dt,expect", [
    (1, 64, 32, (8,), (4,), 0, 4 * 32 * 2 * 64 * 4),
    (1, 512, 256, (16,), (8,), 1, 8 * 256 * 2 * 512 * 2),
    (1, 256, 128, (10,), (5,), 1, 5 * 128 * 2 * 256 * 2),
    (1, 4098, 1, (4096,), (1024,), 0, 1024 * 1 * 4 * 4128 * 4),
    (2, 256, 128, (4, 4), (2, 2), 1, 4 * 128 * 4 * 256 * 2),
    (2, 128, 64, (3, 3), (2, 2), 0, 4 * 64 * 4 * 128 * 4),
    (1, 3, 5, (7,), (3,), 2, 3 * 5 * 3 * 32 * 2),
])
def test_packed_bytes(lib, ndim, C_in, C_out, k, s, dt, expect):
    assert C.ctconv_packed_bytes(ndim, C_in, C_out, k, s, dt) == expect


def test_packed_bytes_rejects(lib):
    for args, st in [((1, 0, 4, (4,), (2,), 0), 2), ((1, 4, 0, (4,), (2,), 0), 2),
                     ((1, 4, 4, (0,), (2,), 0), 3), ((1, 4, 4, (4,), (2,), 7), 4)]:
        with pytest.raises(C.CtconvError) as e:
            C.ctconv_packed_bytes(*args)
        assert e.value.status == st
    a = (ctypes.c_int64 * 3)(4, 4, 4)
    nb = ctypes.c_size_t(0)
    assert lib.ctconv_packed_bytes(3, 4, 4, a, a, 0, ctypes.byref(nb)) == 3
    assert lib.ctconv_packed_bytes(1, 4, 4, a, a, 0, None) == 1


def _fwd(lib, x=0x1000, w=0x2000, b=None, y=0x3000, N=1, C_in=4, C_out=4, sp=(8,), k=4, s=2,
         p=1, op=0, d=1, dt=0, route=0):
    nd = len(sp)
    arr = lambda v: (ctypes.c_int64 * nd)(*C.per_dim(v, nd))  # noqa: E731
    return lib.ctconv_forward_route(x, w, b, y, N, C_in, C_out, nd, arr(sp), arr(k), arr(s),
                                    arr(p), arr(op), arr(d), dt, route, None)


def test_forward_validation_before_launch(lib):
    # Every call below must be rejected on the host: none reaches a launch.
    assert _fwd(lib, x=None) == 1
    # an empty input may come with a NULL pointer (it is never read); its
    # output is then only filled, which would launch, so check N = 0 only
    assert _fwd(lib, x=None, y=None, N=0) == 0
    assert _fwd(lib, y=None, sp=(0,), k=8, s=2, p=0) == 1
    assert _fwd(lib, w=None) == 1
    assert _fwd(lib, y=None) == 1
    assert _fwd(lib, C_in=0) == 2
    assert _fwd(lib, C_out=0) == 2
    assert _fwd(lib, N=-1) == 2
    assert _fwd(lib, dt=9) == 4
    assert _fwd(lib, s=0) == 3
    assert _fwd(lib, op=2) == 3
    assert _fwd(lib, p=9) == 2
    assert _fwd(lib, route=7) == 3
    assert _fwd(lib, x=0x1001) == 5
    assert _fwd(lib, y=0x3008) == 5
    assert _fwd(lib, b=0x4004) == 5
    # polyphase forced on a shape outside the polyphase form (16-bit: fp32
    # shapes with more taps per phase than an instance run as tap groups)
    assert _fwd(lib, d=3, k=5, s=2, dt=1, route=1) == 3   # 7 expanded taps per phase
    assert _fwd(lib, d=2, k=9, s=2, route=1) == 3          # reduced problem with 9 taps
    assert _fwd(lib, k=20, s=4, p=2, dt=1, route=1) == 3   # 5 taps per phase
    assert _fwd(lib, sp=(3,), dt=1, route=1) == 3     # rows shorter than 8 bytes
    # fused activation: an unknown activation is rejected
    nd = 1
    arr = lambda v: (ctypes.c_int64 * nd)(*C.per_dim(v, nd))  # noqa: E731
    assert lib.ctconv_forward_act(0x1000, 0x2000, None, 0x3000, 1, 4, 4, nd, arr((8,)), arr(4),
                                  arr(2), arr(1), arr(0), arr(1), 0, 7, 0, None) == 3
    assert lib.ctconv_elu(None, 0x1000, 4, 0, None) == 1
    assert lib.ctconv_elu(0x1000, 0x2000, -1, 0, None) == 2
    assert lib.ctconv_elu(0x1000, 0x2000, 4, 5, None) == 4
    assert lib.ctconv_elu(0x1002, 0x2000, 4, 1, None) == 5


def test_forward_with_N_zero_enqueues_nothing(lib):
    assert _fwd(lib, N=0) == 0


@pytest.mark.parametrize("name,route", [
    ("upsampler1d_small", 1), ("vocoder_stack", 1), ("istft", 1), ("upsampler2d", 1),
    ("gather2d", 1), ("gather2d_dil2", 1), ("gather2d_s3", 1), ("gather1d_m8", 1),
])
def test_routes_of_workloads(lib, name, route):
    from synth import inputs as I

    wl = I.workload(name)
    dt = {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype]
    sp = wl.in_spatial
    for L in wl.layers:
        r = C.ctconv_query_route(wl.N, L.C_in, L.C_out, sp, L.kernel, L.stride, L.padding,
                                 L.output_padding, L.dilation, dt)
        assert r == route
        sp = C.ctconv_output_shape(sp, L.kernel, L.stride, L.padding, L.output_padding,
                                   L.dilation)


@pytest.mark.parametrize("k,s,p,op,d,route", [
    (8, 4, 2, 0, 1, 1), (6, 3, 0, 0, 1, 1), (4, 1, 1, 0, 1, 1), (3, 2, 1, 0, 1, 1),
    (8, 4, 2, 1, 1, 1), (16, 4, 2, 0, 1, 1), (20, 4, 2, 0, 1, 2),
    (7, 3, 2, 2, 1, 1), (13, 4, 1, 0, 1, 1), (17, 4, 1, 0, 1, 2),
    # dilation: g = gcd(s, d), s' = s / g, d' = d / g, expanded kernel of
    # (k - 1) d' + 1 taps, m = ceil(that / s')
    (8, 4, 2, 0, 2, 1),   # g 2, s' 2, d' 1: m 4
    (3, 2, 1, 1, 2, 1),   # g 2, s' 1: m 3
    (4, 4, 1, 0, 2, 1),   # g 2, s' 2: m 2
    (3, 2, 1, 0, 3, 1),   # g 1, d' 3: 7 taps, m 4
    (4, 3, 1, 0, 2, 1),   # g 1, d' 2: 7 taps, m 3
    (3, 4, 1, 0, 6, 1),   # g 2, s' 2, d' 3: 7 taps, m 4
    (5, 2, 1, 0, 3, 2),   # g 1, d' 3: 13 taps, m 7
    (4, 2, 1, 0, 3, 2),   # g 1, d' 3: 10 taps, m 5
])
def test_route_rule(lib, k, s, p, op, d, route):
    # 1-D: polyphase iff the taps per phase (of the dilation-expanded kernel
    # at the reduced stride) are within the compiled 1 .. 4
    assert C.ctconv_query_route(2, 16, 16, (50,), k, s, p, op, d, 1) == route


@pytest.mark.parametrize("k,s,p,op,d,route", [
    ((3, 3), (2, 2), (1, 1), (1, 1), (2, 2), 1),   # reduced: stride 1, 3 x 3 taps
    ((3, 3), (4, 4), (1, 1), (0, 0), (2, 2), 1),   # reduced: stride 2, 2 x 2 taps
    ((3, 3), (3, 3), (1, 1), (0, 0), (2, 2), 1),   # 9 phases: tiles hold subsets of them
    ((5, 5), (3, 3), (1, 1), (1, 1), (1, 1), 1),   # 9 phases, 2 x 2 taps
    ((4, 4), (4, 4), (0, 0), (0, 0), (1, 1), 1),   # 16 phases, 1 x 1 tap
    ((3, 2), (3, 1), (1, 0), (2, 0), (2, 1), 1),   # y expanded: 5 taps at stride 3, 2 x 2
    ((3, 3), (2, 2), (1, 1), (0, 0), (3, 3), 1),   # expanded: 7 taps at stride 2, 4 x 4 (tap groups)
    ((4, 2), (2, 2), (1, 2), (0, 1), (1, 3), 1),   # x expanded to 4 taps: 2 x 2
    ((3, 3), (1, 1), (1, 1), (0, 0), (1, 1), 1),   # 3 x 3 taps without dilation
    ((5, 5), (2, 2), (2, 2), (1, 1), (1, 1), 1),   # 3 x 3 taps per phase
])
def test_route_rule_2d_dilation(lib, k, s, p, op, d, route):
    # 2-D: per dimension reduction by gcd(s, d) and expansion of the rest of
    # the dilation; the compiled 2-D tap counts are 1 or 2 per dimension, or
    # 3 x 3 (fp32 without a reduction: any count, in tap groups); any number
    # of phases (column tiles take subsets of them)
    assert C.ctconv_query_route(2, 16, 16, (20, 22), k, s, p, op, d, 0) == route


@pytest.mark.parametrize("sp,dt,route", [
    ((1,), 0, 2), ((2,), 0, 1), ((3,), 1, 2), ((4,), 1, 1), ((3,), 2, 2),
    ((9, 3), 1, 2), ((9, 4), 1, 1), ((1, 2), 0, 1),
])
def test_route_short_rows(lib, sp, dt, route):
    # the polyphase kernel loads 8 bytes of an input row at a time: rows
    # shorter than that go to the gather kernel
    k, s, p = ((8,), (4,), (2,)) if len(sp) == 1 else ((4, 4), (2, 2), (1, 1))
    assert C.ctconv_query_route(2, 16, 16, sp, k, s, p, 0, 1, dt) == route


def test_planner_cases_reach_polyphase(lib):
    """The seeded random set aimed at phase subsets and tap groups keeps
    exercising them: most of its shapes are planned onto the polyphase route
    (the rest, 2-D tap groups over 16 phases and rows under 8 bytes, go to
    the gather kernel)."""
    from random_cases import PLANNER_CASES

    dts = {"f32": 0, "bf16": 1, "f16": 2}
    hits = {"subset": 0, "groups": 0}
    for kind, dt, N, C_in, C_out, sp, k, s, p, op, d, _, _ in PLANNER_CASES:
        if C.ctconv_query_route(N, C_in, C_out, sp, k, s, p, op, d, dts[dt]) == 1:
            hits[kind] += 1
    assert hits["subset"] >= 12 and hits["groups"] >= 12, hits


def test_stream_sizes(lib):
    # chunk of L frames: L*s outputs, k - s tail values, conv workspace
    # (the chunk's conv output is fp32 in every dtype)
    assert C.ctconv_stream_sizes(2, 3, 5, 10, 5, 1) == (25, 5, 2 * 3 * 30 * 4)
    assert C.ctconv_stream_sizes(1, 4, 2, 16, 4, 0) == (8, 12, 1 * 4 * 20 * 4)
    assert C.ctconv_stream_sizes(1, 4, 3, 4, 4, 2) == (12, 0, 1 * 4 * 12 * 4)
    assert C.ctconv_stream_sizes(1, 4, 0, 8, 4, 1) == (0, 4, 0)


def test_stream_validation_before_launch(lib):
    # every call below returns before any launch (fake device pointers)
    def step(k=8, s=4, L=3, tin=0x5000, tout=0x6000, act=0, ws=0x7000, N=1):
        return lib.ctconv_stream_step(0x1000, 0x2000, None, 0x3000, tin, tout, ws, N, 4, 4, L, k,
                                      s, 0, act, None)

    assert step(k=3, s=4) == 3            # kernel shorter than stride
    assert step(L=0) == 2                 # empty chunk
    assert step(tin=0x5000, tout=0x5000) == 3  # tail buffers alias
    assert step(act=7) == 3               # unknown activation
    assert step(ws=None) == 1             # no workspace
    assert step(tout=None) == 1           # tail needed (k > s)
    assert step(N=0) == 0                 # nothing to do
    assert lib.ctconv_stream_flush(0x5000, None, 0x3000, 1, 4, 8, 4, 0, 7, None) == 3
    assert lib.ctconv_stream_flush(0x5000, None, 0x3000, 0, 4, 8, 4, 0, 0, None) == 0
    assert lib.ctconv_stream_flush(0x5000, None, 0x3000, 1, 4, 4, 4, 0, 0, None) == 0  # no tail


def test_istft_normalize_validation(lib):
    f = lib.ctconv_istft_normalize
    assert f(0x1000, 0x2000, 0x3000, 2, 100, 60, 41, 0, None) == 2   # trim + L_out > L_in
    assert f(0x1000, 0x2000, 0x3000, 2, 100, -1, 10, 0, None) == 2
    assert f(None, 0x2000, 0x3000, 2, 100, 10, 10, 0, None) == 1
    assert f(0x1001, 0x2000, 0x3000, 2, 100, 10, 10, 0, None) == 5
    assert f(0x1000, 0x2000, 0x3000, 2, 100, 10, 10, 9, None) == 4
    assert f(0x1000, 0x2000, 0x3000, 0, 100, 10, 10, 0, None) == 0   # nothing to do


def _dw(lib, x=0x1000, w=0x2000, b=None, y=0x3000, N=1, C_in=4, C_out=4, sp=(8,), k=4, s=2,
        p=1, op=0, d=1, dt=0, act=0, which=0):
    nd = len(sp)
    arr = lambda v: (ctypes.c_int64 * nd)(*C.per_dim(v, nd))  # noqa: E731
    return lib.ctconv_depthwise_forward_kernel(x, w, b, y, N, C_in, C_out, nd, arr(sp), arr(k),
                                               arr(s), arr(p), arr(op), arr(d), dt, act, which,
                                               None)


def test_depthwise_validation_before_launch(lib):
    # Every call below is rejected on the host: none reaches a launch.
    assert _dw(lib, C_out=6) == 2          # C_out not a multiple of C_in
    assert _dw(lib, C_in=0) == 2
    assert _dw(lib, N=-1) == 2
    assert _dw(lib, x=None) == 1
    assert _dw(lib, w=None) == 1
    assert _dw(lib, y=None) == 1
    assert _dw(lib, x=None, y=None, N=0) == 0  # nothing to do
    assert _dw(lib, dt=3) == 4
    assert _dw(lib, act=5) == 3
    assert _dw(lib, which=3) == 3
    assert _dw(lib, s=0) == 3
    assert _dw(lib, op=2) == 3
    assert _dw(lib, x=0x1004) == 5
    assert _dw(lib, w=0x2002) == 5
    assert _dw(lib, b=0x4008) == 5
    # the row-phase kernel forced on shapes it does not take
    assert _dw(lib, s=3, k=6, which=1) == 3        # row stride 3
    assert _dw(lib, d=2, k=3, which=1) == 3        # dilation along the row
    assert _dw(lib, k=10, s=2, which=1) == 3       # 5 taps per phase


@pytest.mark.parametrize("sp,k,s,p,op,d,which", [
    ((50,), 4, 2, 1, 0, 1, 1),              # k = 2s upsampler
    ((50,), 8, 4, 2, 0, 1, 1),
    ((50,), 3, 1, 1, 0, 1, 1),              # stride 1
    ((50,), 5, 2, 1, 1, 1, 1),              # k mod s != 0, output_padding
    ((50,), 6, 3, 1, 0, 1, 2),              # stride 3: element kernel
    ((50,), 3, 2, 1, 1, 2, 2),              # dilation along the row
    ((50,), 10, 2, 4, 0, 1, 2),             # 5 taps per phase
    ((20, 22), (4, 4), (2, 2), (1, 1), (0, 0), (1, 1), 1),
    ((20, 22), (3, 3), (2, 2), (1, 1), (1, 1), (2, 1), 2),  # dilation along H
    ((20, 22), (8, 4), (4, 2), (2, 1), (0, 0), (1, 1), 1),  # stride 4 along H
    ((20, 22), (5, 4), (5, 2), (2, 1), (0, 0), (1, 1), 2),  # stride 5 along H
    ((20, 22), (10, 4), (2, 2), (4, 1), (0, 0), (1, 1), 2), # 5 row taps per phase
    ((20, 22), (3, 3), (2, 2), (1, 1), (1, 1), (1, 2), 2),
    ((20, 22), (3, 3), (3, 2), (1, 1), (0, 0), (1, 1), 1),  # any stride along H
])
def test_depthwise_kernel_choice(lib, sp, k, s, p, op, d, which):
    assert C.ctconv_depthwise_query_kernel(2, 8, 16, sp, k, s, p, op, d, 1) == which


def test_product_path_imports_no_oracle_and_fails_loudly_without_library(tmp_path):
    """The package and bench's product leg never import the oracle, and the
    binding raises when libctconv.so is missing (no CPU fallback)."""
    import ast
    import importlib

    pkg = os.path.join(ROOT, "vision_upsampler_decoders_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            tree = ast.parse(open(os.path.join(pkg, fn)).read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    assert not any(a.name.split(".")[0] == "oracle" for a in node.names), fn
                if isinstance(node, ast.ImportFrom):
                    assert (node.module or "").split(".")[0] != "oracle", fn
    mod = importlib.import_module("vision_upsampler_decoders_amd.ctconv")
    missing = str(tmp_path / "libctconv_missing.so")
    saved = mod._lib if hasattr(mod, "_lib") else None
    try:
        if hasattr(mod, "_lib"):
            mod._lib = None
        with pytest.raises((ImportError, OSError)):
            mod.load(missing)
    finally:
        if hasattr(mod, "_lib"):
            mod._lib = saved


def test_depthwise_size_limits_choose_element_kernel(lib):
    """Shapes past the row-phase kernels' 32-bit offsets (x of 2 GiB or more)
    go to the element kernel; sizes past int64 are rejected (host only, no
    allocation)."""
    # bf16 x of 8 * 512 * 2^18 * 2 bytes = 2 GiB: element kernel
    assert C.ctconv_depthwise_query_kernel(8, 512, 512, (1 << 18,), 4, 2, 1, 0, 1, 1) == 2
    # just under 2 GiB: row-phase family
    assert C.ctconv_depthwise_query_kernel(8, 512, 512, ((1 << 18) - 64,), 4, 2, 1, 0, 1, 1) == 1
    # element counts beyond int64
    with pytest.raises(C.CtconvError):
        C.ctconv_depthwise_query_kernel(1 << 40, 1 << 20, 1 << 20, (1 << 20,), 4, 2, 1, 0, 1, 1)


def test_workspace_bytes(lib):
    """Only fp32 shapes with too few output tiles split their reduction: the
    iSTFT (one output channel, 8 x 348 rows) asks for slabs the size of y;
    16-bit shapes and the large fp32 ones ask for none."""
    # iSTFT 4098 -> 1, k4096 s1024, 345 frames, N = 8: y has 8 * 356352 floats
    nb = C.ctconv_workspace_bytes(8, 4098, 1, (345,), 4096, 1024, 0, 0, 1, C.CTCONV_F32)
    y_bytes = 8 * 356352 * 4
    assert nb > 0 and nb % y_bytes == 0
    # one image of it (the per-GPU shard of a batch split): still split
    assert C.ctconv_workspace_bytes(1, 4098, 1, (345,), 4096, 1024, 0, 0, 1, C.CTCONV_F32) > 0
    assert C.ctconv_workspace_bytes(8, 512, 256, (2000,), 16, 8, 4, 0, 1, C.CTCONV_BF16) == 0
    assert C.ctconv_workspace_bytes(4, 128, 64, (96, 96), 3, 2, 1, 1, 2, C.CTCONV_F32) == 0
    # gather route and empty input: none
    assert C.ctconv_workspace_bytes(2, 40, 16, (100,), 8, 4, 2, 1, 3, C.CTCONV_F32) == 0
    assert C.ctconv_workspace_bytes(8, 4098, 1, (0,), 4096, 1024, 0, 0, 1, C.CTCONV_F32) == 0
    with pytest.raises(C.CtconvError):
        C.ctconv_workspace_bytes(8, 0, 1, (345,), 4096, 1024, 0, 0, 1, C.CTCONV_F32)


def test_forward_ws_validation_before_launch(lib):
    """A missing or short workspace is rejected on the host (no launch)."""
    nd = 1
    arr = lambda v: (ctypes.c_int64 * nd)(*C.per_dim(v, nd))  # noqa: E731
    need = C.ctconv_workspace_bytes(8, 4098, 1, (345,), 4096, 1024, 0, 0, 1, C.CTCONV_F32)

    def call(ws, nbytes, act=0):
        return lib.ctconv_forward_ws(0x1000, 0x2000, None, 0x3000, 8, 4098, 1, nd, arr((345,)),
                                     arr(4096), arr(1024), arr(0), arr(0), arr(1), 0, act, ws,
                                     nbytes, None)

    assert call(None, 0) == 7
    assert call(0x4000, need - 16) == 7
    assert call(0x4008, need) == 5      # misaligned workspace
    assert call(0x4000, need, act=9) == 3
    assert "workspace" in C.ctconv_status_string(7)


def test_noalloc_rejects_beyond_scratch_before_any_device_call(lib):
    """ctconv_forward_noalloc checks the workspace it needs against the fixed
    scratch on the host: a shape needing more is refused (no device call is
    made, which this GPU-less host would fail)."""
    assert C.ctconv_scratch_bytes() == 64 << 20
    need = C.ctconv_workspace_bytes(1, 2048, 2, (1024,), 4096, 2048, 0, 0, 1, C.CTCONV_F32)
    assert need > C.ctconv_scratch_bytes()
    nd = 1
    arr = lambda v: (ctypes.c_int64 * nd)(*C.per_dim(v, nd))  # noqa: E731
    st = lib.ctconv_forward_noalloc(0x1000, 0x2000, None, 0x3000, 1, 2048, 2, nd, arr((1024,)),
                                    arr(4096), arr(2048), arr(0), arr(0), arr(1), 0, 0, None)
    assert st == 8
    assert "scratch" in C.ctconv_status_string(8)
    # invalid arguments are still reported as such
    st = lib.ctconv_forward_noalloc(0x1000, 0x2000, None, 0x3000, 1, 0, 2, nd, arr((1024,)),
                                    arr(4096), arr(2048), arr(0), arr(0), arr(1), 0, 0, None)
    assert st == 2


def test_clock_probe_validates_before_any_device_call(lib):
    mhz = ctypes.c_double()
    # NULL workspace / NULL result, then an iteration count out of range
    assert lib.ctconv_clock_probe(None, 1 << 20, 4096, ctypes.byref(mhz), None, None) == 1
    assert lib.ctconv_clock_probe(ctypes.c_void_p(4096), 1 << 20, 4096, None, None, None) == 1
    assert lib.ctconv_clock_probe(ctypes.c_void_p(4096), 1 << 20, 0, ctypes.byref(mhz), None,
                                  None) == 3
    assert lib.ctconv_clock_probe(ctypes.c_void_p(4096), 1 << 20, (1 << 24) + 1,
                                  ctypes.byref(mhz), None, None) == 3

"""ctypes binding of libctconv (include/ctconv.h), plus torch-tensor helpers.

This module only marshals arguments: every step of the computation runs in
the HIP kernels of libctconv.so.  Importing it fails loudly when the library
has not been built; there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libctconv.so")

CTCONV_F32, CTCONV_BF16, CTCONV_F16 = 0, 1, 2
ROUTE_AUTO, ROUTE_POLYPHASE, ROUTE_GATHER = 0, 1, 2
# the two polyphase kernels, forced (cross-checks)
ROUTE_POLYPHASE_TILED, ROUTE_POLYPHASE_STREAM = 3, 4
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_PARAM", 4: "ERR_DTYPE",
          5: "ERR_ALIGN", 6: "ERR_HIP", 7: "ERR_WORKSPACE", 8: "ERR_SCRATCH"}

EXPORTED = (
    "ctconv_abi_version", "ctconv_status_string", "ctconv_output_shape", "ctconv_packed_bytes",
    "ctconv_prepack", "ctconv_forward", "ctconv_forward_route", "ctconv_forward_act",
    "ctconv_query_route", "ctconv_elu", "ctconv_stream_sizes", "ctconv_stream_step",
    "ctconv_stream_flush", "ctconv_istft_normalize", "ctconv_depthwise_forward",
    "ctconv_depthwise_forward_kernel", "ctconv_depthwise_query_kernel",
    "ctconv_workspace_bytes", "ctconv_forward_ws", "ctconv_forward_noalloc",
    "ctconv_scratch_bytes", "ctconv_clock_probe_bytes", "ctconv_clock_probe",
)

DW_AUTO, DW_ROW, DW_ELEMENT = 0, 1, 2

ACT_NONE, ACT_ELU = 0, 1


class CtconvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} "
                         f"({_string(status) if _lib is not None else ''})")


_lib = None
_i64p = ctypes.POINTER(ctypes.c_int64)


def load(path: str = LIB_PATH):
    """Load libctconv.so and declare its prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m vision_upsampler_decoders_amd.build`")
    lib = ctypes.CDLL(path)
    c_int, c_i64, c_vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    lib.ctconv_abi_version.argtypes = []
    lib.ctconv_abi_version.restype = c_int
    lib.ctconv_status_string.argtypes = [c_int]
    lib.ctconv_status_string.restype = ctypes.c_char_p
    lib.ctconv_output_shape.argtypes = [c_int] + [_i64p] * 7
    lib.ctconv_output_shape.restype = c_int
    lib.ctconv_packed_bytes.argtypes = [c_int, c_i64, c_i64, _i64p, _i64p, c_int,
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.ctconv_packed_bytes.restype = c_int
    lib.ctconv_prepack.argtypes = [c_vp, c_vp, c_int, c_i64, c_i64, _i64p, _i64p, c_int, c_vp]
    lib.ctconv_prepack.restype = c_int
    fwd = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_int] + [_i64p] * 6 + [c_int]
    lib.ctconv_forward.argtypes = fwd + [c_vp]
    lib.ctconv_forward.restype = c_int
    lib.ctconv_forward_route.argtypes = fwd + [c_int, c_vp]
    lib.ctconv_forward_route.restype = c_int
    lib.ctconv_forward_act.argtypes = fwd + [c_int, c_int, c_vp]
    lib.ctconv_forward_act.restype = c_int
    lib.ctconv_query_route.argtypes = [c_i64, c_i64, c_i64, c_int] + [_i64p] * 6 + [
        c_int, ctypes.POINTER(c_int)]
    lib.ctconv_query_route.restype = c_int
    lib.ctconv_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_int] + [_i64p] * 6 + [
        c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.ctconv_workspace_bytes.restype = c_int
    lib.ctconv_forward_ws.argtypes = fwd + [c_int, c_vp, ctypes.c_size_t, c_vp]
    lib.ctconv_forward_ws.restype = c_int
    lib.ctconv_forward_noalloc.argtypes = fwd + [c_int, c_vp]
    lib.ctconv_forward_noalloc.restype = c_int
    lib.ctconv_scratch_bytes.argtypes = []
    lib.ctconv_scratch_bytes.restype = ctypes.c_size_t
    lib.ctconv_clock_probe_bytes.argtypes = []
    lib.ctconv_clock_probe_bytes.restype = ctypes.c_size_t
    lib.ctconv_clock_probe.argtypes = [c_vp, ctypes.c_size_t, c_int, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double), c_vp]
    lib.ctconv_clock_probe.restype = c_int
    lib.ctconv_depthwise_forward.argtypes = fwd + [c_int, c_vp]
    lib.ctconv_depthwise_forward.restype = c_int
    lib.ctconv_depthwise_forward_kernel.argtypes = fwd + [c_int, c_int, c_vp]
    lib.ctconv_depthwise_forward_kernel.restype = c_int
    lib.ctconv_depthwise_query_kernel.argtypes = [c_i64, c_i64, c_i64, c_int] + [_i64p] * 6 + [
        c_int, ctypes.POINTER(c_int)]
    lib.ctconv_depthwise_query_kernel.restype = c_int
    lib.ctconv_elu.argtypes = [c_vp, c_vp, c_i64, c_int, c_vp]
    lib.ctconv_elu.restype = c_int
    lib.ctconv_stream_sizes.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i64, c_int, _i64p, _i64p,
                                        _i64p]
    lib.ctconv_stream_sizes.restype = c_int
    lib.ctconv_stream_step.argtypes = [c_vp] * 7 + [c_i64] * 6 + [c_int, c_int, c_vp]
    lib.ctconv_stream_step.restype = c_int
    lib.ctconv_stream_flush.argtypes = [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_int,
                                        c_int, c_vp]
    lib.ctconv_stream_flush.restype = c_int
    lib.ctconv_istft_normalize.argtypes = [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_int,
                                           c_vp]
    lib.ctconv_istft_normalize.restype = c_int
    _lib = lib
    return lib


def _string(status: int) -> str:
    return _lib.ctconv_status_string(status).decode()


def _arr(v: Sequence[int]):
    return (ctypes.c_int64 * len(v))(*[int(t) for t in v])


def per_dim(v, ndim: int) -> Tuple[int, ...]:
    """Broadcast a scalar to every spatial dimension (as parse_hw does for 2-D)."""
    if isinstance(v, int):
        return (v,) * ndim
    v = tuple(int(t) for t in v)
    if len(v) != ndim:
        raise ValueError(f"expected {ndim} values, got {v}")
    return v


def _check(fn: str, st: int):
    if st != 0:
        raise CtconvError(fn, st)


# ---------------------------------------------------------------------------
# Raw C-ABI calls with the same names (pointers and sizes only)
# ---------------------------------------------------------------------------


def ctconv_abi_version() -> int:
    return load().ctconv_abi_version()


def ctconv_status_string(status: int) -> str:
    load()
    return _string(status)


def ctconv_output_shape(in_spatial, kernel, stride, padding=0, output_padding=0, dilation=1):
    ndim = len(in_spatial)
    out = (ctypes.c_int64 * ndim)()
    st = load().ctconv_output_shape(ndim, _arr(in_spatial), _arr(per_dim(kernel, ndim)),
                                    _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
                                    _arr(per_dim(output_padding, ndim)),
                                    _arr(per_dim(dilation, ndim)), out)
    _check("ctconv_output_shape", st)
    return tuple(int(v) for v in out)


def ctconv_packed_bytes(ndim: int, C_in: int, C_out: int, kernel, stride, dtype: int) -> int:
    nb = ctypes.c_size_t(0)
    st = load().ctconv_packed_bytes(ndim, C_in, C_out, _arr(per_dim(kernel, ndim)),
                                    _arr(per_dim(stride, ndim)), dtype, ctypes.byref(nb))
    _check("ctconv_packed_bytes", st)
    return int(nb.value)


def ctconv_prepack(w_ptr: int, packed_ptr: int, ndim: int, C_in: int, C_out: int, kernel,
                   stride, dtype: int, stream: int) -> None:
    st = load().ctconv_prepack(w_ptr, packed_ptr, ndim, C_in, C_out,
                               _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), dtype,
                               stream)
    _check("ctconv_prepack", st)


def ctconv_forward_route(x_ptr: int, packed_ptr: int, bias_ptr: Optional[int], y_ptr: int, N: int,
                         C_in: int, C_out: int, in_spatial, kernel, stride, padding,
                         output_padding, dilation, dtype: int, route: int, stream: int) -> None:
    ndim = len(in_spatial)
    st = load().ctconv_forward_route(
        x_ptr, packed_ptr, bias_ptr, y_ptr, N, C_in, C_out, ndim, _arr(in_spatial),
        _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype, route, stream)
    _check("ctconv_forward_route", st)


def ctconv_forward_act(x_ptr: int, packed_ptr: int, bias_ptr: Optional[int], y_ptr: int, N: int,
                       C_in: int, C_out: int, in_spatial, kernel, stride, padding,
                       output_padding, dilation, dtype: int, act: int, route: int,
                       stream: int) -> None:
    ndim = len(in_spatial)
    st = load().ctconv_forward_act(
        x_ptr, packed_ptr, bias_ptr, y_ptr, N, C_in, C_out, ndim, _arr(in_spatial),
        _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype, act, route,
        stream)
    _check("ctconv_forward_act", st)


def ctconv_forward(x_ptr: int, packed_ptr: int, bias_ptr: Optional[int], y_ptr: int, N: int,
                   C_in: int, C_out: int, in_spatial, kernel, stride, padding, output_padding,
                   dilation, dtype: int, stream: int) -> None:
    ndim = len(in_spatial)
    st = load().ctconv_forward(
        x_ptr, packed_ptr, bias_ptr, y_ptr, N, C_in, C_out, ndim, _arr(in_spatial),
        _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype, stream)
    _check("ctconv_forward", st)


def ctconv_workspace_bytes(N: int, C_in: int, C_out: int, in_spatial, kernel, stride, padding=0,
                           output_padding=0, dilation=1, dtype: int = CTCONV_F32) -> int:
    ndim = len(in_spatial)
    nb = ctypes.c_size_t(0)
    st = load().ctconv_workspace_bytes(
        N, C_in, C_out, ndim, _arr(in_spatial), _arr(per_dim(kernel, ndim)),
        _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype,
        ctypes.byref(nb))
    _check("ctconv_workspace_bytes", st)
    return int(nb.value)


def ctconv_forward_ws(x_ptr: int, packed_ptr: int, bias_ptr: Optional[int], y_ptr: int, N: int,
                      C_in: int, C_out: int, in_spatial, kernel, stride, padding, output_padding,
                      dilation, dtype: int, act: int, ws_ptr: Optional[int], ws_bytes: int,
                      stream: int) -> None:
    ndim = len(in_spatial)
    st = load().ctconv_forward_ws(
        x_ptr, packed_ptr, bias_ptr, y_ptr, N, C_in, C_out, ndim, _arr(in_spatial),
        _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype, act, ws_ptr,
        ws_bytes, stream)
    _check("ctconv_forward_ws", st)


def ctconv_forward_noalloc(x_ptr: int, packed_ptr: int, bias_ptr: Optional[int], y_ptr: int,
                           N: int, C_in: int, C_out: int, in_spatial, kernel, stride, padding,
                           output_padding, dilation, dtype: int, act: int, stream: int) -> None:
    ndim = len(in_spatial)
    st = load().ctconv_forward_noalloc(
        x_ptr, packed_ptr, bias_ptr, y_ptr, N, C_in, C_out, ndim, _arr(in_spatial),
        _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype, act, stream)
    _check("ctconv_forward_noalloc", st)


def ctconv_scratch_bytes() -> int:
    return int(load().ctconv_scratch_bytes())


def ctconv_clock_probe_bytes() -> int:
    return int(load().ctconv_clock_probe_bytes())


def ctconv_clock_probe(ws_ptr: int, ws_bytes: int, iters: int, stream: int):
    """(sustained shader clock in MHz, the probe's bf16 MFMA TFLOP/s); synchronous."""
    mhz, tf = ctypes.c_double(), ctypes.c_double()
    st = load().ctconv_clock_probe(ws_ptr, ws_bytes, iters, ctypes.byref(mhz), ctypes.byref(tf),
                                   stream)
    _check("ctconv_clock_probe", st)
    return mhz.value, tf.value


def ctconv_query_route(N: int, C_in: int, C_out: int, in_spatial, kernel, stride, padding=0,
                       output_padding=0, dilation=1, dtype: int = CTCONV_F32) -> int:
    ndim = len(in_spatial)
    r = ctypes.c_int(-1)
    st = load().ctconv_query_route(
        N, C_in, C_out, ndim, _arr(in_spatial), _arr(per_dim(kernel, ndim)),
        _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype,
        ctypes.byref(r))
    _check("ctconv_query_route", st)
    return r.value


def ctconv_depthwise_forward_kernel(x_ptr: int, w_ptr: int, bias_ptr: Optional[int], y_ptr: int,
                                    N: int, C_in: int, C_out: int, in_spatial, kernel, stride,
                                    padding, output_padding, dilation, dtype: int, act: int,
                                    which: int, stream: int) -> None:
    ndim = len(in_spatial)
    st = load().ctconv_depthwise_forward_kernel(
        x_ptr, w_ptr, bias_ptr, y_ptr, N, C_in, C_out, ndim, _arr(in_spatial),
        _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype, act, which,
        stream)
    _check("ctconv_depthwise_forward_kernel", st)


def ctconv_depthwise_forward(x_ptr: int, w_ptr: int, bias_ptr: Optional[int], y_ptr: int, N: int,
                             C_in: int, C_out: int, in_spatial, kernel, stride, padding,
                             output_padding, dilation, dtype: int, act: int,
                             stream: int) -> None:
    ndim = len(in_spatial)
    st = load().ctconv_depthwise_forward(
        x_ptr, w_ptr, bias_ptr, y_ptr, N, C_in, C_out, ndim, _arr(in_spatial),
        _arr(per_dim(kernel, ndim)), _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype, act, stream)
    _check("ctconv_depthwise_forward", st)


def ctconv_depthwise_query_kernel(N: int, C_in: int, C_out: int, in_spatial, kernel, stride,
                                  padding=0, output_padding=0, dilation=1,
                                  dtype: int = CTCONV_F32) -> int:
    ndim = len(in_spatial)
    r = ctypes.c_int(-1)
    st = load().ctconv_depthwise_query_kernel(
        N, C_in, C_out, ndim, _arr(in_spatial), _arr(per_dim(kernel, ndim)),
        _arr(per_dim(stride, ndim)), _arr(per_dim(padding, ndim)),
        _arr(per_dim(output_padding, ndim)), _arr(per_dim(dilation, ndim)), dtype,
        ctypes.byref(r))
    _check("ctconv_depthwise_query_kernel", st)
    return r.value


def ctconv_elu(x_ptr: int, y_ptr: int, n: int, dtype: int, stream: int) -> None:
    _check("ctconv_elu", load().ctconv_elu(x_ptr, y_ptr, n, dtype, stream))


def ctconv_stream_sizes(N: int, C_out: int, L_chunk: int, kernel: int, stride: int,
                        dtype: int) -> Tuple[int, int, int]:
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("ctconv_stream_sizes",
           load().ctconv_stream_sizes(N, C_out, L_chunk, kernel, stride, dtype, ctypes.byref(a),
                                      ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def ctconv_stream_step(x_ptr: int, packed_ptr: int, bias_ptr: Optional[int], y_ptr: int,
                       tail_in_ptr: Optional[int], tail_out_ptr: Optional[int], ws_ptr: int, N: int,
                       C_in: int, C_out: int, L_chunk: int, kernel: int, stride: int, dtype: int,
                       act: int, stream: int) -> None:
    _check("ctconv_stream_step",
           load().ctconv_stream_step(x_ptr, packed_ptr, bias_ptr, y_ptr, tail_in_ptr,
                                     tail_out_ptr, ws_ptr, N, C_in, C_out, L_chunk, kernel,
                                     stride, dtype, act, stream))


def ctconv_stream_flush(tail_in_ptr: Optional[int], bias_ptr: Optional[int], y_ptr: int, N: int,
                        C_out: int, kernel: int, stride: int, dtype: int, act: int,
                        stream: int) -> None:
    _check("ctconv_stream_flush",
           load().ctconv_stream_flush(tail_in_ptr, bias_ptr, y_ptr, N, C_out, kernel, stride,
                                      dtype, act, stream))


def ctconv_istft_normalize(y_ptr: int, env_ptr: int, out_ptr: int, rows: int, L_in: int,
                           trim: int, L_out: int, dtype: int, stream: int) -> None:
    _check("ctconv_istft_normalize",
           load().ctconv_istft_normalize(y_ptr, env_ptr, out_ptr, rows, L_in, trim, L_out, dtype,
                                         stream))


# ---------------------------------------------------------------------------
# torch helpers (device memory and streams only)
# ---------------------------------------------------------------------------


def _torch():
    import torch

    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: CTCONV_F32, torch.bfloat16: CTCONV_BF16, torch.float16: CTCONV_F16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def dtype_code_of(name: str) -> int:
    """"f32" / "bf16" / "f16" -> the ctconv_dtype code."""
    return {"f32": CTCONV_F32, "bf16": CTCONV_BF16, "f16": CTCONV_F16}[name]


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _side_stream(stream, device):
    """The explicit stream when it differs from the current one (else None).
    Inputs made ready on the current stream (copies by .contiguous(), fresh
    allocations) must be visible to it, so it first waits for the current
    stream."""
    torch = _torch()
    if stream is None:
        return None
    cur = torch.cuda.current_stream(device)
    if int(stream.cuda_stream) == int(cur.cuda_stream):
        return None
    stream.wait_stream(cur)
    return stream


def _claim(side, *tensors):
    """Tell the caching allocator that these tensors are used on `side`, so
    their memory is not reused before the work queued there is done."""
    if side is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(side)


def _check_tensor(name, t, dtype, device, shape=None, numel=None):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def sustained_clock(iters: int = 4096, device=None, stream=None):
    """(MHz, TFLOP/s) of ctconv_clock_probe on `device` (a workspace is allocated here)."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    nb = ctconv_clock_probe_bytes()
    ws = torch.empty(max(nb, 8), dtype=torch.uint8, device=dev)
    return ctconv_clock_probe(ws.data_ptr(), ws.numel(), iters, _stream(stream))


def prepack(w, stride, stream=None):
    """Packed phase-major copy of a ConvTranspose weight w [C_in, C_out, k...] (device)."""
    torch = _torch()
    if not w.is_cuda:
        raise ValueError("w must be a device tensor")
    w = w.contiguous()
    ndim = w.dim() - 2
    C_in, C_out = w.shape[0], w.shape[1]
    k = tuple(w.shape[2:])
    dt = dtype_code(w)
    nb = ctconv_packed_bytes(ndim, C_in, C_out, k, stride, dt)
    packed = torch.empty(nb // w.element_size(), dtype=w.dtype, device=w.device)
    side = _side_stream(stream, w.device)
    ctconv_prepack(w.data_ptr(), packed.data_ptr(), ndim, C_in, C_out, k, stride, dt,
                   _stream(stream))
    _claim(side, w, packed)
    return packed


def forward(x, packed, bias, C_out: int, kernel, stride, padding=0, output_padding=0,
            dilation=1, route: int = ROUTE_AUTO, out=None, stream=None, act: int = ACT_NONE,
            workspace=None):
    """y = act(ConvTranspose(x, w, bias)) with w given by its packed form (device tensors).

    packed must be the ctconv_prepack output for this C_in, C_out, kernel,
    stride and dtype: its byte size is checked against ctconv_packed_bytes.
    bias (or None) is [C_out] of x's dtype; out (or None) is the contiguous
    [N, C_out, out_spatial...] tensor of x's dtype to write.  workspace: None
    (ctconv_forward_act), True (ctconv_forward_ws with a workspace allocated
    here) or a device tensor of at least ctconv_workspace_bytes bytes
    (ctconv_forward_ws; route must be ROUTE_AUTO)."""
    torch = _torch()
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    x = x.contiguous()
    ndim = x.dim() - 2
    if ndim not in (1, 2):
        raise ValueError("x must be [N, C_in, L] or [N, C_in, H, W]")
    N, C_in = x.shape[0], x.shape[1]
    sp = tuple(x.shape[2:])
    dt = dtype_code(x)
    kernel = per_dim(kernel, ndim)
    nb = ctconv_packed_bytes(ndim, C_in, C_out, kernel, stride, dt)
    _check_tensor("packed", packed, x.dtype, x.device)
    if not packed.is_contiguous() or packed.numel() * packed.element_size() != nb:
        raise ValueError(f"packed holds {packed.numel() * packed.element_size()} bytes; "
                         f"ctconv_packed_bytes gives {nb} for this weight shape, stride and "
                         f"dtype")
    osp = ctconv_output_shape(sp, kernel, stride, padding, output_padding, dilation)
    if bias is not None:
        _check_tensor("bias", bias, x.dtype, x.device, numel=C_out)
        bias = bias.contiguous()
    if out is not None:
        _check_tensor("out", out, x.dtype, x.device, shape=(N, C_out) + osp)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        y = out
    else:
        y = torch.empty((N, C_out) + osp, dtype=x.dtype, device=x.device)
    ws = None
    if workspace is not None:
        if route != ROUTE_AUTO:
            raise ValueError("a workspace call takes the automatic route")
        need = ctconv_workspace_bytes(N, C_in, C_out, sp, kernel, stride, padding,
                                      output_padding, dilation, dt)
        if workspace is True:
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
        else:
            ws = workspace
            if not ws.is_cuda or ws.device != x.device or not ws.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on x's device")
            if ws.numel() * ws.element_size() < need:
                raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes; "
                                 f"ctconv_workspace_bytes gives {need}")
    side = _side_stream(stream, x.device)
    bptr = None if bias is None else bias.data_ptr()
    if ws is None:
        ctconv_forward_act(x.data_ptr(), packed.data_ptr(), bptr, y.data_ptr(), N, C_in, C_out,
                           sp, kernel, stride, padding, output_padding, dilation, dt, act,
                           route, _stream(stream))
    else:
        ctconv_forward_ws(x.data_ptr(), packed.data_ptr(), bptr, y.data_ptr(), N, C_in, C_out, sp,
                          kernel, stride, padding, output_padding, dilation, dt, act,
                          ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _claim(side, x, packed, bias, y, ws)
    return y


def depthwise_forward(x, w, bias, stride, padding=0, output_padding=0, dilation=1,
                      act: int = ACT_NONE, which: int = DW_AUTO, out=None, stream=None):
    """y = act(ConvTranspose(x, w, bias, groups=C_in)) for w [C_in, M, k...] (device tensors)."""
    torch = _torch()
    if not x.is_cuda or not w.is_cuda:
        raise ValueError("x and w must be device tensors")
    x = x.contiguous()
    w = w.contiguous()
    ndim = x.dim() - 2
    if ndim not in (1, 2):
        raise ValueError("x must be [N, C_in, L] or [N, C_in, H, W]")
    N, C_in = x.shape[0], x.shape[1]
    if w.shape[0] != C_in or w.dim() != ndim + 2:
        raise ValueError("w must be [C_in, M, k...]")
    _check_tensor("w", w, x.dtype, x.device)
    C_out = C_in * w.shape[1]
    kernel = tuple(w.shape[2:])
    sp = tuple(x.shape[2:])
    osp = ctconv_output_shape(sp, kernel, stride, padding, output_padding, dilation)
    if bias is not None:
        _check_tensor("bias", bias, x.dtype, x.device, numel=C_out)
        bias = bias.contiguous()
    if out is not None:
        _check_tensor("out", out, x.dtype, x.device, shape=(N, C_out) + osp)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        y = out
    else:
        y = torch.empty((N, C_out) + osp, dtype=x.dtype, device=x.device)
    side = _side_stream(stream, x.device)
    bptr = None if bias is None else bias.data_ptr()
    ctconv_depthwise_forward_kernel(x.data_ptr(), w.data_ptr(), bptr, y.data_ptr(), N, C_in,
                                    C_out, sp, kernel, stride, padding, output_padding, dilation,
                                    dtype_code(x), act, which, _stream(stream))
    _claim(side, x, w, bias, y)
    return y


def elu(x, out=None, stream=None):
    torch = _torch()
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    x = x.contiguous()
    if out is not None:
        _check_tensor("out", out, x.dtype, x.device, shape=tuple(x.shape))
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        y = out
    else:
        y = torch.empty_like(x)
    side = _side_stream(stream, x.device)
    ctconv_elu(x.data_ptr(), y.data_ptr(), x.numel(), dtype_code(x), _stream(stream))
    _claim(side, x, y)
    return y


class Conv:
    """A transposed convolution with its arguments marshalled once.

    Holds the C arrays of one shape so that each call is a single foreign
    function call (no per-call Python-side shape work).  Buffers are passed as
    device tensors or raw pointers at call time.
    """

    def __init__(self, N: int, C_in: int, C_out: int, in_spatial, kernel, stride, padding=0,
                 output_padding=0, dilation=1, dtype: int = CTCONV_F32,
                 route: int = ROUTE_AUTO, act: int = ACT_NONE):
        nd = len(in_spatial)
        self.ndim = nd
        self.N, self.C_in, self.C_out = int(N), int(C_in), int(C_out)
        self.in_spatial = tuple(int(v) for v in in_spatial)
        self.kernel = per_dim(kernel, nd)
        self.stride = per_dim(stride, nd)
        self.padding = per_dim(padding, nd)
        self.output_padding = per_dim(output_padding, nd)
        self.dilation = per_dim(dilation, nd)
        self.dtype = dtype
        self.route = route
        self.act = act
        self.out_spatial = ctconv_output_shape(self.in_spatial, self.kernel, self.stride,
                                               self.padding, self.output_padding, self.dilation)
        self._args = [_arr(self.in_spatial), _arr(self.kernel), _arr(self.stride),
                      _arr(self.padding), _arr(self.output_padding), _arr(self.dilation)]
        self._fn = load().ctconv_forward_act

    def out_shape(self):
        return (self.N, self.C_out) + self.out_spatial

    def __call__(self, x_ptr: int, packed_ptr: int, bias_ptr, y_ptr: int, stream: int) -> None:
        st = self._fn(x_ptr, packed_ptr, bias_ptr, y_ptr, self.N, self.C_in, self.C_out,
                      self.ndim, *self._args, self.dtype, self.act, self.route, stream)
        if st != 0:
            raise CtconvError("ctconv_forward_act", st)


class DepthwiseConv(Conv):
    """A depthwise transposed convolution (groups = C_in) with its arguments
    marshalled once; called with the unpacked weight [C_in, C_out / C_in, k...]."""

    def __init__(self, *args, which: int = DW_AUTO, **kw):
        kw.pop("route", None)
        super().__init__(*args, **kw)
        self.which = which
        self._fn = load().ctconv_depthwise_forward_kernel

    def __call__(self, x_ptr: int, w_ptr: int, bias_ptr, y_ptr: int, stream: int) -> None:
        st = self._fn(x_ptr, w_ptr, bias_ptr, y_ptr, self.N, self.C_in, self.C_out,
                      self.ndim, *self._args, self.dtype, self.act, self.which, stream)
        if st != 0:
            raise CtconvError("ctconv_depthwise_forward_kernel", st)


class ConvWS(Conv):
    """A transposed convolution through ctconv_forward_ws (deterministic split
    of the reduction when the shape calls for one), arguments marshalled once;
    called with the workspace pointer and its size in bytes."""

    def __init__(self, *args, **kw):
        kw.pop("route", None)
        super().__init__(*args, **kw)
        self._fn = load().ctconv_forward_ws
        self.ws_bytes = ctconv_workspace_bytes(self.N, self.C_in, self.C_out, self.in_spatial,
                                               self.kernel, self.stride, self.padding,
                                               self.output_padding, self.dilation, self.dtype)

    def __call__(self, x_ptr: int, packed_ptr: int, bias_ptr, y_ptr: int, stream: int,
                 ws_ptr=None, ws_bytes: int = 0) -> None:
        st = self._fn(x_ptr, packed_ptr, bias_ptr, y_ptr, self.N, self.C_in, self.C_out,
                      self.ndim, *self._args, self.dtype, self.act, ws_ptr, ws_bytes, stream)
        if st != 0:
            raise CtconvError("ctconv_forward_ws", st)

"""ctconv: dense transposed convolution (ConvTranspose1d/2d) on AMD MI355X.

The computation lives in libctconv.so (HIP, gfx950); see include/ctconv.h for
the C ABI.  This package holds the build script and the ctypes binding.
"""

from .ctconv import (  # noqa: F401
    CTCONV_BF16,
    CTCONV_F16,
    CTCONV_F32,
    ROUTE_AUTO,
    ROUTE_GATHER,
    ROUTE_POLYPHASE,
    CtconvError,
    elu,
    forward,
    load,
    prepack,
)

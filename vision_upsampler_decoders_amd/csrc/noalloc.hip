// ctconv_forward_noalloc: ctconv_forward_ws with the library's own fixed
// scratch as the workspace, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops).  Nothing here calls an
// allocating routine: the scratch is a file-scope device array that the
// runtime creates with the code object, and its address on each device is
// looked up once (hipGetSymbolAddress) with that device current.

#include <mutex>

#include "ctconv_internal.h"

namespace {

// The workspace of every no-allocation call on a device (one copy per
// device, held until the process ends).  Only its device address, looked up
// below, is ever passed to a kernel: on the host, `scratch` names a host-side
// stand-in, not device memory.
static __device__ __align__(256) unsigned char scratch[CTCONV_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // scratch's address per device (write-once)

// The scratch's address on `dev`, looked up on first use with dev current.
ctconv_status scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return CTCONV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return CTCONV_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return CTCONV_ERR_HIP;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return CTCONV_ERR_HIP;
        if (e != hipSuccess || ptr == nullptr) return CTCONV_ERR_HIP;
        g_ptr[dev] = ptr;
    }
    *out = g_ptr[dev];
    return CTCONV_OK;
}

}  // namespace

extern "C" {

size_t ctconv_scratch_bytes(void) { return (size_t)CTCONV_SCRATCH_BYTES; }

ctconv_status ctconv_forward_noalloc(const void* x, const void* packed_w, const void* bias,
                                     void* y, int64_t N, int64_t C_in, int64_t C_out, int ndim,
                                     const int64_t* in_spatial, const int64_t* kernel,
                                     const int64_t* stride, const int64_t* padding,
                                     const int64_t* output_padding, const int64_t* dilation,
                                     ctconv_dtype dtype, ctconv_activation act, void* stream) {
    // host-only checks first: the workspace this call needs must fit the scratch
    size_t need = 0;
    ctconv_status st = ctconv_workspace_bytes(N, C_in, C_out, ndim, in_spatial, kernel, stride,
                                              padding, output_padding, dilation, dtype, &need);
    if (st != CTCONV_OK) return st;
    if (need > (size_t)CTCONV_SCRATCH_BYTES) return CTCONV_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        // the device the work is enqueued on
        int dev = -1;
        const hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                    : hipGetDevice(&dev);
        if (e != hipSuccess) return CTCONV_ERR_HIP;
        st = scratch_on(dev, &ws);
        if (st != CTCONV_OK) return st;
    }
    return ctconv_forward_ws(x, packed_w, bias, y, N, C_in, C_out, ndim, in_spatial, kernel,
                             stride, padding, output_padding, dilation, dtype, act, ws,
                             need > 0 ? (size_t)CTCONV_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"

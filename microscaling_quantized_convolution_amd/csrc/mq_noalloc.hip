// mq_noalloc.hip -- the backward convolution call for callers that cannot allocate.
//
// mq_conv_backward_noalloc computes what mq_conv_backward computes (the weight gradient
// G_W = G_Y . X'^T and the input gradient G_X = col2im(W^T . G_Y) of the onedev.kr MicroQonv
// digest, section "How it differs"), with the same kernels, but the weight gradient's split-K
// partial sums live in a library-owned device array instead of a caller workspace: code under
// HIP graph capture, tight serving loops and harnesses that forbid hipMalloc can call it with
// only their inputs and outputs.
//
// The array is a file-scope __device__ variable of MQ_NOALLOC_SCRATCH_BYTES bytes; every GPU the
// library runs on holds its own copy until the process ends. Host code never uses the array's
// name as an address (on the host it only names the symbol): once per device, with that device
// current, hipGetSymbolAddress gives the device address, which is kept per device and passed to
// the kernels like a workspace pointer. Every call on one GPU shares that GPU's array; the split
// partials are fully written before they are read, so nothing has to start at zero, but calls
// that overlap on one GPU (different streams, or different host threads without ordering) race
// on it.
#include "../../include/mq.h"
#include "mq_kernels.hpp"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

__device__ __align__(256) uint8_t scratch[MQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per device), or null.
void *scratch_on_current_device(mq_status *err)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = MQ_ERR_LAUNCH;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *err = MQ_ERR_LAUNCH;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

} // namespace

extern "C" mq_status mq_conv_backward_noalloc(const mq_conv *p, const mq_qtensor *w,
                                              const mq_qtensor *gy, const mq_qtensor *x,
                                              float *gw_dev, float *gx_dev, hipStream_t stream)
{
    // every host-side check before the device is touched
    const mq_status chk = mq::backward_check(p, w, gy, x, gw_dev, gx_dev);
    if (chk != MQ_OK) return chk;
    if (mq_wgrad_workspace_bytes(p) > MQ_NOALLOC_SCRATCH_BYTES) return MQ_ERR_UNSUPPORTED;
    mq_status err = MQ_OK;
    void *ws = scratch_on_current_device(&err);
    if (!ws) return err;
    return mq_conv_backward(p, w, gy, x, gw_dev, gx_dev, ws, MQ_NOALLOC_SCRATCH_BYTES, stream);
}

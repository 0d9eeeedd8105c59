// tp_linear_row_noalloc: the row-parallel Linear with its workspace taken
// from a fixed device array instead of the caller, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Declared in include/tplinear.h.
//
// `scratch` below is one array per GPU the library runs on, reserved when the
// code object is loaded on that GPU and held until the process ends.  In host
// code its name is only a host-side stand-in, not a device address: the
// device address of each GPU's copy is looked up with hipGetSymbolAddress
// once per device (with that device current) and cached, and only that
// address is ever passed on.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"
#include "tplinear.h"

namespace {

static __device__ __attribute__((aligned(256))) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;        // devices with an id below this are served
std::atomic<void *> scratch_addr[MAX_DEVICES];
std::mutex scratch_mu;

// Device address of the current device's copy of `scratch`.
tp_status current_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TP_ERR_HIP;
    if (dev >= MAX_DEVICES) return TP_ERR_HIP;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *q = nullptr;
            if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
                return TP_ERR_HIP;
            scratch_addr[dev].store(q, std::memory_order_release);
            p = q;
        }
    }
    *out = p;
    return TP_OK;
}

}  // namespace

extern "C" tp_status tp_linear_row_noalloc(const void *X, int64_t ldx, const void *W, int64_t ldw,
                                           void *Y, int64_t ldy, int64_t y_slice_stride,
                                           int32_t mode, int64_t M, int64_t N, int64_t K, int32_t P,
                                           int32_t dtype, void *stream) {
    // tp_linear_row's argument checks first, so both reject the same calls
    // the same way before anything touches a device.
    const tp_status chk = tpl::row_args_status(X, ldx, W, ldw, nullptr, Y, nullptr, ldy,
                                               y_slice_stride, mode, M, N, K, P, dtype);
    if (chk != TP_OK) return chk;
    if (M == 0 || N == 0) return TP_OK;
    tpl::RowPlan plan;
    const tp_status pst = tpl::plan_row(X, ldx, W, ldw, nullptr, Y, nullptr, ldy, y_slice_stride,
                                        mode, M, N, K, P, dtype, TP_NOALLOC_SCRATCH_BYTES, plan);
    if (pst != TP_OK) return pst;
    // Only the partials-and-fold path uses a workspace: the P fp32 partials.
    void *ws = nullptr;
    if (plan.path == tpl::RowPlan::PARTIALS_AND_FOLD) {
        if (tp_row_workspace_bytes(mode, M, N, P) > (size_t)TP_NOALLOC_SCRATCH_BYTES)
            return TP_ERR_WORKSPACE;
        const tp_status st = current_scratch(&ws);
        if (st != TP_OK) return st;
    }
    return tpl::run_row(plan, (float *)ws, (hipStream_t)stream);
}

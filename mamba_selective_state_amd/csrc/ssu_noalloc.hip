// ssu_ssd_prefill_noalloc: the SSD prefill with its workspace in a
// file-scope device array instead of a caller's buffer, for callers that
// cannot allocate. The kernels are ssu_ssd_prefill's own; only where the
// workspace lives differs.
//
// Host code never passes `scratch` itself: in host code that name stands for
// a host-side shadow, not a device address. The array's address on a GPU is
// taken once per device with hipGetSymbolAddress while that device is
// current, and that address is what the kernels receive.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ssu.h"
#include "ssu_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SSU_SSD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // the array's address on each device, once looked up

// The array's device address on the current device (nullptr on failure,
// with the error reported).
void *scratch_on_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        ssu::report_error(SSU_ERR_HIP, "ssu_ssd_prefill_noalloc: no current device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            ssu::report_error(SSU_ERR_HIP, "ssu_ssd_prefill_noalloc: hipGetSymbolAddress of the workspace failed");
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" ssu_status_t ssu_ssd_prefill_noalloc(const ssu_ssd_args_t *a, void *stream) {
    if (!a)
        return ssu::report_error(SSU_ERR_VALUE, "ssu_ssd_prefill_noalloc: args is NULL");
    // the workspace this call needs, from the shapes ssu_ssd_prefill checks
    // in full afterwards
    const bool shaped = a->x.ndim == 3 && a->B.ndim == 3 && a->cu_chunk_seqlens.ndim == 1;
    if (shaped) {
        const int64_t need = ssu_ssd_workspace_bytes(a->x.size[1], a->x.size[2], a->B.size[2],
                                                     a->cu_chunk_seqlens.size[0] - 1);
        if (need > SSU_SSD_SCRATCH_BYTES) {
            char msg[256];
            snprintf(msg, sizeof msg,
                     "ssu_ssd_prefill_noalloc: this call needs %lld bytes of workspace, more than the "
                     "%lld the allocation-free entry point holds (use ssu_ssd_prefill)",
                     (long long)need, (long long)SSU_SSD_SCRATCH_BYTES);
            return ssu::report_error(SSU_ERR_VALUE, msg);
        }
    }
    void *ptr = scratch_on_current_device();
    if (!ptr)
        return SSU_ERR_HIP;
    return ssu_ssd_prefill(a, ptr, SSU_SSD_SCRATCH_BYTES, stream);
}

// ssd_noalloc.hip -- ssd_chunk_scan_fwd_noalloc: the forward pass with the
// library's own device scratch, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The workspace of ssd_chunk_scan_fwd (decay sums, weights, chunk states,
// chunk-start states, C B^T tiles) lives in a file-scope device array of
// SSD_NOALLOC_SCRATCH_BYTES.  Every GPU the library runs on holds its own
// copy of the array, at its own address, from the first call on that device
// until the process ends.  Host code never passes the array's name to a
// kernel: the name is a host-side stand-in, so the device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and that
// address is what the stages receive as their workspace.
//
// Nothing here allocates: no hipMalloc, no hipFree, no allocating library
// call.  The stages ignore the workspace's contents on entry, so nothing
// needs clearing between calls.  All calls on one GPU share its array, so
// calls that overlap in time on one GPU (two streams, two threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ssd.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Per device: the array's device address, found once with that device
// current.  std::call_once makes concurrent first calls on one device safe.
struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t status = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

ssd_status scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERROR_LAUNCH;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d]() {
        void *p = nullptr;
        d.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.status == hipSuccess) d.ptr = p;
    });
    if (d.status != hipSuccess || d.ptr == nullptr) return SSD_ERROR_LAUNCH;
    *out = d.ptr;
    return SSD_OK;
}

}  // namespace

extern "C" ssd_status ssd_chunk_scan_fwd_noalloc(const ssd_shape *shape, const void *x, const void *dt,
                                                 const float *A, const void *B, const void *C,
                                                 const float *D, int64_t chunk_size,
                                                 const float *initial_states, void *y,
                                                 float *final_states, void *stream) {
    if (shape == nullptr) return SSD_ERROR_INVALID_VALUE;
    if (shape->flags != 0) return SSD_ERROR_INVALID_VALUE;  // intermediates are not readable here
    const size_t need = ssd_chunk_scan_fwd_workspace_size(shape, chunk_size);
    if (need == 0) {
        // invalid or unsupported shape: report which, exactly as the forward call would
        ssd_workspace_layout lay;
        const ssd_status st = ssd_chunk_scan_fwd_workspace_layout(shape, chunk_size, &lay);
        if (st != SSD_OK) return st;
    }
    if (need > (size_t)SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERROR_SCRATCH;
    if (shape->batch == 0) {
        // nothing to compute; no device is touched
        return ssd_chunk_scan_fwd(shape, x, dt, A, B, C, D, chunk_size, initial_states, y,
                                  final_states, nullptr, 0, stream);
    }
    void *ws = nullptr;
    const ssd_status st = scratch_for_current_device(&ws);
    if (st != SSD_OK) return st;
    return ssd_chunk_scan_fwd(shape, x, dt, A, B, C, D, chunk_size, initial_states, y, final_states,
                              ws, (size_t)SSD_NOALLOC_SCRATCH_BYTES, stream);
}

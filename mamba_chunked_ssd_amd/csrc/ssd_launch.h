// ssd_launch.h -- launch helpers shared by the kernel translation units
// (device code; the host-only declarations are in ssd_internal.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "ssd_internal.h"

namespace ssd {

// Launch on `stream`; when `ev` holds events they time this dispatch alone.
template <typename... Args, typename F>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                const LaunchEvents &ev, Args... args) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, ev.start, ev.stop, 0u, args...);
    return hipGetLastError();
}

// Opt a kernel in to more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per
// CU).  The template parameter is the kernel itself.  The attribute is set on
// the first call for that kernel through a function-local static, whose
// initialisation C++ makes thread-safe (concurrent first calls wait for the
// one that runs it); afterwards the result is only read, so there is no
// mutable shared state.  A failure is kept and returned to every caller.
template <auto Kernel>
hipError_t allow_lds(size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    static const hipError_t status = hipFuncSetAttribute(
        reinterpret_cast<const void *>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kLdsPerCu);
    return status;
}

// Blocks are dispatched round-robin over the 8 XCDs (each with its own L2).
// Remap a hardware block index so that consecutive logical indices land on
// the same XCD: logical = (hw % 8) * (n / 8) + hw / 8 when n % 8 == 0.
__device__ __forceinline__ int xcd_remap(int hw, int n) {
    if (n % 8 != 0) return hw;
    return (hw % 8) * (n / 8) + hw / 8;
}

}  // namespace ssd

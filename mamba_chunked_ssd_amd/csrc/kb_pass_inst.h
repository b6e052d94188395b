// kb_pass_inst.h -- launch of one backward MFMA pass for one input type and
// headdim (instantiated by kb_pass_q.hip, kb_pass_b.hip, kb_pass_c.hip).
#pragma once

#include "kb_pass.h"

namespace ssd {
namespace bwd {

template <typename In, int NKQ, int DV, int PASS>
hipError_t launch_one(const PassArgs &a, unsigned blocks, size_t lds, hipStream_t stream, const LaunchEvents &ev) {
    constexpr auto kern = kb_pass<In, NKQ, DV, PASS>;
    const hipError_t st = allow_lds<kern>(lds);
    if (st != hipSuccess) return st;
    const int threads = kb_threads(PASS, std::is_same<In, uint16_t>::value, NKQ, a.T);
    if (a.occ != nullptr)  // blocks per CU at this LDS size and the kernel's registers
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(a.occ, kern, threads, lds);
    return launch_kernel(kern, dim3(blocks), dim3(threads), lds, stream, ev, a);
}

// Whether passes B and C are built with `dv`-column tiles for this input type
// and headdim.  bf16: the accumulators (strips per wave x dv / 16 per lane)
// beside the Q fragments (headdim / 32, one bf16 term) fit the waves'
// registers (256 at two strips per wave, 128 at one, where a block holds 16
// waves; at one strip the widest tiles spill a few values) only up to this
// width.  fp32: the scores come from the stored tiles, so the three-term Q
// fragments live only for the state term and 64 columns fit.  The host
// applies the same rule (bwd_dv_ok in ssd_internal.h).
__host__ __device__ constexpr bool bc_dv_ok(bool bf16, int P, int dv) {
    return dv <= (bf16 ? (P <= 64 ? 64 : 32) : 64);
}

// passes B and C: headdim (32 k) and dv-tile dispatch
template <typename In, int PASS>
hipError_t launch_bc(const PassArgs &a, int dv, unsigned blocks, size_t lds, hipStream_t stream,
                     const LaunchEvents &ev) {
#define SSD_KB_DVX(NK, DVV)                                                                 \
    if constexpr (bc_dv_ok(std::is_same<In, uint16_t>::value, 32 * NK, DVV))                \
        return launch_one<In, NK, DVV, PASS>(a, blocks, lds, stream, ev);                   \
    else                                                                                    \
        return hipErrorInvalidValue;
#define SSD_KB_DV(NK)                                                                       \
    switch (dv) {                                                                           \
        case 16: SSD_KB_DVX(NK, 16)                                                         \
        case 32: SSD_KB_DVX(NK, 32)                                                         \
        case 64: SSD_KB_DVX(NK, 64)                                                         \
        default: return hipErrorInvalidValue;                                               \
    }
    switch (a.P) {
        case 32: SSD_KB_DV(1)
        case 64: SSD_KB_DV(2)
        case 128: SSD_KB_DV(4)
        default: return hipErrorInvalidValue;
    }
#undef SSD_KB_DV
#undef SSD_KB_DVX
}

// the entry of each translation unit
hipError_t launch_pass_q(const PassArgs &a, bool bf16, int dv, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev);
hipError_t launch_pass_b(const PassArgs &a, bool bf16, int dv, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev);
hipError_t launch_pass_c(const PassArgs &a, bool bf16, int dv, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev);
hipError_t launch_pass_w(const PassArgs &a, bool bf16, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev);
hipError_t launch_pass_p(const PassArgs &a, unsigned blocks, size_t lds, hipStream_t stream, const LaunchEvents &ev);

}  // namespace bwd
}  // namespace ssd

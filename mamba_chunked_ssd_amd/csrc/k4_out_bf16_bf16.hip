// k4_out_bf16_bf16.hip -- stage 4 (chunk output) instantiated for bf16 inputs and a bf16 y.
// The kernels and their documentation are in k4_chunk_out.h.
#include "k4_chunk_out.h"

namespace ssd {
namespace k4 {

hipError_t launch_bf16_in_bf16_out(const Problem &p, const Plan &plan, const void *x, const void *B,
                                   const void *C, const float *CB, G2View G2, const float *DT, const float *D,
                                   const float *H, void *y, hipStream_t stream, const LaunchEvents &ev) {
    return launch<uint16_t, uint16_t>(p, plan, x, B, C, CB, G2, DT, D, H, y, stream, ev);
}

}  // namespace k4
}  // namespace ssd

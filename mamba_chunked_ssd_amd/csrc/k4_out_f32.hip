// k4_out_f32.hip -- stage 4 (chunk output) instantiated for fp32 inputs and an fp32 y, plus the stage-4 dispatch.
// The kernels and their documentation are in k4_chunk_out.h.
#include "k4_chunk_out.h"

namespace ssd {

hipError_t launch_chunk_out(const Problem &p, const Plan &plan, const void *x, const void *B,
                            const void *C, const float *CB, G2View G2, const float *DT, const float *D,
                            const float *H, void *y, hipStream_t stream, const LaunchEvents &ev) {
    if (!p.bf16) return k4::launch<float, float>(p, plan, x, B, C, CB, G2, DT, D, H, y, stream, ev);
    if (p.y_bf16) return k4::launch_bf16_in_bf16_out(p, plan, x, B, C, CB, G2, DT, D, H, y, stream, ev);
    return k4::launch_bf16_in_f32_out(p, plan, x, B, C, CB, G2, DT, D, H, y, stream, ev);
}

}  // namespace ssd

// kb_pass_b.hip -- the dB pass of the backward pass, the sums of W and the
// decayed score tiles of fp32 problems (kb_pass.h, passes B, W and P).
#include "kb_pass_inst.h"

namespace ssd {
namespace bwd {

hipError_t launch_pass_b(const PassArgs &a, bool bf16, int dv, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev) {
    if (bf16) return launch_bc<uint16_t, kPassB>(a, dv, blocks, lds, stream, ev);
    return launch_bc<float, kPassB>(a, dv, blocks, lds, stream, ev);
}

hipError_t launch_pass_w(const PassArgs &a, bool bf16, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev) {
    switch (a.P) {
        case 32:
            return bf16 ? launch_one<uint16_t, 1, 16, kPassW>(a, blocks, lds, stream, ev)
                        : launch_one<float, 1, 16, kPassW>(a, blocks, lds, stream, ev);
        case 64:
            return bf16 ? launch_one<uint16_t, 2, 16, kPassW>(a, blocks, lds, stream, ev)
                        : launch_one<float, 2, 16, kPassW>(a, blocks, lds, stream, ev);
        case 128:
            return bf16 ? launch_one<uint16_t, 4, 16, kPassW>(a, blocks, lds, stream, ev)
                        : launch_one<float, 4, 16, kPassW>(a, blocks, lds, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pass_p(const PassArgs &a, unsigned blocks, size_t lds, hipStream_t stream, const LaunchEvents &ev) {
    switch (a.P) {
        case 32: return launch_one<float, 1, 16, kPassP>(a, blocks, lds, stream, ev);
        case 64: return launch_one<float, 2, 16, kPassP>(a, blocks, lds, stream, ev);
        case 128: return launch_one<float, 4, 16, kPassP>(a, blocks, lds, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bwd
}  // namespace ssd

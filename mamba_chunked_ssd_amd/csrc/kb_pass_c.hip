// kb_pass_c.hip -- the dC pass of the backward pass (kb_pass.h, pass C).
#include "kb_pass_inst.h"

namespace ssd {
namespace bwd {

hipError_t launch_pass_c(const PassArgs &a, bool bf16, int dv, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev) {
    if (bf16) return launch_bc<uint16_t, kPassC>(a, dv, blocks, lds, stream, ev);
    return launch_bc<float, kPassC>(a, dv, blocks, lds, stream, ev);
}

}  // namespace bwd
}  // namespace ssd

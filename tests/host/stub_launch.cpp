// Stub stage launchers for the host-only sanitizer builds of ssd_api.cpp: each
// records that it was called and enqueues nothing, so the C ABI's host logic
// (validation, workspace layout, plans, stage order) runs under ASan, UBSan
// and TSan on a machine without a GPU.  Not part of the library.
#include <hip/hip_runtime_api.h>

#include <atomic>

#include "../../mamba_chunked_ssd_amd/csrc/ssd_internal.h"

std::atomic<long> g_launches[5];  // calls per stage (4: the decode step)
std::atomic<long> g_bwd_launches;  // backward-only kernels
std::atomic<long> g_event_records;

namespace ssd {

hipError_t launch_chunk_cumsum(const Problem &, const void *, const float *, G2Pair, float *, float *,
                               hipStream_t, const LaunchEvents &, float *) {
    g_launches[0]++;
    return hipSuccess;
}
hipError_t launch_chunk_state(const Problem &, const Plan &, const void *, const void *, const float *,
                              float *, hipStream_t, const LaunchEvents &) {
    g_launches[1]++;
    return hipSuccess;
}
int chunk_state_blocks_per_cu(const Problem &p) { return p.bf16 ? 1 : 2; }
hipError_t launch_state_pass(const Problem &, const float *, float *, G2View, const float *, float *,
                             const void *, const void *, float *, hipStream_t, const LaunchEvents &) {
    g_launches[2]++;
    return hipSuccess;
}
bool state_fused_supported(const Problem &p, int cols) {
    return p.bf16 && (cols == 32 || cols == 64) && p.dstate % cols == 0;
}
hipError_t launch_state_fused(const Problem &, const Plan &, const void *, const void *, const float *,
                              G2View, const float *, float *, float *, const void *, float *, hipStream_t,
                              const LaunchEvents &) {
    g_launches[1]++;
    return hipSuccess;
}
hipError_t launch_decode_step(const Problem &, const void *, const void *, const float *, const void *,
                              const void *, const float *, float *, void *, hipStream_t, const LaunchEvents &) {
    g_launches[4]++;
    return hipSuccess;
}
hipError_t launch_chunk_out(const Problem &, const Plan &, const void *, const void *, const void *,
                            const float *, G2View, const float *, const float *, const float *, void *,
                            hipStream_t, const LaunchEvents &) {
    g_launches[3]++;
    return hipSuccess;
}

hipError_t launch_bwd_scores(const Problem &, const void *, const void *, float *, hipStream_t,
                             const LaunchEvents &) {
    g_bwd_launches++;
    return hipSuccess;
}
hipError_t launch_bwd_carry(const Problem &, const float *, const void *, G2View, const float *, void *, float *,
                            float *, hipStream_t, const LaunchEvents &) {
    g_bwd_launches++;
    return hipSuccess;
}
// the LDS rule of the pass kernels: tables, K (pass 4, and passes 1-3 of bf16
// problems), the W sums' parts (pass 3), V, state tile
size_t bwd_pass_lds(const Problem &p, int pass, int dv, int pad, bool xt) {
    const int64_t esz = p.bf16 ? 2 : 4;
    const int64_t T = p.chunk, P = p.headdim;
    int64_t bytes = 16 * T;
    if (pass == 4 || (pass != 0 && p.bf16)) bytes += T * (P + pad) * esz;
    if (pass == 3) bytes += 8 * T * (T / 32 + 1);
    if (pass == 3 || pass == 4) return bytes <= (int64_t)kLdsPerCu ? (size_t)bytes : 0;
    bytes += T * (dv + pad) * esz;
    const int64_t erow = pass == 0 ? (p.dstate + 31) / 32 * 32 + pad : dv + pad;
    bytes += (pass == 0 ? dv : P) * erow * 4;
    if (xt && (pass == 0 || pass == 2)) bytes += T * (dv + pad) * esz;
    return bytes <= (int64_t)kLdsPerCu ? (size_t)bytes : 0;
}
hipError_t launch_bwd_pass(const Problem &, const BwdPassLaunch &, hipStream_t, const LaunchEvents &) {
    g_bwd_launches++;
    return hipSuccess;
}
int bwd_pass_blocks_per_cu(const Problem &, const BwdPassLaunch &) { return 0; }
hipError_t launch_bwd_tokens(const Problem &, const BwdTokens &, const float *, const float *, const float *, float *,
                             float *, float *, hipStream_t, const LaunchEvents &) {
    g_bwd_launches++;
    return hipSuccess;
}
hipError_t launch_bwd_reduce(const Problem &, const float *, const float *, int, float *, float *, const float *,
                             const float *, float *, float *, hipStream_t, const LaunchEvents &) {
    g_bwd_launches++;
    return hipSuccess;
}

}  // namespace ssd

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
    g_event_records++;
    return hipSuccess;
}

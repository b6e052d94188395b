// ssd_tune.cpp -- ssd_chunk_scan_fwd_tune: a per-shape autotuner over launch
// plans (declared in include/ssd.h).
//
// The pages credit per-shape tuning of the kernels' tile configurations as
// one of the optimisations of the forward pass ("Kernel shorts: Mamba-2 in
// cuTile, CompileIQ + Helion, Deepgram on Trainium2", TL;DR; the video
// description "Mamba-2 en Python con CUDA Tile", chapter on the four
// optimisations).  Here the tunable choices are those of ssd_plan: heads per
// block of the chunk-output launch, the state path (split or fused) with its
// heads per block or dstate columns per block.  The tuner runs the caller's
// own problem under each candidate on the caller's stream, times each stage
// with events recorded by the kernels' own dispatches, and keeps the fastest.
// The chunk output's time does not depend on the state path, so the two are
// tuned one after the other (candidates add, they do not multiply).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/ssd.h"

namespace {

// Heads-per-block candidates for `hpg` heads per group: a geometric-ish set
// and hpg itself, one per distinct number of blocks per group (the smallest
// heads per block giving that count).
std::vector<int> head_candidates(int64_t hpg) {
    static const int kBase[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32, 40, 48, 64, 80, 96, 128};
    std::vector<int> out;
    std::vector<int64_t> seen;
    auto add = [&](int64_t hb) {
        if (hb < 1 || hb > hpg) return;
        const int64_t nhb = (hpg + hb - 1) / hb;
        if (std::find(seen.begin(), seen.end(), nhb) != seen.end()) return;
        seen.push_back(nhb);
        out.push_back((int)hb);
    };
    for (int hb : kBase) add(hb);
    add(hpg);
    return out;
}

struct Events {
    hipEvent_t ev[8] = {};
    bool ok = true;
    Events() {
        for (auto &e : ev)
            if (hipEventCreate(&e) != hipSuccess) {
                e = nullptr;
                ok = false;
            }
    }
    ~Events() {
        for (auto &e : ev)
            if (e != nullptr) hipEventDestroy(e);
    }
};

float median(std::vector<float> v) {
    std::sort(v.begin(), v.end());
    return v.empty() ? 0.f : v[v.size() / 2];
}

}  // namespace

extern "C" ssd_status ssd_chunk_scan_fwd_tune(const ssd_shape *shape, const void *x, const void *dt,
                                              const float *A, const void *B, const void *C, const float *D,
                                              int64_t chunk_size, const float *initial_states, void *y,
                                              float *final_states, void *workspace, size_t workspace_bytes,
                                              void *stream, int reps, ssd_plan *best, float *best_us) {
    if (best == nullptr || reps < 1 || reps > 1000) return SSD_ERROR_INVALID_VALUE;
    ssd_plan base;
    ssd_status st = ssd_chunk_scan_fwd_default_plan(shape, chunk_size, &base);
    if (st != SSD_OK) return st;
    // the initial state may alias the final state: the candidates would then
    // read each other's results, so tuning needs them apart
    if (initial_states != nullptr && (const void *)initial_states == (const void *)final_states)
        return SSD_ERROR_INVALID_VALUE;
    const int64_t hpg = shape->nheads / shape->ngroups;
    hipStream_t s = static_cast<hipStream_t>(stream);

    Events E;
    if (!E.ok) return SSD_ERROR_LAUNCH;
    // runs `plan` once untimed, then `reps` times with stage events; returns
    // the median time of each stage in microseconds (stage_us[4])
    auto measure = [&](const ssd_plan &plan, float *stage_us) -> ssd_status {
        ssd_status r = ssd_chunk_scan_fwd_ex(shape, x, dt, A, B, C, D, chunk_size, initial_states, y,
                                             final_states, workspace, workspace_bytes, stream, &plan, nullptr);
        if (r != SSD_OK) return r;
        std::vector<float> t[4];
        for (int i = 0; i < reps; ++i) {
            r = ssd_chunk_scan_fwd_ex(shape, x, dt, A, B, C, D, chunk_size, initial_states, y, final_states,
                                      workspace, workspace_bytes, stream, &plan,
                                      reinterpret_cast<void *const *>(E.ev));
            if (r != SSD_OK) return r;
            if (hipStreamSynchronize(s) != hipSuccess) return SSD_ERROR_LAUNCH;
            for (int k = 0; k < 4; ++k) {
                float ms = 0.f;
                if (hipEventElapsedTime(&ms, E.ev[2 * k], E.ev[2 * k + 1]) != hipSuccess) return SSD_ERROR_LAUNCH;
                t[k].push_back(ms * 1000.f);
            }
        }
        for (int k = 0; k < 4; ++k) stage_us[k] = median(t[k]);
        return SSD_OK;
    };

    // 1. chunk output: heads per block
    ssd_plan plan = base;
    float best_out = 0.f;
    bool first = true;
    for (int hb : head_candidates(hpg)) {
        ssd_plan c = base;
        c.chunk_out_heads = hb;
        float us[4];
        st = measure(c, us);
        if (st != SSD_OK) return st;
        if (first || us[3] < best_out) {
            best_out = us[3];
            plan.chunk_out_heads = hb;
            first = false;
        }
    }
    // 2. the state stages: split with each chunk-state heads per block, fused
    //    with each supported column count
    float best_state = 0.f;
    first = true;
    std::vector<ssd_plan> cands;
    for (int hb : head_candidates(hpg)) {
        ssd_plan c = plan;
        c.state_path = SSD_STATE_SPLIT;
        c.chunk_state_heads = hb;
        cands.push_back(c);
    }
    for (int cols : {32, 64}) {
        ssd_plan c = plan;
        c.state_path = SSD_STATE_FUSED;
        c.fused_cols = cols;
        uint32_t mask = 0;
        if (ssd_chunk_scan_fwd_stage_launches(shape, chunk_size, &c, &mask) == SSD_OK) cands.push_back(c);
    }
    ssd_plan chosen = plan;
    for (const ssd_plan &c : cands) {
        float us[4];
        st = measure(c, us);
        if (st != SSD_OK) return st;
        const float t = us[1] + us[2];  // chunk state (or the fused launch) + state passing
        if (first || t < best_state) {
            best_state = t;
            chosen = c;
            first = false;
        }
    }
    // 3. the chosen plan once more, so the outputs hold its result, and its time
    float us[4];
    st = measure(chosen, us);
    if (st != SSD_OK) return st;
    *best = chosen;
    if (best_us != nullptr) *best_us = us[0] + us[1] + us[2] + us[3];
    return SSD_OK;
}

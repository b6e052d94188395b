// ssd_bwd.cpp -- ssd_chunk_scan_bwd (declared in include/ssd.h): argument
// validation, the backward workspace layout, the launch plan and the stage
// order.  Host code only; validation touches no HIP API.
//
// Stages (the kernels are described where they are defined):
//   0-2   the forward's cumsum (plus the adjoint weights exp(G)), chunk
//         states and state passing, recomputed: the chunk-start states h_c
//         and the final state (with a forward call's kept states, stage 0
//         only, h_c read from that call's workspace);
//   3     u_c = sum_r exp(G_r) dy_r C_r^T with the forward's chunk-state
//         kernel (dy as x, C as B);
//   4     the reverse carry of the state gradient (kb_aux.hip);
//   5     the per-group score tiles B_r . C_s (kb_aux.hip) and, for fp32
//         problems, each head's decayed x . dy tiles (kb_pass.h, pass P);
//   6-9   the dx, dB and dC passes and the sums of W (kb_pass.h);
//   10-11 ddt and the reductions of dB, dC, dA, dD (kb_aux.hip).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <limits>

#include "../../include/ssd.h"
#include "ssd_host.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

enum { kPassQ = 0, kPassB = 1, kPassC = 2, kPassW = 3, kPassP = 4 };

struct BwdPlan {
    int dvq, padq;    // dx pass: headdim columns per block, LDS row padding
    int dvb, padb;    // dB pass: dstate columns per block, padding
    int dvc, padc;    // dC pass: dstate columns per block, padding
    int hb, nhb;      // dB and dC passes: heads per block, runs of heads per group
    int nvtq;         // dx pass: column tiles (headdim / dvq)
};

struct BwdLayout {
    size_t g2_hi, g2_lo, dt, w, wb, s, h, e, zp, st, pt, ptt, xq, xqi, dyx, cdi, wd, dbp, dcp, dap, ddp, total;
};

bool make_bwd_plan(const Problem &p, BwdPlan *out) {
    BwdPlan q;
    q.dvq = (int)std::min<int64_t>(p.headdim, 64);
    q.padq = bwd_pass_lds(p, kPassQ, q.dvq, 8) != 0 ? 8 : 0;
    if (bwd_pass_lds(p, kPassQ, q.dvq, q.padq) == 0) return false;
    // A block of at most four waves (one per SIMD: fp32 inputs at chunk 128
    // or less) whose headdim tile leaves LDS for one block per CU takes
    // 32-column tiles where two blocks then fit: twice the waves per SIMD for
    // one more pass over the score tiles (fp32 headdim 128, dstate 256,
    // chunk 128: dx pass 12.0 -> 9.2 ms).
    if (q.dvq == 64 && kb_pass_waves(p, kPassQ) <= 4) {
        const size_t wide = bwd_pass_lds(p, kPassQ, 64, q.padq);
        const int pad32 = bwd_pass_lds(p, kPassQ, 32, 8) != 0 ? 8 : 0;
        const size_t narrow = bwd_pass_lds(p, kPassQ, 32, pad32);
        if (narrow != 0 && kLdsPerCu / narrow > kLdsPerCu / wide) {
            q.dvq = 32;
            q.padq = pad32;
        }
    }
    q.nvtq = (int)(p.headdim / q.dvq);
    // widest dstate tile each pass's registers and one CU's LDS hold
    auto widest = [&](int pass, int *dv_out, int *pad_out) {
        for (int dv : {64, 32, 16}) {
            if (!bwd_dv_ok(p.bf16, p.headdim, dv) || p.dstate % dv != 0) continue;
            for (int pad : {8, 0}) {
                if (bwd_pass_lds(p, pass, dv, pad) != 0) {
                    *dv_out = dv;
                    *pad_out = pad;
                    return true;
                }
            }
        }
        return false;
    };
    if (!widest(kPassB, &q.dvb, &q.padb) || !widest(kPassC, &q.dvc, &q.padc)) return false;
    // heads per block of passes B and C: each block stages its group's V tile
    // once and then one head after another; the partial sums it leaves per
    // run of heads cost memory traffic.  One block per CU (LDS), 256 CUs:
    // the smallest makespan in rounds x (heads + 1), fewest runs on ties.
    const int64_t base = p.batch * p.nchunks * p.ngroups * (p.dstate / q.dvb);
    const int64_t hpg = p.heads_per_group;
    const int64_t slots = 256 * std::max<int64_t>(1, (int64_t)(kLdsPerCu / bwd_pass_lds(p, kPassB, q.dvb, q.padb)));
    double best = std::numeric_limits<double>::max();
    int best_hb = (int)hpg;
    for (int64_t hb = hpg; hb >= 1; --hb) {
        const int64_t nhb = (hpg + hb - 1) / hb;
        const int64_t blocks = base * nhb;
        const double rounds = (double)((blocks + slots - 1) / std::max<int64_t>(slots, 1));
        const double cost = rounds * ((double)hb + 1.0);
        if (cost < best - 1e-9) {
            best = cost;
            best_hb = (int)hb;
        }
    }
    q.hb = best_hb;
    q.nhb = (int)((hpg + best_hb - 1) / best_hb);
    *out = q;
    return true;
}

BwdLayout bwd_layout(const Problem &p, const BwdPlan &q) {
    BwdLayout l;
    std::memset(&l, 0, sizeof(l));
    const size_t seq = (size_t)p.batch * p.nheads * p.padded_len * sizeof(float);
    const size_t states = (size_t)p.batch * p.nheads * p.nchunks * p.headdim * p.dstate * sizeof(float);
    const int64_t n = p.chunk / 16;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    l.g2_hi = take(seq);
    l.g2_lo = take(seq);
    l.dt = take(seq);
    l.w = take(seq);
    l.wb = take(seq);
    l.s = take(states);  // chunk states s_c, then the adjoint terms u_c
    l.h = take(states);
    l.e = take(states);
    l.zp = take((size_t)p.batch * p.nheads * p.nchunks * (p.headdim * p.dstate / 256) * sizeof(float));
    l.st = take((size_t)p.batch * p.nchunks * p.ngroups * (n * (n + 1) / 2) * 256 * sizeof(float));
    // fp32 problems: every head's decayed score tiles (kb_pass.h, pass P)
    l.pt = take(p.bf16 ? 0 : (size_t)p.batch * p.nheads * p.nchunks * (n * (n + 1) / 2) * 256 * sizeof(float));
    l.ptt = take(p.bf16 ? 0 : (size_t)p.batch * p.nheads * p.nchunks * (n * (n + 1) / 2) * 256 * sizeof(float));
    const size_t tok = (size_t)p.batch * p.nheads * p.padded_len * sizeof(float);
    l.xq = take(tok * q.nvtq);
    l.xqi = take(tok * q.nvtq);
    l.dyx = take(tok * q.nvtq);
    l.cdi = take(tok * (p.dstate / q.dvc));
    l.wd = take(tok * 2);  // doubles
    const size_t part = (size_t)q.nhb * p.batch * p.padded_len * p.ngroups * p.dstate * sizeof(float);
    l.dbp = take(part);
    l.dcp = take(part);
    l.dap = take((size_t)p.batch * p.nchunks * p.nheads * sizeof(float));
    l.ddp = take((size_t)p.batch * p.nchunks * p.nheads * sizeof(float));
    l.total = off;
    return l;
}

ssd_status prepare(const ssd_shape *shape, int64_t chunk, Problem *p, BwdPlan *q, BwdLayout *l) {
    ssd_status st = check_shape(shape, chunk, p);
    if (st != SSD_OK) return st;
    if (shape->flags != 0) return SSD_ERROR_INVALID_VALUE;
    if (!make_bwd_plan(*p, q)) return SSD_ERROR_UNSUPPORTED;
    if (bwd_pass_lds(*p, kPassW, 16, 0) == 0) return SSD_ERROR_UNSUPPORTED;
    if (!p->bf16 && bwd_pass_lds(*p, kPassP, 16, 0) == 0) return SSD_ERROR_UNSUPPORTED;
    // the passes address one chunk's rows of dy / x / B / C with 32-bit
    // LDS-sized loops and int block counts
    if (p->batch * p->nchunks * p->ngroups * q->nhb * (p->dstate / std::min(q->dvb, q->dvc)) > 0x7fffffff)
        return SSD_ERROR_UNSUPPORTED;
    *l = bwd_layout(*p, *q);
    return SSD_OK;
}

ssd_status backward(const ssd_shape *shape, const void *x, const void *dt, const float *A, const void *B,
                    const void *C, const float *D, int64_t chunk_size, const float *init, const void *dy,
                    const float *dfinal, float *dx, float *ddt, float *dA, float *dB, float *dC,
                    float *dD, float *dinit, void *workspace, size_t workspace_bytes, const void *fwd_ws,
                    size_t fwd_ws_bytes, void *stream_handle, void *const *events) {
    Problem p;
    BwdPlan q;
    BwdLayout lay;
    ssd_status st = prepare(shape, chunk_size, &p, &q, &lay);
    if (st != SSD_OK) return st;
    const size_t esz = p.bf16 ? 2 : 4;
    const size_t tok = (size_t)(p.batch * p.seqlen);
    const size_t x_elems = tok * p.nheads * p.headdim;
    const size_t dt_elems = tok * p.nheads;
    const size_t bc_elems = tok * p.ngroups * p.dstate;
    const size_t hd_bytes = (size_t)p.nheads * sizeof(float);
    const size_t st_bytes = (size_t)p.batch * p.nheads * p.headdim * p.dstate * sizeof(float);
    const bool has_tokens = tok > 0;

    if (has_tokens && (x == nullptr || dt == nullptr || B == nullptr || C == nullptr || dy == nullptr || dx == nullptr || ddt == nullptr || dB == nullptr || dC == nullptr))
        return SSD_ERROR_INVALID_VALUE;
    if (A == nullptr || dA == nullptr) return SSD_ERROR_INVALID_VALUE;
    if (lay.total > 0 && p.batch > 0 && workspace == nullptr) return SSD_ERROR_WORKSPACE;
    if (workspace_bytes < lay.total) return SSD_ERROR_WORKSPACE;
    // a forward call's kept intermediates: its chunk-start states h_c, at the
    // offset of the forward layout with SSD_FLAG_KEEP_INTERMEDIATES
    const unsigned char *saved_h = nullptr;
    size_t saved_h_bytes = 0;
    if (fwd_ws != nullptr) {
        ssd_shape keep = *shape;
        keep.flags = SSD_FLAG_KEEP_INTERMEDIATES;
        ssd_workspace_layout fl;
        if (ssd_chunk_scan_fwd_workspace_layout(&keep, chunk_size, &fl) != SSD_OK) return SSD_ERROR_INVALID_VALUE;
        if (fwd_ws_bytes < fl.total) return SSD_ERROR_WORKSPACE;
        if (!aligned(fwd_ws, kAlign)) return SSD_ERROR_MISALIGNED;
        saved_h = static_cast<const unsigned char *>(fwd_ws) + fl.h;
        saved_h_bytes = (size_t)p.batch * p.nheads * p.nchunks * p.headdim * p.dstate * sizeof(float);
    }
    if (events != nullptr)
        for (int i = 0; i < 2 * SSD_BWD_STAGES; ++i)
            if (events[i] == nullptr) return SSD_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(dy, 16) ||
        !aligned(dt, esz) || !aligned(A, 4) || !aligned(D, 4) || !aligned(init, 16) || !aligned(dfinal, 16) ||
        !aligned(dx, 16) || !aligned(ddt, 4) || !aligned(dA, 4) || !aligned(dB, 16) || !aligned(dC, 16) ||
        !aligned(dD, 4) || !aligned(dinit, 16) || !aligned(workspace, kAlign))
        return SSD_ERROR_MISALIGNED;

    const Range ins[] = {range_of(x, x_elems * esz),  range_of(dt, dt_elems * esz),
                         range_of(A, hd_bytes),       range_of(B, bc_elems * esz),
                         range_of(C, bc_elems * esz), range_of(D, D ? hd_bytes : 0),
                         range_of(init, init ? st_bytes : 0), range_of(dy, x_elems * esz), range_of(dfinal, dfinal ? st_bytes : 0),
                         range_of(saved_h, saved_h_bytes)};
    const Range outs[] = {range_of(dx, x_elems * 4),        range_of(ddt, dt_elems * 4),
                          range_of(dA, hd_bytes),           range_of(dB, bc_elems * 4),
                          range_of(dC, bc_elems * 4),       range_of(dD, dD ? hd_bytes : 0),
                          range_of(dinit, dinit ? st_bytes : 0), range_of(workspace, lay.total)};
    const int nouts = (int)(sizeof(outs) / sizeof(outs[0]));
    for (int i = 0; i < nouts; ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r)) return SSD_ERROR_INVALID_VALUE;
        for (int j = i + 1; j < nouts; ++j)
            if (overlap(outs[i], outs[j])) return SSD_ERROR_INVALID_VALUE;
    }

    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    auto events_of = [&](int i) {
        LaunchEvents ev;
        if (events != nullptr) {
            ev.start = static_cast<hipEvent_t>(events[2 * i]);
            ev.stop = static_cast<hipEvent_t>(events[2 * i + 1]);
        }
        return ev;
    };
    auto skip = [&](int i) -> bool {
        if (events == nullptr) return true;
        const LaunchEvents ev = events_of(i);
        return hipEventRecord(ev.start, stream) == hipSuccess && hipEventRecord(ev.stop, stream) == hipSuccess;
    };
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    auto fp = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
    const G2Pair G2{fp(lay.g2_hi), fp(lay.g2_lo)};
    const G2View G2v{G2.hi, G2.lo};
    float *DTf = fp(lay.dt);
    float *S = fp(lay.s);
    const void *Hs = saved_h != nullptr ? static_cast<const void *>(saved_h) : static_cast<const void *>(fp(lay.h));
    void *E = ws + lay.e;
    float *Zp = fp(lay.zp);

    const bool run = p.batch > 0 && p.nchunks > 0;
    if (run) {
        const Plan fplan = make_plan(p);
        if (launch_chunk_cumsum(p, dt, A, G2, DTf, fp(lay.w), stream, events_of(0), fp(lay.wb)) != hipSuccess)
            return SSD_ERROR_LAUNCH;
        if (saved_h == nullptr) {
            if (launch_chunk_state(p, fplan, x, B, fp(lay.w), S, stream, events_of(1)) != hipSuccess)
                return SSD_ERROR_LAUNCH;
            if (launch_state_pass(p, S, fp(lay.h), G2v, init, nullptr, B, C, nullptr, stream, events_of(2)) !=
                hipSuccess)
                return SSD_ERROR_LAUNCH;
        } else if (!skip(1) || !skip(2)) {
            return SSD_ERROR_LAUNCH;
        }
        // u_c into S's region (s_c has been consumed)
        if (launch_chunk_state(p, fplan, dy, C, fp(lay.wb), S, stream, events_of(3)) != hipSuccess)
            return SSD_ERROR_LAUNCH;
    } else if (!skip(0) || !skip(1) || !skip(2) || !skip(3)) {
        return SSD_ERROR_LAUNCH;
    }
    // the carry also turns d_final_states into d_initial_states when there is no chunk
    if (p.batch > 0) {
        if (launch_bwd_carry(p, S, Hs, G2v, dfinal, E, Zp, dinit, stream, events_of(4)) != hipSuccess)
            return SSD_ERROR_LAUNCH;
    } else if (!skip(4)) {
        return SSD_ERROR_LAUNCH;
    }
    if (run) {
        BwdPassLaunch L;
        std::memset(&L, 0, sizeof(L));
        L.x = x;
        L.dy = dy;
        L.B = B;
        L.C = C;
        L.G2 = G2v;
        L.DT = DTf;
        L.E = E;
        L.H = Hs;
        L.ST = fp(lay.st);
        L.D = D;
        L.xq = fp(lay.xq);
        L.xqi = fp(lay.xqi);
        L.dyx = fp(lay.dyx);
        L.cdi = fp(lay.cdi);
        L.wd = reinterpret_cast<double *>(ws + lay.wd);
        L.pt = fp(lay.pt);
        // the dx and dC passes' epilogue tile (x or C) is staged in LDS where
        // it fits and costs the pass no block per CU (the runtime's occupancy
        // from the kernel's registers and LDS); else it is read from memory
        auto xt_pays = [&](BwdPassLaunch Lx) {
            Lx.xt_lds = 1;
            if (bwd_pass_lds(p, Lx.pass, Lx.dv, Lx.lds_pad, true) == 0) return false;
            const int with = bwd_pass_blocks_per_cu(p, Lx);
            Lx.xt_lds = 0;
            const int without = bwd_pass_blocks_per_cu(p, Lx);
            return with == 0 || without == 0 || with >= without;
        };
        L.ptt = fp(lay.ptt);
        // stage 5: the score tiles B . C per group, and for fp32 problems the
        // decayed x . dy tiles per head (the stage's events span both launches)
        {
            const LaunchEvents ev5 = events_of(5);
            if (p.bf16) {
                if (launch_bwd_scores(p, B, C, fp(lay.st), stream, ev5) != hipSuccess) return SSD_ERROR_LAUNCH;
            } else {
                if (launch_bwd_scores(p, B, C, fp(lay.st), stream, LaunchEvents{ev5.start, nullptr}) != hipSuccess)
                    return SSD_ERROR_LAUNCH;
                L.pass = kPassP;
                L.out = nullptr;
                L.dv = 16;
                L.hb = 1;
                L.lds_pad = bwd_pass_lds(p, kPassP, 16, 8) != 0 ? 8 : 0;
                L.xt_lds = 0;
                if (launch_bwd_pass(p, L, stream, LaunchEvents{nullptr, ev5.stop}) != hipSuccess)
                    return SSD_ERROR_LAUNCH;
            }
        }
        L.pass = kPassQ;
        L.out = dx;
        L.dv = q.dvq;
        L.hb = 1;
        L.lds_pad = q.padq;
        L.xt_lds = xt_pays(L) ? 1 : 0;
        if (launch_bwd_pass(p, L, stream, events_of(6)) != hipSuccess) return SSD_ERROR_LAUNCH;
        L.pass = kPassB;
        L.out = fp(lay.dbp);
        L.dv = q.dvb;
        L.hb = q.hb;
        L.lds_pad = q.padb;
        L.xt_lds = 0;
        if (launch_bwd_pass(p, L, stream, events_of(7)) != hipSuccess) return SSD_ERROR_LAUNCH;
        L.pass = kPassC;
        L.out = fp(lay.dcp);
        L.dv = q.dvc;
        L.lds_pad = q.padc;
        L.xt_lds = xt_pays(L) ? 1 : 0;
        if (launch_bwd_pass(p, L, stream, events_of(8)) != hipSuccess) return SSD_ERROR_LAUNCH;
        L.pass = kPassW;
        L.out = nullptr;
        L.dv = 16;
        L.hb = 1;
        L.lds_pad = bwd_pass_lds(p, kPassW, 16, 8) != 0 ? 8 : 0;
        L.xt_lds = 0;
        if (launch_bwd_pass(p, L, stream, events_of(9)) != hipSuccess) return SSD_ERROR_LAUNCH;
        const BwdTokens tk{fp(lay.xq), fp(lay.xqi), fp(lay.dyx), fp(lay.cdi),
                           reinterpret_cast<const double *>(ws + lay.wd), q.nvtq, (int)(p.dstate / q.dvc)};
        if (launch_bwd_tokens(p, tk, DTf, Zp, A, ddt, fp(lay.dap), fp(lay.ddp), stream, events_of(10)) != hipSuccess)
            return SSD_ERROR_LAUNCH;
    } else if (!skip(5) || !skip(6) || !skip(7) || !skip(8) || !skip(9) || !skip(10)) {
        return SSD_ERROR_LAUNCH;
    }
    // dA and dD are written even with no tokens (as zeros)
    if (launch_bwd_reduce(p, fp(lay.dbp), fp(lay.dcp), q.nhb, dB, dC, fp(lay.dap), fp(lay.ddp), dA, dD, stream,
                          events_of(11)) != hipSuccess)
        return SSD_ERROR_LAUNCH;
    return SSD_OK;
}

}  // namespace
}  // namespace ssd

using namespace ssd;

extern "C" {

size_t ssd_chunk_scan_bwd_workspace_size(const ssd_shape *shape, int64_t chunk_size) {
    Problem p;
    BwdPlan q;
    BwdLayout l;
    if (prepare(shape, chunk_size, &p, &q, &l) != SSD_OK) return 0;
    return l.total;
}

ssd_status ssd_chunk_scan_bwd(const ssd_shape *shape, const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, int64_t chunk_size, const float *initial_states,
                              const void *dy, const float *d_final_states, float *dx, float *ddt,
                              float *dA, float *dB, float *dC, float *dD, float *d_initial_states, void *workspace,
                              size_t workspace_bytes, void *stream) {
    return backward(shape, x, dt, A, B, C, D, chunk_size, initial_states, dy, d_final_states, dx, ddt, dA, dB, dC,
                    dD, d_initial_states, workspace, workspace_bytes, nullptr, 0, stream, nullptr);
}

ssd_status ssd_chunk_scan_bwd_profiled(const ssd_shape *shape, const void *x, const void *dt, const float *A,
                                       const void *B, const void *C, const float *D, int64_t chunk_size,
                                       const float *initial_states, const void *dy, const float *d_final_states, float *dx, float *ddt, float *dA, float *dB,
                                       float *dC, float *dD, float *d_initial_states, void *workspace,
                                       size_t workspace_bytes, void *stream, void *const *stage_events) {
    if (stage_events == nullptr) return SSD_ERROR_INVALID_VALUE;
    return backward(shape, x, dt, A, B, C, D, chunk_size, initial_states, dy, d_final_states, dx, ddt, dA, dB, dC,
                    dD, d_initial_states, workspace, workspace_bytes, nullptr, 0, stream, stage_events);
}

ssd_status ssd_chunk_scan_bwd_saved(const ssd_shape *shape, const void *x, const void *dt, const float *A,
                                    const void *B, const void *C, const float *D, int64_t chunk_size,
                                    const float *initial_states, const void *dy, const float *d_final_states,
                                    const void *fwd_workspace, size_t fwd_workspace_bytes, float *dx, float *ddt,
                                    float *dA, float *dB, float *dC, float *dD, float *d_initial_states,
                                    void *workspace, size_t workspace_bytes, void *stream, void *const *stage_events) {
    if (fwd_workspace == nullptr) return SSD_ERROR_INVALID_VALUE;
    return backward(shape, x, dt, A, B, C, D, chunk_size, initial_states, dy, d_final_states, dx, ddt, dA, dB, dC,
                    dD, d_initial_states, workspace, workspace_bytes, fwd_workspace, fwd_workspace_bytes, stream,
                    stage_events);
}

}  // extern "C"

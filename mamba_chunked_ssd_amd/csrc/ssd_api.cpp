// ssd_api.cpp -- the C ABI of libssd (declared in include/ssd.h).
//
// Host side only: argument validation, workspace layout, the per-shape launch
// plan, and the four stage launches on the caller's stream ("Accelerating
// Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile": the
// three-kernel split of the forward pass listed at the end of section "Mamba-2
// architecture", with the state stage split in two: the parallel per-chunk
// contraction and the sequential carry).  Validation touches no HIP API, so
// every error path runs without a device.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <limits>

#include "../../include/ssd.h"
#include "ssd_host.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int64_t kMaxI32 = std::numeric_limits<int32_t>::max();

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
    *out = a * b;
    return true;
}

bool chunk_supported(int64_t t) { return t == 64 || t == 128 || t == 256; }
bool headdim_supported(int64_t p) { return p == 32 || p == 64 || p == 128; }
bool dstate_supported(int64_t n) { return n >= 16 && n <= 256 && n % 16 == 0; }

}  // namespace

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Shape checks shared by the size queries, the forward and the backward call.
ssd_status check_shape(const ssd_shape *s, int64_t chunk, Problem *p) {
    if (s == nullptr) return SSD_ERROR_INVALID_VALUE;
    if (s->batch < 0 || s->seqlen < 0 || s->nheads < 1 || s->headdim < 1 || s->dstate < 1 ||
        s->ngroups < 1 || chunk < 1)
        return SSD_ERROR_INVALID_VALUE;
    if (s->nheads % s->ngroups != 0) return SSD_ERROR_INVALID_VALUE;
    if (s->dtype != SSD_DTYPE_F32 && s->dtype != SSD_DTYPE_BF16) return SSD_ERROR_INVALID_VALUE;
    if (s->y_dtype != SSD_DTYPE_F32 && s->y_dtype != s->dtype) return SSD_ERROR_INVALID_VALUE;
    if (s->reserved != 0) return SSD_ERROR_INVALID_VALUE;
    if ((s->flags & ~(uint32_t)SSD_FLAG_KEEP_INTERMEDIATES) != 0) return SSD_ERROR_INVALID_VALUE;
    if (!chunk_supported(chunk) || !headdim_supported(s->headdim) || !dstate_supported(s->dstate))
        return SSD_ERROR_UNSUPPORTED;

    Problem q;
    q.batch = s->batch;
    q.seqlen = s->seqlen;
    q.nheads = s->nheads;
    q.headdim = s->headdim;
    q.dstate = s->dstate;
    q.ngroups = s->ngroups;
    q.chunk = chunk;
    q.nchunks = (s->seqlen + chunk - 1) / chunk;
    q.padded_len = q.nchunks * chunk;
    q.heads_per_group = s->nheads / s->ngroups;
    q.bf16 = s->dtype == SSD_DTYPE_BF16;
    q.y_bf16 = s->y_dtype == SSD_DTYPE_BF16;

    // Every element count must fit int64; kernel-side scalar parameters fit int32.
    int64_t t, e;
    if (!mul_ok(q.batch, q.seqlen, &t) || !mul_ok(t, q.nheads, &e) || !mul_ok(e, q.headdim, &e))
        return SSD_ERROR_UNSUPPORTED;
    if (!mul_ok(t, q.ngroups, &e) || !mul_ok(e, q.dstate, &e)) return SSD_ERROR_UNSUPPORTED;
    int64_t st;
    if (!mul_ok(q.batch, q.nheads, &st) || !mul_ok(st, q.nchunks, &st) ||
        !mul_ok(st, q.headdim * q.dstate, &st) || st > std::numeric_limits<int64_t>::max() / 8)
        return SSD_ERROR_UNSUPPORTED;
    if (q.nheads > kMaxI32 || q.nchunks > kMaxI32 || q.ngroups > kMaxI32 || q.batch > 65535)
        return SSD_ERROR_UNSUPPORTED;
    // The chunk output stage addresses one chunk's y rows, and the state
    // stages one chunk's B rows, with 32-bit byte offsets.
    if (q.chunk * q.nheads * q.headdim * 4 > kMaxI32) return SSD_ERROR_UNSUPPORTED;
    if (q.chunk * q.ngroups * q.dstate * 4 > kMaxI32) return SSD_ERROR_UNSUPPORTED;
    // Launch geometry limits (work-items per grid dimension < 2^32).
    const int64_t tiles = q.batch * q.nchunks * q.ngroups * q.heads_per_group;  // upper bound on blocks
    if (tiles > ((int64_t)1 << 31) / 512) return SSD_ERROR_UNSUPPORTED;
    const int64_t k3_threads = q.batch * q.nheads * q.headdim * q.dstate / 4;
    if (k3_threads > ((int64_t)1 << 31)) return SSD_ERROR_UNSUPPORTED;
    if ((q.nheads + 3) / 4 > 65535) return SSD_ERROR_UNSUPPORTED;  // cumsum grid.y
    *p = q;
    return SSD_OK;
}

namespace {

ssd_workspace_layout layout_for(const Problem &p, bool keep) {
    ssd_workspace_layout l;
    std::memset(&l, 0, sizeof(l));
    const size_t seq = (size_t)p.batch * p.nheads * p.padded_len * sizeof(float);
    const size_t states = (size_t)p.batch * p.nheads * p.nchunks * p.headdim * p.dstate * sizeof(float);
    size_t off = 0;
    l.g2_hi = off;
    off = align_up(off + seq);
    l.g2_lo = off;
    off = align_up(off + seq);
    l.dt = off;
    off = align_up(off + seq);
    l.w = off;
    off = align_up(off + seq);
    l.s = off;
    off = align_up(off + states);
    // bf16 problems store h_c split into bf16 hi/lo planes, which cannot be
    // written in place over s_c; fp32 problems without the keep flag reuse S
    const bool own_h = keep || p.bf16;
    l.h = own_h ? off : l.s;
    if (own_h) off = align_up(off + states);
    l.cb = off;
    if (uses_cb_tiles(p))
        off = align_up(off + (size_t)p.batch * p.nchunks * p.ngroups * cb_slots(p.chunk) * 64 * 4 *
                                 sizeof(float));
    l.total = off;
    l.nchunks = p.nchunks;
    l.padded_len = p.padded_len;
    return l;
}


// Pick heads-per-block for a stage whose blocks each handle one (batch, chunk,
// group) and a run of heads: each block pays a fixed set-up cost (staging the
// shared B / C B^T tiles, ~`setup` head-equivalents) plus one unit per head,
// and `slots` blocks run concurrently.  Minimise the modelled makespan.
int pick_heads_per_block(const Problem &p, int64_t slots, double setup) {
    const int64_t base = p.batch * p.nchunks * p.ngroups;
    const int64_t hpg = p.heads_per_group;
    if (base == 0) return 1;
    double best = std::numeric_limits<double>::max();
    int best_hb = (int)hpg;
    for (int64_t hb = 1; hb <= hpg; ++hb) {
        const int64_t nhb = (hpg + hb - 1) / hb;
        if (hb > 1 && (hpg + hb - 2) / (hb - 1) == nhb) continue;  // same split as hb - 1
        const int64_t blocks = base * nhb;
        const double rounds = (double)((blocks + slots - 1) / slots);
        const double cost = rounds * ((double)hb + setup);
        if (cost < best - 1e-9) {
            best = cost;
            best_hb = (int)hb;
        }
    }
    return best_hb;
}

const int kNumCUs = 256;

}  // namespace

Plan make_plan(const Problem &p) {
    Plan plan;
    plan.k2_heads_per_block = pick_heads_per_block(p, chunk_state_blocks_per_cu(p) * kNumCUs, 1.0);
    plan.k4_heads_per_block = pick_heads_per_block(p, kNumCUs, 1.0);
    // The general bf16 chunk output at chunk 256 with dstate > 128 re-reads
    // the chunk's C rows (T x dstate bf16: 128 KiB at dstate 256) in every
    // head.  A chunk's blocks are consecutive, so they run at the same time on
    // one XCD; with at least four of them C is read from that XCD's L2 instead
    // of from memory for each head.  Measured on MI355X with that kernel
    // (65 536 tokens, 32 heads, headdim 64, dstate 256): 8 heads per block
    // 477-514 us against 521-540 us with 32.  The kernel with asynchronous
    // copies (uses_cb_tiles) keeps C in registers and needs no such cap.
    if (p.bf16 && p.chunk == 256 && p.dstate > 128 && p.heads_per_group >= 4 && !uses_cb_tiles(p))
        plan.k4_heads_per_block =
            std::min<int>(plan.k4_heads_per_block, (int)((p.heads_per_group + 3) / 4));
    // The fused state launch (bf16) walks the chunks of one (batch, head,
    // 64 dstate columns) per block in order: it saves the s_c round trip
    // through memory but keeps only that many blocks busy.  Measured on
    // MI355X it wins with two or more blocks per CU (8 x 4096 tokens: 1280
    // blocks, 281-300 us against 334-340 us for the two split launches),
    // is faster warm but slower cold with one to two (2.7B-shaped layer: 320
    // blocks, 77.5 against 79.4 us per forward pass with steps back to back,
    // 98-99 against 91-94 us summed over the stages from a cold cache) and
    // loses below (65 536 tokens, 32 heads, dstate 256: 128 blocks, 666 us
    // against 426 us).
    plan.fused_cols = 64;
    plan.fused_state = p.nchunks > 0 && state_fused_supported(p, 64) &&
                       p.batch * p.nheads * (p.dstate / 64) >= 2 * kNumCUs;
    if (!plan.fused_state) plan.fused_cols = (int)std::min<int64_t>(p.dstate, 64);
    return plan;
}

namespace {

// The fused state path: bf16 inputs, blocks of 32 or 64 dstate columns that
// divide dstate, at least half the headdim (state_fused_supported).
bool fused_cols_ok(const Problem &p, int64_t cols) {
    return cols >= 32 && cols % 32 == 0 && cols <= p.dstate && p.dstate % cols == 0;
}
bool fused_supported(const Problem &p, int cols) { return state_fused_supported(p, cols); }

ssd_plan to_abi(const Plan &q) {
    ssd_plan r;
    std::memset(&r, 0, sizeof(r));
    r.state_path = q.fused_state ? SSD_STATE_FUSED : SSD_STATE_SPLIT;
    r.chunk_state_heads = q.k2_heads_per_block;
    r.chunk_out_heads = q.k4_heads_per_block;
    r.fused_cols = q.fused_cols;
    return r;
}

// Check a caller's plan against the problem; NULL selects the default plan.
ssd_status plan_from_abi(const Problem &p, const ssd_plan *in, Plan *out) {
    if (in == nullptr) {
        *out = make_plan(p);
        return SSD_OK;
    }
    for (int i = 0; i < 4; ++i)
        if (in->reserved[i] != 0) return SSD_ERROR_INVALID_VALUE;
    if (in->state_path != SSD_STATE_SPLIT && in->state_path != SSD_STATE_FUSED)
        return SSD_ERROR_INVALID_VALUE;
    const int64_t hpg = p.heads_per_group;
    if (in->chunk_state_heads < 1 || in->chunk_state_heads > hpg || in->chunk_out_heads < 1 ||
        in->chunk_out_heads > hpg)
        return SSD_ERROR_INVALID_VALUE;
    const bool fused = in->state_path == SSD_STATE_FUSED;
    if (fused && !fused_cols_ok(p, in->fused_cols)) return SSD_ERROR_INVALID_VALUE;
    if (fused && !fused_supported(p, in->fused_cols)) return SSD_ERROR_UNSUPPORTED;
    Plan q;
    q.fused_state = fused;
    q.k2_heads_per_block = in->chunk_state_heads;
    q.k4_heads_per_block = in->chunk_out_heads;
    q.fused_cols = fused ? in->fused_cols : (int)p.dstate;
    *out = q;
    return SSD_OK;
}

}  // namespace
}  // namespace ssd

using namespace ssd;

extern "C" {

size_t ssd_chunk_scan_fwd_workspace_size(const ssd_shape *shape, int64_t chunk_size) {
    Problem p;
    if (check_shape(shape, chunk_size, &p) != SSD_OK) return 0;
    return layout_for(p, (shape->flags & SSD_FLAG_KEEP_INTERMEDIATES) != 0).total;
}

ssd_status ssd_chunk_scan_fwd_workspace_layout(const ssd_shape *shape, int64_t chunk_size,
                                               ssd_workspace_layout *layout) {
    if (layout == nullptr) return SSD_ERROR_INVALID_VALUE;
    Problem p;
    const ssd_status st = check_shape(shape, chunk_size, &p);
    if (st != SSD_OK) return st;
    *layout = layout_for(p, (shape->flags & SSD_FLAG_KEEP_INTERMEDIATES) != 0);
    return SSD_OK;
}

ssd_status ssd_chunk_scan_fwd_default_plan(const ssd_shape *shape, int64_t chunk_size, ssd_plan *plan) {
    if (plan == nullptr) return SSD_ERROR_INVALID_VALUE;
    Problem p;
    const ssd_status st = check_shape(shape, chunk_size, &p);
    if (st != SSD_OK) return st;
    *plan = to_abi(make_plan(p));
    return SSD_OK;
}

static ssd_status forward(const ssd_shape *shape, const void *x, const void *dt, const float *A,
                          const void *B, const void *C, const float *D, int64_t chunk_size,
                          const float *init, void *y, float *final_states, void *workspace,
                          size_t workspace_bytes, void *stream_handle, const ssd_plan *abi_plan,
                          void *const *events) {
    Problem p;
    ssd_status st = check_shape(shape, chunk_size, &p);
    if (st != SSD_OK) return st;
    Plan plan;
    st = plan_from_abi(p, abi_plan, &plan);
    if (st != SSD_OK) return st;
    const bool keep = (shape->flags & SSD_FLAG_KEEP_INTERMEDIATES) != 0;
    const ssd_workspace_layout lay = layout_for(p, keep);
    const size_t esz = p.bf16 ? 2 : 4;
    const size_t ysz = p.y_bf16 ? 2 : 4;

    const size_t tok = (size_t)(p.batch * p.seqlen);
    const size_t x_bytes = tok * p.nheads * p.headdim * esz;
    const size_t dt_bytes = tok * p.nheads * esz;
    const size_t bc_bytes = tok * p.ngroups * p.dstate * esz;
    const size_t hd_bytes = (size_t)p.nheads * sizeof(float);
    const size_t st_bytes = (size_t)p.batch * p.nheads * p.headdim * p.dstate * sizeof(float);
    const bool has_tokens = tok > 0;

    // required pointers
    if (has_tokens && (x == nullptr || dt == nullptr || A == nullptr || B == nullptr ||
                       C == nullptr || y == nullptr))
        return SSD_ERROR_INVALID_VALUE;
    if (p.batch > 0 && lay.total > 0 && workspace == nullptr) return SSD_ERROR_WORKSPACE;
    if (workspace_bytes < lay.total) return SSD_ERROR_WORKSPACE;
    if (events != nullptr)
        for (int i = 0; i < 8; ++i)
            if (events[i] == nullptr) return SSD_ERROR_INVALID_VALUE;

    // alignment
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(dt, esz) || !aligned(A, 4) || !aligned(D, 4) || !aligned(init, 16) ||
        !aligned(final_states, 16) || !aligned(workspace, kAlign))
        return SSD_ERROR_MISALIGNED;

    // aliasing: outputs must not overlap inputs or each other; final_states may
    // be the very same buffer as initial_states.
    const Range ry = range_of(y, x_bytes / esz * ysz);
    const Range rws = range_of(workspace, lay.total);
    const Range rfin = range_of(final_states, final_states ? st_bytes : 0);
    const Range rinit = range_of(init, init ? st_bytes : 0);
    const Range ins[] = {range_of(x, x_bytes), range_of(dt, dt_bytes), range_of(A, hd_bytes),
                         range_of(B, bc_bytes), range_of(C, bc_bytes),
                         range_of(D, D ? hd_bytes : 0), rinit};
    for (const Range &r : ins) {
        if (overlap(ry, r) || overlap(rws, r)) return SSD_ERROR_INVALID_VALUE;
        if (&r != &ins[6] && overlap(rfin, r)) return SSD_ERROR_INVALID_VALUE;
    }
    if (overlap(rfin, rinit) && (void *)final_states != (const void *)init) return SSD_ERROR_INVALID_VALUE;
    if (overlap(ry, rws) || overlap(ry, rfin) || overlap(rws, rfin)) return SSD_ERROR_INVALID_VALUE;

    if (p.batch == 0) return SSD_OK;  // nothing to compute

    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const G2Pair G2{reinterpret_cast<float *>(ws + lay.g2_hi), reinterpret_cast<float *>(ws + lay.g2_lo)};
    const G2View G2v{G2.hi, G2.lo};
    float *DTf = reinterpret_cast<float *>(ws + lay.dt);
    float *Wf = reinterpret_cast<float *>(ws + lay.w);
    float *S = reinterpret_cast<float *>(ws + lay.s);
    float *Hs = reinterpret_cast<float *>(ws + lay.h);
    float *CB = reinterpret_cast<float *>(ws + lay.cb);

    // stage i's (start, stop) events, recorded by its kernel's dispatch; a
    // stage with nothing to do records both at once
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
        return hipEventRecord(ev.start, stream) == hipSuccess &&
               hipEventRecord(ev.stop, stream) == hipSuccess;
    };
    if (p.nchunks > 0 && plan.fused_state) {
        // stage 1 is the fused launch (chunk states and carry); stage 2 has no kernel
        if (launch_chunk_cumsum(p, dt, A, G2, DTf, Wf, stream, events_of(0)) != hipSuccess)
            return SSD_ERROR_LAUNCH;
        if (launch_state_fused(p, plan, x, B, Wf, G2v, init, Hs, final_states, C, CB, stream,
                               events_of(1)) != hipSuccess)
            return SSD_ERROR_LAUNCH;
        if (!skip(2)) return SSD_ERROR_LAUNCH;
    } else {
        if (p.nchunks > 0) {
            if (launch_chunk_cumsum(p, dt, A, G2, DTf, Wf, stream, events_of(0)) != hipSuccess)
                return SSD_ERROR_LAUNCH;
            if (launch_chunk_state(p, plan, x, B, Wf, S, stream, events_of(1)) != hipSuccess)
                return SSD_ERROR_LAUNCH;
        } else if (!skip(0) || !skip(1)) {
            return SSD_ERROR_LAUNCH;
        }
        if (launch_state_pass(p, S, Hs, G2v, init, final_states, B, C, CB, stream, events_of(2)) !=
            hipSuccess)
            return SSD_ERROR_LAUNCH;
    }
    if (p.nchunks > 0) {
        if (launch_chunk_out(p, plan, x, B, C, CB, G2v, DTf, D, Hs, y, stream, events_of(3)) != hipSuccess)
            return SSD_ERROR_LAUNCH;
    } else if (!skip(3)) {
        return SSD_ERROR_LAUNCH;
    }
    return SSD_OK;
}

ssd_status ssd_chunk_scan_fwd(const ssd_shape *shape, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D, int64_t chunk_size,
                              const float *initial_states, void *y, float *final_states,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return forward(shape, x, dt, A, B, C, D, chunk_size, initial_states, y, final_states, workspace,
                   workspace_bytes, stream, nullptr, nullptr);
}

ssd_status ssd_chunk_scan_fwd_ex(const ssd_shape *shape, const void *x, const void *dt, const float *A,
                                 const void *B, const void *C, const float *D, int64_t chunk_size,
                                 const float *initial_states, void *y, float *final_states,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const ssd_plan *plan, void *const *stage_events) {
    return forward(shape, x, dt, A, B, C, D, chunk_size, initial_states, y, final_states, workspace,
                   workspace_bytes, stream, plan, stage_events);
}

ssd_status ssd_chunk_scan_fwd_profiled(const ssd_shape *shape, const void *x, const void *dt,
                                       const float *A, const void *B, const void *C, const float *D,
                                       int64_t chunk_size, const float *initial_states, void *y,
                                       float *final_states, void *workspace, size_t workspace_bytes,
                                       void *stream, void *const *stage_events) {
    if (stage_events == nullptr) return SSD_ERROR_INVALID_VALUE;
    return forward(shape, x, dt, A, B, C, D, chunk_size, initial_states, y, final_states, workspace,
                   workspace_bytes, stream, nullptr, stage_events);
}

ssd_status ssd_chunk_scan_fwd_stage_launches(const ssd_shape *shape, int64_t chunk_size,
                                             const ssd_plan *abi_plan, uint32_t *mask) {
    if (mask == nullptr) return SSD_ERROR_INVALID_VALUE;
    Problem p;
    ssd_status st = check_shape(shape, chunk_size, &p);
    if (st != SSD_OK) return st;
    Plan plan;
    st = plan_from_abi(p, abi_plan, &plan);
    if (st != SSD_OK) return st;
    uint32_t m = 0;
    if (p.batch > 0) {
        if (p.nchunks > 0) m |= 1u | 8u;
        // the fused path is one launch (stage 1) that also carries the state
        // and writes the final state; with no chunks only the carry runs
        if (p.nchunks > 0 && plan.fused_state) m |= 2u;
        else if (p.nchunks > 0) m |= 2u | 4u;
        else m |= 4u;
    }
    *mask = m;
    return SSD_OK;
}

ssd_status ssd_decode_step(const ssd_shape *shape, const void *x, const void *dt, const float *A,
                           const void *B, const void *C, const float *D, float *state, void *y,
                           void *stream_handle, void *const *events) {
    Problem p;
    // the chunk size plays no part in a single step; any supported one validates the rest
    const ssd_status st = check_shape(shape, 64, &p);
    if (st != SSD_OK) return st;
    if (p.seqlen != 1 || shape->flags != 0) return SSD_ERROR_INVALID_VALUE;
    if (events != nullptr && (events[0] == nullptr || events[1] == nullptr)) return SSD_ERROR_INVALID_VALUE;
    if (p.batch == 0) return SSD_OK;
    if (x == nullptr || dt == nullptr || A == nullptr || B == nullptr || C == nullptr ||
        state == nullptr || y == nullptr)
        return SSD_ERROR_INVALID_VALUE;
    const size_t esz = p.bf16 ? 2 : 4, ysz = p.y_bf16 ? 2 : 4;
    if (!aligned(x, esz) || !aligned(dt, esz) || !aligned(A, 4) || !aligned(D, 4) || !aligned(B, 16) ||
        !aligned(C, 16) || !aligned(state, 16) || !aligned(y, ysz))
        return SSD_ERROR_MISALIGNED;
    const size_t bh = (size_t)p.batch * p.nheads;
    const Range rx = range_of(x, bh * p.headdim * esz), rdt = range_of(dt, bh * esz),
                rA = range_of(A, p.nheads * 4), rD = range_of(D, D ? p.nheads * 4 : 0),
                rB = range_of(B, (size_t)p.batch * p.ngroups * p.dstate * esz),
                rC = range_of(C, (size_t)p.batch * p.ngroups * p.dstate * esz),
                rs = range_of(state, bh * p.headdim * p.dstate * 4), ry = range_of(y, bh * p.headdim * ysz);
    for (const Range &r : {rx, rdt, rA, rD, rB, rC})
        if (overlap(r, rs) || overlap(r, ry)) return SSD_ERROR_INVALID_VALUE;
    if (overlap(rs, ry)) return SSD_ERROR_INVALID_VALUE;
    LaunchEvents ev;
    if (events != nullptr) {
        ev.start = static_cast<hipEvent_t>(events[0]);
        ev.stop = static_cast<hipEvent_t>(events[1]);
    }
    if (launch_decode_step(p, x, dt, A, B, C, D, state, y, static_cast<hipStream_t>(stream_handle), ev) !=
        hipSuccess)
        return SSD_ERROR_LAUNCH;
    return SSD_OK;
}

const char *ssd_status_string(ssd_status s) {
    switch (s) {
        case SSD_OK: return "ok";
        case SSD_ERROR_INVALID_VALUE: return "invalid argument (NULL pointer, bad size, or aliasing)";
        case SSD_ERROR_UNSUPPORTED: return "unsupported size (chunk_size 64/128/256, headdim 32/64/128, dstate 16..256 step 16)";
        case SSD_ERROR_MISALIGNED: return "misaligned pointer (16 B for x/B/C/y/states, 256 B for workspace)";
        case SSD_ERROR_WORKSPACE: return "workspace missing or smaller than ssd_chunk_scan_fwd_workspace_size()";
        case SSD_ERROR_LAUNCH: return "the HIP runtime refused a kernel launch or event record";
        case SSD_ERROR_SCRATCH: return "problem needs more workspace than the no-allocation entry point's 128 MiB scratch";
    }
    return "unknown status";
}

int ssd_version(void) { return 200; }

}  // extern "C"

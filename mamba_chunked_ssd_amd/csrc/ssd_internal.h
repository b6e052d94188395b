// ssd_internal.h -- interface between the C-ABI host code (ssd_api.cpp) and
// the kernel translation units.  Not installed; not part of the ABI.  Host
// declarations only (the HIP runtime API, no device code), so the host code
// also builds with a plain C++ compiler (the sanitizer builds of the tests);
// the launch helpers the kernel files share are in ssd_launch.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

// LDS per compute unit on gfx950, the most one block may use.
constexpr size_t kLdsPerCu = 160 * 1024;

// Problem description after validation, with the derived sizes every stage
// needs.  All element counts are int64.
struct Problem {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int64_t nchunks;          // ceil(seqlen / chunk)
    int64_t padded_len;       // nchunks * chunk
    int64_t heads_per_group;  // nheads / ngroups
    bool bf16;                // element type of x, dt, B, C
    bool y_bf16;              // element type of y
};

// Launch configuration chosen on the host per problem (the C ABI's ssd_plan).
struct Plan {
    bool fused_state;         // stages 2 and 3 in one launch (bf16 only)
    int k2_heads_per_block;   // heads of one group sharing a staged B chunk
    int k4_heads_per_block;   // heads of one group sharing one C B^T tile set
    int fused_cols;           // fused path: dstate columns per block
};

Plan make_plan(const Problem &p);

// bf16 problems with headdim 64 and dstate 128, or dstate 256 at chunk 256,
// take the chunk-output kernel with asynchronous copies; it reads the chunk's
// C B^T tiles, which stage 3 writes once per (batch, chunk, group) into the
// workspace: cb_slots(T) tiles of 64 lanes x 4 floats each (the layout is
// described in include/ssd.h).
inline bool uses_cb_tiles(const Problem &p) {
    return p.bf16 && p.headdim == 64 && (p.dstate == 128 || (p.dstate == 256 && p.chunk == 256));
}
inline int64_t cb_slots(int64_t T) { return (T / 32) * (T / 16 + 2); }

// Each launcher enqueues one kernel on `stream` and returns hipSuccess or the
// launch error.  Buffers follow the layouts documented in include/ssd.h.

// Decay sums G2 = log2(e) * per-chunk inclusive cumsum of A dt, summed in fp64
// and stored as a pair of floats (G2 = hi + lo), head-major
// (batch, nheads, padded_len).
struct G2Pair {
    float *hi;
    float *lo;
};
struct G2View {
    const float *hi;
    const float *lo;
};

// Optional (start, stop) events recorded by a kernel's own dispatch.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Stage 1: G2 (hi/lo), dt widened to fp32 -> DT and the chunk-state weights
// W_t = exp2(G2_last - G2_t) DT_t, all head-major.
// With Wb non-null it also writes exp2(G2_t) (0 past seqlen), the backward
// pass's weights for the adjoint chunk terms.
hipError_t launch_chunk_cumsum(const Problem &p, const void *dt, const float *A, G2Pair G2,
                               float *DT, float *W, hipStream_t stream, const LaunchEvents &ev,
                               float *Wb = nullptr);

// Stage 2: per-chunk input state s_c = sum_t W_t x_t B_t^T,
// written as (batch, nheads, nchunks, headdim, dstate) fp32.
hipError_t launch_chunk_state(const Problem &p, const Plan &plan, const void *x, const void *B,
                              const float *W, float *S, hipStream_t stream, const LaunchEvents &ev);
// How many stage-2 blocks one CU holds (set by the kernel variant's LDS use).
int chunk_state_blocks_per_cu(const Problem &p);

// Stage 3: h_0 = init (or 0); for each chunk store h_c then
// h_{c+1} = exp2(G2_last,c) h_c + s_c; final = h_nchunks.  H may equal S.
// When uses_cb_tiles(p), extra blocks of the same launch also write the C B^T
// tiles (CB) from B and C, beside the memory-bound state stream.
hipError_t launch_state_pass(const Problem &p, const float *S, float *H, G2View G2,
                             const float *init, float *final_states, const void *B,
                             const void *C, float *CB, hipStream_t stream, const LaunchEvents &ev);

// Stages 2 and 3 in one launch (bf16 inputs): per (batch, head, block of
// plan.fused_cols dstate columns) the chunks in order, h_c stored as the hi/lo
// bf16 planes of H, final = h_nchunks; no s_c.  When uses_cb_tiles(p), extra
// blocks of the launch also write the C B^T tiles.  Needs nchunks > 0.
bool state_fused_supported(const Problem &p, int cols);
hipError_t launch_state_fused(const Problem &p, const Plan &plan, const void *x, const void *B,
                              const float *W, G2View G2, const float *init, float *H,
                              float *final_states, const void *C, float *CB, hipStream_t stream,
                              const LaunchEvents &ev);

// Recurrent decode step (seqlen 1): state <- exp(A dt) state + dt x B^T in
// place, y = state C + D x.  Layouts as the forward pass with seqlen 1.
hipError_t launch_decode_step(const Problem &p, const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, float *state, void *y, hipStream_t stream,
                              const LaunchEvents &ev);

// Stage 4: chunk output
// y_i = exp2(G2_i) C_i h_c + sum_{j<=i} exp2(G2_i - G2_j) (C_i . B_j) DT_j x_j + D x_i.
// CB: the C B^T tiles of stage 1 when uses_cb_tiles(p), else unused.
hipError_t launch_chunk_out(const Problem &p, const Plan &plan, const void *x, const void *B,
                            const void *C, const float *CB, G2View G2, const float *DT,
                            const float *D, const float *H, void *y, hipStream_t stream,
                            const LaunchEvents &ev);

// ---------------------------------------------------------------------------
// Backward pass (ssd_chunk_scan_bwd)
// ---------------------------------------------------------------------------

// Score tiles B_r . C_s of every (batch, chunk, group), the 16 x 16 blocks on
// and above the diagonal, in the layout the dx pass reads.
hipError_t launch_bwd_scores(const Problem &p, const void *B, const void *C, float *ST, hipStream_t stream,
                             const LaunchEvents &ev);
// Reverse carry of the adjoint state: E (per (b, h, c): hi/lo bf16 planes for
// bf16 problems, fp32 for fp32 problems), per-wave partials of
// exp(G_last) <E_c, h_c> (headdim * dstate / 256 per chunk) and the gradient
// of the initial state (dinit may be null).
hipError_t launch_bwd_carry(const Problem &p, const float *U, const void *H, G2View G2, const float *dfinal,
                            void *E, float *Zp, float *dinit, hipStream_t stream, const LaunchEvents &ev);

// Strips of 16 rows per wave of each backward pass (0 dx, 1 dB, 2 dC, 3 W
// sums; 1 or 2, see kb_pass.h) for bf16 or fp32 inputs and a headdim of
// 32 nkq.
__host__ __device__ constexpr int bwd_spw(int pass, bool bf16, int nkq) {
    return bf16 && (pass == 0 || pass == 1 || (pass == 2 && nkq <= 2)) ? 1 : 2;
}
// waves of one block of a backward pass
inline int kb_pass_waves(const Problem &p, int pass) {
    return (int)(p.chunk / 16) / bwd_spw(pass, p.bf16, (int)(p.headdim / 32));
}

// One of the MFMA passes (kb_pass.h): 0 = dx and the per-token dot products,
// 1 = dB partials, 2 = dC partials, 3 = the row and column sums of W (dv 16),
// 4 = the decayed score tiles of fp32 problems (dv 16, unused).
struct BwdPassLaunch {
    int pass;
    const void *x, *dy, *B, *C;
    G2View G2;
    const float *DT;
    const void *E;
    const void *H;
    const float *ST;
    const float *D;
    float *out;
    float *xq, *xqi, *dyx, *cdi;  // per-token partial sums (kb_pass.h)
    double *wd;
    float *pt, *ptt;  // fp32 problems: decayed score tiles and their transposes (written by pass 4, read by 1-3)
    int dv;      // columns per block (16, 32 or 64)
    int hb;      // heads per block
    int lds_pad; // LDS row padding in elements (0 or 8)
    int xt_lds;  // dx pass: x tile, dC pass: C tile staged in LDS (needs the room)
};
// Column tiles of the dB and dC passes that their registers hold (the rule
// of kb_pass_inst.h's bc_dv_ok).
inline bool bwd_dv_ok(bool bf16, int64_t P, int dv) {
    return dv <= (bf16 ? (P <= 64 ? 64 : 32) : 64);
}
// LDS bytes a pass block needs; 0 if it does not fit one CU.
size_t bwd_pass_lds(const Problem &p, int pass, int dv, int lds_pad, bool xt = false);
hipError_t launch_bwd_pass(const Problem &p, const BwdPassLaunch &L, hipStream_t stream, const LaunchEvents &ev);
// Blocks of a pass (as launch_bwd_pass would run it) that one CU holds at
// once, from the kernel's registers and LDS; 0 if the runtime cannot say.
int bwd_pass_blocks_per_cu(const Problem &p, const BwdPassLaunch &L);

// The per-token partial sums the passes leave, (parts, batch, nheads, Lp).
struct BwdTokens {
    const float *xq, *xqi, *dyx;  // dx pass: nq parts (its column tiles)
    const float *cdi;             // dC pass: nc parts
    const double *wd;             // W sums: W's row sum minus its column sum, 1 part
    int nq, nc;
};
hipError_t launch_bwd_tokens(const Problem &p, const BwdTokens &tk, const float *DT, const float *Zp,
                             const float *A, float *ddt, float *dap, float *ddp, hipStream_t stream,
                             const LaunchEvents &ev);
hipError_t launch_bwd_reduce(const Problem &p, const float *dbp, const float *dcp, int nhb, float *dB, float *dC,
                             const float *dap, const float *ddp, float *dA, float *dD, hipStream_t stream,
                             const LaunchEvents &ev);

}  // namespace ssd

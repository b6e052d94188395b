// k3_state_pass.hip -- stage 3: carry the state across chunks.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Kernel 2: fwd_pass_state" and the log-space state jump
// of section "Mamba-2 architecture": with s_c the state chunk c produces from a
// zero state (stage 2), the state at the start of chunk c + 1 is
//     h_{c+1} = exp(G_last,c) h_c + s_c ,
// and the kernel stores every chunk-start state h_c (the per-chunk state the
// fwd_pass_state section stores before each chunk update) plus the state
// after the last chunk.
//
// Design for gfx950: this is a pure HBM stream (one read of s, one write of h
// per element, 2 flops).  Each thread owns 4 consecutive state elements of one
// (batch, head) and walks the chunks; the loads of a batch of 4 chunks (16
// beyond 128 chunks) are issued before the dependent FMA chain, and
// consecutive threads touch consecutive 16-byte words, so every wave access
// is a fully coalesced 1 KiB.  For fp32 problems h is fp32 and may alias s
// (in place: each element is read before it is overwritten, by the same
// thread).  For bf16 problems the chunk output multiplies h_c as hi + lo bf16
// halves, so h is written split: per (batch, head, chunk) a hi plane and a lo
// plane of (headdim, dstate) bf16 (hi = bf16(h), lo = bf16(h - hi)), in a
// region of its own; the final state stays fp32.
//
// The same launch also computes, in extra blocks at the front of the grid,
// the C B^T tiles that the chunk output reads (bf16 problems with headdim 64
// and dstate 128, or dstate 256 at chunk 256): MFMA work that depends only on
// B and C, so it runs beside the memory-bound stream instead of on the chunk
// output's critical path ("Mamba-2 architecture": the C B^T factor of the
// chunk output).
#include <climits>

#include "k_cb_tiles.h"
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

// Chunks whose loads are issued together before their stores (see
// state_depth): with few chunks per thread a smaller batch lets one batch's
// stores overlap the next batch's loads; with many, a deeper batch keeps more
// bytes in flight.
template <int kDepth, bool kSplit>
__device__ __forceinline__ void state_pass_body(const float *S, float *H, const float *__restrict__ G2hi,
                                                const float *__restrict__ G2lo, const float *init,
                                                float *final_states, int64_t n_vec, int64_t pn_vec,
                                                int64_t nchunks, int64_t Lp, int T, int64_t blk) {
    const int64_t v = blk * 256 + threadIdx.x;  // float4 index over (bh, pn)
    if (v >= n_vec) return;
    const int64_t bh = v / pn_vec;
    const int64_t e = v % pn_vec;
    const float4 *Sv = reinterpret_cast<const float4 *>(S);
    float4 *Hv = reinterpret_cast<float4 *>(H);

    float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init != nullptr) h = reinterpret_cast<const float4 *>(init)[bh * pn_vec + e];
    const float *g2h = G2hi + bh * Lp + (T - 1);
    const float *g2l = G2lo + bh * Lp + (T - 1);

    for (int64_t c0 = 0; c0 < nchunks; c0 += kDepth) {
        float4 s[kDepth];
        float dec[kDepth];
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
            if (c0 + k < nchunks) {
                s[k] = Sv[((bh * nchunks) + c0 + k) * pn_vec + e];
                dec[k] = g2h[(c0 + k) * T] + g2l[(c0 + k) * T];
            }
        }
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
            if (c0 + k < nchunks) {
                if constexpr (kSplit) {
                    // planes of 4 pn_vec bf16 each: hi at chunk base, lo after it
                    uint16_t *hb = reinterpret_cast<uint16_t *>(H) + ((bh * nchunks) + c0 + k) * 8 * pn_vec;
                    const HiLo a = split_bf16(h.x, h.y), bq = split_bf16(h.z, h.w);
                    *reinterpret_cast<u32x2 *>(hb + 4 * e) = u32x2{a.hi, bq.hi};
                    *reinterpret_cast<u32x2 *>(hb + 4 * pn_vec + 4 * e) = u32x2{a.lo, bq.lo};
                } else {
                    Hv[((bh * nchunks) + c0 + k) * pn_vec + e] = h;
                }
                const float a = fast_exp2(dec[k]);
                h.x = fmaf(a, h.x, s[k].x);
                h.y = fmaf(a, h.y, s[k].y);
                h.z = fmaf(a, h.z, s[k].z);
                h.w = fmaf(a, h.w, s[k].w);
            }
        }
    }
    if (final_states != nullptr) reinterpret_cast<float4 *>(final_states)[bh * pn_vec + e] = h;
}

template <int kDepth, bool kSplit>
__global__ __launch_bounds__(256) void k3_state_pass(const float *S, float *H,
                                                     const float *__restrict__ G2hi,
                                                     const float *__restrict__ G2lo,
                                                     const float *init, float *final_states,
                                                     int64_t n_vec, int64_t pn_vec,
                                                     int64_t nchunks, int64_t Lp, int T) {
    state_pass_body<kDepth, kSplit>(S, H, G2hi, G2lo, init, final_states, n_vec, pn_vec, nchunks, Lp, T,
                                    blockIdx.x);
}

// kRows: dstate 256, the tiles by slot rows (cb_rows; `ntiles` counts its
// tasks); otherwise dstate 128, one tile per wave step (cb_tiles).
template <int T, int kDepth, bool kRows>
__global__ __launch_bounds__(256) void k3_state_pass_cb(const float *S, float *H,
                                                        const float *__restrict__ G2hi,
                                                        const float *__restrict__ G2lo,
                                                        const float *init, float *final_states,
                                                        int64_t n_vec, int64_t pn_vec,
                                                        int64_t nchunks, int64_t Lp,
                                                        const uint16_t *__restrict__ Bm,
                                                        const uint16_t *__restrict__ Cm,
                                                        float *__restrict__ CB, int64_t seqlen,
                                                        int G, int64_t ntiles, int ncb) {
    const int bx = (int)blockIdx.x;
    if (bx < ncb) {
        if constexpr (kRows)
            cb_rows<T, 256>(Bm, Cm, CB, seqlen, G, nchunks, ntiles, ncb, bx);
        else
            cb_tiles<T, 128>(Bm, Cm, CB, seqlen, G, nchunks, ntiles, ncb, bx);
    } else {
        state_pass_body<kDepth, true>(S, H, G2hi, G2lo, init, final_states, n_vec, pn_vec, nchunks, Lp,
                                      T, (int64_t)bx - ncb);
    }
}

}  // namespace

hipError_t launch_state_pass(const Problem &p, const float *S, float *H, G2View G2,
                             const float *init, float *final_states, const void *B,
                             const void *C, float *CB, hipStream_t stream, const LaunchEvents &ev) {
    const int64_t pn_vec = p.headdim * p.dstate / 4;
    const int64_t n_vec = p.batch * p.nheads * pn_vec;
    if (n_vec == 0) return hipSuccess;
    const int64_t blocks = (n_vec + 255) / 256;
    // measured on MI355X: batches of 4 chunks up to 128 chunks (2.7B layer
    // 16.9 -> 15.4 us, grouped fp32 workload 1.94 -> 1.84 ms), 16 beyond
    constexpr int kShallow = 4, kDeep = 16;
    const bool deep = p.nchunks > 128;
    const int64_t ntiles = (uses_cb_tiles(p) && CB != nullptr) ? p.batch * p.nchunks * p.ngroups * cb_slots(p.chunk) : 0;
    if (ntiles > 0) {
        // dstate 256: one wave per slot row (cb_rows), else kCbPerWave tiles per wave
        const bool rows = p.dstate == 256;
        const int64_t units = rows ? p.batch * p.nchunks * p.ngroups * (p.chunk / 32) : ntiles;
        const int64_t ncb = rows ? (units + 3) / 4 : (ntiles + 4 * kCbPerWave - 1) / (4 * kCbPerWave);
        // the tile blocks first, then the stream's.  (Placed after the stream,
        // the tiles were no faster at 65 536 tokens, 32 heads, dstate 256:
        // the deep stream's 512 blocks fill every CU.)
        const int64_t total = ncb + blocks;
        if (total > INT_MAX) return hipErrorInvalidValue;
        const auto *Bm = static_cast<const uint16_t *>(B);
        const auto *Cm = static_cast<const uint16_t *>(C);
#define SSD_K3_CB(TT, DD, RR)                                                                          \
    launch_kernel(k3_state_pass_cb<TT, DD, RR>, dim3((unsigned)total), dim3(256), 0, stream, ev, S, H,   \
                  G2.hi, G2.lo, init, final_states, n_vec, pn_vec, p.nchunks, p.padded_len, Bm, Cm, CB, \
                  p.seqlen, (int)p.ngroups, units, (int)ncb)
#define SSD_K3_CB_T(TT)                                                    \
    if (deep) {                                                            \
        if (rows) SSD_K3_CB(TT, kDeep, true); else SSD_K3_CB(TT, kDeep, false); \
    } else {                                                               \
        if (rows) SSD_K3_CB(TT, kShallow, true); else SSD_K3_CB(TT, kShallow, false); \
    }
        switch (p.chunk) {  // slot rows only at chunk 256 (uses_cb_tiles)
            case 64: if (deep) SSD_K3_CB(64, kDeep, false); else SSD_K3_CB(64, kShallow, false); break;
            case 128: if (deep) SSD_K3_CB(128, kDeep, false); else SSD_K3_CB(128, kShallow, false); break;
            case 256: SSD_K3_CB_T(256); break;
            default: return hipErrorInvalidValue;
        }
#undef SSD_K3_CB_T
#undef SSD_K3_CB
        return hipGetLastError();
    }
#define SSD_K3(DD, SPLIT)                                                                          \
    launch_kernel(k3_state_pass<DD, SPLIT>, dim3((unsigned)blocks), dim3(256), 0, stream, ev, S, H, \
                  G2.hi, G2.lo, init, final_states, n_vec, pn_vec, p.nchunks, p.padded_len, (int)p.chunk)
    if (p.bf16) {
        if (deep) SSD_K3(kDeep, true); else SSD_K3(kShallow, true);
    } else {
        if (deep) SSD_K3(kDeep, false); else SSD_K3(kShallow, false);
    }
#undef SSD_K3
    return hipGetLastError();
}

}  // namespace ssd

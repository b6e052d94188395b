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
// (batch, head) and walks the chunks; loads of up to 8 chunks are issued
// before the dependent FMA chain so each thread keeps 128 B in flight, and
// consecutive threads touch consecutive 16-byte words, so every wave access
// is a fully coalesced 1 KiB.  For fp32 problems h is fp32 and may alias s
// (in place: each element is read before it is overwritten, by the same
// thread).  For bf16 problems the chunk output multiplies h_c as hi + lo bf16
// halves, so h is written split: per (batch, head, chunk) a hi plane and a lo
// plane of (headdim, dstate) bf16 (hi = bf16(h), lo = bf16(h - hi)), in a
// region of its own; the final state stays fp32.
#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kDepth = 8;

template <bool kSplit>
__global__ __launch_bounds__(256) void k3_state_pass(const float *S, float *H,
                                                     const float *__restrict__ G2hi,
                                                     const float *__restrict__ G2lo,
                                                     const float *init, float *final_states,
                                                     int64_t n_vec, int64_t pn_vec,
                                                     int64_t nchunks, int64_t Lp, int T) {
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index over (bh, pn)
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

}  // namespace

hipError_t launch_state_pass(const Problem &p, const float *S, float *H, G2View G2,
                             const float *init, float *final_states, hipStream_t stream, const LaunchEvents &ev) {
    const int64_t pn_vec = p.headdim * p.dstate / 4;
    const int64_t n_vec = p.batch * p.nheads * pn_vec;
    if (n_vec == 0) return hipSuccess;
    const int64_t blocks = (n_vec + 255) / 256;
    if (p.bf16)
        launch_kernel(k3_state_pass<true>, dim3((unsigned)blocks), dim3(256), 0, stream, ev, S, H,
                      G2.hi, G2.lo, init, final_states, n_vec, pn_vec, p.nchunks, p.padded_len,
                      (int)p.chunk);
    else
        launch_kernel(k3_state_pass<false>, dim3((unsigned)blocks), dim3(256), 0, stream, ev, S, H,
                      G2.hi, G2.lo, init, final_states, n_vec, pn_vec, p.nchunks, p.padded_len,
                      (int)p.chunk);
    return hipGetLastError();
}

}  // namespace ssd

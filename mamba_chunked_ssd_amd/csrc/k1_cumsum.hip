// k1_cumsum.hip -- stage 1: per-chunk cumulative sum of the log decay.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Kernel 1: Computing cumulative sums": the chunked
// equations need G, the running sum of a_t = A dt_t inside each chunk
// (restarting at every chunk), in both later stages, so it is computed once
// and stored.  It is kept in base-2 units (G2 = log2(e) G) so that the later
// stages use the native exp2.
//
// Design for gfx950: one wave per (batch, chunk, head), eight heads per block.
// The block first copies its chunk's dt for its eight heads into LDS with
// consecutive threads on consecutive heads of one token (dt is token-major,
// so a wave's load covers 8 tokens x 8 heads instead of 64 tokens of one head
// scattered over 64 rows); then every lane sums T/64 consecutive tokens of its
// wave's head serially, the 64 lane totals are scanned with wave shuffles,
// and each lane adds its exclusive prefix.  (Measured on MI355X: 13.3 -> 11.2
// us at 65 536 tokens x 32 heads, 24.1 -> 20.5 us for the grouped fp32
// workload, unchanged at the 2.7B-shaped layer, where the launch dominates.)  The sum runs in fp64 and is stored as two
// floats, G2 = hi + lo: within a chunk |G2| can reach thousands while the
// later stages exponentiate differences G2_i - G2_j of nearby tokens, and
// (hi_i - hi_j) + (lo_i - lo_j) keeps those differences accurate to fp32
// relative precision instead of to ulp(|G2|).  Outputs are head-major
// (batch, nheads, padded_len), so each (head, chunk) is one contiguous run of
// T floats for the later stages, written by each lane as one vector of its
// T/64 tokens; dt is also written there widened to fp32, and so is the weight
// with which each token enters its chunk's state (the log-space state jump of
// the same page's section "Mamba-2 architecture"),
//     W_t = exp2(G2_last - G2_t) dt_t ,
// whose exponent is formed exactly in fp64 before the fp32 exp2.  Tokens past
// seqlen are treated as dt = 0: G2 stays flat and DT, W are 0.  On request
// (the backward pass) it also writes exp2(G2_t), the weight with which the
// output gradient at token t enters the adjoint of its chunk's starting
// state (0 past seqlen).
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kHeadsPerBlock = 8;

template <typename Tin>
__device__ __forceinline__ float load_dt(const Tin *p);
template <>
__device__ __forceinline__ float load_dt<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_dt<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

template <typename Tin, int T>
__global__ __launch_bounds__(64 * kHeadsPerBlock) void k1_cumsum(
    const Tin *__restrict__ dt, const float *__restrict__ A, float *__restrict__ G2hi,
    float *__restrict__ G2lo, float *__restrict__ DT, float *__restrict__ W, float *__restrict__ Wb,
    int64_t seqlen, int nheads, int64_t Lp) {
    constexpr int E = T / 64;  // tokens per lane
    const int c = blockIdx.x;
    const int h = blockIdx.y * kHeadsPerBlock + (threadIdx.x >> 6);
    const int64_t b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    // the chunk's dt of this block's heads, [head][token]; tokens past seqlen
    // and heads past nheads as 0
    __shared__ float dts[kHeadsPerBlock][T + 1];
    {
        const int h0 = blockIdx.y * kHeadsPerBlock;
        for (int idx = threadIdx.x; idx < T * kHeadsPerBlock; idx += 64 * kHeadsPerBlock) {
            const int tt = idx / kHeadsPerBlock, hh = idx % kHeadsPerBlock;
            const int64_t t = (int64_t)c * T + tt;
            dts[hh][tt] = (t < seqlen && h0 + hh < nheads) ? load_dt(dt + (b * seqlen + t) * nheads + h0 + hh) : 0.f;
        }
    }
    __syncthreads();
    if (h >= nheads) return;  // wave-uniform; no barrier follows

    const int64_t t0 = (int64_t)c * T + lane * E;
    float d[E];
#pragma unroll
    for (int e = 0; e < E; ++e) d[e] = dts[threadIdx.x >> 6][lane * E + e];
    float hi[E], lo[E], wt[E];
    chunk_cumsum_wave<E>(d, A[h], lane, hi, lo, wt);
    const int64_t base = (b * nheads + h) * Lp + t0;
    store_vec<E>(G2hi + base, hi);
    store_vec<E>(G2lo + base, lo);
    store_vec<E>(DT + base, d);
    store_vec<E>(W + base, wt);
    if (Wb != nullptr) {
        float eg[E];
#pragma unroll
        for (int e = 0; e < E; ++e) eg[e] = (t0 + e < seqlen) ? fast_exp2(hi[e]) * fast_exp2(lo[e]) : 0.f;
        store_vec<E>(Wb + base, eg);
    }
}

template <typename Tin, int T>
hipError_t launch_t(const Problem &p, const Tin *dt, const float *A, G2Pair G2, float *DT,
                    float *W, float *Wb, hipStream_t stream, const LaunchEvents &ev) {
    dim3 grid((unsigned)p.nchunks, (unsigned)((p.nheads + kHeadsPerBlock - 1) / kHeadsPerBlock),
              (unsigned)p.batch);
    launch_kernel((k1_cumsum<Tin, T>), grid, dim3(64 * kHeadsPerBlock), 0, stream, ev, dt, A,
                  G2.hi, G2.lo, DT, W, Wb, p.seqlen, (int)p.nheads, p.padded_len);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_dtype(const Problem &p, const Tin *dt, const float *A, G2Pair G2, float *DT,
                        float *W, float *Wb, hipStream_t stream, const LaunchEvents &ev) {
    switch (p.chunk) {
        case 64: return launch_t<Tin, 64>(p, dt, A, G2, DT, W, Wb, stream, ev);
        case 128: return launch_t<Tin, 128>(p, dt, A, G2, DT, W, Wb, stream, ev);
        case 256: return launch_t<Tin, 256>(p, dt, A, G2, DT, W, Wb, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Problem &p, const void *dt, const float *A, G2Pair G2,
                               float *DT, float *W, hipStream_t stream, const LaunchEvents &ev, float *Wb) {
    if (p.bf16) return launch_dtype(p, static_cast<const uint16_t *>(dt), A, G2, DT, W, Wb, stream, ev);
    return launch_dtype(p, static_cast<const float *>(dt), A, G2, DT, W, Wb, stream, ev);
}

}  // namespace ssd

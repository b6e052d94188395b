// k5_decode_step.hip -- one step of the recurrence for one new token per
// sequence, the form the pages name for sequential inference.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Mamba-2 architecture": the recurrent form
//     h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t^T ,   y_t = C_t^T h_t + D x_t
// evaluated for a single t, with the state kept between calls.  In the
// stored [headdim, dstate] orientation, per (batch b, head h, row p):
//     s[p][n] <- exp(A[h] dt) s[p][n] + (dt x[p]) B[n] ,
//     y[p]     = sum_n C[n] s[p][n] + D[h] x[p] .
//
// Design for gfx950: a pure HBM stream (the state is read and written once,
// 8 bytes per element against 4 flops), so no MFMA.  Each thread owns 8
// consecutive dstate entries of one state row (two 16-byte loads in flight,
// then two stores); the R = next power of two >= dstate / 8 threads of a row
// sit in one wave,
// and the row's dot product with C is reduced across them with lane
// shuffles.  B and C rows are shared by every head of a group and come from
// L2 after the first head.  Consecutive threads touch consecutive 16-byte
// words of the state, so every wave access is coalesced.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

template <typename T>
__device__ __forceinline__ float load_in(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ floatx4 load_in4(const T *p, int64_t i);  // 4 consecutive, i % 4 == 0
template <>
__device__ __forceinline__ floatx4 load_in4<float>(const float *p, int64_t i) {
    return *reinterpret_cast<const floatx4 *>(p + i);
}
template <>
__device__ __forceinline__ floatx4 load_in4<uint16_t>(const uint16_t *p, int64_t i) {
    const u32x2 v = *reinterpret_cast<const u32x2 *>(p + i);
    return floatx4{bf16lo(v[0]), bf16hi(v[0]), bf16lo(v[1]), bf16hi(v[1])};
}

template <typename T>
__device__ __forceinline__ void store_y(T *p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_y<float>(float *p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_y<uint16_t>(uint16_t *p, int64_t i, float v) {
    p[i] = (uint16_t)(pack_bf16(v, 0.f) & 0xffffu);
}

template <typename Tin, typename Tout, int R>
__global__ __launch_bounds__(256) void k5_decode_step(const Tin *__restrict__ x, const Tin *__restrict__ dt,
                                                      const float *__restrict__ A, const Tin *__restrict__ Bm,
                                                      const Tin *__restrict__ Cm, const float *__restrict__ D,
                                                      float *__restrict__ state, Tout *__restrict__ y,
                                                      int64_t rows, int NH, int P, int N, int HPG) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / R;  // (b, h, p)
    const int q = (int)(gid % R);  // this thread's 8 dstate entries: 8 q .. 8 q + 7
    if (row >= rows) return;       // whole rows: every lane of a row exits together
    const int p = (int)(row % P);
    const int64_t bh = row / P;
    const int h = (int)(bh % NH);
    const int64_t b = bh / NH;
    const int G = NH / HPG, g = h / HPG;

    float part = 0.f;
    float xp = 0.f;
    if (8 * q < N) {
        // both 16-byte state loads first (two in flight per thread), then
        // the small per-row and per-group operands
        float *sp = state + row * N + 8 * q;
        floatx4 s0 = *reinterpret_cast<const floatx4 *>(sp);
        floatx4 s1 = *reinterpret_cast<const floatx4 *>(sp + 4);
        const float dtv = load_in(dt, bh);
        xp = load_in(x, bh * P + p);
        const floatx4 b0 = load_in4(Bm, (b * G + g) * N + 8 * q), b1 = load_in4(Bm, (b * G + g) * N + 8 * q + 4);
        const floatx4 c0 = load_in4(Cm, (b * G + g) * N + 8 * q), c1 = load_in4(Cm, (b * G + g) * N + 8 * q + 4);
        const float alpha = __expf(A[h] * dtv);  // exp(a_t), a_t = A dt <= 0
        const float u = dtv * xp;                // the rank-one update's scale for row p
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s0[k] = fmaf(alpha, s0[k], u * b0[k]);
            s1[k] = fmaf(alpha, s1[k], u * b1[k]);
            part = fmaf(c0[k], s0[k], part);
            part = fmaf(c1[k], s1[k], part);
        }
        *reinterpret_cast<floatx4 *>(sp) = s0;
        *reinterpret_cast<floatx4 *>(sp + 4) = s1;
    }
    // sum the row's partial dot products over its R lanes (aligned in the wave)
#pragma unroll
    for (int off = R / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, R);
    if (q == 0) store_y<Tout>(y, bh * P + p, part + (D != nullptr ? D[h] : 0.f) * xp);
}

template <typename Tin, typename Tout>
hipError_t launch_io(const Problem &p, const void *x, const void *dt, const float *A, const void *B,
                     const void *C, const float *D, float *state, void *y, hipStream_t stream,
                     const LaunchEvents &ev) {
    const int64_t rows = p.batch * p.nheads * p.headdim;
    if (rows == 0) return hipSuccess;
    const int64_t n8 = p.dstate / 8;  // dstate is a multiple of 16
    int R = 1;
    while (R < n8) R <<= 1;  // <= 32 (dstate <= 256)
    const int64_t blocks = (rows * R + 255) / 256;
    auto go = [&](auto kern) {
        return launch_kernel(kern, dim3((unsigned)blocks), dim3(256), 0, stream, ev,
                             static_cast<const Tin *>(x), static_cast<const Tin *>(dt), A,
                             static_cast<const Tin *>(B), static_cast<const Tin *>(C), D, state,
                             static_cast<Tout *>(y), rows, (int)p.nheads, (int)p.headdim, (int)p.dstate,
                             (int)p.heads_per_group);
    };
    switch (R) {
        case 2: return go(k5_decode_step<Tin, Tout, 2>);
        case 4: return go(k5_decode_step<Tin, Tout, 4>);
        case 8: return go(k5_decode_step<Tin, Tout, 8>);
        case 16: return go(k5_decode_step<Tin, Tout, 16>);
        case 32: return go(k5_decode_step<Tin, Tout, 32>);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_step(const Problem &p, const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, float *state, void *y, hipStream_t stream,
                              const LaunchEvents &ev) {
    if (p.bf16)
        return p.y_bf16 ? launch_io<uint16_t, uint16_t>(p, x, dt, A, B, C, D, state, y, stream, ev)
                        : launch_io<uint16_t, float>(p, x, dt, A, B, C, D, state, y, stream, ev);
    return launch_io<float, float>(p, x, dt, A, B, C, D, state, y, stream, ev);
}

}  // namespace ssd

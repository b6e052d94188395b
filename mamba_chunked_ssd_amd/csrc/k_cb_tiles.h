// k_cb_tiles.h -- the C B^T tiles that the chunk output with asynchronous
// copies reads (bf16 inputs, headdim 64, dstate 128), computed by extra
// blocks at the front of the launch that carries the state across chunks
// (the state-passing launch, or the fused state launch): a little MFMA work
// that depends only on B and C, so it runs beside the memory-bound state
// stream instead of on the chunk output's critical path ("Accelerating
// Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile",
// section "Mamba-2 architecture": the C B^T factor of the chunk output).
#pragma once

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// C B^T tiles for the chunk-output stage (bf16 B and C, dstate 128): tile
// (w, k) of (batch, chunk, group) is the 16 x 16 block (I, J) of
// S_ij = C_i . B_j that the chunk output's wave w keeps in its slot k: I = w,
// J = k for k < (w + 2) & ~1, else I = T/16 - 1 - w and J = k minus that.
// Four MFMAs over dstate in the MFMA output layout (lane 16 q + m holds
// S_{16I+m, 16J+4q+r}, r = 0..3), one float4 per lane, 1 KiB per tile.
// Blocks past the diagonal are written as zero.  Each wave takes kCbPerWave
// tiles; these blocks run at the front of the state-passing grid, beside the
// memory-bound stream.
constexpr int kCbPerWave = 4;

// Blocks of 256 threads that compute `ntiles` tiles.
inline int64_t cb_blocks(int64_t ntiles) { return (ntiles + 4 * kCbPerWave - 1) / (4 * kCbPerWave); }

template <int T>
__device__ __forceinline__ void cb_tiles(const uint16_t *__restrict__ Bm,
                                         const uint16_t *__restrict__ Cm, float *__restrict__ CB,
                                         int64_t seqlen, int G, int64_t nc, int64_t ntiles, int ncb) {
    constexpr int N = 128;
    constexpr int NT16 = T / 16, NSLOT = NT16 + 2, NSL = (T / 32) * NSLOT;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    // consecutive tiles (one chunk's) on one XCD, whose L2 then serves B and C
    const int64_t gw = (int64_t)xcd_remap(blockIdx.x, ncb) * 4 + (threadIdx.x >> 6);
    const int64_t GN = (int64_t)G * N;
#pragma unroll 1
    for (int it = 0; it < kCbPerWave; ++it) {
        const int64_t s = gw * kCbPerWave + it;  // (b, c, g, w, k) flattened
        if (s >= ntiles) return;
        const int rem = (int)(s % NSL);
        const int64_t bcg = s / NSL;
        const int g = (int)(bcg % G);
        const int64_t bc = bcg / G;
        const int64_t c = bc % nc, b = bc / nc;
        const int w = rem / NSLOT, k = rem % NSLOT;
        const int I0 = w, I1 = NT16 - 1 - w, base1 = (I0 + 2) & ~1;
        const int I = k < base1 ? I0 : I1, J = k < base1 ? k : k - base1;
        const int64_t t0 = c * T;
        const int rows = (int)min<int64_t>(T, seqlen - t0);
        floatx4 acc = zero4();
        if (J <= I) {
            const uint16_t *Bc = Bm + ((b * seqlen + t0) * G + g) * N;
            const uint16_t *Cc = Cm + ((b * seqlen + t0) * G + g) * N;
            // 16 bytes of a chunk row at dstate n0; rows past seqlen read as zero
            auto row16 = [&](const uint16_t *base, int row, int n0) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(base + (int64_t)min(row, rows - 1) * GN + n0);
                return row < rows ? v : u32x4{0u, 0u, 0u, 0u};
            };
            u32x4 bf[N / 32], cf[N / 32];
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks) {
                bf[ks] = row16(Bc, 16 * J + l16, 32 * ks + 8 * g4);
                cf[ks] = row16(Cc, 16 * I + l16, 32 * ks + 8 * g4);
            }
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks) acc = mfma_bf16(bf[ks], cf[ks], acc);
        }
        reinterpret_cast<floatx4 *>(CB)[s * 64 + lane] = acc;
    }
}

}  // namespace ssd

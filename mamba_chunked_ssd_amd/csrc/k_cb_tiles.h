// k_cb_tiles.h -- the C B^T tiles that the chunk output with asynchronous
// copies reads (bf16 inputs, headdim 64, dstate 128, or dstate 256 at chunk
// 256; uses_cb_tiles), computed by extra blocks at the front of the launch that
// carries the state across chunks (the state-passing launch, or the fused state
// launch): a little MFMA work that depends only on B and C, so it runs beside
// the memory-bound state stream instead of on the chunk output's critical path
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Mamba-2 architecture": the C B^T factor of the chunk
// output).
#pragma once

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// C B^T tiles for the chunk-output stage (bf16 B and C, dstate N = 128 or 256,
// a template argument): tile (w, k) of (batch, chunk, group) is the 16 x 16
// block (I, J) of S_ij = C_i . B_j that the chunk output's wave w keeps in its
// slot k: I = w, J = k for k < (w + 2) & ~1, else I = T/16 - 1 - w and J = k
// minus that.  N / 32 MFMAs over dstate, loaded and issued 128 dstate entries
// at a time (the same registers at either N), in the MFMA output layout
// (lane 16 q + m holds S_{16I+m, 16J+4q+r}, r = 0..3), one float4 per lane,
// 1 KiB per tile.  Blocks past the diagonal are written as zero.  Each wave takes
// kCbPerWave tiles; these blocks run at the front of a state launch's grid,
// beside its memory-bound work.  bid: the block's index among the ncb tile
// blocks.
constexpr int kCbPerWave = 4;

// Blocks of 256 threads that compute `ntiles` tiles.
inline int64_t cb_blocks(int64_t ntiles) { return (ntiles + 4 * kCbPerWave - 1) / (4 * kCbPerWave); }

template <int T, int N>
__device__ __forceinline__ void cb_tiles(const uint16_t *__restrict__ Bm,
                                         const uint16_t *__restrict__ Cm, float *__restrict__ CB,
                                         int64_t seqlen, int G, int64_t nc, int64_t ntiles, int ncb, int bid) {
    constexpr int KH = 4;  // k-steps of 32 dstate entries per load group
    constexpr int NT16 = T / 16, NSLOT = NT16 + 2, NSL = (T / 32) * NSLOT;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    // consecutive tiles (one chunk's) on one XCD, whose L2 then serves B and
    // C (the tile blocks start the grid)
    const int64_t gw = (int64_t)xcd_remap(bid, ncb) * 4 + (threadIdx.x >> 6);
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
#pragma unroll 1
            for (int n0 = 0; n0 < N; n0 += 32 * KH) {
                u32x4 bf[KH], cf[KH];
#pragma unroll
                for (int ks = 0; ks < KH; ++ks) {
                    bf[ks] = row16(Bc, 16 * J + l16, n0 + 32 * ks + 8 * g4);
                    cf[ks] = row16(Cc, 16 * I + l16, n0 + 32 * ks + 8 * g4);
                }
#pragma unroll
                for (int ks = 0; ks < KH; ++ks) acc = mfma_bf16(bf[ks], cf[ks], acc);
            }
        }
        reinterpret_cast<floatx4 *>(CB)[s * 64 + lane] = acc;
    }
}

// The same tiles at dstate N = 256, for launches that can spend the
// registers: one wave per (batch, chunk, group, slot row w) computes the
// row's NSLOT tiles.  The C fragments of its two row tiles are loaded once
// and each B row tile once (the next one during the current one's MFMAs), so
// a chunk's B and C rows are read from L2 about once per slot row rather
// than twice per tile.  ntasks = batch * nchunks * G * T/32; bid as above.
template <int T, int N>
__device__ __forceinline__ void cb_rows(const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm,
                                        float *__restrict__ CB, int64_t seqlen, int G, int64_t nc,
                                        int64_t ntasks, int ncb, int bid) {
    constexpr int NK = N / 32, NT16 = T / 16, NSLOT = NT16 + 2, NW = T / 32;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    const int64_t task = (int64_t)xcd_remap(bid, ncb) * 4 + (threadIdx.x >> 6);  // (b, c, g, w)
    if (task >= ntasks) return;
    const int w = (int)(task % NW);
    const int64_t bcg = task / NW;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int64_t c = bc % nc, b = bc / nc;
    const int I0 = w, I1 = NT16 - 1 - w, base1 = (I0 + 2) & ~1;
    const int64_t t0 = c * T;
    const int rows = (int)min<int64_t>(T, seqlen - t0);
    const int64_t GN = (int64_t)G * N;
    const uint16_t *Bc = Bm + ((b * seqlen + t0) * G + g) * N;
    const uint16_t *Cc = Cm + ((b * seqlen + t0) * G + g) * N;
    // 16 bytes of a chunk row at dstate n0; rows past seqlen read as zero
    auto row16 = [&](const uint16_t *base, int row, int n0) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(base + (int64_t)min(row, rows - 1) * GN + n0);
        return row < rows ? v : u32x4{0u, 0u, 0u, 0u};
    };
    floatx4 *out = reinterpret_cast<floatx4 *>(CB) + task * NSLOT * 64 + lane;
    u32x4 cf[2][NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        cf[0][ks] = row16(Cc, 16 * I0 + l16, 32 * ks + 8 * g4);
        cf[1][ks] = row16(Cc, 16 * I1 + l16, 32 * ks + 8 * g4);
    }
    // slots past the diagonal: first-half slots after I0, and the second
    // half's last slot when it lies past I1
    for (int k = I0 + 1; k < base1; ++k) out[k * 64] = zero4();
    if (base1 + I1 + 1 < NSLOT) out[(base1 + I1 + 1) * 64] = zero4();
    u32x4 bcur[NK], bnxt[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) bcur[ks] = row16(Bc, l16, 32 * ks + 8 * g4);
#pragma unroll 1
    for (int J = 0; J <= I1; ++J) {
        const int Jn = min(J + 1, I1);
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) bnxt[ks] = row16(Bc, 16 * Jn + l16, 32 * ks + 8 * g4);
        floatx4 a1 = zero4();  // block (I1, J): second-half slot base1 + J
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) a1 = mfma_bf16(bcur[ks], cf[1][ks], a1);
        out[(base1 + J) * 64] = a1;
        if (J <= I0) {  // block (I0, J): first-half slot J
            floatx4 a0 = zero4();
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) a0 = mfma_bf16(bcur[ks], cf[0][ks], a0);
            out[J * 64] = a0;
        }
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) bcur[ks] = bnxt[ks];
    }
}

}  // namespace ssd

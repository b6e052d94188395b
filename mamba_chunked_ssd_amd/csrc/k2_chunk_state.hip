// k2_chunk_state.hip -- stage 2: the state each chunk contributes.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Mamba-2 architecture", log-space state jump
//     h_{t+T} = exp(G_last) h_t + (exp(G_last - G) . B) X^T ,
// whose second term is what a chunk adds to a zero state.  In the stored
// [headdim, dstate] orientation, for chunk c of (batch b, head h, group g):
//     s_c[p][n] = sum_t  w_t x_t[p] B_t[n],   w_t = exp2(G2_last - G2_t) dt_t ,
// a (T x P)^T (T x N) contraction over the chunk's tokens: a dense product,
// so it runs on MFMA.  The pages pre-multiply the rows of B (or of X) by the
// exponentials (same section); here the weights go on X, because B is shared
// by every head of a group and is staged once per block, while X is per head.
//
// Design for gfx950.  One block per (batch, chunk, group, run of heads of that
// group); wave w owns the 32 dstate columns [32w, 32w + 32) for all headdim
// rows; the bf16 path adds waves, if needed, so that every 8x8 unit of the
// x tile has a thread (such extra waves only stage x).
//  * bf16 inputs: v_mfma_f32_16x16x32_bf16.  The contraction index (token) is
//    the slow index of both operands in memory, so both are transposed
//    through LDS: each thread loads an 8-token x 8-column tile with 16-byte
//    global loads, transposes it in registers and writes 16-byte rows of the
//    transposed tile.  The 16-byte chunks of each LDS row are XOR-swizzled by
//    (row ^ row >> 3) & 15 (& 7 when a row has only 8 chunks), which makes
//    both those writes and the MFMA operand reads bank-conflict free (measured
//    with the LDS bank-conflict counter on gfx950).  B^T is staged once
//    per block and each wave keeps its B fragments in registers for all of
//    the block's heads.  w_t x_t is fp32-valued; it is split into a hi and a lo
//    bf16 (hi + lo keeps ~16 significant bits) and both halves are multiplied
//    by the exact bf16 B, which keeps the state within fp32-accumulation
//    accuracy instead of bf16 rounding.
//  * fp32 inputs: v_mfma_f32_16x16x4_f32.  Its operands carry one k value per
//    lane, so x and B are read in their natural token-major layout with no
//    transpose; B fragments come straight from global memory into registers,
//    and w_t x_t is staged in LDS in 64-token slabs.
// The next head's x tile is loaded into registers while the current head's
// MFMAs run.  Tokens past seqlen are zero-filled (the chunk is padded).
#include <algorithm>

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

// byte offset of 16-byte chunk `ch` of row `row` in a [rows][T] bf16 tile;
// chunks are XOR-swizzled within each row
template <int T>
__device__ __forceinline__ int tr_off(int row, int ch) {
    constexpr int M = (T / 8 >= 16) ? 15 : 7;  // T / 8 chunks per row
    return row * (T * 2) + ((ch ^ ((row ^ (row >> 3)) & M)) << 4);
}

// Transpose an 8x8 tile of bf16 held as 8 rows of 4 dwords (row r holds
// columns 2i, 2i+1 in dword i) into 8 columns of 4 dwords (column q holds rows
// 2i, 2i+1 in dword i).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int i = q >> 1;
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2)
            out[q][r2] = __builtin_amdgcn_perm(in[2 * r2 + 1][i], in[2 * r2][i], sel);
    }
}

// ---------------------------------------------------------------------------
// bf16 path
// ---------------------------------------------------------------------------
template <int T, int P>
__global__ __launch_bounds__(512) void k2_chunk_state_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const float *__restrict__ G2hi, const float *__restrict__ G2lo, const float *__restrict__ DT,
    float *__restrict__ S, int64_t L, int NH, int N, int G, int NC, int64_t Lp, int HPG, int HB,
    int nhb) {
    constexpr int KS = T / 32;   // k-steps of the contraction over tokens
    constexpr int PT = P / 16;   // 16-row tiles of headdim
    constexpr int TO = T / 8;    // token octets
    constexpr int PO = P / 8;    // headdim octets
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char *xhi = lds;                 // [P][T] bf16, swizzled
    unsigned char *xlo = lds + P * T * 2;     // [P][T] bf16, swizzled

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = bid % nhb;
    const int bcg = bid / nhb;
    const int gi = bcg % G;
    const int bc = bcg / G;
    const int c = bc % NC;
    const int64_t b = bc / NC;
    const int h_begin = gi * HPG + hb * HB;
    const int h_end = min(h_begin + HB, (gi + 1) * HPG);
    const int64_t t0 = (int64_t)c * T;

    // ---- stage B^T for this chunk in pieces that fit the x buffers; each wave
    //      keeps its own B fragments (32 columns, all tokens) in registers.
    u32x4 bfrag[KS][2];
    {
        constexpr int PIECE = 2 * P;  // columns per piece: PIECE * T * 2 B = 2 * P * T * 2 B
        for (int n_base = 0; n_base < N; n_base += PIECE) {
            const int ncols = min(PIECE, N - n_base);
            const int units = TO * (ncols / 8);
            for (int u = tid; u < units; u += nthr) {
                const int no = u % (ncols / 8), to = u / (ncols / 8);
                u32x4 rows[8], cols[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t tok = t0 + to * 8 + r;
                    rows[r] = u32x4{0u, 0u, 0u, 0u};
                    if (tok < L)
                        rows[r] = *reinterpret_cast<const u32x4 *>(
                            Bm + ((b * L + tok) * G + gi) * N + n_base + no * 8);
                }
                transpose8x8(rows, cols);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    *reinterpret_cast<u32x4 *>(lds + tr_off<T>(no * 8 + q, to)) = cols[q];
            }
            __syncthreads();
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int n = 32 * w + 16 * nt + l16;
                const bool mine = (n - n_base) >= 0 && (n - n_base) < ncols;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    if (mine)
                        bfrag[ks][nt] = *reinterpret_cast<const u32x4 *>(
                            lds + tr_off<T>(n - n_base, 4 * ks + g4));
                    else if (n_base == 0)
                        bfrag[ks][nt] = u32x4{0u, 0u, 0u, 0u};
            }
            __syncthreads();
        }
    }

    // ---- per head: x tile -> registers (prefetched one head ahead).  The
    //      launch gives every 8x8 (token, headdim) unit of the tile its own
    //      thread, so one pass covers the tile.
    const int units = TO * PO;
    const int u = tid;
    const int po = u % PO, to = u / PO;
    const bool has_unit = u < units;
    const bool wave_busy = 32 * w < N;  // waves past dstate only stage x
    // The unit's x rows and its 8 tokens' cumsum / dt values, loaded one head
    // ahead through per-head buffer resources (rows past seqlen read as 0).
    struct Pre {
        u32x4 rows[8];
        floatx4 gh[2], gl[2], dd[2];
        float lh, ll;
    };
    const int64_t rows_valid = min<int64_t>(T, L - t0);
    const uint32_t x_bytes = (uint32_t)(((rows_valid - 1) * NH * P + P) * 2);
    auto load_x = [&](int h, Pre &pre) {
        const auto xres = buffer_rsrc(x + ((b * L + t0) * NH + h) * P, x_bytes);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            pre.rows[r] = u32x4{0u, 0u, 0u, 0u};
            if (has_unit) pre.rows[r] = buffer_load_x4(xres, ((to * 8 + r) * NH * P + po * 8) * 2);
        }
        const int64_t hoff = ((int64_t)b * NH + h) * Lp + t0;
        const auto gh = buffer_rsrc(G2hi + hoff, T * 4), gl = buffer_rsrc(G2lo + hoff, T * 4);
        const auto dd = buffer_rsrc(DT + hoff, T * 4);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            pre.gh[q] = __builtin_bit_cast(floatx4, buffer_load_x4(gh, (to * 8 + 4 * q) * 4));
            pre.gl[q] = __builtin_bit_cast(floatx4, buffer_load_x4(gl, (to * 8 + 4 * q) * 4));
            pre.dd[q] = __builtin_bit_cast(floatx4, buffer_load_x4(dd, (to * 8 + 4 * q) * 4));
        }
        pre.lh = buffer_load_f32(gh, (T - 1) * 4);
        pre.ll = buffer_load_f32(gl, (T - 1) * 4);
    };
    // Scale by w_t = exp2(G2_last - G2_t) dt_t (G2 differences formed from the
    // hi/lo pair), split into hi/lo bf16 and
    // write the unit transposed into xhi / xlo.
    auto store_x = [&](const Pre &pre) {
        if (!has_unit) return;
        const u32x4 (&rows)[8] = pre.rows;
        const float lh = pre.lh, ll = pre.ll;
        float wt[8];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const floatx4 a = pre.gh[q], l = pre.gl[q], d = pre.dd[q];
#pragma unroll
            for (int i = 0; i < 4; ++i) wt[4 * q + i] = fast_exp2((lh - a[i]) + (ll - l[i])) * d[i];
        }
        u32x4 hi[8], lo[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
            {
                const HiLo s2 = split_bf16(bf16lo(rows[r][i]) * wt[r], bf16hi(rows[r][i]) * wt[r]);
                hi[r][i] = s2.hi;
                lo[r][i] = s2.lo;
            }
        u32x4 t8[8];
        transpose8x8(hi, t8);
#pragma unroll
        for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4 *>(xhi + tr_off<T>(po * 8 + q, to)) = t8[q];
        transpose8x8(lo, t8);
#pragma unroll
        for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4 *>(xlo + tr_off<T>(po * 8 + q, to)) = t8[q];
    };

    Pre pre;
    if (h_begin < h_end) load_x(h_begin, pre);

    for (int h = h_begin; h < h_end; ++h) {
        store_x(pre);
        __syncthreads();
        if (h + 1 < h_end) load_x(h + 1, pre);
        if (!wave_busy) {
            __syncthreads();
            continue;
        }
        // opaque lane coordinates: keeps the LDS offsets from being hoisted
        // out of the head loop into registers
        int tid_o = tid;
        asm volatile("" : "+v"(tid_o));
        const int l16 = tid_o & 15, g4 = (tid_o >> 4) & 3;

        floatx4 acc[PT][2];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt][0] = acc[pt][1] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int off = tr_off<T>(16 * pt + l16, 4 * ks + g4);
                const u32x4 ah = *reinterpret_cast<const u32x4 *>(xhi + off);
                const u32x4 al = *reinterpret_cast<const u32x4 *>(xlo + off);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    acc[pt][nt] = mfma_bf16(ah, bfrag[ks][nt], acc[pt][nt]);
                    acc[pt][nt] = mfma_bf16(al, bfrag[ks][nt], acc[pt][nt]);
                }
            }
        }
        float *out = S + (((int64_t)b * NH + h) * NC + c) * (int64_t)P * N;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int n = 32 * w + 16 * nt + l16;
                if (n < N)
#pragma unroll
                    for (int r = 0; r < 4; ++r) out[(16 * pt + 4 * g4 + r) * N + n] = acc[pt][nt][r];
            }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
constexpr int kSlab = 64;  // tokens of w*x staged in LDS at a time

template <int T, int P>
__global__ __launch_bounds__(512) void k2_chunk_state_f32(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ G2hi,
    const float *__restrict__ G2lo, const float *__restrict__ DT, float *__restrict__ S, int64_t L,
    int NH, int N, int G, int NC, int64_t Lp, int HPG, int HB, int nhb) {
    constexpr int KS = T / 4;        // k-steps (4 tokens each) over the chunk
    constexpr int PT = P / 16;
    constexpr int LDP = P + 16;      // padded LDS row (floats)
    constexpr int SLAB_KS = kSlab / 4;
    __shared__ __align__(16) float xs[kSlab * LDP];

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int hb = bid % nhb;
    const int bcg = bid / nhb;
    const int gi = bcg % G;
    const int bc = bcg / G;
    const int c = bc % NC;
    const int64_t b = bc / NC;
    const int h_begin = gi * HPG + hb * HB;
    const int h_end = min(h_begin + HB, (gi + 1) * HPG);
    const int64_t t0 = (int64_t)c * T;

    // B fragments: lane holds B[t = 4ks + g4][n = 32w + 16nt + l16]
    float bfrag[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = 32 * w + 16 * nt + l16;
            const int64_t tok = t0 + 4 * ks + g4;
            bfrag[ks][nt] = (n < N && tok < L) ? Bm[((b * L + tok) * G + gi) * N + n] : 0.f;
        }

    for (int h = h_begin; h < h_end; ++h) {
        const int64_t hoff = ((int64_t)b * NH + h) * Lp + t0;
        const float *gh = G2hi + hoff;
        const float *gl = G2lo + hoff;
        const float *dd = DT + hoff;
        const float lh = gh[T - 1], ll = gl[T - 1];
        int tid_o = tid;  // opaque lane coordinates, as in the bf16 kernel
        asm volatile("" : "+v"(tid_o));
        const int l16 = tid_o & 15, g4 = (tid_o >> 4) & 3;
        floatx4 acc[PT][2];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt][0] = acc[pt][1] = zero4();
#pragma unroll
        for (int slab = 0; slab < T / kSlab; ++slab) {
            // stage w_t x_t for tokens [slab*64, slab*64 + 64)
            for (int v = tid; v < kSlab * (P / 4); v += nthr) {
                const int tt = v / (P / 4), p4 = v % (P / 4);
                const int t = slab * kSlab + tt;
                float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (t0 + t < L) {
                    xv = *reinterpret_cast<const float4 *>(x + ((b * L + t0 + t) * NH + h) * P + 4 * p4);
                    const float wt = fast_exp2((lh - gh[t]) + (ll - gl[t])) * dd[t];
                    xv.x *= wt; xv.y *= wt; xv.z *= wt; xv.w *= wt;
                }
                *reinterpret_cast<float4 *>(&xs[tt * LDP + 4 * p4]) = xv;
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < SLAB_KS; ++ks) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const float a = xs[(4 * ks + g4) * LDP + 16 * pt + l16];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        acc[pt][nt] = mfma_f32(a, bfrag[slab * SLAB_KS + ks][nt], acc[pt][nt]);
                }
            }
            __syncthreads();
        }
        float *out = S + (((int64_t)b * NH + h) * NC + c) * (int64_t)P * N;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int n = 32 * w + 16 * nt + l16;
                if (n < N)
#pragma unroll
                    for (int r = 0; r < 4; ++r) out[(16 * pt + 4 * g4 + r) * N + n] = acc[pt][nt][r];
            }
    }
}

template <int T, int P>
hipError_t launch_tp(const Problem &p, const Plan &plan, const void *x, const void *B,
                     G2View G2, const float *DT, float *S, hipStream_t stream) {
    const int HB = plan.k2_heads_per_block;
    const int nhb = (int)((p.heads_per_group + HB - 1) / HB);
    const int64_t blocks = p.batch * p.nchunks * p.ngroups * nhb;
    if (blocks == 0) return hipSuccess;
    if (p.bf16) {
        // one 8x8 (token, headdim) unit of the x tile per thread
        const int waves = (int)std::max<int64_t>((p.dstate + 31) / 32, (T / 8) * (P / 8) / 64);
        constexpr size_t lds = (size_t)2 * P * T * 2;
        static_assert(lds <= 160 * 1024, "stage-2 LDS budget exceeded");
        if (allow_lds<k2_chunk_state_bf16<T, P>>(lds) != hipSuccess) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k2_chunk_state_bf16<T, P>), dim3((unsigned)blocks), dim3(64 * waves),
                           lds, stream, static_cast<const uint16_t *>(x),
                           static_cast<const uint16_t *>(B), G2.hi, G2.lo, DT, S, p.seqlen,
                           (int)p.nheads,
                           (int)p.dstate, (int)p.ngroups, (int)p.nchunks, p.padded_len,
                           (int)p.heads_per_group, HB, nhb);
    } else {
        const int waves = (int)((p.dstate + 31) / 32);
        hipLaunchKernelGGL((k2_chunk_state_f32<T, P>), dim3((unsigned)blocks), dim3(64 * waves), 0,
                           stream, static_cast<const float *>(x), static_cast<const float *>(B),
                           G2.hi, G2.lo, DT, S, p.seqlen, (int)p.nheads, (int)p.dstate,
                           (int)p.ngroups,
                           (int)p.nchunks, p.padded_len, (int)p.heads_per_group, HB, nhb);
    }
    return hipGetLastError();
}

template <int T>
hipError_t launch_t(const Problem &p, const Plan &plan, const void *x, const void *B,
                    G2View G2, const float *DT, float *S, hipStream_t stream) {
    switch (p.headdim) {
        case 32: return launch_tp<T, 32>(p, plan, x, B, G2, DT, S, stream);
        case 64: return launch_tp<T, 64>(p, plan, x, B, G2, DT, S, stream);
        case 128: return launch_tp<T, 128>(p, plan, x, B, G2, DT, S, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_state(const Problem &p, const Plan &plan, const void *x, const void *B,
                              G2View G2, const float *DT, float *S, hipStream_t stream) {
    switch (p.chunk) {
        case 64: return launch_t<64>(p, plan, x, B, G2, DT, S, stream);
        case 128: return launch_t<128>(p, plan, x, B, G2, DT, S, stream);
        case 256: return launch_t<256>(p, plan, x, B, G2, DT, S, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd

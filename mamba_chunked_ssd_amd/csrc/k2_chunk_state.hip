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
#include <type_traits>
#include <utility>

#include "ssd_device.h"
#include "ssd_launch.h"

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

// compile-time loop
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// bf16 path
// ---------------------------------------------------------------------------
template <int T, int P>
__global__ __launch_bounds__(512) void k2_chunk_state_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const float *__restrict__ W, float *__restrict__ S, int64_t L, int NH, int N, int G, int NC, int64_t Lp, int HPG, int HB,
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

    // ---- per head: x tile -> registers (prefetched one head ahead).  The
    //      launch gives every 8x8 (token, headdim) unit of the tile its own
    //      thread, so one pass covers the tile.
    const int units = TO * PO;
    const int u = tid;
    const int po = u % PO, to = u / PO;
    const bool has_unit = u < units;
    const bool wave_busy = 32 * w < N;  // waves past dstate only stage x
    // The unit's x rows and its 8 tokens' weights, loaded one head ahead
    // through per-head buffer resources (rows past seqlen read as 0).
    struct Pre {
        u32x4 rows[8];
        floatx4 wv[2];
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
        const auto wr = buffer_rsrc(W + ((int64_t)b * NH + h) * Lp + t0, T * 4);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            pre.wv[q] = __builtin_bit_cast(floatx4, buffer_load_x4(wr, (to * 8 + 4 * q) * 4));
    };
    // Scale by w_t, split into hi/lo bf16 and write the unit transposed into
    // xhi / xlo.
    auto store_x = [&](const Pre &pre) {
        if (!has_unit) return;
        const u32x4 (&rows)[8] = pre.rows;
        float wt[8];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) wt[4 * q + i] = pre.wv[q][i];
        // one pair of columns (dword i of every row) at a time: split, then
        // transpose into LDS rows 8 po + 2i and 8 po + 2i + 1 of both tiles
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t hi[8], lo[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const HiLo s2 = split_bf16(bf16lo(rows[r][i]) * wt[r], bf16hi(rows[r][i]) * wt[r]);
                hi[r] = s2.hi;
                lo[r] = s2.lo;
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t sel = half ? 0x07060302u : 0x05040100u;
                const int row = po * 8 + 2 * i + half;
                u32x4 th, tl;
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) {
                    th[r2] = __builtin_amdgcn_perm(hi[2 * r2 + 1], hi[2 * r2], sel);
                    tl[r2] = __builtin_amdgcn_perm(lo[2 * r2 + 1], lo[2 * r2], sel);
                }
                *reinterpret_cast<u32x4 *>(xhi + tr_off<T>(row, to)) = th;
                *reinterpret_cast<u32x4 *>(xlo + tr_off<T>(row, to)) = tl;
            }
        }
    };

    Pre pre;
    if (h_begin < h_end) load_x(h_begin, pre);  // in flight during the B^T staging

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


    // A head's states are stored after the next head's staging: on this
    // architecture one counter tracks both loads and stores, so the wait for
    // the prefetched loads would otherwise also wait for the stores to land.
    floatx4 accd[PT][2];  // the previous head's states
    auto store_states = [&](int h, const auto &acc) {
        // lane coordinates from an opaque copy of the thread index, so the
        // store addresses are formed here rather than hoisted out of the loop
        int tid_o = tid;
        asm volatile("" : "+v"(tid_o));
        const int l16 = tid_o & 15, g4 = (tid_o >> 4) & 3;
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
    };
    for (int h = h_begin; h < h_end; ++h) {
        store_x(pre);
        if (h > h_begin && wave_busy) store_states(h - 1, accd);
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
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) accd[pt][0] = acc[pt][0], accd[pt][1] = acc[pt][1];
        __syncthreads();
    }
    if (h_begin < h_end && wave_busy) store_states(h_end - 1, accd);
}

// ---------------------------------------------------------------------------
// bf16 path with producer and consumer waves
// ---------------------------------------------------------------------------
// When two x^T hi/lo tile pairs fit in LDS (8 P T bytes) and dstate <= 128
// (at most 4 consumer waves, so 8 waves hold the B fragments without
// spilling), kProducers waves
// stage head k + 1 (x and weights loaded one head further ahead; scale, split,
// transpose) into one buffer while ceil(N / 32) consumer waves run head k's
// MFMAs from the other and store its states: one block barrier per head, and
// the staging (VALU) of one head overlaps the MFMAs of the previous one on
// every SIMD.  Consumers keep their B fragments in registers for the block's
// heads; they never load from global memory in the head loop, and producers
// never store to it, so neither role waits on the other's memory traffic.
constexpr int kProducers = 4;

template <int T, int P>
struct K2WsLds {
    static constexpr size_t buf = (size_t)2 * P * T * 2;  // hi + lo tiles of one head
    static constexpr size_t total = 2 * buf;
    static constexpr bool fits = total <= 160 * 1024;
    // dstate 128: each consumer wave's 32 B columns (T rows of 64 bytes) fit
    // in the second buffer
    static constexpr bool b_cols_fit = (size_t)T * 256 <= buf;
};

// A consumer wave's 32 columns of the chunk's B rows in LDS: T rows of 64
// bytes, the 16-byte chunk q of row t at chunk q ^ b_swz(t).  A transposing
// read (4 consecutive tokens x 16 columns per 16 lanes) by half a wave covers
// rows t .. t + 3 and t + 8 .. t + 11 (t a multiple of 4): four 64-byte bank
// quarters (t mod 4), each shared by two rows that the swizzle puts in
// different halves -- no bank conflicts.
__device__ __forceinline__ int b_swz(int t) { return 2 * ((t >> 3) & 1); }

template <int T, int P, int NCW>
__global__ __launch_bounds__(64 * (kProducers + NCW)) void k2_chunk_state_bf16_ws(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm, const float *__restrict__ W,
    float *__restrict__ S, int64_t L, int NH, int N, int G, int NC, int64_t Lp, int HPG, int HB,
    int nhb) {
    constexpr int KS = T / 32;   // k-steps of the contraction over tokens
    constexpr int PT = P / 16;   // 16-row tiles of headdim
    constexpr int TO = T / 8;    // token octets
    constexpr int PO = P / 8;    // headdim octets
    constexpr int NTHR = 64 * (kProducers + NCW);
    constexpr int PTHR = 64 * kProducers;
    constexpr size_t BUF = K2WsLds<T, P>::buf;
    constexpr int XU = TO * PO;  // x units of 8 tokens x 8 columns
    constexpr int XPASS = (XU + PTHR - 1) / PTHR;
    static_assert(K2WsLds<T, P>::fits, "two x^T buffers must fit in LDS");
    extern __shared__ __align__(16) unsigned char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const bool producer = w < kProducers;
    const int cw = w - kProducers;  // consumer wave: dstate columns [32 cw, 32 cw + 32)

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

    // ---- producer side: x rows and weights of XPASS units, one head ahead,
    //      through per-head buffer resources (rows past seqlen read as 0)
    struct Pre {
        u32x4 rows[8];
        floatx4 wv[2];
    };
    Pre pre[XPASS];
    const int64_t rows_valid = min<int64_t>(T, L - t0);
    const uint32_t x_bytes = (uint32_t)(((rows_valid - 1) * NH * P + P) * 2);
    auto unit = [&](int ps, int &po, int &to) __attribute__((always_inline)) {
        const int u = tid + ps * PTHR;
        po = u % PO;
        to = u / PO;
        return u < XU;
    };
    auto load_x = [&](int h) __attribute__((always_inline)) {
        const auto xres = buffer_rsrc(x + ((b * L + t0) * NH + h) * P, x_bytes);
        const auto wr = buffer_rsrc(W + ((int64_t)b * NH + h) * Lp + t0, T * 4);
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            int po, to;
            if (!unit(ps, po, to)) continue;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                pre[ps].rows[r] = buffer_load_x4(xres, ((to * 8 + r) * NH * P + po * 8) * 2);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                pre[ps].wv[q] = __builtin_bit_cast(floatx4, buffer_load_x4(wr, (to * 8 + 4 * q) * 4));
        }
    };
    // scale by w_t, split into hi/lo bf16, write transposed into buffer `bf`
    auto store_x = [&](int bf) __attribute__((always_inline)) {
        unsigned char *xhi = lds + bf * BUF;
        unsigned char *xlo = xhi + P * T * 2;
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            int po, to;
            if (!unit(ps, po, to)) continue;
            float wt[8];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) wt[4 * q + i] = pre[ps].wv[q][i];
            // one pair of columns (dword i of every row) at a time
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hi[8], lo[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const uint32_t v = pre[ps].rows[r][i];
                    const HiLo s2 = split_bf16(bf16lo(v) * wt[r], bf16hi(v) * wt[r]);
                    hi[r] = s2.hi;
                    lo[r] = s2.lo;
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t sel = half ? 0x07060302u : 0x05040100u;
                    const int row = po * 8 + 2 * i + half;
                    u32x4 th, tl;
#pragma unroll
                    for (int r2 = 0; r2 < 4; ++r2) {
                        th[r2] = __builtin_amdgcn_perm(hi[2 * r2 + 1], hi[2 * r2], sel);
                        tl[r2] = __builtin_amdgcn_perm(lo[2 * r2 + 1], lo[2 * r2], sel);
                    }
                    *reinterpret_cast<u32x4 *>(xhi + tr_off<T>(row, to)) = th;
                    *reinterpret_cast<u32x4 *>(xlo + tr_off<T>(row, to)) = tl;
                }
            }
        }
    };
    if (producer && h_begin < h_end) load_x(h_begin);  // in flight during the B^T staging

    // ---- B for this chunk; each consumer wave keeps its fragments in
    //      registers.  With dstate 128 each consumer wave copies its own 32
    //      columns of the chunk's rows straight into the second buffer
    //      (asynchronous copies, 16 bytes per lane; rows past seqlen read as
    //      zero) and reads them back transposed, 4 tokens per read -- no
    //      barrier, and the producers stage head 0 into the first buffer
    //      meanwhile.  Otherwise all threads stage B^T through registers.
    u32x4 bfrag[KS][2];
    const bool b_async = K2WsLds<T, P>::b_cols_fit && N == 128;
    if (b_async) {
        if (!producer && K2WsLds<T, P>::b_cols_fit) {
            const int64_t rows_b = min<int64_t>(T, L - t0);
            const int cwu = __builtin_amdgcn_readfirstlane(cw);
            const i32x4 bd = buffer_desc(Bm + ((b * L + t0) * G + gi) * 128 + 32 * cwu,
                                         (uint32_t)(((rows_b - 1) * G * 128 + 32) * 2));
            unsigned char *breg = lds + BUF + cwu * (T * 64);
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int k = 0; k < T / 16; ++k) {  // 1-KiB copies: 16 rows of 64 bytes
                const int t = 16 * k + (ln >> 2);
                lds_dma_x4(bd, lds_addr(breg + k * 1024), (t * G * 128 + 8 * ((ln & 3) ^ b_swz(t))) * 2);
            }
            lds_dma_wait();
            const int r = l16 >> 2, a = l16 & 3;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int ch = 2 * nt + (a >> 1);
                    u32x2 v[2];
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int t = 32 * ks + 8 * g4 + 4 * hf + r;
                        v[hf] = tr_read(breg + t * 64 + ((ch ^ b_swz(t)) << 4) + 8 * (a & 1));
                    }
                    bfrag[ks][nt] = u32x4{v[0][0], v[0][1], v[1][0], v[1][1]};
                }
        }
    } else {
        constexpr int PIECE = (int)(2 * BUF / (T * 2)) < 256 ? (int)(2 * BUF / (T * 2)) : 256;
        for (int n_base = 0; n_base < N; n_base += PIECE) {
            const int ncols = min(PIECE, N - n_base);
            const int units = TO * (ncols / 8);
            for (int u = tid; u < units; u += NTHR) {
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
            if (!producer) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int n = 32 * cw + 16 * nt + l16;
                    const bool mine = (n - n_base) >= 0 && (n - n_base) < ncols;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        if (mine)
                            bfrag[ks][nt] = *reinterpret_cast<const u32x4 *>(
                                lds + tr_off<T>(n - n_base, 4 * ks + g4));
                        else if (n_base == 0)
                            bfrag[ks][nt] = u32x4{0u, 0u, 0u, 0u};
                }
            }
            __syncthreads();
        }
    }

    // ---- heads: producers stage head i + 1 while consumers compute head i
    if (producer && h_begin < h_end) {
        store_x(0);
        if (h_begin + 1 < h_end) load_x(h_begin + 1);
    }
    __syncthreads();
    for (int i = 0; h_begin + i < h_end; ++i) {
        const int h = h_begin + i;
        if (producer) {
            if (h + 1 < h_end) {
                store_x((i + 1) & 1);
                if (h + 2 < h_end) load_x(h + 2);
            }
        } else if (32 * cw < N) {
            // opaque lane coordinates: keeps the LDS and store offsets from
            // being hoisted out of the head loop into registers
            int tid_o = tid;
            asm volatile("" : "+v"(tid_o));
            const int ol16 = tid_o & 15, og4 = (tid_o >> 4) & 3;
            const unsigned char *xhi = lds + (i & 1) * BUF;
            const unsigned char *xlo = xhi + P * T * 2;
            floatx4 acc[PT][2];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt][0] = acc[pt][1] = zero4();
            // x^T fragments of one k-step, read one step ahead of their MFMAs
            struct Frags {
                u32x4 h[PT], l[PT];
            };
            auto read = [&](int ks) {
                Frags f;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int off = tr_off<T>(16 * pt + ol16, 4 * ks + og4);
                    f.h[pt] = *reinterpret_cast<const u32x4 *>(xhi + off);
                    f.l[pt] = *reinterpret_cast<const u32x4 *>(xlo + off);
                }
                return f;
            };
            Frags cur = read(0);
            static_for<KS>([&](auto kc) {
                constexpr int ks = decltype(kc)::value;
                Frags nxt;
                if constexpr (ks + 1 < KS) nxt = read(ks + 1);
                // hi products of every tile first, then lo: dependent MFMAs
                // (same accumulator) are never adjacent.  B is the A operand
                // and x^T the B operand, so a tile comes out transposed: lane
                // (l16, g4) holds the state's row 16 pt + l16, columns
                // 16 nt + 4 g4 .. +3 -- one 16-byte store.
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) acc[pt][nt] = mfma_bf16(bfrag[ks][nt], cur.h[pt], acc[pt][nt]);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) acc[pt][nt] = mfma_bf16(bfrag[ks][nt], cur.l[pt], acc[pt][nt]);
                if constexpr (ks + 1 < KS) cur = nxt;
                __builtin_amdgcn_sched_barrier(0);
            });
            float *out = S + (((int64_t)b * NH + h) * NC + c) * (int64_t)P * N;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int n0 = 32 * cw + 16 * nt;  // dstate is a multiple of 16
                    if (n0 < N)
                        *reinterpret_cast<floatx4 *>(out + (16 * pt + ol16) * N + n0 + 4 * og4) = acc[pt][nt];
                }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
constexpr int kSlab = 64;  // tokens of w*x staged in LDS at a time

// With PF (eight waves, dstate > 224; not chunk 256 with headdim 128, which
// has no registers left for it) the x rows and weights of the next
// (head, slab) step are loaded into registers while the current slab's MFMAs
// run, instead of after them.
template <int T, int P, bool PF>
__global__ __launch_bounds__(512) void k2_chunk_state_f32(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ W,
    float *__restrict__ S, int64_t L,
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

    constexpr int NSL = T / kSlab;
    constexpr int XV = kSlab * (P / 4);              // float4 units of a slab
    constexpr int XPT = PF ? (XV + 511) / 512 : 1;   // per thread (PF: 512 threads)
    struct XPre {
        float4 v[XPT];
        float wt[XPT];
    };
    XPre pre;
    auto pre_load = [&](int h, int slab) {
        const float *wh = W + ((int64_t)b * NH + h) * Lp + t0;
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int v = tid + q * 512;
            const int tt = v / (P / 4), p4 = v % (P / 4);
            const int t = slab * kSlab + tt;
            pre.v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            pre.wt[q] = 0.f;
            if (v < XV && t0 + t < L) {
                pre.v[q] = *reinterpret_cast<const float4 *>(x + ((b * L + t0 + t) * NH + h) * P + 4 * p4);
                pre.wt[q] = wh[t];
            }
        }
    };
    if constexpr (PF)
        if (h_begin < h_end) pre_load(h_begin, 0);

    for (int h = h_begin; h < h_end; ++h) {
        const float *wh = W + ((int64_t)b * NH + h) * Lp + t0;
        int tid_o = tid;  // opaque lane coordinates, as in the bf16 kernel
        asm volatile("" : "+v"(tid_o));
        const int l16 = tid_o & 15, g4 = (tid_o >> 4) & 3;
        floatx4 acc[PT][2];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt][0] = acc[pt][1] = zero4();
#pragma unroll
        for (int slab = 0; slab < NSL; ++slab) {
            // stage w_t x_t for tokens [slab*64, slab*64 + 64)
            if constexpr (PF) {
#pragma unroll
                for (int q = 0; q < XPT; ++q) {
                    const int v = tid + q * 512;
                    if (v < XV) {
                        const int tt = v / (P / 4), p4 = v % (P / 4);
                        float4 xv = pre.v[q];
                        const float wt = pre.wt[q];
                        xv.x *= wt; xv.y *= wt; xv.z *= wt; xv.w *= wt;
                        *reinterpret_cast<float4 *>(&xs[tt * LDP + 4 * p4]) = xv;
                    }
                }
            } else {
                for (int v = tid; v < XV; v += nthr) {
                    const int tt = v / (P / 4), p4 = v % (P / 4);
                    const int t = slab * kSlab + tt;
                    float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (t0 + t < L) {
                        xv = *reinterpret_cast<const float4 *>(x + ((b * L + t0 + t) * NH + h) * P + 4 * p4);
                        const float wt = wh[t];
                        xv.x *= wt; xv.y *= wt; xv.z *= wt; xv.w *= wt;
                    }
                    *reinterpret_cast<float4 *>(&xs[tt * LDP + 4 * p4]) = xv;
                }
            }
            __syncthreads();
            if constexpr (PF) {  // the next step's rows, in flight during this slab's MFMAs
                if (slab + 1 < NSL)
                    pre_load(h, slab + 1);
                else if (h + 1 < h_end)
                    pre_load(h + 1, 0);
            }
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
                     const float *W, float *S, hipStream_t stream, const LaunchEvents &ev) {
    const int HB = plan.k2_heads_per_block;
    const int nhb = (int)((p.heads_per_group + HB - 1) / HB);
    const int64_t blocks = p.batch * p.nchunks * p.ngroups * nhb;
    if (blocks == 0) return hipSuccess;
    if (p.bf16 && p.dstate <= 128 && K2WsLds<T, P>::fits) {
        if constexpr (K2WsLds<T, P>::fits) {
            constexpr size_t lds = K2WsLds<T, P>::total;
            auto go = [&](auto kern, int ncw) -> hipError_t {
                if (allow_lds<decltype(kern)::value>(lds) != hipSuccess) return hipErrorInvalidValue;
                launch_kernel(decltype(kern)::value, dim3((unsigned)blocks),
                                   dim3(64 * (kProducers + ncw)), lds, stream, ev,
                                   static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B),
                                   W, S, p.seqlen, (int)p.nheads, (int)p.dstate, (int)p.ngroups,
                                   (int)p.nchunks, p.padded_len, (int)p.heads_per_group, HB, nhb);
                return hipSuccess;
            };
            const hipError_t e =
                p.dstate <= 64
                    ? go(std::integral_constant<decltype(&k2_chunk_state_bf16_ws<T, P, 2>),
                                                &k2_chunk_state_bf16_ws<T, P, 2>>{}, 2)
                    : go(std::integral_constant<decltype(&k2_chunk_state_bf16_ws<T, P, 4>),
                                                &k2_chunk_state_bf16_ws<T, P, 4>>{}, 4);
            if (e != hipSuccess) return e;
        }
    } else if (p.bf16) {
        // one 8x8 (token, headdim) unit of the x tile per thread
        const int waves = (int)std::max<int64_t>((p.dstate + 31) / 32, (T / 8) * (P / 8) / 64);
        constexpr size_t lds = (size_t)2 * P * T * 2;
        static_assert(lds <= 160 * 1024, "stage-2 LDS budget exceeded");
        if (allow_lds<k2_chunk_state_bf16<T, P>>(lds) != hipSuccess) return hipErrorInvalidValue;
        launch_kernel((k2_chunk_state_bf16<T, P>), dim3((unsigned)blocks), dim3(64 * waves),
                           lds, stream, ev, static_cast<const uint16_t *>(x),
                           static_cast<const uint16_t *>(B), W, S, p.seqlen, (int)p.nheads,
                           (int)p.dstate, (int)p.ngroups, (int)p.nchunks, p.padded_len,
                           (int)p.heads_per_group, HB, nhb);
    } else {
        const int waves = (int)((p.dstate + 31) / 32);
        // (chunk 256 with headdim 128 has no registers left for the prefetch)
        constexpr bool kPfOk = !(T == 256 && P == 128);
        if (kPfOk && waves == 8)
            launch_kernel((k2_chunk_state_f32<T, P, kPfOk>), dim3((unsigned)blocks), dim3(512), 0, stream, ev,
                          static_cast<const float *>(x), static_cast<const float *>(B), W, S, p.seqlen,
                          (int)p.nheads, (int)p.dstate, (int)p.ngroups, (int)p.nchunks, p.padded_len,
                          (int)p.heads_per_group, HB, nhb);
        else
            launch_kernel((k2_chunk_state_f32<T, P, false>), dim3((unsigned)blocks), dim3(64 * waves), 0,
                          stream, ev, static_cast<const float *>(x), static_cast<const float *>(B), W, S,
                          p.seqlen, (int)p.nheads, (int)p.dstate, (int)p.ngroups, (int)p.nchunks,
                          p.padded_len, (int)p.heads_per_group, HB, nhb);
    }
    return hipGetLastError();
}

template <int T>
hipError_t launch_t(const Problem &p, const Plan &plan, const void *x, const void *B,
                    const float *W, float *S, hipStream_t stream, const LaunchEvents &ev) {
    switch (p.headdim) {
        case 32: return launch_tp<T, 32>(p, plan, x, B, W, S, stream, ev);
        case 64: return launch_tp<T, 64>(p, plan, x, B, W, S, stream, ev);
        case 128: return launch_tp<T, 128>(p, plan, x, B, W, S, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int chunk_state_blocks_per_cu(const Problem &p) {
    size_t lds = 0;
    if (p.bf16) {
        // producer/consumer variant (two x^T hi/lo buffers) when it applies
        const size_t ws = (size_t)8 * p.headdim * p.chunk;
        lds = (ws <= 160 * 1024 && p.dstate <= 128) ? ws : (size_t)4 * p.headdim * p.chunk;
    } else {
        lds = (size_t)kSlab * (p.headdim + 16) * 4;
    }
    const size_t by_lds = (160 * 1024) / std::max<size_t>(lds, 1);
    return (int)std::max<size_t>(1, std::min<size_t>(2, by_lds));
}

hipError_t launch_chunk_state(const Problem &p, const Plan &plan, const void *x, const void *B,
                              const float *W, float *S, hipStream_t stream, const LaunchEvents &ev) {
    switch (p.chunk) {
        case 64: return launch_t<64>(p, plan, x, B, W, S, stream, ev);
        case 128: return launch_t<128>(p, plan, x, B, W, S, stream, ev);
        case 256: return launch_t<256>(p, plan, x, B, W, S, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd

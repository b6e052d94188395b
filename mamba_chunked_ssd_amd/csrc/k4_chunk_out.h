// k4_chunk_out.h -- stage 4: the chunk output, fused (kernel templates; the
// k4_*.hip translation units instantiate them per input/output type).
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Mamba-2 architecture", chunk output with decay
//     Y = exp(G) C h_c + (exp(G - G^T) . (C B^T) . M) X + D X ,
// M the causal mask that keeps the diagonal, B the dt-scaled rows, h_c the
// state at the chunk start (stage 3).  Element-wise, for row i of the chunk:
//     y_i = exp2(G2_i) C_i h_c + sum_{j<=i} exp2(G2_i - G2_j) (C_i . B_j) dt_j x_j + D x_i .
// The masked decay factors for j > i would be exponentials of positive numbers;
// they are never used (the mask is a select applied before they could enter a
// product), which is the stability argument of the same section.  The
// interaction matrix exists only in registers: it never touches LDS or HBM.
//
// Design for gfx950.  One block per (batch, chunk, group, run of heads of that
// group), T/32 waves.  The chunk's 16-token row tiles are dealt to waves in
// pairs (w, T/16 - 1 - w) so every wave owns the same number of lower-
// triangular 16x16 tiles.  C B^T depends on the group only, so each wave
// computes its tiles of it once, in fp32 MFMA accumulators, and keeps them in
// registers for all of the block's heads; per head it only re-applies the
// head's decay and dt.  The tiles are computed transposed (A = B rows,
// B = C rows), which leaves every lane holding 4 consecutive columns j of one
// row i: an A-operand fragment of the next product, up to a fixed relabelling
// of the contraction index that the X operand reads mirror.
//  * bf16 inputs: v_mfma_f32_16x16x32_bf16.  X is staged per head in LDS
//    transposed ([headdim][token]); h_c arrives from the state-passing stage
//    as hi/lo bf16 planes and is staged as is.  The
//    fp32-valued operands -- the decay-masked tile and h_c -- are split into
//    hi + lo bf16 halves and multiplied by the exact bf16 inputs, so the
//    result keeps fp32-accumulation accuracy.
//  * fp32 inputs: v_mfma_f32_16x16x4_f32 on the fp32 values directly; X is
//    staged in its natural layout, h_c and C fragments are read from global
//    memory (L2) as 16-byte vectors.
// Per head, the block tabulates in LDS what every lane would otherwise
// recompute: exp2(G2_i) (row decay of the carried-state term), the column
// factor exp2(G2_e - G2_j) dt_j with e the last token of j's 16-token tile,
// and the row factor exp2(G2_i - G2_e(J)) for every row i and earlier tile J.
// An off-diagonal tile (J < I) then takes exp2(G2_i - G2_j) dt_j as
// rowfactor(i, J) * colfactor(j): both factors have exponents <= 0, so neither
// can overflow.  Only the diagonal tile evaluates per-element exponentials.
// All G2 differences are formed from the fp64-derived hi/lo pair.
//
// LDS layouts (bank-conflict free on gfx950, measured with
// SQ_LDS_BANK_CONFLICT): the transposed x tile uses rows of 2T + 16 bytes
// (64-bit operand reads by 32 lanes hit 32 distinct 8-byte bank groups); the
// h tile uses rows of 2 NPAD + 32 bytes (128-bit reads).  Both are read at a
// per-lane base plus compile-time immediates.  When it fits, each wave parks
// its C fragments in an unpadded C tile whose 16-byte chunks are XOR-swizzled
// by (row & 15) instead of holding them in registers for the whole block.  The next head's x, h_c and
// decay data are loaded into registers while the current head computes.
#pragma once

#include <utility>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace k4 {

// gfx950 LDS per CU (and the most one block may use)
constexpr size_t kLdsBytes = 160 * 1024;


// Wave w owns row tiles I0 = w and I1 = T/16 - 1 - w.  Its S slots are laid
// out as [I0: J = 0..I0][pad to even][I1: J = 0..I1][pad to even]; the total
// is always T/16 + 2 and a pair (2q, 2q + 1) never straddles the two tiles.
__device__ __forceinline__ int slot_base1(int I0) { return (I0 + 2) & ~1; }

// Per-head tables in LDS (T floats each):
//   gh[t] + gl[t] = G2_t (hi/lo),  dt[t],  e2[t] = exp2(G2_t),
//   cf[t] = exp2(G2_e(t) - G2_t) dt_t,  e(t) = last token of t's 16-tile.
template <int T>
struct Tables {
    float *gh, *gl, *dt, *e2, *cf;
    static constexpr size_t bytes = (size_t)5 * T * 4;
    __device__ Tables(float *base)
        : gh(base), gl(base + T), dt(base + 2 * T), e2(base + 3 * T), cf(base + 4 * T) {}
    // G2 at the last token before row tile I (G2 before the chunk is 0)
    __device__ float before_hi(int I) const { return I > 0 ? gh[16 * I - 1] : 0.f; }
    __device__ float before_lo(int I) const { return I > 0 ? gl[16 * I - 1] : 0.f; }
};

// Per-token part of the tables (thread t < T), from its G2 pair, the pair at
// its tile end, and dt.
template <int T>
__device__ __forceinline__ void token_tables(const Tables<T> &tb, int t, float gh, float gl,
                                             float geh, float gel, float d) {
    tb.gh[t] = gh;
    tb.gl[t] = gl;
    tb.dt[t] = d;
    tb.e2[t] = fast_exp2(gh + gl);
    tb.cf[t] = fast_exp2((geh - gh) + (gel - gl)) * d;
}

// Off-diagonal decay weights.  For row i in tile I and column j in tile J < I,
//     exp2(G2_i - G2_j) dt_j = rs(i) * m(I, J) * cf(j),
//     rs(i)   = exp2(G2_i - G2_{16 I - 1})        (per row, one per lane and row tile)
//     m(I, J) = exp2(G2_{16 I - 1} - G2_{16 J + 15})  (per tile pair, wave-uniform)
//     cf(j)   = exp2(G2_{16 J + 15} - G2_j) dt_j     (per column, tabulated)
// Every exponent is <= 0 (G2 never increases), so no factor can overflow, and
// a factor that underflows bounds a product that is at least as small.
template <int T>
__device__ __forceinline__ float tile_pair_factor(const Tables<T> &tb, int I, int J) {
    return fast_exp2((tb.before_hi(I) - tb.gh[16 * J + 15]) + (tb.before_lo(I) - tb.gl[16 * J + 15]));
}
template <int T>
__device__ __forceinline__ float row_factor(const Tables<T> &tb, int I, float gih, float gil) {
    return fast_exp2((gih - tb.before_hi(I)) + (gil - tb.before_lo(I)));
}

// Decay-and-dt weighted values of one S tile slot for this lane: row
// i = 16 I + l16, columns j = 16 J + 4 g4 + r; rm = rs(i) m(I, J) when J < I.
// On the diagonal tile the exponent is the exact difference G2_i - G2_j (0
// for j = i) and the mask is a select taken before exp2.
template <int T>
__device__ __forceinline__ void tile_values(const floatx4 &s, int J, int I, int l16, int g4,
                                            float gih, float gil, float rm, const Tables<T> &tb,
                                            float (&v)[4]) {
    if (J > I) {
        v[0] = v[1] = v[2] = v[3] = 0.f;
    } else if (J < I) {
        const float4 cf = *reinterpret_cast<const float4 *>(tb.cf + 16 * J + 4 * g4);
        v[0] = s[0] * (rm * cf.x);
        v[1] = s[1] * (rm * cf.y);
        v[2] = s[2] * (rm * cf.z);
        v[3] = s[3] * (rm * cf.w);
    } else {
        const float4 jh = *reinterpret_cast<const float4 *>(tb.gh + 16 * J + 4 * g4);
        const float4 jl = *reinterpret_cast<const float4 *>(tb.gl + 16 * J + 4 * g4);
        const float4 dj = *reinterpret_cast<const float4 *>(tb.dt + 16 * J + 4 * g4);
        const float hv[4] = {jh.x, jh.y, jh.z, jh.w};
        const float lv[4] = {jl.x, jl.y, jl.z, jl.w};
        const float dv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool keep = (4 * g4 + r) <= l16;  // j <= i (diagonal kept)
            const float arg = keep ? ((gih - hv[r]) + (gil - lv[r])) : -INFINITY;
            v[r] = keep ? s[r] * (fast_exp2(arg) * dv[r]) : 0.f;
        }
    }
}

// y is written with raw buffer stores: the resource covers a chunk's rows of
// one head up to the last valid row, so the hardware drops the stores of rows
// past the sequence end, and the row offsets stay 32-bit.  A buffer store
// reads its data register after it issues (later still when copies are
// queued ahead of it), and the compiler does not wait for that before it
// reuses the register (measured: such reuse corrupted stored values).  So
// values go out four at a time, at off + r * stride, followed by an expcnt
// wait that takes the four data registers as operands: they stay untouched
// until the stores have read them (not until the stores complete).
template <typename OutT>
__device__ __forceinline__ void store_out4(__amdgpu_buffer_rsrc_t r, int off, int stride, const float (&v)[4]);
template <>
__device__ __forceinline__ void store_out4<float>(__amdgpu_buffer_rsrc_t r, int off, int stride,
                                                  const float (&v)[4]) {
    uint32_t d[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        d[k] = __float_as_uint(v[k]);
        __builtin_amdgcn_raw_buffer_store_b32(d[k], r, off + k * stride, 0, 0);
    }
    asm volatile("s_waitcnt expcnt(0)" ::"v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]) : "memory");
}
template <>
__device__ __forceinline__ void store_out4<uint16_t>(__amdgpu_buffer_rsrc_t r, int off, int stride,
                                                     const float (&v)[4]) {
    uint32_t d[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        d[k] = pack_bf16(v[k], 0.f) & 0xffffu;
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)d[k], r, off + k * stride, 0, 0);
    }
    asm volatile("s_waitcnt expcnt(0)" ::"v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]) : "memory");
}

__device__ __forceinline__ uint32_t sel_half(int q) { return (q & 1) ? 0x07060302u : 0x05040100u; }

// Lane coordinates re-derived from an opaque copy of the thread index inside
// a loop, so the compiler recomputes the cheap per-lane offsets instead of
// hoisting every one of them out of the head loop into registers.
struct LaneIds {
    int l16, g4, w;
};
__device__ __forceinline__ LaneIds opaque_lane_ids(int tid) {
    int t = tid;
    asm volatile("" : "+v"(t));
    LaneIds r;
    r.l16 = t & 15;
    r.g4 = (t >> 4) & 3;
    r.w = __builtin_amdgcn_readfirstlane(t >> 6);
    return r;
}

// ---------------------------------------------------------------------------
// bf16 path
// ---------------------------------------------------------------------------
// LDS of the bf16 kernel: x^T tile, the h hi/lo tiles when they fit, tables.
template <int T, int P, int NKMAX>
struct Bf16Lds {
    static constexpr int XRS = 2 * T + 32;           // x^T row stride (bytes)
    static constexpr int HRS = 2 * NKMAX * 32 + 32;  // h / C row stride (bytes)
    static constexpr size_t x = (size_t)P * XRS;
    static constexpr size_t h = (size_t)2 * P * HRS;
    static constexpr int CRS = 2 * NKMAX * 32;       // C row stride (bytes), XOR-swizzled
    static constexpr size_t c = (size_t)T * CRS;     // the chunk's C rows
    static constexpr size_t tables = Tables<T>::bytes;
    // h is staged in LDS when everything fits; otherwise its fragments are read
    // from global memory (L2) and split into hi/lo in registers.
    static constexpr bool h_in_lds = x + h + tables <= kLdsBytes;
    // The C fragments of a wave's row tiles live in LDS (rather than in 8 NKMAX
    // registers per lane for the whole block) when that still fits.
    static constexpr bool c_in_lds = h_in_lds && x + h + c + tables <= kLdsBytes;
    static constexpr size_t heads_total = x + (h_in_lds ? h : 0) + (c_in_lds ? c : 0) + tables;
    static_assert(heads_total <= kLdsBytes, "stage-4 LDS budget exceeded");
    // Before the first head the x / h / table space is free: B rows are staged
    // there (from offset 0) in pieces of KSP dstate slices of 32, as many as fit
    // below the C tile, or else in max(heads_total, half the LDS).
    static constexpr size_t b_avail =
        c_in_lds ? x + h : (heads_total > kLdsBytes / 2 ? heads_total : kLdsBytes / 2);
    static constexpr int KSP = (size_t)T * 64 * NKMAX <= b_avail       ? NKMAX
                               : (size_t)T * 64 * (NKMAX / 2) <= b_avail ? NKMAX / 2
                                                                         : NKMAX / 4;
    static constexpr int NPIECE = NKMAX / KSP;
    static constexpr size_t b_bytes = (size_t)T * 64 * KSP;
    static_assert(KSP >= 1 && b_bytes <= b_avail, "stage-4 B staging does not fit");
    // what the block allocates
    static constexpr size_t total = heads_total > b_bytes ? heads_total : b_bytes;
};

// Compile-time loops and the wave-index dispatch: every wave runs straight-line
// code specialised for its own pair of row tiles, so no tile-pair step sits
// behind a runtime branch and the compiler can schedule across steps.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int NW, typename F>
__device__ __forceinline__ void dispatch_wave(int w, F &&f) {
    static_for<NW>([&](auto wc) {
        if (w == decltype(wc)::value) f(wc);
    });
}

// Slot layout of wave W (see slot_base1) as compile-time functions.
template <int T, int W>
struct WaveTiles {
    static constexpr int NT16 = T / 16;
    static constexpr int NSLOT = NT16 + 2;
    static constexpr int I0 = W, I1 = NT16 - 1 - W;
    static constexpr int base1 = (I0 + 2) & ~1;
    static constexpr int ii_of(int k) { return k < base1 ? 0 : 1; }
    static constexpr int I_of(int k) { return k < base1 ? I0 : I1; }
    static constexpr int J_of(int k) { return k < base1 ? k : k - base1; }
    // the q-th pair processed: pairs of I0 (0 .. base1/2 - 1) and of I1
    // (base1/2 .. NSLOT/2 - 1) alternate while both last
    static constexpr int pair_order(int q) {
        const int n0 = base1 / 2, n1 = NSLOT / 2 - n0;
        const int m = n0 < n1 ? n0 : n1;
        if (q < 2 * m) return (q % 2 == 0) ? q / 2 : n0 + q / 2;
        return n0 > n1 ? q - m : n0 + (q - m);
    }
};

// tile_values with the tile relation known at compile time.  With kSkip the
// diagonal tile also carries the skip term: D is added to the weight of j = i
// (y_i = sum_j W_ij x_j + D x_i), so no separate pass over x is needed.
template <int T, int J, int I, bool kSkip = false>
__device__ __forceinline__ void tile_values_ct(const floatx4 &s, int l16, int g4, float gih, float gil,
                                               float rm, const Tables<T> &tb, float (&v)[4],
                                               float Dh = 0.f) {
    if constexpr (J > I) {
        v[0] = v[1] = v[2] = v[3] = 0.f;
    } else if constexpr (J < I) {
        const float4 cf = *reinterpret_cast<const float4 *>(tb.cf + 16 * J + 4 * g4);
        v[0] = s[0] * (rm * cf.x);
        v[1] = s[1] * (rm * cf.y);
        v[2] = s[2] * (rm * cf.z);
        v[3] = s[3] * (rm * cf.w);
    } else {
        const float4 jh = *reinterpret_cast<const float4 *>(tb.gh + 16 * J + 4 * g4);
        const float4 jl = *reinterpret_cast<const float4 *>(tb.gl + 16 * J + 4 * g4);
        const float4 dj = *reinterpret_cast<const float4 *>(tb.dt + 16 * J + 4 * g4);
        const float hv[4] = {jh.x, jh.y, jh.z, jh.w};
        const float lv[4] = {jl.x, jl.y, jl.z, jl.w};
        const float dv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool keep = (4 * g4 + r) <= l16;  // j <= i (diagonal kept)
            const float arg = keep ? ((gih - hv[r]) + (gil - lv[r])) : -INFINITY;
            if constexpr (kSkip)
                v[r] = keep ? fmaf(s[r], fast_exp2(arg) * dv[r], (4 * g4 + r) == l16 ? Dh : 0.f) : 0.f;
            else
                v[r] = keep ? s[r] * (fast_exp2(arg) * dv[r]) : 0.f;
        }
    }
}

// C B^T tiles of wave W (transposed: lane holds S[i = 16 I + l16][j = 16 J + 4 g4 + r]),
// contribution of the dstate slices ks = KSP * PC .. KSP * PC + KSP - 1.  The
// slices' B rows are staged in LDS (row stride 64 KSP bytes, 16-byte chunk c
// of row t stored at chunk c ^ (t & SWM)); bl = that tile + l16 * row stride.
// C fragments come from the swizzled C tile (CLDS, cl = tile + l16 * CRS) or
// from registers.
template <int T, int NKMAX, int KSP, int PC, bool CLDS, int CRS, int W>
__device__ __forceinline__ void cbt_piece(floatx4 (&S)[T / 16 + 2], const u32x4 (&cfr)[2][NKMAX],
                                          const unsigned char *bl, const unsigned char *cl, int l16,
                                          int g4) {
    using WT = WaveTiles<T, W>;
    constexpr int BROW = 64 * KSP;
    constexpr int SWM = (4 * KSP >= 16 ? 16 : 4 * KSP) - 1;
    static_for<KSP>([&](auto kc) {
        constexpr int ksl = decltype(kc)::value;
        constexpr int ks = KSP * PC + ksl;
        u32x4 c0, c1;
        if constexpr (CLDS) {
            c0 = *reinterpret_cast<const u32x4 *>(cl + 16 * WT::I0 * CRS + (((4 * ks + g4) ^ l16) << 4));
            c1 = *reinterpret_cast<const u32x4 *>(cl + 16 * WT::I1 * CRS + (((4 * ks + g4) ^ l16) << 4));
        } else {
            c0 = cfr[0][ks];
            c1 = cfr[1][ks];
        }
        const unsigned char *bk = bl + (((4 * ksl + g4) ^ (l16 & SWM)) << 4);
        static_for<WT::I1 + 1>([&](auto jc) {
            constexpr int J = decltype(jc)::value;
            const u32x4 bf = *reinterpret_cast<const u32x4 *>(bk + 16 * J * BROW);
            if constexpr (J <= WT::I0) S[J] = mfma_bf16(bf, c0, S[J]);
            S[WT::base1 + J] = mfma_bf16(bf, c1, S[WT::base1 + J]);
        });
    });
}

// Everything one wave computes for one head.
template <int T, int P, int NKMAX, typename OutT>
struct HeadCtx {
    const unsigned char *xl;  // x^T + l16 * XRS + 16 g4
    const unsigned char *hl;  // h hi tile + l16 * HRS + 16 g4 (when staged in LDS)
    const unsigned char *cl;  // C tile + l16 * CRS (when staged in LDS)
    const uint16_t *hp;       // h_c hi plane in global memory (lo plane follows; when not staged)
    const uint16_t *cg[2];    // C rows 16 I0 + l16 and 16 I1 + l16 (clamped; when re-read per head)
    bool cok[2];              // those rows are within the sequence
    Tables<T> tb;
    __amdgpu_buffer_rsrc_t yr;  // y[b, t0 .., h, :] through the chunk's last valid row
    int NHP;                  // nheads * headdim (row stride of y)
    int N;
    float Dh;
    int l16, g4;
};

template <int T, int P, int NKMAX, bool HLDS, bool CLDS, bool CG, typename OutT, int W, typename Mid>
__device__ __forceinline__ void head_wave(const floatx4 (&S)[T / 16 + 2],
                                          const u32x4 (&cfr)[2][NKMAX],
                                          const HeadCtx<T, P, NKMAX, OutT> &cx, Mid &&mid) {
    using Lds = Bf16Lds<T, P, NKMAX>;
    using WT = WaveTiles<T, W>;
    constexpr int XRS = Lds::XRS, HRS = Lds::HRS;
    constexpr int PT = P / 16;
    constexpr int NT16 = T / 16;
    constexpr int I0 = WT::I0, I1 = WT::I1;
    const int l16 = cx.l16, g4 = cx.g4;

    floatx4 acc[2][PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[0][pt] = acc[1][pt] = zero4();

    // inter-chunk term C_i h_c (h split into hi + lo); fragments past dstate are 0.
    // With CG the C fragments are re-read from global memory (L2) two k-steps
    // ahead instead of being held in registers for the whole block.
    constexpr int CGD = 2;  // prefetch distance (k-steps)
    u32x4 cq[CG ? CGD + 1 : 1][2];
    auto cg_load = [&](int ks, u32x4 (&dst)[2]) {
        const int n0 = 32 * ks + 8 * g4;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(cx.cg[ii] + min(n0, cx.N - 8));
            dst[ii] = (cx.cok[ii] && n0 < cx.N) ? v : u32x4{0u, 0u, 0u, 0u};
        }
    };
    if constexpr (CG) {
#pragma unroll
        for (int d = 0; d < CGD && d < NKMAX; ++d) cg_load(d, cq[d]);
    }
#pragma unroll
    for (int ks = 0; ks < NKMAX; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        u32x4 cf[2];
        if constexpr (CG) {
            if (ks + CGD < NKMAX) cg_load(ks + CGD, cq[(ks + CGD) % (CGD + 1)]);
        }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            if constexpr (CLDS)  // 16-byte chunk (4 ks + g4) of row 16 I + l16, swizzled by l16
                cf[ii] = *reinterpret_cast<const u32x4 *>(
                    cx.cl + (16 * (ii ? I1 : I0)) * Lds::CRS + (((4 * ks + g4) ^ l16) << 4));
            else if constexpr (CG)
                cf[ii] = cq[ks % (CGD + 1)][ii];
            else
                cf[ii] = cfr[ii][ks];
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            u32x4 hh, hlv;
            if constexpr (HLDS) {
                hh = *reinterpret_cast<const u32x4 *>(cx.hl + pt * 16 * HRS + 64 * ks);
                hlv = *reinterpret_cast<const u32x4 *>(cx.hl + Lds::h / 2 + pt * 16 * HRS + 64 * ks);
            } else {
                hh = hlv = u32x4{0u, 0u, 0u, 0u};
                const int n0 = 32 * ks + 8 * g4;
                if (n0 < cx.N) {
                    const uint16_t *src = cx.hp + (16 * pt + l16) * cx.N + n0;
                    hh = *reinterpret_cast<const u32x4 *>(src);
                    hlv = *reinterpret_cast<const u32x4 *>(src + P * cx.N);
                }
            }
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                acc[ii][pt] = mfma_bf16(cf[ii], hh, acc[ii][pt]);
                acc[ii][pt] = mfma_bf16(cf[ii], hlv, acc[ii][pt]);
            }
        }
    }
    // rows i = 16 I + 4 g4 + r take exp2(G2_i)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const float4 e = *reinterpret_cast<const float4 *>(cx.tb.e2 + 16 * (ii ? I1 : I0) + 4 * g4);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            acc[ii][pt][0] *= e.x;
            acc[ii][pt][1] *= e.y;
            acc[ii][pt][2] *= e.z;
            acc[ii][pt][3] *= e.w;
        }
    }
    mid();  // h_c is no longer read in this head
    // tile-pair factors m(I, J): lane k evaluates the one of slot k, which is
    // then read back as a wave-uniform value
    float mk;
    {
        const int k = l16 + 16 * g4;
        const int Ik = k < WT::base1 ? I0 : I1;
        const int Jk = k < WT::base1 ? k : k - WT::base1;
        const bool off = k < WT::NSLOT && Jk < Ik;
        const float m = tile_pair_factor(cx.tb, off ? Ik : 1, off ? Jk : 0);  // in-range reads
        mk = off ? m : 0.f;
    }
    // intra-chunk term: slot pairs (J, J + 1) of one row tile, K = 32.  The
    // A operand (masked, decay-weighted values, hi/lo) of pair q + 1 is built
    // while the MFMAs of pair q run; the x fragments are read just before use.
    const float rs[2] = {row_factor(cx.tb, I0, cx.tb.gh[16 * I0 + l16], cx.tb.gl[16 * I0 + l16]),
                         row_factor(cx.tb, I1, cx.tb.gh[16 * I1 + l16], cx.tb.gl[16 * I1 + l16])};
    // G2 of the lane's row, re-read from LDS where a diagonal tile needs it
    // (an opaque offset keeps the reads from being merged and held in registers)
    auto row_g2 = [&](int I, float &h, float &lo) {
        int off = 16 * I + l16;
        asm volatile("" : "+v"(off));
        h = cx.tb.gh[off];
        lo = cx.tb.gl[off];
    };
    constexpr int NP = WT::NSLOT / 2;
    struct AOps {
        u32x4 hi, lo;
        u32x4 xb[PT];  // x fragments of the pair, one per 16 headdim columns
    };
    auto prep = [&](auto qc) {
        constexpr int k0 = 2 * decltype(qc)::value;
        constexpr int ii = k0 < WT::base1 ? 0 : 1;
        constexpr int I = ii ? I1 : I0;
        constexpr int Ja = k0 - (ii ? WT::base1 : 0), Jb = Ja + 1;
        const float rma = rs[ii] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), k0));
        const float rmb = rs[ii] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), k0 + 1));
        float gih = 0.f, gil = 0.f;
        if constexpr (Ja == I || Jb == I) row_g2(I, gih, gil);
        float va[4], vb[4];
        tile_values_ct<T, Ja, I>(S[k0], l16, g4, gih, gil, rma, cx.tb, va);
        tile_values_ct<T, Jb, I>(S[k0 + 1], l16, g4, gih, gil, rmb, cx.tb, vb);
        const HiLo p0 = split_bf16(va[0], va[1]), p1 = split_bf16(va[2], va[3]);
        const HiLo p2 = split_bf16(vb[0], vb[1]), p3 = split_bf16(vb[2], vb[3]);
        AOps o;
        o.hi = u32x4{p0.hi, p1.hi, p2.hi, p3.hi};
        o.lo = u32x4{p0.lo, p1.lo, p2.lo, p3.lo};
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)  // chunk (Ja / 2, g4): tokens 16 Ja + 4 g4 .. +3, 16 Jb + 4 g4 .. +3
            o.xb[pt] = *reinterpret_cast<const u32x4 *>(cx.xl + pt * 16 * XRS + 32 * Ja);
        return o;
    };
    // pairs of the two row tiles alternate, so consecutive MFMAs go to
    // different accumulators (8 independent chains instead of 4)
    AOps cur = prep(std::integral_constant<int, WT::pair_order(0)>{});
    static_for<NP>([&](auto qc) {
        constexpr int q = WT::pair_order(decltype(qc)::value);
        constexpr int k0 = 2 * q;
        constexpr int ii = k0 < WT::base1 ? 0 : 1;
        constexpr int qn = decltype(qc)::value + 1;
        AOps nxt;
        if constexpr (qn < NP) nxt = prep(std::integral_constant<int, WT::pair_order(qn < NP ? qn : 0)>{});
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[ii][pt] = mfma_bf16(cur.hi, cur.xb[pt], acc[ii][pt]);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[ii][pt] = mfma_bf16(cur.lo, cur.xb[pt], acc[ii][pt]);
        if constexpr (qn < NP) cur = nxt;
        __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_sched_barrier(0);
    // skip term and store: lane holds rows 16 I + 4 g4 + r, column 16 pt + l16
    constexpr int ES = (int)sizeof(OutT);
    const int lane_off = ((4 * g4) * cx.NHP + l16) * ES;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = ii ? I1 : I0;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const u32x2 xv2 = *reinterpret_cast<const u32x2 *>(cx.xl + pt * 16 * XRS + 32 * (I & ~1) + 8 * (I & 1));
            const float xv[4] = {bf16lo(xv2[0]), bf16hi(xv2[0]), bf16lo(xv2[1]), bf16hi(xv2[1])};
            const float yv[4] = {acc[ii][pt][0] + cx.Dh * xv[0], acc[ii][pt][1] + cx.Dh * xv[1],
                                 acc[ii][pt][2] + cx.Dh * xv[2], acc[ii][pt][3] + cx.Dh * xv[3]};
            store_out4<OutT>(cx.yr, lane_off + 16 * I * cx.NHP * ES + 16 * pt * ES, cx.NHP * ES, yv);
        }
    }
}

template <int T, int P, int NKMAX, typename OutT>
__global__ __launch_bounds__(2 * T) void k4_chunk_out_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ G2hi, const float *__restrict__ G2lo,
    const float *__restrict__ DT, const float *__restrict__ Dv, const uint16_t *__restrict__ H,
    OutT *__restrict__ y, int64_t L, int NH, int N, int G, int NC, int64_t Lp, int HPG, int HB,
    int nhb) {
    using Lds = Bf16Lds<T, P, NKMAX>;
    constexpr bool kHinLds = Lds::h_in_lds;
    constexpr int XRS = Lds::XRS, HRS = Lds::HRS;
    constexpr int NT16 = T / 16;
    constexpr int NSLOT = NT16 + 2;
    constexpr int NW = T / 32;
    constexpr int NTHR = 2 * T;
    // x staging unit: 4 tokens x 8 headdim columns; within a wave 16 token
    // quads x 4 column octets (conflict-free transposing LDS writes)
    constexpr int XUNITS = (T / 4) * (P / 8);
    constexpr int XPASS = (XUNITS + NTHR - 1) / NTHR;
    constexpr int TQH = T / 64;                       // token-quad groups of 16
    constexpr int HCH = NKMAX * 4;                    // 8-element chunks per h row
    constexpr int HUNITS = P * HCH;
    constexpr int HPASS = (HUNITS + NTHR - 1) / NTHR;
    constexpr int HREG = kHinLds ? HPASS : 1;

    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char *xt = lds;                               // [P][XRS]
    unsigned char *hhi = xt + Lds::x;                      // [P][HRS] (if kHinLds)
    unsigned char *hlo = hhi + Lds::h / 2;                 // [P][HRS] (if kHinLds)
    constexpr bool kCinLds = Lds::c_in_lds;
    // Eight waves of 256 registers each cannot hold the C fragments of the
    // larger tiles beside the C B^T tiles and the next head's prefetch; those
    // shapes re-read C (L2-resident) in every head instead.
    constexpr bool kCglb = !kCinLds && T == 256 && (NKMAX == 8 || P == 128);
    // Those shapes also copy h_c straight into LDS (asynchronous copies, no
    // registers): issued once every wave is past the inter-chunk term of the
    // current head, landing during its intra-chunk term.
    constexpr bool kHdma = kCglb && kHinLds;
    unsigned char *ct = xt + Lds::x + (kHinLds ? Lds::h : 0);  // [T][HRS] (if kCinLds)
    const Tables<T> tb(reinterpret_cast<float *>(ct + (kCinLds ? Lds::c : 0)));

    const int tid = threadIdx.x;
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
    const int rows = (int)min<int64_t>(T, L - t0);  // valid tokens in this chunk
    const bool full = rows == T;

    // ---------------- per-head data, loaded one head ahead ----------------
    u32x4 xr[XPASS][4];
    u32x4 hr[HREG][2];  // hi, lo bf16 of 8 consecutive dstate entries
    float sgh = 0.f, sgl = 0.f, seh = 0.f, sel = 0.f, sdt = 0.f;
    auto xunit = [&](int ps, int &tq, int &po) {
        const int u = tid + ps * NTHR;
        const int wv = u >> 6, ln = u & 63;
        tq = 16 * (wv % TQH) + (ln & 15);
        po = 4 * (wv / TQH) + (ln >> 4);
        return u < XUNITS;
    };
    auto load_head = [&](int h) {
        const uint16_t *xh = x + ((b * L + t0) * NH + h) * P;
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            int tq, po;
            const bool ok = xunit(ps, tq, po);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * tq + r;
                xr[ps][r] = u32x4{0u, 0u, 0u, 0u};
                if (ok && (full || t < rows))
                    xr[ps][r] = *reinterpret_cast<const u32x4 *>(xh + (int64_t)t * NH * P + po * 8);
            }
        }
        if constexpr (kHinLds && !kHdma) {
            const uint16_t *hp = H + (((int64_t)b * NH + h) * NC + c) * (int64_t)2 * P * N;
#pragma unroll
            for (int ps = 0; ps < HPASS; ++ps) {
                const int u = tid + ps * NTHR;
                const int ch = u % HCH, p = u / HCH;
                hr[ps][0] = hr[ps][1] = u32x4{0u, 0u, 0u, 0u};
                if (u < HUNITS && 8 * ch < N) {
                    hr[ps][0] = *reinterpret_cast<const u32x4 *>(hp + p * N + 8 * ch);
                    hr[ps][1] = *reinterpret_cast<const u32x4 *>(hp + P * N + p * N + 8 * ch);
                }
            }
        }
        if (tid < T) {
            const int64_t hoff = ((int64_t)b * NH + h) * Lp + t0;
            sgh = G2hi[hoff + tid];
            sgl = G2lo[hoff + tid];
            seh = G2hi[hoff + (tid | 15)];
            sel = G2lo[hoff + (tid | 15)];
            sdt = DT[hoff + tid];
        }
    };
    auto stage_head = [&]() {
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            int tq, po;
            if (xunit(ps, tq, po)) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t s = sel_half(q);
                    const u32x2 v = {__builtin_amdgcn_perm(xr[ps][1][q >> 1], xr[ps][0][q >> 1], s),
                                     __builtin_amdgcn_perm(xr[ps][3][q >> 1], xr[ps][2][q >> 1], s)};
                    // tokens 4 tq .. +3 (tile J = tq / 4, quad tq % 4) of column 8 po + q
                    *reinterpret_cast<u32x2 *>(xt + (8 * po + q) * XRS + 32 * ((tq >> 2) & ~1) +
                                               16 * (tq & 3) + 8 * ((tq >> 2) & 1)) = v;
                }
            }
        }
        if constexpr (kHinLds && !kHdma) {
#pragma unroll
            for (int ps = 0; ps < HPASS; ++ps) {
                const int u = tid + ps * NTHR;
                if (u < HUNITS) {
                    const int ch = u % HCH, p = u / HCH;
                    *reinterpret_cast<u32x4 *>(hhi + p * HRS + 16 * ch) = hr[ps][0];
                    *reinterpret_cast<u32x4 *>(hlo + p * HRS + 16 * ch) = hr[ps][1];
                }
            }
        }
        if (tid < T) token_tables(tb, tid, sgh, sgl, seh, sel, sdt);
    };
    // h_c planes of head h into hhi / hlo (rows of HRS bytes): the region is
    // copied as consecutive 1-KiB pieces, lane l of piece q landing at byte
    // 1024 q + 16 l; a lane whose bytes fall in a row's padding or past
    // dstate reads past the resource, which returns zeros.
    auto issue_h_dma = [&](int h) {
        constexpr int HBYTES = (int)Lds::h;  // both planes
        constexpr int PLANE = HBYTES / 2;
        constexpr int NQ = HBYTES / 1024;
        static_assert(HBYTES % 1024 == 0, "h region is whole 1-KiB pieces");
        const uint32_t src_bytes = (uint32_t)(2 * P * N * 2);
        const i32x4 hd = buffer_desc(H + (((int64_t)b * NH + h) * NC + c) * (int64_t)2 * P * N, src_bytes);
        const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
        int ln = tid & 63;
        asm volatile("" : "+v"(ln));
        for (int q = wu; q < NQ; q += NW) {
            const int o = 1024 * q + 16 * ln;
            const int pl = o / PLANE, r = o % PLANE;
            const int row = r / HRS, within = r % HRS;
            const bool ok = within < 2 * N;
            const int voff = ok ? (pl * P * N + row * N) * 2 + within : (int)src_bytes;
            lds_dma_x4(hd, lds_addr(hhi + 1024 * q), voff);
        }
    };

    // (with kCglb the first head's prefetch waits until the C B^T tiles are
    // done, so its registers are not live beside the tiles' operands)
    if (!kCglb && h_begin < h_end) load_head(h_begin);

    // ---------------- C B^T tiles (transposed), once per block -------------
    // All threads stage the chunk's C rows (into the C tile, when it lives in
    // LDS) and its B rows (piece by piece) with coalesced 16-byte loads at
    // clamped addresses; chunks past the chunk's rows or past dstate are zero.
    // Each wave then reads its fragments from LDS.
    const int I0 = w, I1 = NT16 - 1 - w;
    const uint16_t *Bc = Bm + ((b * L + t0) * G + gi) * N;
    const uint16_t *Cc = Cm + ((b * L + t0) * G + gi) * N;
    const int64_t GN = (int64_t)G * N;
    auto chunk16 = [&](const uint16_t *base, int row, int n0) {
        const bool ok = row < rows && n0 < N;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(base + (int64_t)min(row, rows - 1) * GN +
                                                          min(n0, N - 8));
        return ok ? v : u32x4{0u, 0u, 0u, 0u};
    };
    u32x4 cfr[2][NKMAX];
    if constexpr (kCinLds) {
        constexpr int CCH = 4 * NKMAX;                   // 16-byte chunks per C row
        constexpr int CPT = T * CCH / NTHR;              // per thread
        u32x4 cv[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int u = tid + k * NTHR;
            cv[k] = chunk16(Cc, u / CCH, 8 * (u % CCH));
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int u = tid + k * NTHR;
            const int row = u / CCH, ch = u % CCH;
            *reinterpret_cast<u32x4 *>(ct + row * Lds::CRS + ((ch ^ (row & 15)) << 4)) = cv[k];
        }
    } else if constexpr (!kCglb) {
        // lane holds C[t0 + 16 I + l16][32 ks + 8 g4 .. +7]
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int ks = 0; ks < NKMAX; ++ks)
                cfr[ii][ks] = chunk16(Cc, 16 * (ii ? I1 : I0) + l16, 32 * ks + 8 * g4);
    }
    floatx4 S[NSLOT];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) S[k] = zero4();
    static_for<Lds::NPIECE>([&](auto pcc) {
        constexpr int PC = decltype(pcc)::value;
        constexpr int KSP = Lds::KSP;
        constexpr int BCH = 4 * KSP;                     // 16-byte chunks per staged B row
        constexpr int BPT = T * BCH / NTHR;              // per thread
        constexpr int SWM = (BCH >= 16 ? 16 : BCH) - 1;
        if constexpr (PC > 0) __syncthreads();           // previous piece consumed
        if constexpr (kCglb) {  // only this piece's C fragments
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int ksl = 0; ksl < KSP; ++ksl)
                    cfr[ii][KSP * PC + ksl] = chunk16(Cc, 16 * (ii ? I1 : I0) + l16, 32 * (KSP * PC + ksl) + 8 * g4);
        }
        u32x4 bv[BPT];
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + k * NTHR;
            bv[k] = chunk16(Bc, u / BCH, 8 * (BCH * PC + u % BCH));
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int u = tid + k * NTHR;
            const int row = u / BCH, ch = u % BCH;
            *reinterpret_cast<u32x4 *>(lds + row * (16 * BCH) + ((ch ^ (row & SWM)) << 4)) = bv[k];
        }
        __syncthreads();
        dispatch_wave<NW>(w, [&](auto wc) {
            cbt_piece<T, NKMAX, KSP, PC, kCinLds, Lds::CRS, decltype(wc)::value>(
                S, cfr, lds + l16 * (16 * BCH), ct + l16 * Lds::CRS, l16, g4);
        });
    });
    __syncthreads();  // the B rows are overwritten by the first head's staging
    if (kCglb && h_begin < h_end) load_head(h_begin);
    if constexpr (kHdma)
        if (h_begin < h_end) issue_h_dma(h_begin);

    // ---------------- heads -------------------------------------------------
    for (int h = h_begin; h < h_end; ++h) {
        stage_head();
        if constexpr (kHdma) lds_dma_wait();  // this wave's h_c copies have landed
        __syncthreads();
        if (h + 1 < h_end) load_head(h + 1);
        const LaneIds id = opaque_lane_ids(tid);
        const int ra = 16 * id.w + id.l16, rb = 16 * (NT16 - 1 - id.w) + id.l16;  // rows of I0, I1
        HeadCtx<T, P, NKMAX, OutT> cx{xt + id.l16 * XRS + 16 * id.g4,
                                      hhi + id.l16 * HRS + 16 * id.g4,
                                      ct + id.l16 * Lds::CRS,
                                      H + (((int64_t)b * NH + h) * NC + c) * (int64_t)2 * P * N,
                                      {Cc + (int64_t)min(ra, rows - 1) * GN, Cc + (int64_t)min(rb, rows - 1) * GN},
                                      {ra < rows, rb < rows},
                                      tb,
                                      buffer_rsrc(y + ((b * L + t0) * NH + h) * P,
                                                  (uint32_t)(((rows - 1) * NH * P + P) * sizeof(OutT))),
                                      NH * P,
                                      N,
                                      (Dv != nullptr) ? Dv[h] : 0.f,
                                      id.l16,
                                      id.g4};
        dispatch_wave<NW>(id.w, [&](auto wc) {
            head_wave<T, P, NKMAX, kHinLds, kCinLds, kCglb, OutT, decltype(wc)::value>(S, cfr, cx, [&]() {
                if constexpr (kHdma) {
                    __syncthreads();  // every wave is done reading this head's h_c
                    if (h + 1 < h_end) issue_h_dma(h + 1);
                }
            });
        });
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
template <int T, int P>
struct F32Lds {
    static constexpr int LDP = P + 4;                 // padded row of the x tile (floats)
    static constexpr size_t x = (size_t)T * LDP * 4;
    static constexpr size_t total = x + Tables<T>::bytes;
    static_assert(total <= kLdsBytes, "stage-4 LDS budget exceeded");
};

template <int T, int P, typename OutT>
__global__ __launch_bounds__(2 * T) void k4_chunk_out_f32(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ Cm,
    const float *__restrict__ G2hi, const float *__restrict__ G2lo, const float *__restrict__ DT,
    const float *__restrict__ Dv, const float *__restrict__ H, OutT *__restrict__ y, int64_t L,
    int NH, int N, int G, int NC, int64_t Lp, int HPG, int HB, int nhb) {
    using Lds = F32Lds<T, P>;
    constexpr int NT16 = T / 16;
    constexpr int NSLOT = NT16 + 2;
    constexpr int PT = P / 16;
    constexpr int NTHR = 2 * T;
    constexpr int LDP = Lds::LDP;
    constexpr int XV = T * (P / 4);                  // float4 units of the x tile
    constexpr int XPASS = (XV + NTHR - 1) / NTHR;

    extern __shared__ __align__(16) unsigned char lds[];
    float *xs = reinterpret_cast<float *>(lds);       // [T][LDP]
    const Tables<T> tb(reinterpret_cast<float *>(lds + Lds::x));

    const int tid = threadIdx.x;
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
    const int ns = N / 16;
    const bool full = t0 + T <= L;

    floatx4 xr[XPASS];
    float sgh = 0.f, sgl = 0.f, seh = 0.f, sel = 0.f, sdt = 0.f;
    auto load_head = [&](int h) {
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            const int v = tid + ps * NTHR;
            const int t = v / (P / 4), p4 = v % (P / 4);
            xr[ps] = zero4();
            if (v < XV && (full || t0 + t < L))
                xr[ps] = *reinterpret_cast<const floatx4 *>(x + ((b * L + t0 + t) * NH + h) * P + 4 * p4);
        }
        if (tid < T) {
            const int64_t hoff = ((int64_t)b * NH + h) * Lp + t0;
            sgh = G2hi[hoff + tid];
            sgl = G2lo[hoff + tid];
            seh = G2hi[hoff + (tid | 15)];
            sel = G2lo[hoff + (tid | 15)];
            sdt = DT[hoff + tid];
        }
    };
    auto stage_head = [&]() {
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            const int v = tid + ps * NTHR;
            if (v < XV) {
                const int t = v / (P / 4), p4 = v % (P / 4);
                *reinterpret_cast<floatx4 *>(xs + t * LDP + 4 * p4) = xr[ps];
            }
        }
        if (tid < T) token_tables(tb, tid, sgh, sgl, seh, sel, sdt);
    };

    if (h_begin < h_end) load_head(h_begin);

    const int I0 = w, I1 = NT16 - 1 - w;
    const int base1 = slot_base1(I0);
    const int64_t rowC[2] = {t0 + 16 * I0 + l16, t0 + 16 * I1 + l16};

    // C B^T tiles (transposed), once per block.  K = 4 per MFMA: instruction q
    // of a 16-wide dstate step s contracts n = 16 s + 4 g4 + q.
    floatx4 S[NSLOT];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) S[k] = zero4();
    if constexpr (T <= 128) {
        // per dstate step: both C rows and the B row of every column tile J
        // <= I1 are loaded once, then all of the step's (I, J) MFMAs run (a
        // B row serves both row tiles)
        // (code specialised per wave, so every slot index is a constant)
        const bool cok[2] = {full || rowC[0] < L, full || rowC[1] < L};
        const float *crow[2] = {Cm + ((b * L + (cok[0] ? rowC[0] : 0)) * G + gi) * N,
                                Cm + ((b * L + (cok[1] ? rowC[1] : 0)) * G + gi) * N};
        dispatch_wave<T / 32>(w, [&](auto wc) {
            constexpr int WI0 = decltype(wc)::value, WI1 = NT16 - 1 - WI0, WB1 = (WI0 + 2) & ~1;
            for (int s = 0; s < ns; ++s) {
                floatx4 cv[2], bv[WI1 + 1];
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
                    cv[ii] = cok[ii] ? *reinterpret_cast<const floatx4 *>(crow[ii] + 16 * s + 4 * g4) : zero4();
#pragma unroll
                for (int J = 0; J <= WI1; ++J) {  // WI1 >= WI0
                    bv[J] = zero4();
                    const int64_t row = t0 + 16 * J + l16;
                    if (full || row < L)
                        bv[J] = *reinterpret_cast<const floatx4 *>(Bm + ((b * L + row) * G + gi) * N + 16 * s + 4 * g4);
                }
#pragma unroll
                for (int J = 0; J <= WI1; ++J) {
                    if (J <= WI0)
#pragma unroll
                        for (int q = 0; q < 4; ++q) S[J] = mfma_f32(bv[J][q], cv[0][q], S[J]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) S[WB1 + J] = mfma_f32(bv[J][q], cv[1][q], S[WB1 + J]);
                }
            }
        });
    } else {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = ii ? I1 : I0;
        const int kb = ii ? base1 : 0, kend = ii ? NSLOT : base1;
        const bool crow_ok = full || rowC[ii] < L;
        const float *crow = Cm + ((b * L + (crow_ok ? rowC[ii] : 0)) * G + gi) * N;
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int J = k - kb;
            if (k < kb || k >= kend || J > I) continue;  // wave-uniform
            const int64_t row = t0 + 16 * J + l16;
            const bool brow_ok = full || row < L;
            const float *brow = Bm + ((b * L + (brow_ok ? row : 0)) * G + gi) * N;
            for (int s = 0; s < ns; ++s) {
                floatx4 bv = zero4(), cv = zero4();
                if (brow_ok) bv = *reinterpret_cast<const floatx4 *>(brow + 16 * s + 4 * g4);
                if (crow_ok) cv = *reinterpret_cast<const floatx4 *>(crow + 16 * s + 4 * g4);
#pragma unroll
                for (int q = 0; q < 4; ++q) S[k] = mfma_f32(bv[q], cv[q], S[k]);
            }
        }
    }
    }

    for (int h = h_begin; h < h_end; ++h) {
        stage_head();
        __syncthreads();
        if (h + 1 < h_end) load_head(h + 1);
        const float Dh = (Dv != nullptr) ? Dv[h] : 0.f;
        const float *hp = H + (((int64_t)b * NH + h) * NC + c) * (int64_t)P * N;
        const LaneIds id = opaque_lane_ids(tid);
        const int I0h = id.w, I1h = NT16 - 1 - id.w;
        const int base1h = slot_base1(I0h);
        const int64_t rc[2] = {t0 + 16 * I0h + id.l16, t0 + 16 * I1h + id.l16};

        floatx4 acc[2][PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[0][pt] = acc[1][pt] = zero4();

        // inter-chunk term C_i h_c.  Headdim 128 at chunk <= 128 runs one
        // wave per SIMD (the register budget), so the C and h fragments of
        // dstate step s + 2 are loaded while step s's MFMAs run: three
        // register sets in rotation.  Other shapes keep one set (the
        // second would cost them occupancy or spill).
        struct InterOps {
            floatx4 c[2], h[PT];
        };
        auto inter_load = [&](int s, InterOps &o) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                o.c[ii] = zero4();
                if (full || rc[ii] < L)
                    o.c[ii] = *reinterpret_cast<const floatx4 *>(Cm + ((b * L + rc[ii]) * G + gi) * N + 16 * s + 4 * id.g4);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                o.h[pt] = *reinterpret_cast<const floatx4 *>(hp + (16 * pt + id.l16) * N + 16 * s + 4 * id.g4);
        };
        auto inter_mfma = [&](const InterOps &o) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[0][pt] = mfma_f32(o.c[0][q], o.h[pt][q], acc[0][pt]);
                    acc[1][pt] = mfma_f32(o.c[1][q], o.h[pt][q], acc[1][pt]);
                }
        };
        if constexpr (T <= 128 && P == 128) {
            InterOps opa, opb, opc;
            inter_load(0, opa);
            if (1 < ns) inter_load(1, opb);
            for (int s = 0; s < ns; s += 3) {
                if (s + 2 < ns) inter_load(s + 2, opc);
                inter_mfma(opa);
                if (s + 1 < ns) {
                    if (s + 3 < ns) inter_load(s + 3, opa);
                    inter_mfma(opb);
                }
                if (s + 2 < ns) {
                    if (s + 4 < ns) inter_load(s + 4, opb);
                    inter_mfma(opc);
                }
            }
        } else {
            for (int s = 0; s < ns; ++s) {
                InterOps o;
                inter_load(s, o);
                inter_mfma(o);
            }
        }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const float4 e = *reinterpret_cast<const float4 *>(tb.e2 + 16 * (ii ? I1h : I0h) + 4 * id.g4);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                acc[ii][pt][0] *= e.x;
                acc[ii][pt][1] *= e.y;
                acc[ii][pt][2] *= e.z;
                acc[ii][pt][3] *= e.w;
            }
        }
        // intra-chunk term: instruction r of a slot contracts j = 16 J + 4 g4 + r
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int I = ii ? I1h : I0h;
            const int kb = ii ? base1h : 0, kend = ii ? NSLOT : base1h;
            const float gih = tb.gh[16 * I + id.l16], gil = tb.gl[16 * I + id.l16];
            const float rs = row_factor(tb, I, gih, gil);
#pragma unroll
            for (int k = 0; k < NSLOT; ++k) {
                const int J = k - kb;
                if (k < kb || k >= kend || J > I) continue;  // wave-uniform
                const float rm = J < I ? rs * tile_pair_factor(tb, I, J) : 0.f;
                float v[4];
                tile_values<T>(S[k], J, I, id.l16, id.g4, gih, gil, rm, tb, v);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float *xrow = xs + (16 * J + 4 * id.g4 + r) * LDP + id.l16;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        acc[ii][pt] = mfma_f32(v[r], xrow[16 * pt], acc[ii][pt]);
                }
            }
        }
        const int rows = (int)min<int64_t>(T, L - t0);
        const __amdgpu_buffer_rsrc_t yr = buffer_rsrc(
            y + ((b * L + t0) * NH + h) * P, (uint32_t)(((rows - 1) * NH * P + P) * sizeof(OutT)));
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int I = ii ? I1h : I0h;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int p = 16 * pt + id.l16;
                const int i0 = 16 * I + 4 * id.g4;
                float yv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) yv[r] = acc[ii][pt][r] + Dh * xs[(i0 + r) * LDP + p];
                store_out4<OutT>(yr, (i0 * NH * P + p) * (int)sizeof(OutT), NH * P * (int)sizeof(OutT), yv);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// bf16 path with asynchronous copies (headdim 64; dstate 128, or 256 at chunk
// 256)
// ---------------------------------------------------------------------------
// Same computation and tile assignment as k4_chunk_out_bf16, with the per-head
// data moved by the hardware: the x rows and the h_c hi/lo planes of head
// k + 1 are copied from global memory straight into a second LDS buffer
// (buffer loads with an LDS destination, 16 bytes per lane) while head k
// computes from the first, so no registers hold the next head and no VALU
// stages it; one block barrier per head.  x stays row-major ([token][p]) in
// LDS: the MFMA x operand, whose contraction index is the token, is read with
// the gfx950 transposing LDS read (ds_read_b64_tr_b16: within each 16-lane
// group, lane l receives element l % 4 of lanes 4r + (l % 16) / 4, r = 0..3),
// which hands every lane 4 tokens of its column; the same read returns the
// skip term's x in the MFMA output layout.  C fragments live in registers.
// Rows past the sequence end read as zero (the buffer resource ends at the
// chunk's last valid row).
//
// At dstate 256 the h_c planes (64 KiB) fit only once beside the two x
// buffers, and the C fragments take 64 registers per lane: the h_c planes are
// single-buffered, every wave takes the inter-chunk term first, and the
// next head's h_c copies go out after a block barrier behind it, landing
// during the intra-chunk term; the x rows and tables stay double-buffered.
// The C fragments then never leave registers, where the general kernel
// re-reads them from L2 in every head.
namespace acfg {
constexpr int P = 64, PT = P / 16;
}

template <int T, int N>
struct AsyncLds {
    static constexpr bool h_single = N > 128;                 // one h_c buffer
    static constexpr size_t x = (size_t)T * acfg::P * 2;      // row-major x tile
    static constexpr size_t plane = (size_t)acfg::P * N * 2;  // one h_c plane
    static constexpr size_t hb = 2 * plane;                   // one head's h_c planes
    static constexpr size_t tab = Tables<T>::bytes;
    // buffer k's x tile and h_c planes (dstate 128: x and h_c of one head side
    // by side; dstate 256: both x tiles, then the h_c planes), then the tables
    static constexpr size_t xoff(int k) { return h_single ? k * x : k * (x + hb); }
    static constexpr size_t hoff(int k) { return h_single ? 2 * x : k * (x + hb) + x; }
    static constexpr size_t tab0 = h_single ? 2 * x + hb : 2 * (x + hb);  // buffer k's tables at tab0 + k tab
    static constexpr size_t total = tab0 + 2 * tab;
    static_assert(total <= kLdsBytes, "async chunk-output LDS budget");
};

// x tile (128-byte token rows): 16-byte chunk c of row t is stored at chunk
// c ^ xswz(t), which spreads the 16 rows of one transposing read over all banks
__device__ __forceinline__ int xswz(int t) { return 2 * ((t >> 1) & 3); }


// One wave's output tile of one head (skip term included), from buffers
// xt (x tile) and hp (h_c hi plane, lo plane after it) and tables tb.
// Rows 16 I + 4 g4 + r (r = 0..3), column 16 pt + l16 of one head's y.
template <typename OutT>
__device__ __forceinline__ void store_quad(const floatx4 &v, __amdgpu_buffer_rsrc_t yr, int NHP,
                                           int I, int pt, int l16, int g4) {
    constexpr int ES = (int)sizeof(OutT);
    int lane_off = ((4 * g4) * NHP + l16) * ES;
    asm volatile("" : "+v"(lane_off));
    const float yv[4] = {v[0], v[1], v[2], v[3]};
    store_out4<OutT>(yr, lane_off + 16 * I * NHP * ES + 16 * pt * ES, NHP * ES, yv);
}

// acc holds this head's tile on return.  dstate 128: for the first-half
// waves it holds the previous head's finished tile on entry, stored through
// yprev, spread over the inter-chunk MFMAs and the first intra-chunk pairs (a
// resource of 0 bytes drops the stores); the second-half waves store their
// tile after the call.  pre(s), s = 0 .. 8 (first-half waves), issues piece s
// of the next head's copies: x and h_c pieces in the inter-chunk steps, the
// G2 / dt copies after them.  Issued any later, the copies land after the
// head's MFMAs and the end-of-head wait shows their latency; the stores, which
// need not land early, are spread further so that the memory queue never
// fills and blocks the MFMA issue.  dstate 256 (single h_c buffer): every wave
// stores its tile after the call; the x and G2 / dt pieces go out in the
// inter-chunk steps, the h_c pieces over the first intra-chunk pairs, after
// the block barrier that ends every wave's reads of h_c.
template <int T, int N, int W, typename OutT, typename Pre>
__device__ __forceinline__ void head_wave_async(const floatx4 (&S)[T / 16 + 2],
                                                const u32x4 (&cfr)[2][N / 32],
                                                const unsigned char *xt, const unsigned char *hp,
                                                const Tables<T> &tb, float Dh, int l16, int g4,
                                                floatx4 (&acc)[2][acfg::PT],
                                                __amdgpu_buffer_rsrc_t yprev, int NHP, Pre &&pre) {
    using WT = WaveTiles<T, W>;
    using LD = AsyncLds<T, N>;
    constexpr int PT = acfg::PT, NK = N / 32;
    constexpr int I0 = WT::I0, I1 = WT::I1;
    constexpr int XROW = acfg::P * 2, HROW = N * 2;
    constexpr bool kSingle = LD::h_single;
    constexpr bool kIssuer = W < T / 64;  // the waves that issue the next head's copies
    // the previous head's tile stored during this head (dstate 128, issuers)
    constexpr bool kDefer = !kSingle && kIssuer;
    static_assert(kSingle || NK == PT, "one (row tile, column tile) pair of stores per step and tile");

    // Waves of the first half take the inter-chunk term first, with the next
    // head's copies and the previous head's stores; waves of the second half
    // (which share SIMDs with the first) take the VALU-heavy intra-chunk term
    // first and store their tile at the end, so each SIMD overlaps one wave's
    // memory traffic with the other's VALU work.
    constexpr bool kIntraFirst = !kSingle && W >= T / 64;
    floatx4 prev[kDefer ? 2 : 1][kDefer ? PT : 1];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        if constexpr (kDefer) {
            prev[0][pt] = acc[0][pt];
            prev[1][pt] = acc[1][pt];
        }
        acc[0][pt] = acc[1][pt] = zero4();
    }

    // ---- inter-chunk term C_i h_c (h_c as hi + lo planes) into a; the
    // first-half waves issue the memory pieces between its steps
    auto inter = [&](floatx4 (&a)[2][PT]) {
        static_for<NK>([&](auto kc) {
            constexpr int ks = decltype(kc)::value;
            const int cofs = ((4 * ks + g4) ^ l16) << 4;  // chunk 4 ks + g4 of row 16 pt + l16
            u32x4 hh[PT], hl[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                hh[pt] = *reinterpret_cast<const u32x4 *>(hp + (16 * pt + l16) * HROW + cofs);
                hl[pt] = *reinterpret_cast<const u32x4 *>(hp + LD::plane + (16 * pt + l16) * HROW + cofs);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) a[ii][pt] = mfma_bf16(cfr[ii][ks], hh[pt], a[ii][pt]);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) a[ii][pt] = mfma_bf16(cfr[ii][ks], hl[pt], a[ii][pt]);
            if constexpr (kDefer) {
                pre(ks);
                pre(4 + ks);
                store_quad<OutT>(prev[0][ks], yprev, NHP, I0, ks, l16, g4);
            } else if constexpr (kSingle && kIssuer && ks % 2 == 0) {
                pre(ks / 2);  // x pieces only: h_c is still being read
            }
        });
        if constexpr (kIssuer) pre(8);
    };
    // exp2(G2_i) of rows i = 16 I + 4 g4 + r
    auto e2_rows = [&](int ii) {
        return *reinterpret_cast<const float4 *>(tb.e2 + 16 * (ii ? I1 : I0) + 4 * g4);
    };
    if constexpr (!kIntraFirst) {
        inter(acc);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const float4 e = e2_rows(ii);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                acc[ii][pt][0] *= e.x;
                acc[ii][pt][1] *= e.y;
                acc[ii][pt][2] *= e.z;
                acc[ii][pt][3] *= e.w;
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kSingle) __syncthreads();  // every wave is done reading this head's h_c

    // ---- intra-chunk term
    float mk;  // tile-pair factor of slot k = lane, read back wave-uniformly
    {
        const int k = l16 + 16 * g4;
        const int Ik = k < WT::base1 ? I0 : I1;
        const int Jk = k < WT::base1 ? k : k - WT::base1;
        const bool off = k < WT::NSLOT && Jk < Ik;
        const float m = tile_pair_factor(tb, off ? Ik : 1, off ? Jk : 0);  // in-range reads
        mk = off ? m : 0.f;
    }
    const float rs[2] = {row_factor(tb, I0, tb.gh[16 * I0 + l16], tb.gl[16 * I0 + l16]),
                         row_factor(tb, I1, tb.gh[16 * I1 + l16], tb.gl[16 * I1 + l16])};
    auto row_g2 = [&](int I, float &h, float &lo) {
        int off = 16 * I + l16;
        asm volatile("" : "+v"(off));
        h = tb.gh[off];
        lo = tb.gl[off];
    };
    // transposing-read offsets: this lane supplies row 4 g4 + (l16 >> 2) of a
    // 16-row tile and columns 16 pt + 4 (l16 & 3) .. +3
    int trb[PT];
    {
        const int tr_row = 4 * g4 + (l16 >> 2), tr_a = l16 & 3;
        const int f = xswz(tr_row);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            trb[pt] = tr_row * XROW + ((((2 * pt) ^ f) | (tr_a >> 1)) << 4) + 8 * (tr_a & 1);
            asm volatile("" : "+v"(trb[pt]));
        }
    }
    constexpr int NP = WT::NSLOT / 2;
    static_assert(!kSingle || NP >= 4, "the h_c pieces go out over the first four pairs");
    struct AOps {
        u32x4 hi, lo;
        u32x4 xb[PT];
    };
    auto prep = [&](auto qc) {
        constexpr int k0 = 2 * decltype(qc)::value;
        constexpr int ii = k0 < WT::base1 ? 0 : 1;
        constexpr int I = ii ? I1 : I0;
        constexpr int Ja = k0 - (ii ? WT::base1 : 0), Jb = Ja + 1;
        const float rma = rs[ii] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), k0));
        const float rmb = rs[ii] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), k0 + 1));
        float gih = 0.f, gil = 0.f;
        if constexpr (Ja == I || Jb == I) row_g2(I, gih, gil);
        float va[4], vb[4];
        tile_values_ct<T, Ja, I, true>(S[k0], l16, g4, gih, gil, rma, tb, va, Dh);
        tile_values_ct<T, Jb, I, true>(S[k0 + 1], l16, g4, gih, gil, rmb, tb, vb, Dh);
        const HiLo p0 = split_bf16(va[0], va[1]), p1 = split_bf16(va[2], va[3]);
        const HiLo p2 = split_bf16(vb[0], vb[1]), p3 = split_bf16(vb[2], vb[3]);
        AOps o;
        o.hi = u32x4{p0.hi, p1.hi, p2.hi, p3.hi};
        o.lo = u32x4{p0.lo, p1.lo, p2.lo, p3.lo};
        constexpr int JbR = Jb < WT::NT16 ? Jb : WT::NT16 - 1;  // padded tile: weights are 0
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            // tokens 16 Ja + 4 g4 .. +3 then 16 Jb + 4 g4 .. +3 of column 16 pt + l16
            const u32x2 a = tr_read(xt + 16 * Ja * XROW + trb[pt]);
            const u32x2 bq = tr_read(xt + 16 * JbR * XROW + trb[pt]);
            o.xb[pt] = u32x4{a[0], a[1], bq[0], bq[1]};
        }
        return o;
    };
    // dstate 128: the operands of pair q + 1 are built during the MFMAs of
    // pair q.  dstate 256: the C fragments leave no registers for a second
    // operand set; each pair's operands are built just before its MFMAs, and
    // the other wave of the SIMD fills the gap.
    AOps cur = prep(std::integral_constant<int, WT::pair_order(0)>{});
    static_for<NP>([&](auto qc) {
        constexpr int q = WT::pair_order(decltype(qc)::value);
        constexpr int ii = 2 * q < WT::base1 ? 0 : 1;
        constexpr int qn = decltype(qc)::value + 1;
        if constexpr (kSingle && decltype(qc)::value > 0) cur = prep(std::integral_constant<int, q>{});
        AOps nxt;
        if constexpr (!kSingle && qn < NP)
            nxt = prep(std::integral_constant<int, WT::pair_order(qn < NP ? qn : 0)>{});
        // the previous head's second row tile goes out over the first pairs
        if constexpr (kDefer && decltype(qc)::value < PT)
            store_quad<OutT>(prev[1][decltype(qc)::value], yprev, NHP, I1, decltype(qc)::value, l16, g4);
        // single h_c buffer: the next head's h_c copies over the first pairs
        if constexpr (kSingle && kIssuer && decltype(qc)::value < 4) pre(4 + decltype(qc)::value);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[ii][pt] = mfma_bf16(cur.hi, cur.xb[pt], acc[ii][pt]);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[ii][pt] = mfma_bf16(cur.lo, cur.xb[pt], acc[ii][pt]);
        if constexpr (!kSingle) {
            if constexpr (qn < NP) cur = nxt;
            // Interleave the next pair's VALU work with this pair's MFMAs: a
            // wave64 VALU op takes 4 cycles and an MFMA 16, so four or five of
            // them run under each MFMA instead of waiting for the whole group.
#pragma unroll
            for (int k = 0; k < 2 * PT; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    static_for<PT>([&](auto kc) {  // stores left over when there are fewer pairs than tiles
        if constexpr (kDefer && decltype(kc)::value >= NP)
            store_quad<OutT>(prev[1][decltype(kc)::value], yprev, NHP, I1, decltype(kc)::value, l16, g4);
    });
    if constexpr (kIntraFirst) {
        __builtin_amdgcn_sched_barrier(0);
        floatx4 t[2][PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) t[0][pt] = t[1][pt] = zero4();
        inter(t);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const float4 e = e2_rows(ii);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                acc[ii][pt][0] = fmaf(e.x, t[ii][pt][0], acc[ii][pt][0]);
                acc[ii][pt][1] = fmaf(e.y, t[ii][pt][1], acc[ii][pt][1]);
                acc[ii][pt][2] = fmaf(e.z, t[ii][pt][2], acc[ii][pt][2]);
                acc[ii][pt][3] = fmaf(e.w, t[ii][pt][3], acc[ii][pt][3]);
            }
        }
    }
}

// Store a wave's two output tiles (rows 16 I + 4 g4 + r, column 16 pt + l16).
template <typename OutT>
__device__ __forceinline__ void store_tile(const floatx4 (&acc)[2][acfg::PT], __amdgpu_buffer_rsrc_t yr,
                                           int NHP, int I0, int I1, int l16, int g4) {
    constexpr int ES = (int)sizeof(OutT);
    int lane_off = ((4 * g4) * NHP + l16) * ES;
    asm volatile("" : "+v"(lane_off));
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = ii ? I1 : I0;
#pragma unroll
        for (int pt = 0; pt < acfg::PT; ++pt) {
            const float yv[4] = {acc[ii][pt][0], acc[ii][pt][1], acc[ii][pt][2], acc[ii][pt][3]};
            store_out4<OutT>(yr, lane_off + 16 * I * NHP * ES + 16 * pt * ES, NHP * ES, yv);
        }
    }
}

// Derived per-token tables (exp2(G2_t) and the column factor) from the G2
// pair and dt already in the tables; thread t < T, same arithmetic as
// token_tables.
template <int T>
__device__ __forceinline__ void token_derived(const Tables<T> &tb, int t) {
    const float gh = tb.gh[t], gl = tb.gl[t], geh = tb.gh[t | 15], gel = tb.gl[t | 15];
    tb.e2[t] = fast_exp2(gh + gl);
    tb.cf[t] = fast_exp2((geh - gh) + (gel - gl)) * tb.dt[t];
}

template <int T, int N, typename OutT>
__global__ __launch_bounds__(2 * T) void k4_chunk_out_bf16_async(
    const uint16_t *__restrict__ x, const float *__restrict__ CBt,
    const uint16_t *__restrict__ Cm, const float *__restrict__ G2hi, const float *__restrict__ G2lo,
    const float *__restrict__ DT, const float *__restrict__ Dv, const uint16_t *__restrict__ H,
    OutT *__restrict__ y, int64_t L, int NH, int G, int NC, int64_t Lp, int HPG, int HB, int nhb) {
    using LD = AsyncLds<T, N>;
    constexpr int P = acfg::P, NK = N / 32, PT = acfg::PT;
    constexpr int NT16 = T / 16;
    constexpr int NSLOT = NT16 + 2;
    constexpr int NW = T / 32;
    constexpr int NTHR = 2 * T;

    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
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
    const int rows = (int)min<int64_t>(T, L - t0);  // valid tokens in this chunk
    const int64_t GN = (int64_t)G * N;
    const int NHP = NH * P;
    const uint16_t *Cc = Cm + ((b * L + t0) * G + gi) * N;

    // (a constant offset from lds plus k tab: the table reads then pair up)
    auto tables = [&](int k) { return Tables<T>(reinterpret_cast<float *>(lds + LD::tab0 + k * LD::tab)); };
    // ---- copies of one head's x rows, h_c planes, G2 pair and dt into buffer k.
    // x: 1-KiB blocks of 8 token rows; lane l takes 16-byte chunk l % 8 of row
    // 8 q + l / 8, from the global chunk that the row's swizzle puts there.
    // h_c: 1-KiB blocks of 1024 / (2 N) rows of the two stacked planes, the
    // 16-byte chunks XOR-swizzled by row.
    // G2 / dt: waves w < T / 64 copy tokens 64 w .. +63 (which they also
    // derive the tables of).
    const uint32_t x_bytes = (uint32_t)(((rows - 1) * NHP + P) * 2);
    // Pieces of head h's copies, issued by the first NW / 2 waves: s = 0 .. 3
    // a quarter of the x rows, 4 .. 7 a quarter of the h_c planes, 8 the
    // G2 / dt copies; the pieces go out spread over the previous head's MFMAs.
    constexpr int MW = NW / 2;  // copy-issuing waves
    constexpr int XQ = (int)(LD::x / 1024), HQ = (int)(2 * LD::plane / 1024);
    constexpr int XPW = XQ / MW, HPW = HQ / MW;  // copies per issuing wave
    static_assert(XQ % MW == 0 && HQ % MW == 0 && XPW % 4 == 0 && HPW % 4 == 0, "copy split");
    static_assert(T / 64 == MW, "the issuing waves also derive the tables");
    constexpr int HCPR = N / 8;                  // 16-byte chunks per h_c row
    constexpr int HRPK = 64 / HCPR;              // h_c rows per 1-KiB block
    constexpr int HCSH = N == 128 ? 4 : 5;       // log2(HCPR)
    static_assert(HCPR == 1 << HCSH, "h_c row chunks");
    auto issue_piece = [&](int h, int k, int s) {
        const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);  // < MW
        int ln = tid & 63;
        asm volatile("" : "+v"(ln));
        const uint32_t xb = lds_addr(lds + LD::xoff(k));
        if (s < 4) {
            const i32x4 xd = buffer_desc(x + ((b * L + t0) * NH + h) * P, x_bytes);
            const int xr = ln >> 3, xl = ((ln & 7) ^ xswz(ln >> 3)) * 16;
#pragma unroll
            for (int kk = s * (XPW / 4); kk < (s + 1) * (XPW / 4); ++kk) {
                const int q = wu + kk * MW;
                lds_dma_x4(xd, xb + q * 1024, (8 * q + xr) * NHP * 2 + xl);
            }
        } else if (s < 8) {
            const i32x4 hd = buffer_desc(H + (((int64_t)b * NH + h) * NC + c) * (int64_t)2 * P * N,
                                         (uint32_t)(2 * LD::plane));
            const uint32_t hbase = LD::h_single ? lds_addr(lds + LD::hoff(k)) : xb + (uint32_t)LD::x;
#pragma unroll
            for (int kk = (s - 4) * (HPW / 4); kk < (s - 3) * (HPW / 4); ++kk) {
                const int qh = wu + kk * MW;
                const int row = HRPK * qh + (ln >> HCSH);  // row of the two stacked planes
                lds_dma_x4(hd, hbase + qh * 1024, row * (2 * N) + (((ln & (HCPR - 1)) ^ (row & 15)) << 4));
            }
        } else {
            const int64_t hoff = ((int64_t)b * NH + h) * Lp + t0;
            const Tables<T> tb = tables(k);
            const int voff = (64 * wu + ln) * 4;
            lds_dma_x1(buffer_desc(G2hi + hoff, T * 4), lds_addr(tb.gh + 64 * wu), voff);
            lds_dma_x1(buffer_desc(G2lo + hoff, T * 4), lds_addr(tb.gl + 64 * wu), voff);
            lds_dma_x1(buffer_desc(DT + hoff, T * 4), lds_addr(tb.dt + 64 * wu), voff);
        }
    };
    auto issue = [&](int h, int k) {
#pragma unroll
        for (int s = 0; s < 9; ++s) issue_piece(h, k, s);
    };

    // 16 bytes of row `row` of a (rows x N) bf16 matrix at dstate n0; rows past
    // the chunk's valid rows read as zero (clamped address, value selected)
    auto chunk16 = [&](const uint16_t *base, int row, int n0) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(base + (int64_t)min(row, rows - 1) * GN + n0);
        return row < rows ? v : u32x4{0u, 0u, 0u, 0u};
    };
    // ---- C fragments (registers): lane holds C[t0 + 16 I + l16][32 ks + 8 g4 .. +7]
    const int I0 = w, I1 = NT16 - 1 - w;
    u32x4 cfr[2][NK];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
            cfr[ii][ks] = chunk16(Cc, 16 * (ii ? I1 : I0) + l16, 32 * ks + 8 * g4);

    // ---- C B^T tiles of this wave's slots, computed once per chunk by the
    // state-passing launch; then the first head's copies (after every
    // compiler-visible load, whose waits would otherwise count them)
    floatx4 S[NSLOT];
    {
        const floatx4 *cb = reinterpret_cast<const floatx4 *>(CBt) +
                            ((((b * NC + c) * G + gi) * NW + w) * NSLOT) * 64 + lane;
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) S[k] = cb[k * 64];
    }
    if (h_begin < h_end && w < MW) issue(h_begin, 0);
    lds_dma_wait();  // this wave's copies of the first head have landed
    if (h_begin < h_end && tid < T) token_derived(tables(0), tid);
    __syncthreads();  // every wave's copies are visible

    // ---- heads: the copies for head i + 1 run while head i computes
    floatx4 acc[2][PT];
    const uint32_t y_bytes = (uint32_t)(((rows - 1) * NHP + P) * sizeof(OutT));
    auto y_head = [&](int h) { return buffer_rsrc(y + ((b * L + t0) * NH + h) * P, y_bytes); };
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[0][pt] = acc[1][pt] = zero4();
    for (int i = 0; h_begin + i < h_end; ++i) {
        const int h = h_begin + i, cur = i & 1;
        const LaneIds id = opaque_lane_ids(tid);
        const bool issuer = id.w < MW;  // wave-uniform
        const bool more = h + 1 < h_end;
        auto pre = [&](int s) {
            if (more) issue_piece(h + 1, cur ^ 1, s);
        };
        const float Dh = (Dv != nullptr) ? Dv[h] : 0.f;
        // dstate 128: the previous head's y goes out during this head's first MFMAs
        const auto yprev = buffer_rsrc(y + ((b * L + t0) * NH + (i > 0 ? h - 1 : h)) * P,
                                       (!LD::h_single && i > 0) ? y_bytes : 0u);
        dispatch_wave<NW>(id.w, [&](auto wc) {
            head_wave_async<T, N, decltype(wc)::value, OutT>(S, cfr, lds + LD::xoff(cur), lds + LD::hoff(cur),
                                                             tables(cur), Dh, id.l16, id.g4, acc, yprev, NHP,
                                                             pre);
        });
        if (issuer) {
            lds_dma_wait();  // this wave's copies of the next head have landed
            if (more) token_derived(tables(cur ^ 1), tid);
            if constexpr (LD::h_single)
                store_tile<OutT>(acc, y_head(h), NHP, id.w, NT16 - 1 - id.w, id.l16, id.g4);
        } else {
            store_tile<OutT>(acc, y_head(h), NHP, id.w, NT16 - 1 - id.w, id.l16, id.g4);
        }
        __syncthreads();
    }
    if (!LD::h_single && h_begin < h_end && w < MW)
        store_tile<OutT>(acc, y_head(h_end - 1), NHP, I0, I1, l16, g4);
}

// ---------------------------------------------------------------------------
// launch: InT is the input element type, OutT the element type of y
// ---------------------------------------------------------------------------
template <int T, int P, int NKMAX, typename OutT>
hipError_t launch_bf16_in(const Problem &p, int HB, int nhb, int64_t blocks, const void *x,
                          const void *B, const void *C, const float *CB, G2View G2, const float *DT, const float *D,
                          const float *H, void *y, hipStream_t stream, const LaunchEvents &ev) {
    constexpr auto kern = k4_chunk_out_bf16<T, P, NKMAX, OutT>;
    constexpr size_t lds = Bf16Lds<T, P, NKMAX>::total;
    if (allow_lds<kern>(lds) != hipSuccess) return hipErrorInvalidValue;
    launch_kernel(kern, dim3((unsigned)blocks), dim3(2 * T), lds, stream, ev,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B),
                       static_cast<const uint16_t *>(C), G2.hi, G2.lo, DT, D,
                       reinterpret_cast<const uint16_t *>(H),  // hi/lo bf16 planes
                       static_cast<OutT *>(y), p.seqlen, (int)p.nheads, (int)p.dstate,
                       (int)p.ngroups, (int)p.nchunks, p.padded_len, (int)p.heads_per_group, HB,
                       nhb);
    return hipGetLastError();
}

template <int T, int P, typename OutT>
hipError_t launch_f32_in(const Problem &p, int HB, int nhb, int64_t blocks, const void *x,
                         const void *B, const void *C, const float *CB, G2View G2, const float *DT, const float *D,
                         const float *H, void *y, hipStream_t stream, const LaunchEvents &ev) {
    constexpr auto kern = k4_chunk_out_f32<T, P, OutT>;
    constexpr size_t lds = F32Lds<T, P>::total;
    if (allow_lds<kern>(lds) != hipSuccess) return hipErrorInvalidValue;
    launch_kernel(kern, dim3((unsigned)blocks), dim3(2 * T), lds, stream, ev,
                       static_cast<const float *>(x), static_cast<const float *>(B),
                       static_cast<const float *>(C), G2.hi, G2.lo, DT, D, H,
                       static_cast<OutT *>(y), p.seqlen, (int)p.nheads, (int)p.dstate,
                       (int)p.ngroups, (int)p.nchunks, p.padded_len, (int)p.heads_per_group, HB,
                       nhb);
    return hipGetLastError();
}

template <int T, int N, typename OutT>
hipError_t launch_bf16_async(const Problem &p, int HB, int nhb, int64_t blocks, const void *x,
                             const void *B, const void *C, const float *CB, G2View G2, const float *DT, const float *D,
                             const float *H, void *y, hipStream_t stream, const LaunchEvents &ev) {
    constexpr auto kern = k4_chunk_out_bf16_async<T, N, OutT>;
    constexpr size_t lds = AsyncLds<T, N>::total;
    if (allow_lds<kern>(lds) != hipSuccess) return hipErrorInvalidValue;
    launch_kernel(kern, dim3((unsigned)blocks), dim3(2 * T), lds, stream, ev,
                  static_cast<const uint16_t *>(x), CB, static_cast<const uint16_t *>(C), G2.hi,
                  G2.lo, DT, D,
                  reinterpret_cast<const uint16_t *>(H),  // hi/lo bf16 planes
                  static_cast<OutT *>(y), p.seqlen, (int)p.nheads, (int)p.ngroups, (int)p.nchunks,
                  p.padded_len, (int)p.heads_per_group, HB, nhb);
    return hipGetLastError();
}

template <typename InT, typename OutT, int T, int P>
hipError_t launch_tp(const Problem &p, const Plan &plan, const void *x, const void *B, const void *C,
                     const float *CB, G2View G2, const float *DT, const float *D, const float *H, void *y,
                     hipStream_t stream, const LaunchEvents &ev) {
    const int HB = plan.k4_heads_per_block;
    const int nhb = (int)((p.heads_per_group + HB - 1) / HB);
    const int64_t blocks = p.batch * p.nchunks * p.ngroups * nhb;
    if (blocks == 0) return hipSuccess;
    if constexpr (sizeof(InT) == 2) {
        if constexpr (P == acfg::P) {
            if (uses_cb_tiles(p) && p.dstate == 128)
                return launch_bf16_async<T, 128, OutT>(p, HB, nhb, blocks, x, B, C, CB, G2, DT, D, H, y, stream, ev);
            if constexpr (T == 256)
                if (uses_cb_tiles(p) && p.dstate == 256)
                    return launch_bf16_async<T, 256, OutT>(p, HB, nhb, blocks, x, B, C, CB, G2, DT, D, H, y,
                                                           stream, ev);
        }
        if (p.dstate <= 128)
            return launch_bf16_in<T, P, 4, OutT>(p, HB, nhb, blocks, x, B, C, CB, G2, DT, D, H, y, stream, ev);
        return launch_bf16_in<T, P, 8, OutT>(p, HB, nhb, blocks, x, B, C, CB, G2, DT, D, H, y, stream, ev);
    } else {
        return launch_f32_in<T, P, OutT>(p, HB, nhb, blocks, x, B, C, CB, G2, DT, D, H, y, stream, ev);
    }
}

template <typename InT, typename OutT>
hipError_t launch(const Problem &p, const Plan &plan, const void *x, const void *B, const void *C,
                  const float *CB, G2View G2, const float *DT, const float *D, const float *H, void *y,
                  hipStream_t stream, const LaunchEvents &ev) {
#define SSD_K4_P(T)                                                                              \
    switch (p.headdim) {                                                                         \
        case 32: return launch_tp<InT, OutT, T, 32>(p, plan, x, B, C, CB, G2, DT, D, H, y, stream, ev);  \
        case 64: return launch_tp<InT, OutT, T, 64>(p, plan, x, B, C, CB, G2, DT, D, H, y, stream, ev);  \
        case 128: return launch_tp<InT, OutT, T, 128>(p, plan, x, B, C, CB, G2, DT, D, H, y, stream, ev); \
        default: return hipErrorInvalidValue;                                                    \
    }
    switch (p.chunk) {
        case 64: SSD_K4_P(64)
        case 128: SSD_K4_P(128)
        case 256: SSD_K4_P(256)
        default: return hipErrorInvalidValue;
    }
#undef SSD_K4_P
}

// One explicit instantiation per translation unit (compiled in parallel).
hipError_t launch_bf16_in_f32_out(const Problem &p, const Plan &plan, const void *x, const void *B,
                                  const void *C, const float *CB, G2View G2, const float *DT, const float *D,
                                  const float *H, void *y, hipStream_t stream, const LaunchEvents &ev);
hipError_t launch_bf16_in_bf16_out(const Problem &p, const Plan &plan, const void *x, const void *B,
                                   const void *C, const float *CB, G2View G2, const float *DT, const float *D,
                                   const float *H, void *y, hipStream_t stream, const LaunchEvents &ev);

}  // namespace k4
}  // namespace ssd

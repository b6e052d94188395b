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
//    transposed ([headdim][token], 8-byte units XOR-swizzled by
//    (row ^ row >> 3) & 15: conflict-free for the transposing writes and the
//    operand reads).  The fp32-valued operands -- the decay-masked tile and the
//    carried state h_c -- are split into hi + lo bf16 halves and multiplied by
//    the exact bf16 inputs, so the result keeps fp32-accumulation accuracy.
//  * fp32 inputs: v_mfma_f32_16x16x4_f32 on the fp32 values directly; X is
//    staged in its natural layout, h_c and C fragments are read from global
//    memory (L2) as 16-byte vectors.
// Off-diagonal tiles (J < I) use exp2(G2_i - G2_j) = exp2(G2_i - G2_e) *
// exp2(G2_e - G2_j) with e the last token of tile J: both exponents are <= 0,
// and the second factor (times dt_j) is tabulated once per head and token, so
// a lane needs one exp2 per tile instead of four.  The next head's x, h_c and
// decay data are loaded into registers while the current head computes.
#pragma once

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace k4 {

// Wave w owns row tiles I0 = w and I1 = T/16 - 1 - w.  Its S slots are laid
// out as [I0: J = 0..I0][pad to even][I1: J = 0..I1][pad to even]; the total
// is always T/16 + 2 and a pair (2q, 2q + 1) never straddles the two tiles.
__device__ __forceinline__ int slot_base1(int I0) { return (I0 + 2) & ~1; }

// Per-head decay tables (T floats each, in LDS) for the tokens of the chunk:
//   gh[t] + gl[t] = G2_t (the hi/lo pair),  dts[t] = dt_t,
//   cfs[t] = exp2(G2_e(t) - G2_t) dt_t with e(t) the last token of t's 16-tile.
// Every exponent below is a difference formed as (hi_i - hi_j) + (lo_i - lo_j).
struct Tables {
    float *gh, *gl, *cfs, *dts;
};

__device__ __forceinline__ void head_tables(const Tables &tb, int t, float gh, float gl, float geh,
                                            float gel, float d) {
    tb.gh[t] = gh;
    tb.gl[t] = gl;
    tb.cfs[t] = fast_exp2((geh - gh) + (gel - gl)) * d;
    tb.dts[t] = d;
}

// Decay-and-dt weighted values of one S tile slot for this lane: row
// i = 16 I + l16 (G2_i = gih + gil), columns j = 16 J + 4 g4 + r.  On the
// diagonal tile the exponent is the exact difference G2_i - G2_j (0 for j = i)
// and the mask is a select taken before exp2; off the diagonal both factors of
// exp2(G2_i - G2_e) exp2(G2_e - G2_j) have exponents <= 0.
__device__ __forceinline__ void tile_values(const floatx4 &s, int J, int I, float gih, float gil,
                                            const Tables &tb, int l16, int g4, float (&v)[4]) {
    if (J > I) {
        v[0] = v[1] = v[2] = v[3] = 0.f;
    } else if (J < I) {
        const int e = 16 * J + 15;
        const float rf = fast_exp2((gih - tb.gh[e]) + (gil - tb.gl[e]));
        const float4 cf = *reinterpret_cast<const float4 *>(tb.cfs + 16 * J + 4 * g4);
        v[0] = s[0] * (rf * cf.x);
        v[1] = s[1] * (rf * cf.y);
        v[2] = s[2] * (rf * cf.z);
        v[3] = s[3] * (rf * cf.w);
    } else {
        const float4 jh = *reinterpret_cast<const float4 *>(tb.gh + 16 * J + 4 * g4);
        const float4 jl = *reinterpret_cast<const float4 *>(tb.gl + 16 * J + 4 * g4);
        const float4 dj = *reinterpret_cast<const float4 *>(tb.dts + 16 * J + 4 * g4);
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

// exp2(G2) of the four accumulator rows 16 I + 4 g4 + r
__device__ __forceinline__ void row_decay(const Tables &tb, int I, int g4, float (&e)[4]) {
    const float4 h = *reinterpret_cast<const float4 *>(tb.gh + 16 * I + 4 * g4);
    const float4 l = *reinterpret_cast<const float4 *>(tb.gl + 16 * I + 4 * g4);
    e[0] = fast_exp2(h.x + l.x);
    e[1] = fast_exp2(h.y + l.y);
    e[2] = fast_exp2(h.z + l.z);
    e[3] = fast_exp2(h.w + l.w);
}

template <typename OutT>
__device__ __forceinline__ void store_out(OutT *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float v) {
    *p = (uint16_t)(pack_bf16(v, 0.f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// bf16 path
// ---------------------------------------------------------------------------
// 8-byte-unit swizzle of the transposed x tile ([P][T] bf16).
__device__ __forceinline__ int swz16(int row) { return (row ^ (row >> 3)) & 15; }
template <int T>
__device__ __forceinline__ int xt_off(int row, int unit) {  // unit = token / 4
    return row * (T * 2) + ((unit ^ swz16(row)) << 3);
}
// 16-byte-chunk swizzle of the h tile ([P][NPAD] bf16).
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }
template <int NPAD>
__device__ __forceinline__ int h_off(int row, int chunk) {  // chunk = n / 8
    return row * (NPAD * 2) + ((chunk ^ swz8(row)) << 4);
}

__device__ __forceinline__ uint32_t sel_half(int q) { return (q & 1) ? 0x07060302u : 0x05040100u; }

// gfx950 LDS per CU (and the most one block may use)
constexpr size_t kLdsBytes = 160 * 1024;

// LDS of the bf16 kernel: x^T tile, the h hi/lo tiles when they fit, decay tables.
template <int T, int P, int NKMAX>
struct Bf16Lds {
    static constexpr size_t x = (size_t)P * T * 2;
    static constexpr size_t h = (size_t)2 * P * (NKMAX * 32) * 2;
    static constexpr size_t tables = (size_t)4 * T * 4;
    // h is staged in LDS when everything fits; otherwise its fragments are read
    // from global memory (L2) and split into hi/lo in registers.
    static constexpr bool h_in_lds = x + h + tables <= kLdsBytes;
    static constexpr size_t total = x + (h_in_lds ? h : 0) + tables;
    static_assert(total <= kLdsBytes, "stage-4 LDS budget exceeded");
};

template <int T, int P, int NKMAX, typename OutT>
__global__ __launch_bounds__(2 * T) void k4_chunk_out_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ G2hi, const float *__restrict__ G2lo,
    const float *__restrict__ DT, const float *__restrict__ Dv, const float *__restrict__ H,
    OutT *__restrict__ y,
    int64_t L, int NH, int N, int G, int NC, int64_t Lp, int HPG, int HB, int nhb) {
    constexpr int NT16 = T / 16;
    constexpr int NSLOT = NT16 + 2;
    constexpr int PT = P / 16;
    constexpr int NPAD = NKMAX * 32;
    constexpr int NTHR = 2 * T;
    constexpr int PO = P / 8;
    constexpr int XUNITS = (T / 4) * PO;              // 4-token x 8-column units of x
    constexpr int XPASS = (XUNITS + NTHR - 1) / NTHR;
    constexpr int HCH = NPAD / 8;                     // 8-element chunks per h row
    constexpr int HUNITS = P * HCH;
    constexpr int HPASS = (HUNITS + NTHR - 1) / NTHR;
    constexpr int HREG = Bf16Lds<T, P, NKMAX>::h_in_lds ? HPASS : 1;

    using Lds = Bf16Lds<T, P, NKMAX>;
    constexpr bool kHinLds = Lds::h_in_lds;
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char *xt = lds;                          // [P][T] bf16
    unsigned char *hhi = xt + Lds::x;                 // [P][NPAD] bf16 (if kHinLds)
    unsigned char *hlo = hhi + Lds::h / 2;            // [P][NPAD] bf16 (if kHinLds)
    float *tbase = reinterpret_cast<float *>(xt + Lds::x + (kHinLds ? Lds::h : 0));
    const Tables tb{tbase, tbase + T, tbase + 2 * T, tbase + 3 * T};

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
    const int nk = (N + 31) / 32;

    const int I0 = w, I1 = NT16 - 1 - w;
    const int base1 = slot_base1(I0);

    // ---------------- per-head data, loaded one head ahead ----------------
    u32x4 xr[XPASS][4];   // unit: 4 tokens x 8 headdim columns
    floatx4 hr[HREG][2];  // unit: 8 consecutive fp32 of one h row
    float sgh = 0.f, sgl = 0.f, seh = 0.f, sel = 0.f, sdt = 0.f;
    auto load_head = [&](int h) {
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            const int u = tid + ps * NTHR;
            const int po = u % PO, tq = u / PO;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t tok = t0 + 4 * tq + r;
                xr[ps][r] = u32x4{0u, 0u, 0u, 0u};
                if (u < XUNITS && tok < L)
                    xr[ps][r] = *reinterpret_cast<const u32x4 *>(x + ((b * L + tok) * NH + h) * P + po * 8);
            }
        }
        const float *hp = H + (((int64_t)b * NH + h) * NC + c) * (int64_t)P * N;
        if constexpr (kHinLds) {
#pragma unroll
            for (int ps = 0; ps < HPASS; ++ps) {
                const int u = tid + ps * NTHR;
                const int ch = u % HCH, p = u / HCH;
                hr[ps][0] = hr[ps][1] = zero4();
                if (u < HUNITS && 8 * ch < N) {
                    hr[ps][0] = *reinterpret_cast<const floatx4 *>(hp + p * N + 8 * ch);
                    hr[ps][1] = *reinterpret_cast<const floatx4 *>(hp + p * N + 8 * ch + 4);
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
            const int u = tid + ps * NTHR;
            if (u < XUNITS) {
                const int po = u % PO, tq = u / PO;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t s = sel_half(q);
                    const u32x2 v = {__builtin_amdgcn_perm(xr[ps][1][q >> 1], xr[ps][0][q >> 1], s),
                                     __builtin_amdgcn_perm(xr[ps][3][q >> 1], xr[ps][2][q >> 1], s)};
                    *reinterpret_cast<u32x2 *>(xt + xt_off<T>(8 * po + q, tq)) = v;
                }
            }
        }
#pragma unroll
        for (int ps = 0; ps < HPASS; ++ps) {
            const int u = tid + ps * NTHR;
            if (kHinLds && u < HUNITS) {
                const int ch = u % HCH, p = u / HCH;
                u32x4 hi, lo;
                { const HiLo s2 = split_bf16(hr[ps][0][0], hr[ps][0][1]); hi[0] = s2.hi; lo[0] = s2.lo; }
                { const HiLo s2 = split_bf16(hr[ps][0][2], hr[ps][0][3]); hi[1] = s2.hi; lo[1] = s2.lo; }
                { const HiLo s2 = split_bf16(hr[ps][1][0], hr[ps][1][1]); hi[2] = s2.hi; lo[2] = s2.lo; }
                { const HiLo s2 = split_bf16(hr[ps][1][2], hr[ps][1][3]); hi[3] = s2.hi; lo[3] = s2.lo; }
                *reinterpret_cast<u32x4 *>(hhi + h_off<NPAD>(p, ch)) = hi;
                *reinterpret_cast<u32x4 *>(hlo + h_off<NPAD>(p, ch)) = lo;
            }
        }
        if (tid < T) head_tables(tb, tid, sgh, sgl, seh, sel, sdt);
    };

    if (h_begin < h_end) load_head(h_begin);

    // ---------------- C fragments of the wave's two row tiles -------------
    // lane holds C[t0 + 16 I + l16][32 ks + 8 g4 .. +7]
    u32x4 cfr[2][NKMAX];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int64_t row = t0 + 16 * (ii ? I1 : I0) + l16;
#pragma unroll
        for (int ks = 0; ks < NKMAX; ++ks) {
            const int n0 = 32 * ks + 8 * g4;
            cfr[ii][ks] = u32x4{0u, 0u, 0u, 0u};
            if (ks < nk && row < L && n0 < N)
                cfr[ii][ks] = *reinterpret_cast<const u32x4 *>(Cm + ((b * L + row) * G + gi) * N + n0);
        }
    }

    // ---------------- C B^T tiles (transposed), once per block -------------
    floatx4 S[NSLOT];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) S[k] = zero4();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = ii ? I1 : I0;
        const int kb = ii ? base1 : 0, kend = ii ? NSLOT : base1;
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int J = k - kb;
            if (k < kb || k >= kend || J > I) continue;  // wave-uniform
            const int64_t row = t0 + 16 * J + l16;
#pragma unroll
            for (int ks = 0; ks < NKMAX; ++ks) {
                if (ks >= nk) continue;
                const int n0 = 32 * ks + 8 * g4;
                u32x4 bfr = u32x4{0u, 0u, 0u, 0u};
                if (row < L && n0 < N)
                    bfr = *reinterpret_cast<const u32x4 *>(Bm + ((b * L + row) * G + gi) * N + n0);
                S[k] = mfma_bf16(bfr, cfr[ii][ks], S[k]);
            }
        }
    }

    // ---------------- heads -------------------------------------------------
    for (int h = h_begin; h < h_end; ++h) {
        stage_head();
        __syncthreads();
        if (h + 1 < h_end) load_head(h + 1);
        const float Dh = (Dv != nullptr) ? Dv[h] : 0.f;
        // Re-derive the lane coordinates from an opaque copy each head, so the
        // compiler recomputes the (cheap) swizzled LDS offsets instead of
        // hoisting all of them out of the head loop into registers.
        int tid_o = tid;
        asm volatile("" : "+v"(tid_o));
        const int l16 = tid_o & 15, g4 = (tid_o >> 4) & 3;
        const int w_o = __builtin_amdgcn_readfirstlane(tid_o >> 6);
        const int I0 = w_o, I1 = NT16 - 1 - w_o;
        const int base1 = slot_base1(I0);

        floatx4 acc[2][PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[0][pt] = acc[1][pt] = zero4();

        // inter-chunk term C_i h_c (h split into hi + lo)
        const float *hp = H + (((int64_t)b * NH + h) * NC + c) * (int64_t)P * N;
#pragma unroll
        for (int ks = 0; ks < NKMAX; ++ks) {
            if (ks >= nk) continue;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                u32x4 hh, hl;
                if constexpr (kHinLds) {
                    const int off = h_off<NPAD>(16 * pt + l16, 4 * ks + g4);
                    hh = *reinterpret_cast<const u32x4 *>(hhi + off);
                    hl = *reinterpret_cast<const u32x4 *>(hlo + off);
                } else {
                    // lane reads h[p][32 ks + 8 g4 .. +7]; columns past dstate are 0
                    floatx4 v0 = zero4(), v1 = zero4();
                    const int n0 = 32 * ks + 8 * g4;
                    if (n0 < N) {
                        const float *src = hp + (16 * pt + l16) * N + n0;
                        v0 = *reinterpret_cast<const floatx4 *>(src);
                        v1 = *reinterpret_cast<const floatx4 *>(src + 4);
                    }
                    const HiLo a = split_bf16(v0[0], v0[1]), bq = split_bf16(v0[2], v0[3]);
                    const HiLo cq = split_bf16(v1[0], v1[1]), dq = split_bf16(v1[2], v1[3]);
                    hh = u32x4{a.hi, bq.hi, cq.hi, dq.hi};
                    hl = u32x4{a.lo, bq.lo, cq.lo, dq.lo};
                }
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    acc[ii][pt] = mfma_bf16(cfr[ii][ks], hh, acc[ii][pt]);
                    acc[ii][pt] = mfma_bf16(cfr[ii][ks], hl, acc[ii][pt]);
                }
            }
        }
        // rows i = 16 I + 4 g4 + r take exp2(G2_i)
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            float e[4];
            row_decay(tb, ii ? I1 : I0, g4, e);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[ii][pt][r] *= e[r];
        }
        // intra-chunk term: slot pairs (J, J + 1) of one row tile, K = 32
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int I = ii ? I1 : I0;
            const int kb = ii ? base1 : 0, kend = ii ? NSLOT : base1;
            const float gih = tb.gh[16 * I + l16], gil = tb.gl[16 * I + l16];
#pragma unroll
            for (int q = 0; q < NSLOT / 2; ++q) {
                const int k0 = 2 * q;
                if (k0 < kb || k0 >= kend) continue;  // wave-uniform
                const int Ja = k0 - kb, Jb = Ja + 1;
                float va[4], vb[4];
                tile_values(S[k0], Ja, I, gih, gil, tb, l16, g4, va);
                tile_values(S[k0 + 1], Jb, I, gih, gil, tb, l16, g4, vb);
                u32x4 ahi, alo;
                { const HiLo s2 = split_bf16(va[0], va[1]); ahi[0] = s2.hi; alo[0] = s2.lo; }
                { const HiLo s2 = split_bf16(va[2], va[3]); ahi[1] = s2.hi; alo[1] = s2.lo; }
                { const HiLo s2 = split_bf16(vb[0], vb[1]); ahi[2] = s2.hi; alo[2] = s2.lo; }
                { const HiLo s2 = split_bf16(vb[2], vb[3]); ahi[3] = s2.hi; alo[3] = s2.lo; }
                const int JbR = Jb < NT16 ? Jb : NT16 - 1;  // padded tile: weights are 0
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int p = 16 * pt + l16;
                    const u32x2 xa = *reinterpret_cast<const u32x2 *>(xt + xt_off<T>(p, 4 * Ja + g4));
                    const u32x2 xb = *reinterpret_cast<const u32x2 *>(xt + xt_off<T>(p, 4 * JbR + g4));
                    const u32x4 bop = {xa[0], xa[1], xb[0], xb[1]};
                    acc[ii][pt] = mfma_bf16(ahi, bop, acc[ii][pt]);
                    acc[ii][pt] = mfma_bf16(alo, bop, acc[ii][pt]);
                }
            }
        }
        // skip term and store: lane holds rows 16 I + 4 g4 + r, column 16 pt + l16
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int I = ii ? I1 : I0;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int p = 16 * pt + l16;
                const u32x2 xi = *reinterpret_cast<const u32x2 *>(xt + xt_off<T>(p, 4 * I + g4));
                const float xv[4] = {bf16lo(xi[0]), bf16hi(xi[0]), bf16lo(xi[1]), bf16hi(xi[1])};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = t0 + 16 * I + 4 * g4 + r;
                    if (row < L) {
                        store_out(&y[((b * L + row) * NH + h) * P + p], acc[ii][pt][r] + Dh * xv[r]);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
template <int T, int P, typename OutT>
__global__ __launch_bounds__(2 * T) void k4_chunk_out_f32(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ Cm,
    const float *__restrict__ G2hi, const float *__restrict__ G2lo, const float *__restrict__ DT,
    const float *__restrict__ Dv, const float *__restrict__ H, OutT *__restrict__ y, int64_t L,
    int NH, int N, int G, int NC,
    int64_t Lp, int HPG, int HB, int nhb) {
    constexpr int NT16 = T / 16;
    constexpr int NSLOT = NT16 + 2;
    constexpr int PT = P / 16;
    constexpr int NTHR = 2 * T;
    constexpr int LDP = P + 4;                       // padded LDS row (floats)
    constexpr int XV = T * (P / 4);                  // float4 units of the x tile
    constexpr int XPASS = (XV + NTHR - 1) / NTHR;

    extern __shared__ __align__(16) unsigned char lds[];
    float *xs = reinterpret_cast<float *>(lds);       // [T][LDP]
    const Tables tb{xs + T * LDP, xs + T * LDP + T, xs + T * LDP + 2 * T, xs + T * LDP + 3 * T};

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

    const int I0 = w, I1 = NT16 - 1 - w;
    const int base1 = slot_base1(I0);
    const int64_t rowC[2] = {t0 + 16 * I0 + l16, t0 + 16 * I1 + l16};
    const float *crow[2] = {Cm + ((b * L + rowC[0]) * G + gi) * N, Cm + ((b * L + rowC[1]) * G + gi) * N};

    floatx4 xr[XPASS];
    float sgh = 0.f, sgl = 0.f, seh = 0.f, sel = 0.f, sdt = 0.f;
    auto load_head = [&](int h) {
#pragma unroll
        for (int ps = 0; ps < XPASS; ++ps) {
            const int v = tid + ps * NTHR;
            const int t = v / (P / 4), p4 = v % (P / 4);
            xr[ps] = zero4();
            if (v < XV && t0 + t < L)
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
        if (tid < T) head_tables(tb, tid, sgh, sgl, seh, sel, sdt);
    };

    if (h_begin < h_end) load_head(h_begin);

    // C B^T tiles (transposed), once per block.  K = 4 per MFMA: instruction q
    // of a 16-wide dstate step s contracts n = 16 s + 4 g4 + q.
    floatx4 S[NSLOT];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) S[k] = zero4();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int I = ii ? I1 : I0;
        const int kb = ii ? base1 : 0, kend = ii ? NSLOT : base1;
        const bool crow_ok = rowC[ii] < L;
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int J = k - kb;
            if (k < kb || k >= kend || J > I) continue;  // wave-uniform
            const int64_t row = t0 + 16 * J + l16;
            const float *brow = Bm + ((b * L + row) * G + gi) * N;
            for (int s = 0; s < ns; ++s) {
                floatx4 bv = zero4(), cv = zero4();
                if (row < L) bv = *reinterpret_cast<const floatx4 *>(brow + 16 * s + 4 * g4);
                if (crow_ok) cv = *reinterpret_cast<const floatx4 *>(crow[ii] + 16 * s + 4 * g4);
#pragma unroll
                for (int q = 0; q < 4; ++q) S[k] = mfma_f32(bv[q], cv[q], S[k]);
            }
        }
    }

    for (int h = h_begin; h < h_end; ++h) {
        stage_head();
        __syncthreads();
        if (h + 1 < h_end) load_head(h + 1);
        const float Dh = (Dv != nullptr) ? Dv[h] : 0.f;
        const float *hp = H + (((int64_t)b * NH + h) * NC + c) * (int64_t)P * N;
        int tid_o = tid;  // opaque lane coordinates: see the bf16 kernel
        asm volatile("" : "+v"(tid_o));
        const int l16 = tid_o & 15, g4 = (tid_o >> 4) & 3;
        const int w_o = __builtin_amdgcn_readfirstlane(tid_o >> 6);
        const int I0 = w_o, I1 = NT16 - 1 - w_o;
        const int base1 = slot_base1(I0);

        floatx4 acc[2][PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[0][pt] = acc[1][pt] = zero4();

        // inter-chunk term C_i h_c
        for (int s = 0; s < ns; ++s) {
            floatx4 cv[2];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                cv[ii] = zero4();
                if (rowC[ii] < L) cv[ii] = *reinterpret_cast<const floatx4 *>(crow[ii] + 16 * s + 4 * g4);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const floatx4 hv = *reinterpret_cast<const floatx4 *>(hp + (16 * pt + l16) * N + 16 * s + 4 * g4);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[0][pt] = mfma_f32(cv[0][q], hv[q], acc[0][pt]);
                    acc[1][pt] = mfma_f32(cv[1][q], hv[q], acc[1][pt]);
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            float e[4];
            row_decay(tb, ii ? I1 : I0, g4, e);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[ii][pt][r] *= e[r];
        }
        // intra-chunk term: instruction r of a slot contracts j = 16 J + 4 g4 + r
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int I = ii ? I1 : I0;
            const int kb = ii ? base1 : 0, kend = ii ? NSLOT : base1;
            const float gih = tb.gh[16 * I + l16], gil = tb.gl[16 * I + l16];
#pragma unroll
            for (int k = 0; k < NSLOT; ++k) {
                const int J = k - kb;
                if (k < kb || k >= kend || J > I) continue;  // wave-uniform
                float v[4];
                tile_values(S[k], J, I, gih, gil, tb, l16, g4, v);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float *xrow = xs + (16 * J + 4 * g4 + r) * LDP + l16;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        acc[ii][pt] = mfma_f32(v[r], xrow[16 * pt], acc[ii][pt]);
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int I = ii ? I1 : I0;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const int p = 16 * pt + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * g4 + r;
                    const int64_t row = t0 + i;
                    if (row < L)
                        store_out(&y[((b * L + row) * NH + h) * P + p], acc[ii][pt][r] + Dh * xs[i * LDP + p]);
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launch: InT is the input element type, OutT the element type of y
// ---------------------------------------------------------------------------
template <int T, int P, int NKMAX, typename OutT>
hipError_t launch_bf16_in(const Problem &p, int HB, int nhb, int64_t blocks, const void *x,
                          const void *B, const void *C, G2View G2, const float *DT, const float *D,
                          const float *H, void *y, hipStream_t stream) {
    constexpr auto kern = k4_chunk_out_bf16<T, P, NKMAX, OutT>;
    const size_t lds = Bf16Lds<T, P, NKMAX>::total;
    if (allow_lds<kern>(lds) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(2 * T), lds, stream,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B),
                       static_cast<const uint16_t *>(C), G2.hi, G2.lo, DT, D, H,
                       static_cast<OutT *>(y), p.seqlen, (int)p.nheads, (int)p.dstate,
                       (int)p.ngroups, (int)p.nchunks, p.padded_len, (int)p.heads_per_group, HB,
                       nhb);
    return hipGetLastError();
}

template <int T, int P, typename OutT>
hipError_t launch_f32_in(const Problem &p, int HB, int nhb, int64_t blocks, const void *x,
                         const void *B, const void *C, G2View G2, const float *DT, const float *D,
                         const float *H, void *y, hipStream_t stream) {
    constexpr auto kern = k4_chunk_out_f32<T, P, OutT>;
    constexpr size_t lds = (size_t)T * (P + 4) * 4 + (size_t)4 * T * 4;
    static_assert(lds <= kLdsBytes, "stage-4 LDS budget exceeded");
    if (allow_lds<kern>(lds) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(2 * T), lds, stream,
                       static_cast<const float *>(x), static_cast<const float *>(B),
                       static_cast<const float *>(C), G2.hi, G2.lo, DT, D, H,
                       static_cast<OutT *>(y), p.seqlen, (int)p.nheads, (int)p.dstate,
                       (int)p.ngroups, (int)p.nchunks, p.padded_len, (int)p.heads_per_group, HB,
                       nhb);
    return hipGetLastError();
}

template <typename InT, typename OutT, int T, int P>
hipError_t launch_tp(const Problem &p, const Plan &plan, const void *x, const void *B, const void *C,
                     G2View G2, const float *DT, const float *D, const float *H, void *y,
                     hipStream_t stream) {
    const int HB = plan.k4_heads_per_block;
    const int nhb = (int)((p.heads_per_group + HB - 1) / HB);
    const int64_t blocks = p.batch * p.nchunks * p.ngroups * nhb;
    if (blocks == 0) return hipSuccess;
    if constexpr (sizeof(InT) == 2) {
        if (p.dstate <= 128)
            return launch_bf16_in<T, P, 4, OutT>(p, HB, nhb, blocks, x, B, C, G2, DT, D, H, y, stream);
        return launch_bf16_in<T, P, 8, OutT>(p, HB, nhb, blocks, x, B, C, G2, DT, D, H, y, stream);
    } else {
        return launch_f32_in<T, P, OutT>(p, HB, nhb, blocks, x, B, C, G2, DT, D, H, y, stream);
    }
}

template <typename InT, typename OutT>
hipError_t launch(const Problem &p, const Plan &plan, const void *x, const void *B, const void *C,
                  G2View G2, const float *DT, const float *D, const float *H, void *y,
                  hipStream_t stream) {
#define SSD_K4_P(T)                                                                              \
    switch (p.headdim) {                                                                         \
        case 32: return launch_tp<InT, OutT, T, 32>(p, plan, x, B, C, G2, DT, D, H, y, stream);  \
        case 64: return launch_tp<InT, OutT, T, 64>(p, plan, x, B, C, G2, DT, D, H, y, stream);  \
        case 128: return launch_tp<InT, OutT, T, 128>(p, plan, x, B, C, G2, DT, D, H, y, stream); \
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
                                  const void *C, G2View G2, const float *DT, const float *D,
                                  const float *H, void *y, hipStream_t stream);
hipError_t launch_bf16_in_bf16_out(const Problem &p, const Plan &plan, const void *x, const void *B,
                                   const void *C, G2View G2, const float *DT, const float *D,
                                   const float *H, void *y, hipStream_t stream);

}  // namespace k4
}  // namespace ssd

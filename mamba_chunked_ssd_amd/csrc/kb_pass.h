// kb_pass.h -- the three MFMA passes of the backward pass (gfx950).
//
// The pages name the backward pass as what training depends on ("Accelerating
// Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile",
// section "Mamba-2 architecture", where the chunked form is said to serve
// training and prefill) and derive none.  What follows is the chain rule
// applied to the chunked form of the same section.  Per (batch b, chunk c,
// head h), with chunk-local tokens r, s, the per-chunk cumsum G (natural-log
// units here; the kernels use G2 = log2(e) G), h_c the state at the chunk's
// start and E_c the gradient of the loss with respect to the state at the
// chunk's end:
//
//   q_r   = sum_{s >= r} exp(G_s - G_r) (B_r . C_s) dy_s + exp(G_last - G_r) E_c B_r
//           -> dx_r = dt_r q_r + D dy_r, and ddt_r = x_r . q_r + A da_r
//   dB_r  = sum_heads dt_r [ sum_{s >= r} exp(G_s - G_r) (x_r . dy_s) C_s
//                            + exp(G_last - G_r) E_c^T x_r ]
//   dC_r  = sum_heads [ sum_{s <= r} exp(G_r - G_s) (dy_r . x_s) dt_s B_s
//                       + exp(G_r) h_c^T dy_r ]
//
// The gradient of the chunk's decays, da_r = dL/da_r (a = A dt, G its cumsum
// in the chunk), is, from the same expansion,
//   da_r = sum_{s >= r > k} W[s][k]  +  sum_{s >= r} exp(G_s) dy_s . (h_c C_s)
//          + sum_{k < r} dt_k exp(G_last - G_k) x_k . (E_c B_k)  +  exp(G_last) <E_c, h_c> ,
//   W[s][k] = exp(G_s - G_k) (C_s . B_k) (dy_s . x_k) dt_k   (s >= k) :
// every path from an input at token k < r to an output or the chunk's end
// beyond r crosses a_r.  The first sum is taken as a telescoping sum of the
// row and column sums of W (sum_{j >= r} of rowsum_j - colsum_j, the diagonal
// cancelling), both from the same computed W, so that its per-entry errors
// cancel as the exact terms do; the state terms are computed directly.  (The
// same quantity written with the forward output, dy_r . y_r - dt_r x_r . q_r,
// cancels two separately computed sums and loses the precision of fp32.)
//
// Each is one instance of a decayed, masked attention over the chunk,
//   O_r = sum_{s in mask(r)} exp2(G2_later - G2_earlier) w_s (Q_r . K_s) V_s
//         + exp2(e_r) Hm Q_r ,
// the shape of the forward chunk output with the roles of the operands moved:
//   pass Q: Q = B, K = C, V = dy (dv = headdim), anti-causal, Hm = E_c,
//           e_r = G2_last - G2_r; the scores B_r . C_s are shared by the heads
//           of a group and come precomputed (score tiles);
//   pass B: Q = x, K = dy, V = C (dv = dstate), anti-causal, Hm = E_c^T;
//   pass W: pass B's scores x_k . dy_s alone, decayed and times the score
//           tiles and dt_k: the entries of W, whose row and column sums it
//           accumulates (fp64 for fp32 problems, fp32 for bf16; no V, no
//           state term);
//   pass C: Q = dy, K = x, V = B, w_s = dt_s, causal, Hm = h_c^T, e_r = G2_r;
//           C_r . (its state term) gives the second sum's terms;
// and pass Q's state term dotted with x_r the third's.
//
// Design for gfx950.  One block per (batch, chunk, group, run of heads,
// dv-tile); each wave owns one or two 16-row strips (below), so the
// triangular work is even across waves.  Per head the block
// stages K, V and the state Hm into LDS; Q fragments come straight from
// memory into registers.  For a strip and a pair of key strips the scores
// arrive in the MFMA output layout (lane = row, four keys per lane), are
// decayed (on the diagonal tile from exact exponents, masked by a select
// before exp2; off it as a product of three factors, each at most 1: the
// row's decay to its strip's end, the decay between the two strips' near
// ends, and the key's decay to its strip's end, a per-head table) and split
// into bf16 terms, and feed the
// next MFMA directly as its A operand, with the k index relabelled to match:
// the V rows for that relabelling come from transposing LDS reads.  The state
// term is one more MFMA chain per strip.
//
// Precision.  Every MFMA is bf16 x bf16 -> fp32.  A value that is not an exact
// bf16 is a sum of bf16 terms (hi = bf16(v), mid = bf16(v - hi), ...): bf16
// problems keep their inputs exact (one term) and split fp32-valued data (the
// decayed scores, the states) in two (about 17 significant bits); fp32
// problems split everything in three (about 24 bits, fp32's own precision),
// because the gradient of the decays sums per-token terms that largely cancel
// and so magnifies any per-term error.  A product keeps the term pairs
// (i, j) with i + j below the larger term count (1, 2, 3 or 6 MFMAs).  fp32
// data stays fp32 in LDS and is split per fragment; bf16 data is staged as is,
// the states of bf16 problems as their hi and lo planes.
//
// Sums over the heads of a group (dB, dC) accumulate in registers over the
// block's heads and leave as one partial per run of heads, reduced by a later
// kernel in a fixed order (deterministic).
#pragma once

#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace bwd {

enum { kPassQ = 0, kPassB = 1, kPassC = 2, kPassW = 3, kPassP = 4 };

// fp32 problems: pass P stores each head's decayed scores once,
//   P_ab = exp2(G2_b - G2_a) (x_a . dy_b),  a <= b (0 for a > b),
// as 16 x 16 fp32 tiles (a-strip I <= b-strip J), row-major [a][b] for passes
// B and W (row a, key b) and transposed times dt_a, [b][a], for pass C (row b,
// key a), so that every pass reads its tile with one 16-byte load per lane;
// passes B, C and W read them instead of staging K and recomputing the
// scores with three-term splits.  That frees the
// registers the three-term Q fragments held in the key loop and the LDS of the
// K tile, so the fp32 dB and dC passes take 64-column dstate tiles instead of
// 16 and do not redo the scores for each.  bf16 problems recompute the scores
// (one-term fragments are cheap, and the tiles would cost more memory traffic
// than they save).
template <typename In, int PASS>
__host__ __device__ constexpr bool kb_ptiles() {
    return !std::is_same<In, uint16_t>::value && (PASS == kPassB || PASS == kPassC || PASS == kPassW);
}
// whether a pass stages the chunk's K rows in LDS
__host__ __device__ constexpr bool kb_stages_k(int pass, bool f32_in) {
    return pass == kPassP || (pass != kPassQ && !f32_in);
}

// 16-row strips per wave (bwd_spw, shared with the host in ssd_internal.h):
// 2 pairs strip w with strip n - 1 - w (T/32 waves, the pair's K and V
// fragments read once for both); 1 gives one strip per wave (T/16 waves, more
// waves per SIMD to hide latency, the per-SIMD work staying even: SIMD s holds
// the strips s, s + 4, s + 8, ...).  Measured at the 2.7B layer: one strip
// per wave for the dx and dB passes (121 -> 93 and 117 -> 93 us) and for the
// dC pass up to headdim 64 (136 -> 131 us, although its 128 registers then
// spill some values); two for the W sums (two blocks per CU instead of one)
// and every pass with fp32 inputs (three-term fragments: one strip per wave
// spills heavily).
__host__ __device__ constexpr int kb_threads(int pass, bool bf16, int nkq, int T) {
    return 64 * (T / 16) / bwd_spw(pass, bf16, nkq);
}

struct PassArgs {
    const void *x, *dy, *Bm, *Cm;  // inputs, element type In
    const float *G2hi, *G2lo, *DT;  // (batch, nheads, Lp)
    const void *E;                  // adjoint end-of-chunk states per (b, h, c): bf16 hi/lo planes, or fp32
    const void *H;                  // pass C: chunk-start states (bf16 hi/lo planes, or fp32)
    const float *ST;                // pass Q: score tiles
    const float *D;                 // pass Q: skip weights or null
    float *out;                     // pass Q: dx; passes B, C: partial sums per run of heads
    // per-token partial sums, each (parts, batch, nheads, Lp), part-major so
    // that the token pass reads each part as one coalesced vector:
    float *xq, *xqi, *dyx;          // pass Q (parts = its dv-tiles): x . q, x . (state term of q), dy . x
    float *cdi;                     // pass C (parts = its dv-tiles): C . (state term of dC)
    double *wd;                     // pass W (one part): W's row sum minus its column sum
    float *pt, *ptt;                // fp32 problems: the decayed score tiles of each (batch, head, chunk),
                                    // row-major and transposed times dt
    int64_t seqlen, Lp;
    int batch, NH, P, N, G, HPG, T, NC, hb, nhb, nvt;
    int krow, vrow, erow;           // LDS row strides (elements)
    int xt_lds;                     // pass Q: x tile, pass C: C tile staged in LDS (else read from memory)
    int *occ;                       // host only: when set, the launch reports blocks per CU instead
};

// LDS bytes of one block: tables (G2 hi, G2 lo, dt, key factors), K (passes B and C) and V
// in the input element type, the state tile as two bf16 planes or one fp32, and
// (where it fits) the tile the epilogue reads beside O: x for pass Q, C for pass C.
__host__ __device__ inline int kb_lds_bytes(int pass, bool f32_in, int T, int P, int N, int DV, int krow,
                                            int vrow, int erow, bool xt) {
    const int esz = f32_in ? 4 : 2;
    int bytes = 16 * T;  // G2 hi, G2 lo, dt, key factors
    if (kb_stages_k(pass, f32_in)) bytes += T * krow * esz;
    // pass W: one part per wave of W's row sums and the column sums, fp64,
    // summed in the block before they are written
    if (pass == kPassW) return bytes + 8 * T * (T / 16 / bwd_spw(kPassW, !f32_in, P / 32) + 1);
    if (pass == kPassP) return bytes;
    bytes += T * vrow * esz;
    const int erows = pass == kPassQ ? DV : P;
    bytes += erows * erow * 4;
    if (xt && (pass == kPassQ || pass == kPassC)) bytes += T * vrow * esz;  // the epilogue's x or C tile
    return bytes;
}

// A value as a sum of NT bf16 terms, 8 per lane (one MFMA operand each).
template <int NT>
struct Frag {
    u32x4 t[NT];
};

// split 8 floats into NT (1, 2 or 3) bf16 terms
template <int NT>
__device__ __forceinline__ Frag<NT> split8(const float (&v)[8]) {
    Frag<NT> f;
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = v[i];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = pack_bf16(r[2 * i], r[2 * i + 1]);
            if (k + 1 < NT) {
                r[2 * i] -= bf16lo(w[i]);
                r[2 * i + 1] -= bf16hi(w[i]);
            }
        }
        f.t[k] = w;
    }
    return f;
}

// A x B over the term pairs (i, j) with i + j < max(NA, NB), small terms first.
template <int NA, int NB>
__device__ __forceinline__ floatx4 mmf(const Frag<NA> &a, const Frag<NB> &b, floatx4 c) {
    constexpr int M = NA > NB ? NA : NB;
#pragma unroll
    for (int s = M - 1; s >= 0; --s)
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int j = s - i;
            if (j >= 0 && j < NB) c = mfma_bf16(a.t[i], b.t[j], c);
        }
    return c;
}

// Transposing read of 8 bf16 of one column of an LDS plane: rows k0 + 4 g + r
// and k1 + 4 g + r (r = 0..3) of column c0 + l % 16 (see tr_read).
__device__ __forceinline__ u32x4 tr_pair(const uint16_t *plane, int ld, int k0, int k1, int c0, int g4, int l16) {
    const unsigned char *base = reinterpret_cast<const unsigned char *>(plane);
    const int r = l16 >> 2, a = l16 & 3;
    const u32x2 u = tr_read(base + ((k0 + 4 * g4 + r) * ld + c0 + 4 * a) * 2);
    const u32x2 v = tr_read(base + ((k1 + 4 * g4 + r) * ld + c0 + 4 * a) * 2);
    return u32x4{u[0], u[1], v[0], v[1]};
}

// Input element type traits: term counts, global and LDS fragment access.
template <typename In>
struct Io;

template <>
struct Io<uint16_t> {
    static constexpr int NI = 1;  // terms of an input value (exact)
    static constexpr int NF = 2;  // terms of an fp32-valued state operand
    static constexpr int NP = 2;  // terms of a decayed score (one bf16 term gives dx errors of several
                                  // per cent of its rms: too coarse)
    typedef uint16_t Lds;
    // 8 consecutive inputs from memory
    __device__ static Frag<1> load8(const uint16_t *p) { return Frag<1>{{*reinterpret_cast<const u32x4 *>(p)}}; }
    __device__ static float load1(const uint16_t *p) { return bf16_to_f32(*p); }
    // 8 consecutive elements of an LDS row
    __device__ static Frag<1> row8(const uint16_t *lds) { return Frag<1>{{*reinterpret_cast<const u32x4 *>(lds)}}; }
    // column c0 + l16 at rows k0 + 4 g + r and k1 + 4 g + r of an LDS plane
    __device__ static Frag<1> col8(const uint16_t *plane, int ld, int k0, int k1, int c0, int g4, int l16) {
        return Frag<1>{{tr_pair(plane, ld, k0, k1, c0, g4, l16)}};
    }
    // the state tile: 8 consecutive elements of a row, or of a column in
    // natural k order (rows k0 + 8 g .. k0 + 8 g + 7); hi and lo planes
    __device__ static Frag<2> srow8(const unsigned char *st, int ld, int rows, int r, int c) {
        const uint16_t *h = reinterpret_cast<const uint16_t *>(st), *l = h + rows * ld;
        return Frag<2>{{*reinterpret_cast<const u32x4 *>(h + r * ld + c), *reinterpret_cast<const u32x4 *>(l + r * ld + c)}};
    }
    __device__ static Frag<2> scol8(const unsigned char *st, int ld, int rows, int k0, int c0, int g4, int l16) {
        const uint16_t *h = reinterpret_cast<const uint16_t *>(st), *l = h + rows * ld;
        return Frag<2>{{tr_pair(h, ld, k0 + 8 * g4, k0 + 8 * g4 + 4, c0, 0, l16),
                        tr_pair(l, ld, k0 + 8 * g4, k0 + 8 * g4 + 4, c0, 0, l16)}};
    }
};

template <>
struct Io<float> {
    static constexpr int NI = 3;
    static constexpr int NF = 3;
    static constexpr int NP = 3;
    typedef float Lds;
    __device__ static Frag<3> load8(const float *p) {
        const floatx4 a = *reinterpret_cast<const floatx4 *>(p), b = *reinterpret_cast<const floatx4 *>(p + 4);
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        return split8<3>(v);
    }
    __device__ static float load1(const float *p) { return *p; }
    __device__ static Frag<3> row8(const float *lds) { return load8(lds); }
    __device__ static Frag<3> col8(const float *plane, int ld, int k0, int k1, int c0, int g4, int l16) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v[r] = plane[(k0 + 4 * g4 + r) * ld + c0 + l16];
            v[4 + r] = plane[(k1 + 4 * g4 + r) * ld + c0 + l16];
        }
        return split8<3>(v);
    }
    __device__ static Frag<3> srow8(const unsigned char *st, int ld, int, int r, int c) {
        return load8(reinterpret_cast<const float *>(st) + r * ld + c);
    }
    __device__ static Frag<3> scol8(const unsigned char *st, int ld, int, int k0, int c0, int g4, int l16) {
        const float *f = reinterpret_cast<const float *>(st);
        float v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = f[(k0 + 8 * g4 + r) * ld + c0 + l16];
        return split8<3>(v);
    }
};

// Sum over the 16 lanes of each row of the wave (lanes 16 q .. 16 q + 15),
// every lane receiving its row's sum, with DPP lane moves (VALU) rather than
// LDS-crossbar shuffles: row mirror, half-row mirror, then the two quad
// exchanges reach all 16 lanes.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));  // row_mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));  // row_half_mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));   // quad_perm 2,3,0,1
    return v;
}
__device__ __forceinline__ double row16_sum(double v) {
    v += dpp_move_f64<0x140, 0xf>(v);
    v += dpp_move_f64<0x141, 0xf>(v);
    v += dpp_move_f64<0xb1, 0xf>(v);
    v += dpp_move_f64<0x4e, 0xf>(v);
    return v;
}

// rows [0, nrows) x cols [0, ncols) (ncols % 8 == 0) of a row-major source
// (row stride src_ld elements) into an LDS array of row stride `ld`, element
// type unchanged; rows >= vrows and columns >= vcols read as zero.
template <typename T>
__device__ __forceinline__ void stage_rows(T *dst, int ld, const T *src, int64_t src_ld, int nrows, int vrows,
                                           int ncols, int vcols, int tid, int nthr) {
    constexpr int V = 16 / sizeof(T);  // elements per 16-byte word
    const int cpr = ncols / V;
    for (int idx = tid; idx < nrows * cpr; idx += nthr) {
        const int r = idx / cpr, cc = (idx - r * cpr) * V;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (r < vrows && cc < vcols) v = *reinterpret_cast<const u32x4 *>(src + (int64_t)r * src_ld + cc);
        *reinterpret_cast<u32x4 *>(dst + r * ld + cc) = v;
    }
}

// The state tile of (b, h, c): rows [r0, r0 + nrows), cols [c0, c0 + ncols)
// of a (P, N) state, columns >= vcols zero.  bf16 problems: the hi and lo
// planes, one after the other in LDS; fp32 problems: fp32.
template <typename In>
__device__ __forceinline__ void stage_state(unsigned char *st, int ld, const void *base, int P, int N, int r0,
                                            int nrows, int c0, int ncols, int vcols, int tid, int nthr) {
    if constexpr (std::is_same<In, uint16_t>::value) {
        const uint16_t *hi = static_cast<const uint16_t *>(base), *lo = hi + (int64_t)P * N;
        uint16_t *dh = reinterpret_cast<uint16_t *>(st), *dl = dh + nrows * ld;
        stage_rows<uint16_t>(dh, ld, hi + (int64_t)r0 * N + c0, N, nrows, nrows, ncols, vcols, tid, nthr);
        stage_rows<uint16_t>(dl, ld, lo + (int64_t)r0 * N + c0, N, nrows, nrows, ncols, vcols, tid, nthr);
    } else {
        stage_rows<float>(reinterpret_cast<float *>(st), ld, static_cast<const float *>(base) + (int64_t)r0 * N + c0,
                          N, nrows, nrows, ncols, vcols, tid, nthr);
    }
}

__device__ __forceinline__ float lds1(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float lds1(const float *p) { return *p; }

template <typename In, int NKQ, int DV, int PASS>
__global__ __launch_bounds__(kb_threads(PASS, std::is_same<In, uint16_t>::value, NKQ, 256)) void kb_pass(PassArgs a) {
    typedef Io<In> IO;
    typedef typename IO::Lds L;
    constexpr int kSPW = bwd_spw(PASS, std::is_same<In, uint16_t>::value, NKQ);
    // pass W: what the W entries are summed in.  The row and column sums are
    // differenced later, and the difference's sums over the chunk cancel
    // heavily: fp32 problems sum in fp64 (fp32 sums per 16-token tile left dA
    // errors up to 4e-4 of its rms, over the 1e-4 bound; fp64 sums 2e-7);
    // bf16 problems sum in fp32 (dA error 1.2e-5 of its rms, against a 2e-2
    // bound; emulated on a bf16 problem of the 2.7B layer's head shapes).
    typedef typename std::conditional<std::is_same<In, uint16_t>::value, float, double>::type WAcc;
    constexpr bool kPT = kb_ptiles<In, PASS>();  // scores from the stored tiles
    constexpr bool kKS = kb_stages_k(PASS, !std::is_same<In, uint16_t>::value);
    constexpr int NI = IO::NI, NF = IO::NF, NP = IO::NP;
    constexpr int NCT = DV / 16;
    extern __shared__ __align__(16) unsigned char lds[];
    const int T = a.T, n = T / 16;
    const int tid = threadIdx.x, nthr = kb_threads(PASS, std::is_same<In, uint16_t>::value, NKQ, T);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so strip logic stays scalar
    const int l = tid & 63, g4 = l >> 4, l16 = l & 15;

    // The column tiles of one (batch, chunk, group, run of heads) read the
    // same rows of x and dy.  Workgroups are dealt to the 8 XCDs in turn, so
    // the tiles of one run are placed 8 dispatch slots apart: on one XCD,
    // where the second tile's reads hit that XCD's L2 (the grid's tail past a
    // multiple of 8 runs is laid out plainly).
    int64_t u;
    int vt;
    {
        const int64_t bx = blockIdx.x, nfull = ((int64_t)gridDim.x / a.nvt) / 8 * 8;
        if (bx < nfull * a.nvt) {
            const int64_t s = bx >> 3;
            u = (s / a.nvt) * 8 + (bx & 7);
            vt = (int)(s % a.nvt);
        } else {
            const int64_t r = bx - nfull * a.nvt;
            u = nfull + r / a.nvt;
            vt = (int)(r % a.nvt);
        }
    }
    const int hblk = (int)(u % a.nhb);
    u /= a.nhb;
    const int g = (int)(u % a.G);
    u /= a.G;
    const int c = (int)(u % a.NC);
    const int b = (int)(u / a.NC);
    const int h0 = g * a.HPG + hblk * a.hb;
    const int h1 = min(h0 + a.hb, (g + 1) * a.HPG);
    const int64_t t0 = (int64_t)c * T;
    const int vrows = (int)max<int64_t>(0, min<int64_t>(T, a.seqlen - t0));  // valid tokens of the chunk

    float *g2h = reinterpret_cast<float *>(lds);
    float *g2l = g2h + T;
    float *dtt = g2l + T;
    float *kft = dtt + T;  // key factors of the off-diagonal tiles (see below)
    L *KS = reinterpret_cast<L *>(kft + T);
    const int kelems = kKS ? T * a.krow : 0;
    L *VS = KS + kelems;
    unsigned char *ES = reinterpret_cast<unsigned char *>(VS + T * a.vrow);
    const int erows = PASS == kPassQ ? DV : a.P;
    L *XS = reinterpret_cast<L *>(ES + erows * a.erow * 4);  // x (pass Q) or C (pass C) tile, if staged
    // pass W: nwv parts of W's row sums, then its column sums, T doubles each
    const int nwv = T / 16 / kSPW;
    double *wsum = reinterpret_cast<double *>(KS + kelems);

    const In *xin = static_cast<const In *>(a.x);
    const In *dyin = static_cast<const In *>(a.dy);
    const In *Bin = static_cast<const In *>(a.Bm);
    const In *Cin = static_cast<const In *>(a.Cm);
    const int64_t NHP = (int64_t)a.NH * a.P, GN = (int64_t)a.G * a.N;
    const int64_t PN = (int64_t)a.P * a.N;
    const int64_t ssz = std::is_same<In, uint16_t>::value ? 2 * PN * 2 : PN * 4;  // bytes of one state

    // V for passes B and C is the group's C or B tile: staged once per block
    if constexpr (PASS == kPassB || PASS == kPassC) {
        const In *vsrc = (PASS == kPassB ? Cin : Bin) + ((int64_t)b * a.seqlen + t0) * GN + (int64_t)g * a.N +
                         (int64_t)vt * DV;
        stage_rows<L>(VS, a.vrow, reinterpret_cast<const L *>(vsrc), GN, T, vrows, DV, DV, tid, nthr);
        if (PASS == kPassC && a.xt_lds) {
            const In *csrc = Cin + ((int64_t)b * a.seqlen + t0) * GN + (int64_t)g * a.N + (int64_t)vt * DV;
            stage_rows<L>(XS, a.vrow, reinterpret_cast<const L *>(csrc), GN, T, vrows, DV, DV, tid, nthr);
        }
    }

    // strips of this wave and their (pass B, C) accumulators over the heads
    const int strips[2] = {w, kSPW == 2 ? n - 1 - w : w};
    floatx4 acc[kSPW][NCT];
#pragma unroll
    for (int k = 0; k < kSPW; ++k)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[k][ct] = zero4();

    for (int h = h0; h < h1; ++h) {
        const int64_t bh = (int64_t)b * a.NH + h;
        __syncthreads();  // the previous head's reads of LDS are done
        for (int t = tid; t < T; t += nthr) {
            const int64_t gi = bh * a.Lp + t0 + t;
            const float gh = a.G2hi[gi], gl = a.G2lo[gi], d = a.DT[gi];
            g2h[t] = gh;
            g2l[t] = gl;
            dtt[t] = d;
            // decay between token t and the near end of its 16-token strip:
            // exp2(G2_t - G2_start) for the passes whose keys follow the row,
            // exp2(G2_end - G2_t) dt_t for pass C, whose keys precede it (<= 1)
            if constexpr (PASS == kPassC) {
                const int64_t ai = gi - (t & 15) + 15;
                kft[t] = fast_exp2((a.G2hi[ai] - gh) + (a.G2lo[ai] - gl)) * d;
            } else {
                const int64_t ai = gi - (t & 15);
                kft[t] = fast_exp2((gh - a.G2hi[ai]) + (gl - a.G2lo[ai]));
            }
        }
        const int64_t rowbase = ((int64_t)b * a.seqlen + t0) * NHP + (int64_t)h * a.P;  // token t0, head h
        const int64_t pbase = ((int64_t)vt * a.batch * a.NH + bh) * a.Lp + t0;        // part vt of the token sums
        const unsigned char *sbase =
            static_cast<const unsigned char *>(PASS == kPassC ? a.H : a.E) + (bh * a.NC + c) * ssz;
        // this head's stored score tiles (fp32 problems), and their transposes
        float *ptile = a.pt + (bh * a.NC + c) * (int64_t)(n * (n + 1) / 2) * 256;
        float *ptilet = a.ptt + (bh * a.NC + c) * (int64_t)(n * (n + 1) / 2) * 256;
        if constexpr (PASS == kPassQ) {
            stage_rows<L>(VS, a.vrow, reinterpret_cast<const L *>(dyin + rowbase + vt * DV), NHP, T, vrows, DV, DV,
                          tid, nthr);
            if (a.xt_lds)
                stage_rows<L>(XS, a.vrow, reinterpret_cast<const L *>(xin + rowbase + vt * DV), NHP, T, vrows, DV, DV,
                              tid, nthr);
            // E_c rows p of this dv-tile, all dstate columns (zero past dstate)
            stage_state<In>(ES, a.erow, sbase, a.P, a.N, vt * DV, DV, 0, (a.N + 31) & ~31, a.N, tid, nthr);
        } else {
            if constexpr (kKS)
                stage_rows<L>(KS, a.krow, reinterpret_cast<const L *>((PASS == kPassC ? xin : dyin) + rowbase), NHP,
                              T, vrows, a.P, a.P, tid, nthr);
            // E_c (pass B) or h_c (pass C): all rows p, the tile's columns
            if constexpr (PASS == kPassB || PASS == kPassC)
                stage_state<In>(ES, a.erow, sbase, a.P, a.N, 0, a.P, vt * DV, DV, DV, tid, nthr);
        }
        __syncthreads();

        const float Dh = (PASS == kPassQ && a.D != nullptr) ? a.D[h] : 0.f;
        // pass W: sums of W[s][r] over this wave's rows r, for the keys
        // s = 16 J + 4 g4 + i of key strip J = l16
        WAcc colacc[4] = {0, 0, 0, 0};

        // 1. per strip: Q fragments (rows 16 I + l16, 32 kk + 8 g4 ..), the
        //    row's decay tables, and the state term, which starts O
        Frag<NI> qf[kSPW][NKQ];
        floatx4 O[kSPW][NCT];  // the state term first, then the chunk's own tokens on top
        float grh[kSPW], grl[kSPW], rfac[kSPW];
        WAcc rowacc[kSPW];  // pass W: sums over this lane's keys s of W[s][r]
#pragma unroll
        for (int k = 0; k < kSPW; ++k) rowacc[k] = 0;
#pragma unroll
        for (int k = 0; k < kSPW; ++k) {
            const int I = strips[k];
            const int r = 16 * I + l16;  // this lane's row for the score / A-operand layout
            if constexpr (PASS != kPassQ && !(kPT && PASS == kPassW)) {
                const In *qsrc = (PASS == kPassC ? dyin : xin) + rowbase + (int64_t)r * NHP + 8 * g4;
#pragma unroll
                for (int kk = 0; kk < NKQ; ++kk) {
#pragma unroll
                    for (int j = 0; j < NI; ++j) qf[k][kk].t[j] = u32x4{0u, 0u, 0u, 0u};
                    if (r < vrows) qf[k][kk] = IO::load8(qsrc + 32 * kk);
                }
            }
            grh[k] = g2h[r];
            grl[k] = g2l[r];
            // decay between this lane's row and the near end of its strip (<= 1)
            rfac[k] = PASS == kPassC ? fast_exp2((grh[k] - g2h[16 * I]) + (grl[k] - g2l[16 * I]))
                                     : fast_exp2((g2h[16 * I + 15] - grh[k]) + (g2l[16 * I + 15] - grl[k]));
            if constexpr (PASS != kPassW && PASS != kPassP) {
                // state term: Oi = Q Hm^T, scaled per row by exp2(e_r)
                floatx4 Oi[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Oi[ct] = zero4();
                if constexpr (PASS == kPassQ) {
                    const In *bsrc = Bin + (((int64_t)b * a.seqlen + t0 + r) * a.G + g) * a.N + 8 * g4;
                    const int nk = (a.N + 31) / 32;
                    for (int kk = 0; kk < nk; ++kk) {
                        Frag<NI> bf;
#pragma unroll
                        for (int j = 0; j < NI; ++j) bf.t[j] = u32x4{0u, 0u, 0u, 0u};
                        if (r < vrows && 32 * kk + 8 * g4 < a.N) bf = IO::load8(bsrc + 32 * kk);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            const Frag<NF> ef = IO::srow8(ES, a.erow, erows, 16 * ct + l16, 32 * kk + 8 * g4);
                            Oi[ct] = mmf<NI, NF>(bf, ef, Oi[ct]);
                        }
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < NKQ; ++kk) {
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            const Frag<NF> ef = IO::scol8(ES, a.erow, erows, 32 * kk, 16 * ct, g4, l16);
                            Oi[ct] = mmf<NI, NF>(qf[k][kk], ef, Oi[ct]);
                        }
                    }
                }
                // output rows of the D layout: 16 I + 4 g4 + i
                float rf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ro = 16 * I + 4 * g4 + i;
                    if constexpr (PASS == kPassC)
                        rf[i] = fast_exp2(g2h[ro] + g2l[ro]);
                    else
                        rf[i] = fast_exp2((g2h[T - 1] - g2h[ro]) + (g2l[T - 1] - g2l[ro]));
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) O[k][ct][i] = rf[i] * Oi[ct][i];
                if constexpr (PASS == kPassQ) {
                    // x_r . (state term of q_r) over this tile's columns
                    float xs[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xs[i] = 0.f;
                        const int ro = 16 * I + 4 * g4 + i;
                        if (ro < vrows) {
#pragma unroll
                            for (int ct = 0; ct < NCT; ++ct)
                                xs[i] = fmaf(a.xt_lds ? lds1(XS + ro * a.vrow + 16 * ct + l16)
                                                      : IO::load1(xin + rowbase + (int64_t)ro * NHP + vt * DV + 16 * ct + l16),
                                             O[k][ct][i],
                                             xs[i]);
                        }
                        xs[i] = row16_sum(xs[i]);
                    }
                    if (l16 == 0) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) a.xqi[pbase + 16 * I + 4 * g4 + i] = xs[i];
                    }
                }
                if constexpr (PASS == kPassC) {
                    // C_r . (state term of dC_r) over this tile's columns
                    float cd[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        cd[i] = 0.f;
                        const int ro = 16 * I + 4 * g4 + i;
                        if (ro < vrows) {
                            const In *crow = Cin + (((int64_t)b * a.seqlen + t0 + ro) * a.G + g) * a.N + vt * DV + l16;
#pragma unroll
                            for (int ct = 0; ct < NCT; ++ct)
                                cd[i] = fmaf(a.xt_lds ? lds1(XS + ro * a.vrow + 16 * ct + l16) : IO::load1(crow + 16 * ct),
                                             O[k][ct][i], cd[i]);
                        }
                        cd[i] = row16_sum(cd[i]);
                    }
                    if (l16 == 0) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) a.cdi[pbase + 16 * I + 4 * g4 + i] = cd[i];
                    }
                }
            }
        }

        // 2. the key-strip pairs, each pair's K and V fragments read once for
        //    both row strips of the wave
        const int I0 = strips[0], I1 = strips[kSPW - 1];  // I0 <= I1
        const int jlo = PASS == kPassC ? 0 : (I0 & ~1);
        const int jhi = PASS == kPassC ? (I1 & ~1) : n - 2;  // inclusive, even
        const int64_t stb = (((int64_t)b * a.NC + c) * a.G + g) * (int64_t)(n * (n + 1) / 2);
        for (int J0 = jlo; J0 <= jhi; J0 += 2) {
            // the pair's V fragments and (bf16) K fragments of its two key
            // strips, read once for both strips of the wave
            Frag<NI> vf[NCT];
            if constexpr (PASS != kPassW && PASS != kPassP) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) vf[ct] = IO::col8(VS, a.vrow, 16 * J0, 16 * J0 + 16, 16 * ct, g4, l16);
            }
            Frag<NI> kfr[2][NKQ];
            if constexpr (kKS && NI == 1) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int kk = 0; kk < NKQ; ++kk)
                        kfr[jj][kk] = IO::row8(KS + (16 * (J0 + jj) + l16) * a.krow + 32 * kk + 8 * g4);
            }
            // the scores of both strips first (or their tiles' loads, pass Q),
            // so that one strip's MFMA latency hides behind the other's VALU work
            floatx4 Sall[kSPW][2];
#pragma unroll
            for (int k = 0; k < kSPW; ++k) {
                const int I = strips[k];
                const bool act = !(PASS == kPassC ? (J0 > (I & ~1)) : (J0 + 1 < I));
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int J = J0 + jj;
                    floatx4 S = zero4();
                    if (!kPT && act && (PASS == kPassC ? (J <= I) : (J >= I))) {
                        if constexpr (PASS == kPassQ) {
                            const int tile = I * n - (I * (I - 1)) / 2 + (J - I);
                            S = *reinterpret_cast<const floatx4 *>(a.ST + ((stb + tile) * 64 + l) * 4);
                        } else {
#pragma unroll
                            for (int kk = 0; kk < NKQ; ++kk) {
                                if constexpr (NI == 1) {
                                    S = mmf<NI, NI>(kfr[jj][kk], qf[k][kk], S);
                                } else {
                                    const Frag<NI> kf = IO::row8(KS + (16 * J + l16) * a.krow + 32 * kk + 8 * g4);
                                    S = mmf<NI, NI>(kf, qf[k][kk], S);
                                }
                            }
                        }
                    }
                    Sall[k][jj] = S;
                }
            }
#pragma unroll
            for (int k = 0; k < kSPW; ++k) {
                const int I = strips[k];
                if (PASS == kPassC ? (J0 > (I & ~1)) : (J0 + 1 < I)) continue;  // no live key strip
                const int r = 16 * I + l16;
                float pv[8];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int J = J0 + jj;
                    const floatx4 S = Sall[k][jj];
                    const bool live = PASS == kPassC ? (J <= I) : (J >= I);
                    if constexpr (kPT) {
                        // the stored tiles: (I, J) row-major for passes B and W
                        // (row r = a, key s = b); (J, I) transposed, times dt_s, for
                        // pass C (row r = b, key s = a).  Entries with a > b are 0.
                        if (live) {
                            if constexpr (PASS == kPassC) {
                                const floatx4 v = *reinterpret_cast<const floatx4 *>(
                                    ptilet + (J * n - (J * (J - 1)) / 2 + (I - J)) * 256 + l16 * 16 + 4 * g4);
#pragma unroll
                                for (int i = 0; i < 4; ++i) pv[4 * jj + i] = v[i];
                            } else {
                                const floatx4 v = *reinterpret_cast<const floatx4 *>(
                                    ptile + (I * n - (I * (I - 1)) / 2 + (J - I)) * 256 + l16 * 16 + 4 * g4);
#pragma unroll
                                for (int i = 0; i < 4; ++i) pv[4 * jj + i] = v[i];
                            }
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) pv[4 * jj + i] = 0.f;
                        }
                    } else if (J == I) {
                        // the diagonal tile: exact exponents, masked (select before exp2)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int s_ = 16 * J + 4 * g4 + i;
                            float e;
                            bool ok;
                            if constexpr (PASS == kPassC) {
                                ok = s_ <= r;
                                e = (grh[k] - g2h[s_]) + (grl[k] - g2l[s_]);
                            } else {
                                ok = s_ >= r;
                                e = (g2h[s_] - grh[k]) + (g2l[s_] - grl[k]);
                            }
                            float v = S[i] * fast_exp2(ok ? e : -INFINITY);
                            if constexpr (PASS == kPassC) v *= dtt[s_];
                            pv[4 * jj + i] = v;
                        }
                    } else if (live) {
                        // off the diagonal every key is live and the decay factors
                        // through the strips' near ends, each factor <= 1: the row's
                        // to its strip end, strip end to strip end, and the key's
                        // (table) -- two products per entry
                        float se;
                        if constexpr (PASS == kPassC)
                            se = (g2h[16 * I] - g2h[16 * J + 15]) + (g2l[16 * I] - g2l[16 * J + 15]);
                        else
                            se = (g2h[16 * J] - g2h[16 * I + 15]) + (g2l[16 * J] - g2l[16 * I + 15]);
                        const float rowj = rfac[k] * fast_exp2(se);
                        const floatx4 kv = *reinterpret_cast<const floatx4 *>(kft + 16 * J + 4 * g4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) pv[4 * jj + i] = S[i] * rowj * kv[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) pv[4 * jj + i] = 0.f;
                    }
                    if constexpr (PASS == kPassW) {
                        if (live) {
                            // W[s][r] = (x_r . dy_s) exp2(G2_s - G2_r) (B_r . C_s) dt_r for this
                            // lane's row r and keys s = 16 J + 4 g4 + i: sums over s stay in
                            // the lane, sums over the strip's 16 rows go to lane l16 = J
                            // (entries in fp32, their sums in WAcc)
                            const int tile = I * n - (I * (I - 1)) / 2 + (J - I);
                            const floatx4 sc = *reinterpret_cast<const floatx4 *>(a.ST + ((stb + tile) * 64 + l) * 4);
                            const float dtr = dtt[r];
                            WAcc wv[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                wv[i] = (WAcc)(pv[4 * jj + i] * sc[i] * dtr);
                                rowacc[k] += wv[i];
                            }
#pragma unroll
                            for (int i = 0; i < 4; ++i) wv[i] = row16_sum(wv[i]);
#pragma unroll
                            for (int i = 0; i < 4; ++i) colacc[i] += (l16 == J) ? wv[i] : 0.0;
                        }
                    }
                }
                if constexpr (PASS == kPassP) {
                    // store the decayed scores: tile (I, J), row a = r, keys b;
                    // and the transposed tile, [b][a], times dt_a
                    const float da = dtt[r];
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int J = J0 + jj;
                        if (J >= I) {
                            const int64_t to = (I * n - (I * (I - 1)) / 2 + (J - I)) * 256;
                            *reinterpret_cast<floatx4 *>(ptile + to + l16 * 16 + 4 * g4) =
                                floatx4{pv[4 * jj], pv[4 * jj + 1], pv[4 * jj + 2], pv[4 * jj + 3]};
#pragma unroll
                            for (int i = 0; i < 4; ++i) ptilet[to + (4 * g4 + i) * 16 + l16] = pv[4 * jj + i] * da;
                        }
                    }
                } else if constexpr (PASS != kPassW) {
                    const Frag<NP> pf = split8<NP>(pv);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O[k][ct] = mmf<NP, NI>(pf, vf[ct], O[k][ct]);
                }
            }
        }

        // 3. per strip: outputs
#pragma unroll
        for (int k = 0; k < kSPW; ++k) {
            const int I = strips[k];
            const int r = 16 * I + l16;
            if constexpr (PASS == kPassW) {
                // sum over s of W[s][r] (W's column r): this lane's keys, then
                // the 4 lane groups
                WAcc ra = rowacc[k];
                ra += __shfl_xor(ra, 16, 64);
                ra += __shfl_xor(ra, 32, 64);
                if (g4 == 0) wsum[T * nwv + r] = (double)ra;
            } else if constexpr (PASS == kPassQ) {
                float xq[4], dyx[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xq[i] = 0.f;
                    dyx[i] = 0.f;
                    const int ro = 16 * I + 4 * g4 + i;
                    if (ro < vrows) {
                        const float dtv = dtt[ro];
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            const int64_t e = rowbase + (int64_t)ro * NHP + vt * DV + 16 * ct + l16;
                            const float q = O[k][ct][i];
                            const float xv = a.xt_lds ? lds1(XS + ro * a.vrow + 16 * ct + l16) : IO::load1(xin + e);
                            const float dv = lds1(VS + ro * a.vrow + 16 * ct + l16);  // dy: pass Q's V tile
                            a.out[e] = fmaf(dtv, q, Dh * dv);
                            xq[i] = fmaf(xv, q, xq[i]);
                            dyx[i] = fmaf(dv, xv, dyx[i]);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xq[i] = row16_sum(xq[i]);
                    dyx[i] = row16_sum(dyx[i]);
                }
                if (l16 == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ro = 16 * I + 4 * g4 + i;
                        const int64_t ti = pbase + ro;
                        a.xq[ti] = xq[i];
                        a.dyx[ti] = dyx[i];
                    }
                }
            } else if constexpr (PASS == kPassB || PASS == kPassC) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sc = PASS == kPassB ? dtt[16 * I + 4 * g4 + i] : 1.f;
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) acc[k][ct][i] = fmaf(sc, O[k][ct][i], acc[k][ct][i]);
                }
            }
        }
        if constexpr (PASS == kPassW) {
            if (l16 < n) {
                // sums over this wave's rows r of W[s][r] (W's row s), one part per wave
#pragma unroll
                for (int i = 0; i < 4; ++i) wsum[T * w + 16 * l16 + 4 * g4 + i] = (double)colacc[i];
            }
            __syncthreads();
            // the waves' parts in a fixed order, less the column sum: one
            // double per token (the next head writes wsum only after the
            // barriers at its start)
            for (int t = tid; t < T; t += nthr) {
                double rs = 0.0;
                for (int v = 0; v < nwv; ++v) rs += wsum[T * v + t];
                a.wd[bh * a.Lp + t0 + t] = rs - wsum[T * nwv + t];
            }
        }
    }

    if constexpr (PASS == kPassB || PASS == kPassC) {
        // this run of heads' partial sum: (hblk, batch, Lp, G, N)
#pragma unroll
        for (int k = 0; k < kSPW; ++k) {
            const int I = strips[k];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ro = 16 * I + 4 * g4 + i;
                float *dst = a.out + ((((int64_t)hblk * a.batch + b) * a.Lp + t0 + ro) * a.G + g) * a.N +
                             (int64_t)vt * DV + l16;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) dst[16 * ct] = acc[k][ct][i];
            }
        }
    }
}

}  // namespace bwd
}  // namespace ssd

// kb_aux.hip -- the backward pass's smaller kernels (gfx950): the shared
// score tiles, the reverse carry of the adjoint state, and the two finishing
// reductions.
//
// Notation as in kb_pass.h: per (batch, head), chunk c has end-of-chunk
// adjoint E_c (the gradient of the loss with respect to the state after the
// chunk's last token).  The chain rule through the carry of the log-space
// state jump ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels
// in NVIDIA CUDA Tile", section "Mamba-2 architecture": h_{c+1} =
// exp(G_last,c) h_c + s_c) runs it backwards,
//     Lambda_NC = dL/dh_final ,   E_c = Lambda_{c+1} ,
//     Lambda_c = exp(G_last,c) Lambda_{c+1} + u_c ,  u_c = sum_r exp(G_r) dy_r C_r^T ,
// with Lambda_0 the gradient of the initial state.  u_c has the form of a
// chunk state (dy in place of x, C in place of B, weights exp(G_r)) and comes
// from the forward's chunk-state kernel.
//
// The gradient of the per-chunk log decays (kb_pass.h gives the expansion),
//     da_r = sum_{j >= r} (rowW_j - colW_j + cdi_j) + sum_{k < r} dt_k xqi_k + Z_c ,
// with rowW, colW the row and column sums of W, cdi_j = exp(G_j) dy_j . (h_c C_j),
// xqi_k = exp(G_last - G_k) x_k . (E_c B_k) and Z_c = exp(G_last) <E_c, h_c>;
// then ddt_r = x_r . q_r + A da_r, dA = sum dt_r da_r, dD = sum dy_r . x_r.
#include <climits>
#include <type_traits>

#include "ssd_device.h"
#include "ssd_internal.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

// 8 consecutive inputs as NT bf16 terms (bf16 inputs: exact, one term;
// fp32 inputs: hi, mid, lo, about 24 significant bits)
template <typename In>
struct Terms;
template <>
struct Terms<uint16_t> {
    static constexpr int NT = 1;
    __device__ static void load(const uint16_t *p, u32x4 (&t)[1]) { t[0] = *reinterpret_cast<const u32x4 *>(p); }
};
template <>
struct Terms<float> {
    static constexpr int NT = 3;
    __device__ static void load(const float *p, u32x4 (&t)[3]) {
        const floatx4 a = *reinterpret_cast<const floatx4 *>(p), b = *reinterpret_cast<const floatx4 *>(p + 4);
        float r[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t[k][i] = pack_bf16(r[2 * i], r[2 * i + 1]);
                r[2 * i] -= bf16lo(t[k][i]);
                r[2 * i + 1] -= bf16hi(t[k][i]);
            }
    }
};

// ---------------------------------------------------------------------------
// Score tiles: per (batch, chunk, group), S'[r][s] = B_r . C_s for the 16 x 16
// blocks (I, J >= I) of the chunk, in the MFMA output layout the dx pass
// consumes (lane l holds row 16 I + l % 16, keys 16 J + 4 (l / 16) + i,
// i = 0..3).  Tile (I, J) sits at I n - I (I - 1) / 2 + (J - I), n = T / 16.
// One wave per tile; rows past seqlen are zero.
// ---------------------------------------------------------------------------
template <typename In>
__global__ __launch_bounds__(256) void kb_scores(const In *__restrict__ Bm, const In *__restrict__ Cm,
                                                 float *__restrict__ ST, int64_t seqlen, int G, int N, int T,
                                                 int NC, int ntile, int64_t total) {
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= total) return;  // whole waves
    const int l = threadIdx.x & 63, g4 = l >> 4, l16 = l & 15;
    const int tile = (int)(wv % ntile);
    const int64_t bcg = wv / ntile;  // (b * NC + c) * G + g
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % NC);
    const int64_t b = bc / NC;
    const int n = T / 16;
    int I = 0, rem = tile;
    while (rem >= n - I) {
        rem -= n - I;
        ++I;
    }
    const int J = I + rem;
    const int64_t tr = (int64_t)c * T + 16 * I + l16, ts = (int64_t)c * T + 16 * J + l16;
    const In *brow = Bm + ((b * seqlen + tr) * G + g) * N + 8 * g4;
    const In *crow = Cm + ((b * seqlen + ts) * G + g) * N + 8 * g4;
    constexpr int NT = Terms<In>::NT;
    floatx4 S = zero4();
    for (int k0 = 0; k0 < N; k0 += 32) {
        u32x4 bt[NT], ct[NT];
#pragma unroll
        for (int k = 0; k < NT; ++k) bt[k] = ct[k] = u32x4{0u, 0u, 0u, 0u};
        if (k0 + 8 * g4 < N) {
            if (tr < seqlen) Terms<In>::load(brow + k0, bt);
            if (ts < seqlen) Terms<In>::load(crow + k0, ct);
        }
        // D[m = key][n = row]: A = C rows (keys), B = B rows; term pairs
        // (i, j) with i + j < NT, small ones first
#pragma unroll
        for (int sum = NT - 1; sum >= 0; --sum)
#pragma unroll
            for (int i = 0; i <= sum; ++i) S = mfma_bf16(ct[i], bt[sum - i], S);
    }
    *reinterpret_cast<floatx4 *>(ST + (wv * 64 + l) * 4) = S;
}

// ---------------------------------------------------------------------------
// Reverse carry: one thread per 4 consecutive state elements of one (batch,
// head), chunks walked last to first.  Writes E_c per (b, h, c) -- for bf16
// problems as bf16 hi/lo planes (the layout of the forward's bf16 chunk-start
// states), for fp32 problems in fp32 -- the
// per-wave partial sums of Z_c = exp(G_last,c) <E_c, h_c> (h_c the forward's
// chunk-start states), and Lambda_0.
// A wave never straddles two (batch, head) pairs: headdim * dstate / 4 is a
// multiple of 128.
// ---------------------------------------------------------------------------
template <bool kHSplit>
__global__ __launch_bounds__(256) void kb_carry(const float *__restrict__ U, const void *__restrict__ H,
                                                const float *__restrict__ G2hi,
                                                const float *__restrict__ G2lo, const float *__restrict__ dfinal,
                                                void *__restrict__ E, float *__restrict__ Zp,
                                                float *__restrict__ dinit, int64_t n_vec, int64_t pn_vec,
                                                int64_t nchunks, int64_t Lp, int T) {
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= n_vec) return;  // whole waves (n_vec is a multiple of 128)
    const int64_t bh = v / pn_vec, e = v % pn_vec;
    const int64_t nzw = pn_vec / 64, zw = e / 64;
    floatx4 lam = zero4();
    if (dfinal != nullptr) lam = reinterpret_cast<const floatx4 *>(dfinal)[bh * pn_vec + e];
    for (int64_t c = nchunks - 1; c >= 0; --c) {
        const int64_t bhc = bh * nchunks + c;
        // prefetch what this step reads
        const floatx4 uc = reinterpret_cast<const floatx4 *>(U)[bhc * pn_vec + e];
        floatx4 hc;  // h_c, the state at the chunk's start
        if constexpr (kHSplit) {
            const uint16_t *hb = static_cast<const uint16_t *>(H) + bhc * 8 * pn_vec;
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(hb + 4 * e);
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(hb + 4 * pn_vec + 4 * e);
            hc = floatx4{bf16lo(hi[0]) + bf16lo(lo[0]), bf16hi(hi[0]) + bf16hi(lo[0]),
                         bf16lo(hi[1]) + bf16lo(lo[1]), bf16hi(hi[1]) + bf16hi(lo[1])};
        } else {
            hc = reinterpret_cast<const floatx4 *>(H)[bhc * pn_vec + e];
        }
        const float dec = G2hi[bh * Lp + c * T + T - 1] + G2lo[bh * Lp + c * T + T - 1];
        // E_c = Lambda_{c+1}
        if constexpr (kHSplit) {
            uint16_t *eb = static_cast<uint16_t *>(E) + bhc * 8 * pn_vec;
            const HiLo p = split_bf16(lam[0], lam[1]), q = split_bf16(lam[2], lam[3]);
            *reinterpret_cast<u32x2 *>(eb + 4 * e) = u32x2{p.hi, q.hi};
            *reinterpret_cast<u32x2 *>(eb + 4 * pn_vec + 4 * e) = u32x2{p.lo, q.lo};
        } else {
            reinterpret_cast<floatx4 *>(E)[bhc * pn_vec + e] = lam;
        }
        const float a = fast_exp2(dec);
        float z = lam[0] * hc[0] + lam[1] * hc[1] + lam[2] * hc[2] + lam[3] * hc[3];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
        if ((threadIdx.x & 63) == 0) Zp[bhc * nzw + zw] = a * z;
#pragma unroll
        for (int k = 0; k < 4; ++k) lam[k] = fmaf(a, lam[k], uc[k]);
    }
    if (dinit != nullptr) reinterpret_cast<floatx4 *>(dinit)[bh * pn_vec + e] = lam;
}

// ---------------------------------------------------------------------------
// Per-token finish: one wave per (batch, chunk, head), T / 64 consecutive
// tokens per lane.  The partial dot products of the passes are summed, da
// formed with a suffix and a prefix scan over the chunk in fp64 (wave scans),
// then ddt and the chunk's partial sums of dA and dD.  The parts are stored
// part-major, so each lane reads one part of its tokens as one vector and
// the loads of all parts are independent of one another (the kernel's time
// is their latency, not their bytes).
// ---------------------------------------------------------------------------
// E consecutive floats as one vector load (p aligned to 4 E bytes)
template <int E>
__device__ __forceinline__ void load_vec(const float *p, float (&v)[E]) {
    const typename VecF<E>::type t = *reinterpret_cast<const typename VecF<E>::type *>(p);
    if constexpr (E == 1) {
        v[0] = t;
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = t[e];
    }
}

struct TokParts {
    const float *xq, *xqi, *dyx;  // nq parts each
    const float *cdi;             // nc parts
    const double *wd;             // 1 part
    int64_t ps;                   // elements of one part: batch * nheads * Lp
    int nq, nc;
};

// inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (the
// pattern of the cumsum's wave scan): shifts by 1, 2, 4, 8 within rows, then
// row 0's total into rows 1 and 3... by the two row broadcasts
__device__ __forceinline__ double wave_prefix(double v) {
    v += dpp_move_f64<0x111, 0xf>(v);  // row_shr:1
    v += dpp_move_f64<0x112, 0xf>(v);  // row_shr:2
    v += dpp_move_f64<0x114, 0xf>(v);  // row_shr:4
    v += dpp_move_f64<0x118, 0xf>(v);  // row_shr:8
    v += dpp_move_f64<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
    v += dpp_move_f64<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
    return v;
}
__device__ __forceinline__ double lane63(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum(double v) { return lane63(wave_prefix(v)); }

template <int E>
__global__ __launch_bounds__(256) void kb_tokens(TokParts tp, const float *__restrict__ DT,
                                                 const float *__restrict__ Zp, const float *__restrict__ A,
                                                 float *__restrict__ ddt, float *__restrict__ dap,
                                                 float *__restrict__ ddp, int64_t seqlen, int64_t Lp, int NH,
                                                 int NC, int nzw, int64_t total) {
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= total) return;  // whole waves
    const int lane = threadIdx.x & 63;
    const int h = (int)(wv % NH);
    const int64_t bc = wv / NH;
    const int c = (int)(bc % NC);
    const int64_t b = bc / NC;
    const int64_t bh = b * NH + h;
    const int T = 64 * E;
    const int64_t tb = (int64_t)c * T + lane * E;  // first token of this lane

    // this lane's tokens of every part, summed in fp64 (all loads independent)
    const int64_t it0 = bh * Lp + tb;
    double xqv[E], xqiv[E], dyxv[E], cdv[E], dtv[E], wdv[E];
    {
        float d[E];
        load_vec<E>(DT + it0, d);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            dtv[e] = d[e];
            xqv[e] = xqiv[e] = dyxv[e] = cdv[e] = 0.0;
        }
        if constexpr (E == 1) {
            wdv[0] = tp.wd[it0];
        } else {
#pragma unroll
            for (int e = 0; e < E; e += 2) {
                const double2 w2 = *reinterpret_cast<const double2 *>(tp.wd + it0 + e);
                wdv[e] = w2.x;
                wdv[e + 1] = w2.y;
            }
        }
    }
#pragma unroll 2
    for (int v = 0; v < tp.nq; ++v) {
        float q[E], qi[E], yx[E];
        load_vec<E>(tp.xq + v * tp.ps + it0, q);
        load_vec<E>(tp.xqi + v * tp.ps + it0, qi);
        load_vec<E>(tp.dyx + v * tp.ps + it0, yx);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            xqv[e] += q[e];
            xqiv[e] += qi[e];
            dyxv[e] += yx[e];
        }
    }
#pragma unroll 4
    for (int v = 0; v < tp.nc; ++v) {
        float cd[E];
        load_vec<E>(tp.cdi + v * tp.ps + it0, cd);
#pragma unroll
        for (int e = 0; e < E; ++e) cdv[e] += cd[e];
    }
    double suf[E], pre[E];  // per token: suffix and prefix terms
    double dyx = 0.0, lsuf = 0.0, lpre = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (tb + e >= seqlen) {  // padding tokens of the last chunk take no part
            xqv[e] = xqiv[e] = dyxv[e] = cdv[e] = dtv[e] = wdv[e] = 0.0;
        }
        dyx += dyxv[e];
        suf[e] = wdv[e] + cdv[e];
        pre[e] = dtv[e] * xqiv[e];
        lsuf += suf[e];
        lpre += pre[e];
    }
    // sums over the lanes after (suffix terms) and before (prefix terms) this one
    const double isuf = wave_prefix(lsuf), ipre = wave_prefix(lpre);
    const double tsuf = lane63(isuf);
    double z = 0.0;
    for (int k = lane; k < nzw; k += 64) z += (double)Zp[(bh * NC + c) * nzw + k];
    z = wave_sum(z);
    double sacc = tsuf - isuf;  // suffix from the later lanes
    double pacc = ipre - lpre;  // prefix from the earlier lanes
    double da[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {  // exclusive prefix within the lane
        da[e] = pacc;
        pacc += pre[e];
    }
#pragma unroll
    for (int e = E - 1; e >= 0; --e) {  // inclusive suffix within the lane
        sacc += suf[e];
        da[e] += sacc + z;
    }
    double da_sum = 0.0;
    const float Ah = A[h];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t t = tb + e;
        if (t < seqlen) ddt[(b * seqlen + t) * NH + h] = (float)(xqv[e] + (double)Ah * da[e]);
        da_sum += dtv[e] * da[e];
    }
    da_sum = wave_sum(da_sum);
    dyx = wave_sum(dyx);
    if (lane == 0) {
        dap[wv] = (float)da_sum;
        ddp[wv] = (float)dyx;
    }
}

// ---------------------------------------------------------------------------
// Final reductions, one launch: blocks [0, nblk_bc) sum the per-run-of-heads
// partials of dB and of dC (float4 per thread, the runs in order); the last
// blocks sum dA and dD per head over (batch, chunk).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kb_reduce(const float *__restrict__ dbp, const float *__restrict__ dcp,
                                                 float *__restrict__ dB, float *__restrict__ dC,
                                                 const float *__restrict__ dap, const float *__restrict__ ddp,
                                                 float *__restrict__ dA, float *__restrict__ dD, int nhb,
                                                 int64_t batch, int64_t seqlen, int64_t Lp, int64_t gn4,
                                                 int64_t n4, int64_t nblk_bc, int NH, int64_t nbc) {
    if ((int64_t)blockIdx.x < nblk_bc) {
        const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
        if (v >= 2 * n4) return;
        const bool isc = v >= n4;
        const int64_t i = isc ? v - n4 : v;  // float4 index over (batch, seqlen, G N / 4)
        const int64_t bt = i / gn4, r = i % gn4;
        const int64_t b = bt / seqlen, t = bt % seqlen;
        const float *src = isc ? dcp : dbp;
        const int64_t stride = batch * Lp * gn4;  // one run of heads
        const int64_t base = (b * Lp + t) * gn4 + r;
        floatx4 s = zero4();
        for (int k = 0; k < nhb; ++k) s += reinterpret_cast<const floatx4 *>(src)[k * stride + base];
        reinterpret_cast<floatx4 *>(isc ? dC : dB)[i] = s;
        return;
    }
    const int h = (int)(((int64_t)blockIdx.x - nblk_bc) * 256 + threadIdx.x);
    if (h >= NH) return;
    double sa = 0.0, sd = 0.0;
    for (int64_t k = 0; k < nbc; ++k) {
        sa += dap[k * NH + h];
        sd += ddp[k * NH + h];
    }
    dA[h] = (float)sa;
    if (dD != nullptr) dD[h] = (float)sd;
}

}  // namespace

hipError_t launch_bwd_scores(const Problem &p, const void *B, const void *C, float *ST, hipStream_t stream,
                             const LaunchEvents &ev) {
    const int n = (int)(p.chunk / 16), ntile = n * (n + 1) / 2;
    const int64_t total = p.batch * p.nchunks * p.ngroups * ntile;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 3) / 4;
    if (blocks > INT_MAX) return hipErrorInvalidValue;
    if (p.bf16)
        return launch_kernel(kb_scores<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream, ev,
                      static_cast<const uint16_t *>(B), static_cast<const uint16_t *>(C), ST, p.seqlen,
                      (int)p.ngroups, (int)p.dstate, (int)p.chunk, (int)p.nchunks, ntile, total);
    return launch_kernel(kb_scores<float>, dim3((unsigned)blocks), dim3(256), 0, stream, ev,
                      static_cast<const float *>(B), static_cast<const float *>(C), ST, p.seqlen,
                         (int)p.ngroups, (int)p.dstate, (int)p.chunk, (int)p.nchunks, ntile, total);
}

hipError_t launch_bwd_carry(const Problem &p, const float *U, const void *H, G2View G2, const float *dfinal,
                            void *E, float *Zp, float *dinit, hipStream_t stream, const LaunchEvents &ev) {
    const int64_t pn_vec = p.headdim * p.dstate / 4;
    const int64_t n_vec = p.batch * p.nheads * pn_vec;
    if (n_vec == 0) return hipSuccess;
    const int64_t blocks = (n_vec + 255) / 256;
    if (p.bf16)
        return launch_kernel(kb_carry<true>, dim3((unsigned)blocks), dim3(256), 0, stream, ev, U, H, G2.hi, G2.lo,
                      dfinal, E, Zp, dinit, n_vec, pn_vec, p.nchunks, p.padded_len, (int)p.chunk);
    return launch_kernel(kb_carry<false>, dim3((unsigned)blocks), dim3(256), 0, stream, ev, U, H, G2.hi,
                         G2.lo, dfinal, E, Zp, dinit, n_vec, pn_vec, p.nchunks, p.padded_len, (int)p.chunk);
}

hipError_t launch_bwd_tokens(const Problem &p, const BwdTokens &tk, const float *DT, const float *Zp,
                             const float *A, float *ddt, float *dap, float *ddp, hipStream_t stream,
                             const LaunchEvents &ev) {
    const int64_t total = p.batch * p.nchunks * p.nheads;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 3) / 4;
    const int nzw = (int)(p.headdim * p.dstate / 256);
    TokParts tp{tk.xq, tk.xqi, tk.dyx, tk.cdi, tk.wd, p.batch * p.nheads * p.padded_len, tk.nq, tk.nc};
#define SSD_KB_TOK(EE)                                                                                        \
    launch_kernel(kb_tokens<EE>, dim3((unsigned)blocks), dim3(256), 0, stream, ev, tp, DT, Zp, A, ddt, dap, ddp, \
                  p.seqlen, p.padded_len, (int)p.nheads, (int)p.nchunks, nzw, total)
    switch (p.chunk) {
        case 64: return SSD_KB_TOK(1);
        case 128: return SSD_KB_TOK(2);
        case 256: return SSD_KB_TOK(4);
        default: return hipErrorInvalidValue;
    }
#undef SSD_KB_TOK
}

hipError_t launch_bwd_reduce(const Problem &p, const float *dbp, const float *dcp, int nhb, float *dB, float *dC,
                             const float *dap, const float *ddp, float *dA, float *dD, hipStream_t stream,
                             const LaunchEvents &ev) {
    const int64_t gn4 = p.ngroups * p.dstate / 4;
    const int64_t n4 = p.batch * p.seqlen * gn4;
    const int64_t nblk_bc = (2 * n4 + 255) / 256;
    const int64_t nblk_h = (p.nheads + 255) / 256;
    if (nblk_bc + nblk_h > INT_MAX) return hipErrorInvalidValue;
    return launch_kernel(kb_reduce, dim3((unsigned)(nblk_bc + nblk_h)), dim3(256), 0, stream, ev, dbp, dcp, dB, dC,
                         dap, ddp, dA, dD, nhb, p.batch, p.seqlen, p.padded_len, gn4, n4, nblk_bc, (int)p.nheads,
                         p.batch * p.nchunks);
}

}  // namespace ssd

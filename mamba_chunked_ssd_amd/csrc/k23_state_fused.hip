// k23_state_fused.hip -- stages 2 and 3 in one launch: the chunk states and
// the carry across chunks (bf16 inputs).
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Kernel 2: fwd_pass_state": one program per (batch,
// head, state tile) walks the chunks in order, stores the running state at
// each chunk's start, and updates it with the log-space state jump of section
// "Mamba-2 architecture",
//     h_{c+1} = exp(G_last,c) h_c + (exp(G_last,c - G) . B) X^T ,
// so the per-chunk states s_c never travel through memory (the split path
// writes them once and reads them back).  In the stored [headdim, dstate]
// orientation, with w_t = exp2(G2_last - G2_t) dt_t from the cumsum stage:
//     h_{c+1}[p][n] = exp2(G2_last,c) h_c[p][n] + sum_t w_t x_t[p] B_t[n] .
//
// Design for gfx950.
//  * Block = (batch, head, NT dstate columns): one consumer wave per 16
//    headdim rows plus one producer wave.  A consumer keeps its rows of the
//    state tile in MFMA accumulators for the whole chunk loop:
//    v_mfma_f32_16x16x32_bf16 with M = dstate, N = headdim and K = tokens,
//    so lane l holds h[p = 16 w + l % 16][n = 16 mt + 4 (l / 16) + r],
//    r = 0..3 -- four consecutive dstate entries, one 8-byte store per plane.
//  * Tokens arrive in slabs of 64 (x rows of the head, B rows of the NT
//    columns, the 64 weights) by asynchronous copies straight into a ring of
//    LDS slots (buffer_load ... lds, the gfx950 counterpart of a bulk tensor
//    copy), RING - 1 slabs ahead of the MFMAs, across chunk boundaries.  The
//    producer wave issues every copy and waits for them with partial vmcnt
//    waits; one barrier per slab hands a landed slab to the consumers and
//    frees the slot they finished.  Stores and loads share the vmcnt counter
//    and complete in order, so the h_c stores are left to the consumers,
//    which never wait on it: a copy never waits behind a store.  Rows past
//    seqlen read as zero (buffer range check).
//  * Both MFMA operands come from LDS through the transposing read (four
//    tokens of one column per lane), so token-major x and B rows need no
//    register transposes; the 16-byte chunks of each LDS row are XOR-swizzled
//    so a read's eight rows per half wave fall in distinct banks.  A consumer
//    reads every operand of a slab first and scales the second k-step while
//    the first k-step's MFMAs run.
//  * w_t x_t is fp32-valued: each consumer scales its x fragment and splits
//    it into hi + lo bf16, both multiplied by the exact bf16 B (about 16
//    significant bits, as the split path's chunk-state kernel does).
//  * The state at each chunk start is written as the hi and lo bf16 planes the
//    chunk-output stage reads (hi = bf16(h), lo = bf16(h - hi)); the final
//    state is fp32.  Chunk decays exp2(G2_last) for 256 chunks at a time sit
//    in registers (64 per register, read back with readlane).
//  * For bf16 problems with headdim 64 and dstate 128 (or 256 at chunk 256),
//    extra blocks at the front of the grid compute the chunk output's C B^T
//    tiles.
#include "k_cb_tiles.h"
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kSlab = 64;  // tokens per slab

template <int T, int P, int NT>
struct FusedCfg {
    static constexpr int NCW = P / 16;          // consumer waves: one per 16 headdim rows
    static constexpr int NTHR = 64 * (NCW + 1); // + one producer wave
    static constexpr int RBX = 2 * P;           // bytes of an x row
    static constexpr int RBB = 2 * NT;          // bytes of a B row (this block's columns)
    static constexpr int XB = kSlab * RBX;      // x bytes per slab
    static constexpr int BB = kSlab * RBB;      // B bytes per slab
    static constexpr int WB = kSlab * 4;        // weights per slab
    static constexpr int SLOT = XB + BB + WB;
    static constexpr int KP = XB / 1024 + BB / 1024 + 1;  // producer copy instructions per slab
    static constexpr int SPC = T / kSlab;       // slabs per chunk
    static constexpr int MT = NT / 16;          // 16-column dstate tiles
    // ring depth: as deep as LDS allows while two blocks share a CU, at most
    // 8 slots, with every wait immediate (RING - 2) * KP in the vmcnt field
    static constexpr int pick_ring() {
        int best = 3;
        for (int r = 3; r <= 8; ++r)
            if (2 * r * SLOT <= (int)kLdsPerCu && (r - 2) * KP <= 63) best = r;
        return best;
    }
    static constexpr int RING = pick_ring();
    static constexpr size_t LDS = (size_t)RING * SLOT;
    static_assert(LDS <= kLdsPerCu && (RING - 2) * KP <= 63, "ring of LDS slots");
};

// XOR swizzle of the 32-byte column pairs of an LDS row of RB bytes, chosen
// so that the eight rows {t .. t+3, t+8 .. t+11} one half wave reads with the
// transposing read (32 bytes each, at the same column pair) occupy distinct
// banks: the row's position within a 256-byte bank span plus row bits that
// differ between the eight rows (bank conflicts measured zero on gfx950).
template <int RB>
__device__ __forceinline__ int pair_swz(int row) {
    if constexpr (RB == 64)
        return (row >> 3) & 1;
    else if constexpr (RB == 128)
        return ((row >> 1) & 1) | (((row >> 3) & 1) << 1);
    else
        return (row & 3) | (((row >> 3) & 1) << 2);
}
// LDS byte offset of 16-byte chunk q of row `row`
template <int RB>
__device__ __forceinline__ int slab_off(int row, int q) {
    return row * RB + ((q ^ (2 * pair_swz<RB>(row))) << 4);
}
// Transposing read of column tile `tile` (16 bf16 columns) for k-step ks of a
// slab: lane (16 g + 4 r + a) addresses row 32 ks + 8 g + 4 hf + r, columns
// 16 tile + 4 a .. + 3, so lane l receives the 8 tokens 32 ks + 8 g .. + 7 of
// column 16 tile + l % 16 (two bf16 per dword, token order).
template <int RB>
__device__ __forceinline__ u32x4 tr_frag(const unsigned char *slab, int ks, int tile, int l16, int g4) {
    const int r = l16 >> 2, a = l16 & 3;
    u32x2 v[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int row = 32 * ks + 8 * g4 + 4 * hf + r;
        v[hf] = tr_read(slab + slab_off<RB>(row, 2 * tile + (a >> 1)) + 8 * (a & 1));
    }
    return u32x4{v[0][0], v[0][1], v[1][0], v[1][1]};
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most KP * yc copy instructions are outstanding (yc < YCN)
template <int KP, int YCN, int YC = 0>
__device__ __forceinline__ void vm_wait_copies(int yc) {
    if constexpr (YC + 1 < YCN) {
        if (yc == YC) {
            vm_wait<KP * YC>();
            return;
        }
        vm_wait_copies<KP, YCN, YC + 1>(yc);
    } else {
        vm_wait<KP * YC>();
    }
}

// w_t x_t of a lane's 8 tokens, split into hi and lo bf16 operands
__device__ __forceinline__ void scale_split(const u32x4 &xv, const floatx4 &w0, const floatx4 &w1,
                                            u32x4 &xh, u32x4 &xl) {
    const float wt[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const HiLo s2 = split_bf16(bf16lo(xv[d]) * wt[2 * d], bf16hi(xv[d]) * wt[2 * d + 1]);
        xh[d] = s2.hi;
        xl[d] = s2.lo;
    }
}

template <int T, int P, int NT>
__global__ __launch_bounds__(64 * (P / 16 + 1)) void k23_state_fused_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm, const float *__restrict__ W,
    const float *__restrict__ G2hi, const float *__restrict__ G2lo, const float *__restrict__ init,
    uint16_t *__restrict__ H, float *__restrict__ final_states, int64_t L, int NH, int N, int G,
    int NC, int64_t Lp, int HPG, int ntiles, int nfused,
    // C B^T tiles (the problems of uses_cb_tiles; ncb = 0 otherwise)
    const uint16_t *__restrict__ Cm, float *__restrict__ CB, int64_t cb_ntiles, int ncb) {
    using Cfg = FusedCfg<T, P, NT>;
    constexpr int NCW = Cfg::NCW, RING = Cfg::RING, KP = Cfg::KP, SPC = Cfg::SPC, MT = Cfg::MT;
    extern __shared__ __align__(16) unsigned char lds[];

    if constexpr (P == 64) {
        if ((int)blockIdx.x < ncb) {
            if (threadIdx.x < 256) {
                if (N == 256)
                    cb_tiles<T, 256>(Bm, Cm, CB, L, G, NC, cb_ntiles, ncb, blockIdx.x);
                else
                    cb_tiles<T, 128>(Bm, Cm, CB, L, G, NC, cb_ntiles, ncb, blockIdx.x);
            }
            return;
        }
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    // ncb is a multiple of 8, so the hardware XCD of this block is f % 8
    const int f = (int)blockIdx.x - ncb;
    const int bid = xcd_remap(f, nfused);
    const int nt = bid % ntiles;
    const int bh = bid / ntiles;
    const int h = bh % NH;
    const int64_t b = bh / NH;
    const int gi = h / HPG;
    const int n0 = nt * NT;
    const int nslabs = NC * SPC;

    if (w == NCW) {
        // ---- producer wave: asynchronous copies of slab i into ring slot
        //      i % RING, RING - 1 slabs ahead; it issues nothing else, so its
        //      vector-memory counter holds only copies (they complete in
        //      issue order): slab i has landed when no more than the copies
        //      of the slabs after it are outstanding
        const int64_t xrow = (int64_t)NH * P;  // elements between token rows of x
        const int64_t brow = (int64_t)G * N;   // ... of B
        int ln = lane;
        asm volatile("" : "+v"(ln));
        auto issue = [&](int i) {
            const int64_t ts = (int64_t)i * kSlab;
            const int rows = (int)min<int64_t>(kSlab, L - ts);
            unsigned char *slot = lds + (i % RING) * Cfg::SLOT;
            const uint32_t sx = lds_addr(slot), sb = lds_addr(slot + Cfg::XB),
                           sw = lds_addr(slot + Cfg::XB + Cfg::BB);
            const i32x4 xd = buffer_desc(x + ((b * L + ts) * NH + h) * P,
                                         rows > 0 ? (uint32_t)(((rows - 1) * xrow + P) * 2) : 0u);
            const i32x4 bd = buffer_desc(Bm + ((b * L + ts) * G + gi) * N + n0,
                                         rows > 0 ? (uint32_t)(((rows - 1) * brow + NT) * 2) : 0u);
            const i32x4 wd = buffer_desc(W + (int64_t)bh * Lp + ts, kSlab * 4);
            // 1-KiB copy j covers LDS bytes [1024 j, 1024 j + 1024) of the
            // region: lane l lands at row (1024 j + 16 l) / RB, chunk position
            // pos, which holds the row's global chunk pos ^ 2 swz(row)
#pragma unroll
            for (int j = 0; j < Cfg::XB / 1024; ++j) {
                const int byte = 1024 * j + 16 * ln;
                const int row = byte / Cfg::RBX, pos = (byte % Cfg::RBX) >> 4;
                const int q = pos ^ (2 * pair_swz<Cfg::RBX>(row));
                lds_dma_x4(xd, sx + 1024 * j, (int)(row * xrow * 2) + 16 * q);
            }
#pragma unroll
            for (int j = 0; j < Cfg::BB / 1024; ++j) {
                const int byte = 1024 * j + 16 * ln;
                const int row = byte / Cfg::RBB, pos = (byte % Cfg::RBB) >> 4;
                const int q = pos ^ (2 * pair_swz<Cfg::RBB>(row));
                lds_dma_x4(bd, sb + 1024 * j, (int)(row * brow * 2) + 16 * q);
            }
            lds_dma_x1(wd, sw, 4 * ln);
        };
        const int pre = min(RING - 1, nslabs);
        for (int i = 0; i < pre; ++i) issue(i);
        for (int i = 0; i < nslabs; ++i) {
            vm_wait_copies<KP, RING - 1>(min(RING - 2, nslabs - 1 - i));
            __syncthreads();  // slab i is visible; every consumer is done with slot (i - 1) % RING
            if (i + RING - 1 < nslabs) issue(i + RING - 1);
        }
        return;
    }

    // ---- consumer waves: wave w owns headdim rows 16 w .. 16 w + 15 and all
    //      NT columns; acc[mt] lane holds h[16 w + l16][n0 + 16 mt + 4 g4 + r]
    //      Chunk decays exp2(G2_last,c): chunk 256 k + 64 j + l in lane l of
    //      decv[j] for the current k.
    constexpr int DV = 4;
    float decv[DV];
    const float *g2h = G2hi + (int64_t)bh * Lp + (T - 1);
    const float *g2l = G2lo + (int64_t)bh * Lp + (T - 1);
    auto load_decays = [&](int c0) {
#pragma unroll
        for (int j = 0; j < DV; ++j) {
            const int c = c0 + 64 * j + lane;
            decv[j] = c < NC ? fast_exp2(g2h[(int64_t)c * T] + g2l[(int64_t)c * T]) : 0.f;
        }
    };
    load_decays(0);
    floatx4 acc[MT];
    const int prow = 16 * w + l16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = zero4();
        if (init != nullptr)
            acc[mt] = *reinterpret_cast<const floatx4 *>(init + ((int64_t)bh * P + prow) * N + n0 + 16 * mt + 4 * g4);
    }
    // the (batch, head) region of H: nchunks x (hi, lo) planes of P x N bf16;
    // per-lane byte offsets within a chunk's planes, fixed for the loop
    const __amdgpu_buffer_rsrc_t hres =
        buffer_rsrc(H + (int64_t)bh * NC * 2 * P * N, (uint32_t)((int64_t)NC * 4 * P * N));
    const int hoff = (prow * N + n0 + 4 * g4) * 2;
    const int plane = P * N * 2;
    int i = 0;
    for (int c = 0; c < NC; ++c) {
        if (c > 0 && (c & 255) == 0) load_decays(c);
        float dec = 0.f;
        {
            const int j = (c >> 6) & (DV - 1), li = c & 63;
#pragma unroll
            for (int q = 0; q < DV; ++q) {
                const float dq =
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, decv[q]), li));
                dec = (j == q) ? dq : dec;
            }
        }
        // h_c: the hi and lo bf16 planes of (batch, head, chunk), then the
        // decay exp2(G2_last,c).  A buffer store reads its data registers
        // after it issues (later still behind the producer's copies), and the
        // compiler does not wait for that before it reuses them; an expcnt
        // wait that takes the data registers as operands holds them until
        // the stores have read them -- not until the stores complete, which
        // under load takes microseconds (the wait a plain global store gets).
        {
            const int cbase = __builtin_amdgcn_readfirstlane(c * 4 * P * N);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const HiLo a = split_bf16(acc[mt][0], acc[mt][1]), q = split_bf16(acc[mt][2], acc[mt][3]);
                const u32x2 dh = u32x2{a.hi, q.hi}, dl = u32x2{a.lo, q.lo};
                __builtin_amdgcn_raw_buffer_store_b64(dh, hres, hoff + 32 * mt, cbase, 0);
                __builtin_amdgcn_raw_buffer_store_b64(dl, hres, hoff + 32 * mt + plane, cbase, 0);
                asm volatile("s_waitcnt expcnt(0)" ::"v"(dh), "v"(dl) : "memory");
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] *= dec;
        }
        for (int s = 0; s < SPC; ++s, ++i) {
            __syncthreads();  // the producer's copies of slab i are visible
            const unsigned char *slot = lds + (i % RING) * Cfg::SLOT;
            const unsigned char *xs = slot;
            const unsigned char *bs = slot + Cfg::XB;
            const float *ws = reinterpret_cast<const float *>(slot + Cfg::XB + Cfg::BB);
            // every operand of the slab's two k-steps first, then the MFMAs of
            // k-step 0 with k-step 1's scaling between them
            u32x4 xv[2], bt[2][MT];
            floatx4 wv[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                xv[ks] = tr_frag<Cfg::RBX>(xs, ks, w, l16, g4);
                wv[ks][0] = *reinterpret_cast<const floatx4 *>(ws + 32 * ks + 8 * g4);
                wv[ks][1] = *reinterpret_cast<const floatx4 *>(ws + 32 * ks + 8 * g4 + 4);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) bt[ks][mt] = tr_frag<Cfg::RBB>(bs, ks, mt, l16, g4);
            }
            u32x4 xh0, xl0, xh1, xl1;
            scale_split(xv[0], wv[0][0], wv[0][1], xh0, xl0);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(bt[0][mt], xh0, acc[mt]);
            scale_split(xv[1], wv[1][0], wv[1][1], xh1, xl1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(bt[0][mt], xl0, acc[mt]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(bt[1][mt], xh1, acc[mt]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(bt[1][mt], xl1, acc[mt]);
        }
    }
    if (final_states != nullptr) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            *reinterpret_cast<floatx4 *>(final_states + ((int64_t)bh * P + prow) * N + n0 + 16 * mt + 4 * g4) =
                acc[mt];
    }
}

template <int T, int P, int NT>
hipError_t launch_tpn(const Problem &p, const void *x, const void *B, const float *W, G2View G2,
                      const float *init, float *H, float *final_states, const void *C, float *CB,
                      hipStream_t stream, const LaunchEvents &ev) {
    using Cfg = FusedCfg<T, P, NT>;
    constexpr auto kern = k23_state_fused_bf16<T, P, NT>;
    const int ntiles = (int)(p.dstate / NT);
    const int64_t nfused = p.batch * p.nheads * ntiles;
    int64_t ncb = 0, cb_ntiles = 0;
    if (uses_cb_tiles(p)) {
        cb_ntiles = p.batch * p.nchunks * p.ngroups * cb_slots(p.chunk);
        ncb = (cb_blocks(cb_ntiles) + 7) / 8 * 8;  // keeps the fused blocks' XCD mapping
    }
    if (nfused + ncb > INT32_MAX) return hipErrorInvalidValue;
    if (allow_lds<kern>(Cfg::LDS) != hipSuccess) return hipErrorInvalidValue;
    return launch_kernel(kern, dim3((unsigned)(nfused + ncb)), dim3(Cfg::NTHR), Cfg::LDS, stream, ev,
                         static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B), W, G2.hi,
                         G2.lo, init, reinterpret_cast<uint16_t *>(H), final_states, p.seqlen,
                         (int)p.nheads, (int)p.dstate, (int)p.ngroups, (int)p.nchunks, p.padded_len,
                         (int)p.heads_per_group, ntiles, (int)nfused, static_cast<const uint16_t *>(C), CB,
                         cb_ntiles, (int)ncb);
}

template <int T, int P>
hipError_t launch_tp(const Problem &p, int cols, const void *x, const void *B, const float *W, G2View G2,
                     const float *init, float *H, float *final_states, const void *C, float *CB,
                     hipStream_t stream, const LaunchEvents &ev) {
    if (cols == 32) return launch_tpn<T, P, 32>(p, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
    if (cols == 64) return launch_tpn<T, P, 64>(p, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
    return hipErrorInvalidValue;
}

template <int T>
hipError_t launch_t(const Problem &p, int cols, const void *x, const void *B, const float *W, G2View G2,
                    const float *init, float *H, float *final_states, const void *C, float *CB,
                    hipStream_t stream, const LaunchEvents &ev) {
    switch (p.headdim) {
        case 32: return launch_tp<T, 32>(p, cols, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
        case 64: return launch_tp<T, 64>(p, cols, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
        case 128: return launch_tp<T, 128>(p, cols, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool state_fused_supported(const Problem &p, int cols) {
    // the stores address one (batch, head)'s chunk-start states with 32-bit
    // byte offsets
    const int64_t h_bytes = p.nchunks * 4 * p.headdim * p.dstate;
    return p.bf16 && (cols == 32 || cols == 64) && p.dstate % cols == 0 && h_bytes <= INT32_MAX;
}

hipError_t launch_state_fused(const Problem &p, const Plan &plan, const void *x, const void *B,
                              const float *W, G2View G2, const float *init, float *H,
                              float *final_states, const void *C, float *CB, hipStream_t stream,
                              const LaunchEvents &ev) {
    if (p.batch * p.nheads == 0 || p.nchunks == 0) return hipSuccess;
    switch (p.chunk) {
        case 64: return launch_t<64>(p, plan.fused_cols, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
        case 128: return launch_t<128>(p, plan.fused_cols, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
        case 256: return launch_t<256>(p, plan.fused_cols, x, B, W, G2, init, H, final_states, C, CB, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd

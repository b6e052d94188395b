// ssd_device.h -- device-side helpers shared by the libssd kernels (gfx950).
//
// Vector types for the MFMA operands, bf16 storage conversions (round to
// nearest even through the hardware pack instruction), the hi/lo bf16 split
// used for fp32-valued MFMA operands, and the MFMA wrappers.
//
// MFMA lane layouts used throughout (64-lane wave, l = lane, g = l / 16):
//   v_mfma_f32_16x16x32_bf16:  A lane holds A[m = l%16][k = 8g .. 8g+7]
//                              B lane holds B[k = 8g .. 8g+7][n = l%16]
//   v_mfma_f32_16x16x4_f32:    A lane holds A[m = l%16][k = g]
//                              B lane holds B[k = g][n = l%16]
//   both:                      D lane holds D[m = 4g + r][n = l%16], r = 0..3
// A contraction is a sum over k, so any fixed relabelling of k applied to both
// operands gives the same product; the kernels use that freedom to feed MFMA
// output fragments back in as A operands without a register shuffle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
// Low / high bf16 of a packed dword, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> one dword of two bf16 (a in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    floatx2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// hi = bf16(v), lo = bf16(v - hi) for two values at once; hi + lo carries
// about 16 significant bits of v.
struct HiLo {
    uint32_t hi, lo;
};
__device__ __forceinline__ HiLo split_bf16(float a, float b) {
    HiLo r;
    r.hi = pack_bf16(a, b);
    r.lo = pack_bf16(a - bf16lo(r.hi), b - bf16hi(r.hi));
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// E consecutive floats as one vector store
template <int E>
struct VecF;
template <>
struct VecF<1> { typedef float type; };
template <>
struct VecF<2> { typedef floatx2 type; };
template <>
struct VecF<4> { typedef floatx4 type; };

template <int E>
__device__ __forceinline__ void store_vec(float *p, const float (&v)[E]) {
    typename VecF<E>::type t;
    if constexpr (E == 1) {
        t = v[0];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) t[e] = v[e];
    }
    *reinterpret_cast<typename VecF<E>::type *>(p) = t;
}

// A double moved across lanes by one DPP control (both 32-bit halves); a lane
// with no source lane (or in a row the row mask leaves out) gets 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_move_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Per-chunk log-decay cumsum of one head by one wave ("Kernel 1: Computing
// cumulative sums" of the CUDA Tile post): lane l holds dt of the chunk's
// tokens E l .. E l + E - 1 (0 past seqlen).  The running sum of
// log2(e) A dt_t is taken in fp64 (serial within the lane, then a wave scan)
// and returned as hi + lo floats, together with the weight with which each
// token enters its chunk's state, W_t = exp2(G2_last - G2_t) dt_t, whose
// exponent is formed in fp64 before the fp32 exp2.
template <int E>
__device__ __forceinline__ void chunk_cumsum_wave(const float (&d)[E], float A, int lane, float (&hi)[E],
                                                  float (&lo)[E], float (&wt)[E]) {
    const double a2 = (double)A * 1.4426950408889634;  // log2(e)
    double run[E];
    double tot = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        tot += a2 * (double)d[e];
        run[e] = tot;
    }
    // inclusive scan of the lane totals across the wave, with DPP lane moves:
    // shifts by 1, 2, 4, 8 within each row of 16 lanes, then the last lane of
    // row 0 (2) added to row 1 (3), then lane 31 added to rows 2 and 3
    double inc = tot;
    inc += dpp_move_f64<0x111, 0xf>(inc);  // row_shr:1
    inc += dpp_move_f64<0x112, 0xf>(inc);  // row_shr:2
    inc += dpp_move_f64<0x114, 0xf>(inc);  // row_shr:4
    inc += dpp_move_f64<0x118, 0xf>(inc);  // row_shr:8
    inc += dpp_move_f64<0x142, 0xa>(inc);  // row_bcast:15 into rows 1, 3
    inc += dpp_move_f64<0x143, 0xc>(inc);  // row_bcast:31 into rows 2, 3
    const double excl = inc - tot;
    const uint64_t lb = (uint64_t)__double_as_longlong(inc);
    const uint32_t llo = __builtin_amdgcn_readlane((int)(uint32_t)lb, 63);
    const uint32_t lhi = __builtin_amdgcn_readlane((int)(uint32_t)(lb >> 32), 63);
    const double last = __longlong_as_double((long long)(((uint64_t)lhi << 32) | llo));  // chunk's last token
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const double g = excl + run[e];
        hi[e] = (float)g;
        lo[e] = (float)(g - (double)hi[e]);
        wt[e] = __builtin_amdgcn_exp2f((float)(last - g)) * d[e];
    }
}

__device__ __forceinline__ floatx4 mfma_bf16(const u32x4 &a, const u32x4 &b, const floatx4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_f32(float a, float b, const floatx4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Raw buffer access (gfx9 resource word 3 = 0x00020000: 32-bit data format,
// no swizzle, byte-granular range).  Loads past `bytes` read 0 and stores past
// it are dropped; offsets are 32-bit byte offsets from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load_x4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Copies from a raw buffer straight into LDS (the load's LDS-destination
// form): lane l's 16 (or 4) bytes land at lds_addr + 16 l (+ 4 l), where
// lds_addr is a wave-uniform LDS byte address (it goes through M0, which
// needs one wait state before the load).  The range check applies to voffset
// only, so every per-lane offset goes there.  They are issued as inline
// assembly: the compiler neither tracks nor waits for them (it would
// otherwise wait for every pending copy before any LDS read it cannot prove
// disjoint), so the caller waits (lds_dma_wait) before the destination is
// read -- by the issuing wave, or by others after a barrier.
// The descriptor and the LDS address must live in scalar registers; they are
// wave-uniform by construction, and readfirstlane says so to the compiler
// (which otherwise may keep a value it cannot prove uniform in vector
// registers, which the instruction does not accept).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_desc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int32_t)((a >> 32) & 0xffffu)),
                 __builtin_amdgcn_readfirstlane((int32_t)bytes), 0x00020000};
}
template <typename Ptr>
__device__ __forceinline__ uint32_t lds_addr(Ptr p) {
    typedef __attribute__((address_space(3))) const unsigned char lds_byte;
    return (uint32_t)reinterpret_cast<uintptr_t>((lds_byte *)(p));
}
__device__ __forceinline__ void lds_dma_x4(const i32x4 &desc, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(desc)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_x1(const i32x4 &desc, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(desc)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// gfx950 transposing LDS read of 16-bit data (8 bytes per lane): within each
// 16-lane group, lane l receives element l % 4 of the 4 elements addressed by
// lanes 4 r + (l % 16) / 4, r = 0..3.  So when lane 4 r + a addresses row k_r,
// columns 4 a .. 4 a + 3 of a bf16 matrix X, lane l gets X[k_r][l % 16] for
// r = 0..3 (two bf16 per dword, r = 0 in the low half).
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 tr_read(const unsigned char *p) {
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)p));
}

}  // namespace ssd

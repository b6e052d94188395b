// kb_pass_q.hip -- the dx pass of the backward pass (kb_pass.h, pass Q), and
// the host-side dispatch of all three passes.
#include "kb_pass_inst.h"

namespace ssd {
namespace bwd {

hipError_t launch_pass_q(const PassArgs &a, bool bf16, int dv, unsigned blocks, size_t lds, hipStream_t stream,
                         const LaunchEvents &ev) {
    if (bf16) {
        if (dv == 32) return launch_one<uint16_t, 1, 32, kPassQ>(a, blocks, lds, stream, ev);
        if (dv == 64) return launch_one<uint16_t, 1, 64, kPassQ>(a, blocks, lds, stream, ev);
    } else {
        if (dv == 32) return launch_one<float, 1, 32, kPassQ>(a, blocks, lds, stream, ev);
        if (dv == 64) return launch_one<float, 1, 64, kPassQ>(a, blocks, lds, stream, ev);
    }
    return hipErrorInvalidValue;
}

namespace {
void rows_for(const Problem &p, int pass, int dv, int pad, int *krow, int *vrow, int *erow) {
    *krow = (int)p.headdim + pad;
    *vrow = dv + pad;
    *erow = pass == kPassQ ? (int)((p.dstate + 31) / 32 * 32) + pad : dv + pad;
}
}  // namespace

}  // namespace bwd

size_t bwd_pass_lds(const Problem &p, int pass, int dv, int lds_pad, bool xt) {
    int krow, vrow, erow;
    bwd::rows_for(p, pass, dv, lds_pad, &krow, &vrow, &erow);
    const size_t bytes = (size_t)bwd::kb_lds_bytes(pass, !p.bf16, (int)p.chunk, (int)p.headdim, (int)p.dstate, dv,
                                                   krow, vrow, erow, xt);
    return bytes <= kLdsPerCu ? bytes : 0;
}

namespace {
hipError_t run_pass(const Problem &p, const BwdPassLaunch &L, hipStream_t stream, const LaunchEvents &ev, int *occ);
}

hipError_t launch_bwd_pass(const Problem &p, const BwdPassLaunch &L, hipStream_t stream, const LaunchEvents &ev) {
    return run_pass(p, L, stream, ev, nullptr);
}

int bwd_pass_blocks_per_cu(const Problem &p, const BwdPassLaunch &L) {
    int n = 0;
    return run_pass(p, L, nullptr, LaunchEvents{}, &n) == hipSuccess ? n : 0;
}

namespace {
hipError_t run_pass(const Problem &p, const BwdPassLaunch &L, hipStream_t stream, const LaunchEvents &ev, int *occ) {
    using namespace bwd;
    const size_t lds = bwd_pass_lds(p, L.pass, L.dv, L.lds_pad, L.xt_lds != 0);
    if (lds == 0) return hipErrorInvalidValue;
    const int64_t dvtot = L.pass == kPassQ ? p.headdim : (L.pass == kPassW || L.pass == kPassP) ? L.dv : p.dstate;
    if (L.pass == kPassP && p.bf16) return hipErrorInvalidValue;  // fp32 problems only
    if (L.dv <= 0 || dvtot % L.dv != 0 || L.hb < 1 || L.hb > p.heads_per_group) return hipErrorInvalidValue;
    PassArgs a;
    a.x = L.x;
    a.dy = L.dy;
    a.Bm = L.B;
    a.Cm = L.C;
    a.G2hi = L.G2.hi;
    a.G2lo = L.G2.lo;
    a.DT = L.DT;
    a.E = L.E;
    a.H = L.H;
    a.ST = L.ST;
    a.D = L.D;
    a.out = L.out;
    a.xq = L.xq;
    a.xqi = L.xqi;
    a.dyx = L.dyx;
    a.cdi = L.cdi;
    a.wd = L.wd;
    a.pt = L.pt;
    a.ptt = L.ptt;
    a.seqlen = p.seqlen;
    a.Lp = p.padded_len;
    a.batch = (int)p.batch;
    a.NH = (int)p.nheads;
    a.P = (int)p.headdim;
    a.N = (int)p.dstate;
    a.G = (int)p.ngroups;
    a.HPG = (int)p.heads_per_group;
    a.T = (int)p.chunk;
    a.NC = (int)p.nchunks;
    a.nvt = (int)(dvtot / L.dv);
    if (L.pass == kPassQ || L.pass == kPassW || L.pass == kPassP) {
        // one block per head (the head's rows are its own)
        a.hb = 1;
        a.nhb = (int)p.heads_per_group;
    } else {
        a.hb = L.hb;
        a.nhb = (int)((p.heads_per_group + L.hb - 1) / L.hb);
    }
    rows_for(p, L.pass, L.dv, L.lds_pad, &a.krow, &a.vrow, &a.erow);
    a.xt_lds = L.xt_lds ? 1 : 0;
    a.occ = occ;
    const int64_t blocks = p.batch * p.nchunks * p.ngroups * a.nhb * a.nvt;
    if (blocks == 0 && occ == nullptr) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    switch (L.pass) {
        case kPassQ: return launch_pass_q(a, p.bf16, L.dv, (unsigned)blocks, lds, stream, ev);
        case kPassB: return launch_pass_b(a, p.bf16, L.dv, (unsigned)blocks, lds, stream, ev);
        case kPassC: return launch_pass_c(a, p.bf16, L.dv, (unsigned)blocks, lds, stream, ev);
        case kPassW: return launch_pass_w(a, p.bf16, (unsigned)blocks, lds, stream, ev);
        case kPassP: return launch_pass_p(a, (unsigned)blocks, lds, stream, ev);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

}  // namespace ssd

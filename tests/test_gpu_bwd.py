"""Parity of the backward pass (ssd_chunk_scan_bwd, through the C ABI) with
the fp64 oracle's adjoint (oracle.scan_bwd): every gradient -- dx, ddt, dA,
dB, dC, dD and the initial state's -- element by element, over shapes that
span several chunks, ragged last chunks, every supported chunk size and
headdim, dstate values that are not powers of two, grouped heads, runs of
heads per block, and the edge cases.

Bound per gradient: max |gpu - oracle| / rms(oracle) <= 1e-4
for fp32 inputs and 2e-2 for bf16 inputs, as for the forward pass.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_chunked_ssd_amd as ssd
import oracle
import ssd_inputs as si
from tests.gpu_util import TOL, nerr, to_device

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "d_initial_states")


def _run(w, final=True, with_d=True, seed=None):
    inp = si.generate(w, seed=seed)
    if not with_d:
        inp["D"] = None
    cot = si.cotangents(w, final=final)
    t = to_device(inp, w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dy = torch.from_numpy(cot["dy"]).cuda().to(tdt)
    dfin = None if cot["dfinal"] is None else torch.from_numpy(cot["dfinal"]).cuda()
    g = ssd.chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dy, chunk_size=w.chunk_size,
                           initial_states=t["h0"], d_final_states=dfin)
    torch.cuda.synchronize()
    got = {k: v.double().cpu().numpy() for k, v in g.items()}
    ref = oracle.scan_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                          cot["dy"], cot["dfinal"])
    ref["d_initial_states"] = ref.pop("dh0")
    return got, ref


def _check(got, ref, dtype, label):
    errs = {k: nerr(got[k], ref[k]) for k in GRADS if k in got}
    bad = {k: e for k, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, "%s: %s (all: %s)" % (label, bad, errs)
    return errs


# (dtype, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, init_std)
SHAPES = [
    ("f32", 1, 256, 4, 32, 16, 1, 64, 0.0),       # the tiny workload's shape
    ("bf16", 1, 256, 4, 32, 16, 1, 64, 0.0),
    ("f32", 2, 200, 4, 64, 64, 2, 64, 0.1),       # ragged, grouped, initial state
    ("bf16", 2, 200, 4, 64, 64, 2, 64, 0.1),
    ("bf16", 1, 700, 4, 64, 128, 1, 256, 0.1),    # the 2.7B layer's tile shape, ragged
    ("f32", 1, 700, 4, 64, 128, 1, 256, 0.1),
    ("bf16", 1, 384, 6, 128, 48, 3, 128, 0.1),    # headdim 128, dstate 48
    ("f32", 1, 384, 6, 128, 48, 3, 128, 0.0),
    ("bf16", 1, 300, 2, 32, 256, 1, 128, 0.1),    # dstate 256
    ("f32", 1, 300, 2, 128, 256, 1, 256, 0.1),    # fp32, chunk 256, headdim 128 (narrow tiles)
    ("bf16", 1, 300, 2, 128, 256, 1, 256, 0.0),
    ("bf16", 2, 130, 4, 64, 80, 1, 64, 0.0),      # dstate 80 (not a multiple of 32)
    ("f32", 1, 129, 2, 32, 16, 2, 128, 0.1),      # one token past a chunk
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "%s-b%d-L%d-h%d-p%d-n%d-g%d-T%d" % c[:8])
def test_backward_matches_oracle(case):
    dtype, b, L, nh, p, n, g, T, init = case
    w = si.small(dtype=dtype, batch=b, seqlen=L, nheads=nh, headdim=p, dstate=n, ngroups=g, chunk_size=T,
                 dt_mu=-1.0, init_std=init, seed=2000 + L + n)
    print("bwd case", case, flush=True)
    got, ref = _run(w)
    _check(got, ref, dtype, str(case))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_without_D_and_final_gradient(dtype):
    w = si.small(dtype=dtype, batch=2, seqlen=150, nheads=4, headdim=32, dstate=32, ngroups=1, chunk_size=64,
                 dt_mu=-1.0, init_std=0.1, seed=2101)
    got, ref = _run(w, final=False, with_d=False)
    _check(got, ref, dtype, "no D, no dfinal")


def test_backward_slow_decay_long_chunks():
    # small |A dt| keeps the decays near 1 across whole chunks, the regime
    # where the gradient of the decays sums the most terms
    w = si.small(dtype="f32", batch=1, seqlen=512, nheads=4, headdim=64, dstate=64, ngroups=1, chunk_size=256,
                 dt_mu=-4.0, init_std=0.1, seed=2102)
    got, ref = _run(w)
    _check(got, ref, "f32", "slow decay")


def test_backward_runs_of_heads_per_block():
    # enough (batch, chunk) work that the dB / dC passes put several heads in
    # one block: the 2.7B layer's head count and tile shape on a shorter sequence
    w = si.small(dtype="bf16", batch=2, seqlen=2048, nheads=80, headdim=64, dstate=128, ngroups=1,
                 chunk_size=256, dt_mu=-2.0, init_std=0.0, seed=2103)
    got, ref = _run(w)
    _check(got, ref, "bf16", "2.7B layer")


def test_backward_tiny_workload_full():
    w = si.BY_NAME["tiny_f32"]
    got, ref = _run(w)
    _check(got, ref, "f32", w.name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_single_token_and_zero_dt(dtype):
    w = si.small(dtype=dtype, batch=2, seqlen=1, nheads=2, headdim=32, dstate=16, ngroups=1, chunk_size=64,
                 dt_mu=-1.0, init_std=0.1, seed=2104)
    got, ref = _run(w)
    _check(got, ref, dtype, "seqlen 1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_empty_sequence(dtype):
    # seqlen 0: d_initial = d_final, dA = dD = 0
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    b, nh, p, n = 2, 2, 32, 16
    x = torch.zeros((b, 0, nh, p), dtype=tdt, device="cuda")
    dt = torch.zeros((b, 0, nh), dtype=tdt, device="cuda")
    Bm = torch.zeros((b, 0, 1, n), dtype=tdt, device="cuda")
    A = -torch.ones(nh, device="cuda")
    D = torch.ones(nh, device="cuda")
    h0 = torch.randn((b, nh, p, n), device="cuda")
    dfin = torch.randn((b, nh, p, n), device="cuda")
    g = ssd.chunk_scan_bwd(x, dt, A, Bm, Bm.clone(), D, x.clone(), chunk_size=64, initial_states=h0,
                           d_final_states=dfin)
    torch.cuda.synchronize()
    assert torch.equal(g["d_initial_states"], dfin)
    assert not g["dA"].any() and not g["dD"].any()


def test_backward_is_deterministic():
    w = si.small(dtype="bf16", batch=1, seqlen=600, nheads=8, headdim=64, dstate=128, ngroups=2, chunk_size=256,
                 dt_mu=-1.0, init_std=0.1, seed=2105)
    inp = si.generate(w)
    cot = si.cotangents(w)
    t = to_device(inp, "bf16")
    dy = torch.from_numpy(cot["dy"]).cuda().to(torch.bfloat16)
    dfin = torch.from_numpy(cot["dfinal"]).cuda()
    runs = [ssd.chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dy, chunk_size=256,
                               initial_states=t["h0"], d_final_states=dfin) for _ in range(2)]
    torch.cuda.synchronize()
    for k in runs[0]:
        assert torch.equal(runs[0][k], runs[1][k]), k


# (dtype, forward plan or None for the default, batch, seqlen, nheads, headdim, dstate, ngroups, chunk)
SAVED_CASES = [
    ("bf16", None, 2, 600, 8, 64, 128, 2, 256),     # the 2.7B layer's tile shape, ragged, grouped
    ("bf16", "fused", 2, 600, 8, 64, 128, 2, 256),  # states from the fused state launch
    ("f32", None, 1, 300, 4, 128, 48, 2, 128),      # fp32: H a region of its own only with the flag
    ("bf16", None, 1, 129, 2, 32, 16, 1, 64),       # one token past a chunk
]


@pytest.mark.parametrize("case", SAVED_CASES, ids=lambda c: "%s-%s-b%d-L%d-h%d-p%d-n%d-g%d-T%d" % c)
def test_backward_from_saved_forward_states(case):
    # the forward's kept chunk-start states in place of the recomputed ones:
    # the gradients match the oracle's adjoint and the recomputing backward
    dtype, plan, b, L, nh, p, n, g, T = case
    w = si.small(dtype=dtype, batch=b, seqlen=L, nheads=nh, headdim=p, dstate=n, ngroups=g, chunk_size=T,
                 dt_mu=-1.0, init_std=0.1, seed=2300 + L + n)
    print("bwd saved case", case, flush=True)
    inp = si.generate(w)
    cot = si.cotangents(w)
    t = to_device(inp, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dy = torch.from_numpy(cot["dy"]).cuda().to(tdt)
    dfin = torch.from_numpy(cot["dfinal"]).cuda()
    shape = ssd.make_shape(b, L, nh, p, n, g, dtype, True)
    fws = torch.empty(ssd.workspace_size(shape, T), dtype=torch.uint8, device="cuda")
    fplan = None if plan is None else ssd.make_plan(plan, 1, 1, 64)
    ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=T, initial_states=t["h0"],
                       workspace=fws, keep_intermediates=True, plan=fplan)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dy)
    kw = dict(chunk_size=T, initial_states=t["h0"], d_final_states=dfin)
    saved = ssd.chunk_scan_bwd(*args, **kw, saved_workspace=fws)
    plain = ssd.chunk_scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    got = {k: v.double().cpu().numpy() for k, v in saved.items()}
    ref = oracle.scan_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                          cot["dy"], cot["dfinal"])
    ref["d_initial_states"] = ref.pop("dh0")
    _check(got, ref, dtype, str(case))
    # the same states give the same gradients; the fused launch's states
    # differ from the split path's in rounding only
    for k in plain:
        a, e = saved[k].double(), plain[k].double()
        scale = max(float(e.pow(2).mean().sqrt()), 1e-30)
        d = float((a - e).abs().max()) / scale
        assert d <= (1e-3 if plan == "fused" else 1e-6), (k, d)


def test_backward_saved_with_stage_events():
    # the saved-states call with a (start, stop) event pair per stage: the
    # same gradients as without events; the two stages it skips record their
    # pairs back to back
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(2 * len(ssd.BWD_STAGES)):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h.value)
    w = si.small(dtype="bf16", batch=1, seqlen=600, nheads=4, headdim=64, dstate=128, ngroups=1, chunk_size=256,
                 dt_mu=-1.0, init_std=0.1, seed=2411)
    inp = si.generate(w)
    cot = si.cotangents(w)
    t = to_device(inp, "bf16")
    dy = torch.from_numpy(cot["dy"]).cuda().to(torch.bfloat16)
    dfin = torch.from_numpy(cot["dfinal"]).cuda()
    shape = ssd.make_shape(1, 600, 4, 64, 128, 1, "bf16", True)
    fws = torch.empty(ssd.workspace_size(shape, 256), dtype=torch.uint8, device="cuda")
    ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=256, initial_states=t["h0"],
                       workspace=fws, keep_intermediates=True)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dy)
    kw = dict(chunk_size=256, initial_states=t["h0"], d_final_states=dfin, saved_workspace=fws)
    plain = ssd.chunk_scan_bwd(*args, **kw)
    timed = ssd.chunk_scan_bwd(*args, **kw, events=evs)
    torch.cuda.synchronize()
    try:
        for k in plain:
            assert torch.equal(plain[k], timed[k]), k
        ms = []
        for i in range(len(ssd.BWD_STAGES)):
            m = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(m), evs[2 * i], evs[2 * i + 1]) == 0
            ms.append(m.value)
        assert all(v >= 0 for v in ms), ms
        assert ms[1] < 0.05 and ms[2] < 0.05, ms  # skipped: back-to-back records
    finally:
        for e in evs:
            hip.hipEventDestroy(e)

"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Every comparison uses max |gpu - oracle| / rms(oracle) with the north-star
bounds: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32 accumulation).  The
same seeded inputs feed both sides; bf16 inputs are rounded once on the host
and the oracle widens those exact bits.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_chunked_ssd_amd as ssd
import oracle
import ssd_inputs as si
from tests.gpu_util import LOG2E, TOL, nerr, run, to_device

pytestmark = pytest.mark.gpu


def _oracle_all(inp, T):
    y, fin, ck = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                             ckpt_stride=T)
    return y, fin, ck


# (batch, seqlen, nheads, headdim, dstate, ngroups, chunk): several tiles and a
# ragged tail in most cases, every supported chunk size and headdim, odd
# multiples of 16 in dstate, ngroups in {1, 2, nheads}, L = 1 and L < chunk.
STAGE_SHAPES = [
    (2, 300, 4, 64, 128, 1, 64),
    (1, 700, 6, 32, 64, 2, 256),
    (1, 520, 4, 128, 256, 4, 128),
    (2, 200, 2, 64, 16, 1, 64),
    (1, 389, 3, 64, 48, 1, 128),
    (1, 1, 2, 32, 32, 1, 64),
    (1, 100, 2, 64, 128, 1, 256),
    (1, 512, 2, 64, 256, 2, 256),
    (2, 130, 4, 128, 80, 2, 64),
    (1, 600, 8, 64, 128, 1, 128),
    (2, 1000, 6, 64, 128, 2, 256),
    # chunk 256 with dstate > 128 or headdim 128: the chunk output re-reads C
    # per head and copies h_c asynchronously; ragged tails, dstate not a
    # multiple of 32
    (1, 389, 3, 64, 144, 1, 256),
    (1, 700, 2, 32, 256, 1, 256),
    (1, 300, 2, 128, 96, 1, 256),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shp", STAGE_SHAPES, ids=lambda s: "b%d_L%d_h%d_p%d_n%d_g%d_T%d" % s)
def test_stage_parity(dtype, shp):
    b, L, nh, p, n, g, T = shp
    w = si.small(dtype=dtype, batch=b, seqlen=L, nheads=nh, headdim=p, dstate=n, ngroups=g,
                 chunk_size=T, dt_mu=-1.0, init_std=0.1, seed=sum(shp))
    inp = si.generate(w)
    print("case", dtype, shp, flush=True)
    out = run(inp, dtype, T, keep=True)
    tol = TOL[dtype]
    # stage 1: G2 = log2(e) * per-chunk cumsum of A dt; DT = dt
    G = oracle.chunk_cumsum(inp["dt"], inp["A"], T)
    assert nerr(out["G2"] / LOG2E, G) < 1e-9
    nc = -(-L // T)
    dtp = np.zeros((b, nc * T, nh))
    dtp[:, :L] = inp["dt"]
    assert np.array_equal(out["DT"], dtp.transpose(0, 2, 1))
    # chunk-state weights exp(G_last - G_t) dt_t (fp64 exponent, fp32 exp2)
    Wref = oracle.chunk_state_weights(inp["dt"], inp["A"], T)
    assert nerr(out["W"], Wref) < 1e-5, ("W", nerr(out["W"], Wref))
    # C B^T tiles (bf16, headdim 64, dstate 128): fp32 sums of exact bf16
    # products, lower block triangle (blocks past the diagonal are zero).
    # Bound per entry: n fp32 additions, |err| <= n 2^-24 sum_k |C_ik B_jk|.
    if dtype == "bf16" and p == 64 and n == 128:
        blk = np.arange(T) // 16
        lower = (blk[:, None] >= blk[None, :])
        cb = oracle.chunk_cb(inp["B"], inp["C"], T) * lower
        bound = n * 2.0 ** -24 * oracle.chunk_cb(np.abs(inp["B"]), np.abs(inp["C"]), T) * lower
        assert np.all(np.abs(out["CB"] - cb) <= bound), ("CB", nerr(out["CB"], cb))
    else:
        assert "CB" not in out
    # stage 2: per-chunk input states
    S = oracle.chunk_states(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], T)
    assert nerr(out["S"], S) < tol, ("S", nerr(out["S"], S))
    # stage 3: chunk-start states and final state
    y_ref, fin_ref, ck = _oracle_all(inp, T)
    assert nerr(out["H"], ck) < tol, ("H", nerr(out["H"], ck))
    assert nerr(out["final"], fin_ref) < tol, ("final", nerr(out["final"], fin_ref))
    # stage 4: output
    ey = nerr(out["y"], y_ref)
    print("  y err %.3e  final err %.3e" % (ey, nerr(out["final"], fin_ref)))
    assert ey < tol, ("y", ey)


def test_tiny_workload_full_parity():
    w = si.WORKLOADS[0]
    inp = si.generate(w)
    out = run(inp, w.dtype, w.chunk_size)
    y_ref, fin_ref, _ = _oracle_all(inp, w.chunk_size)
    assert nerr(out["y"], y_ref) < TOL["f32"]
    assert nerr(out["final"], fin_ref) < TOL["f32"]


def _sample_units(w, k=3, seed=0):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (w.batch - 1, w.nheads - 1)}
    while len(units) < k:
        units.add((int(rng.integers(w.batch)), int(rng.integers(w.nheads))))
    return sorted(units)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_full_size_sampled(k):
    """Full-size workload in the launch configuration the benchmark times;
    the oracle recomputes sampled (batch, head) units one by one."""
    w = si.WORKLOADS[k]
    print("workload", w.name, flush=True)
    inp = si.generate(w)
    t = to_device(inp, w.dtype)
    y, fin = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                chunk_size=w.chunk_size, initial_states=t["h0"],
                                return_final_states=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool(torch.isfinite(fin).all())
    hpg = w.nheads // w.ngroups
    for bi, h in _sample_units(w):
        g = h // hpg
        sl = lambda a: a[bi:bi + 1, :, h:h + 1]  # noqa: E731
        h0 = None if inp["h0"] is None else inp["h0"][bi:bi + 1, h:h + 1]
        yr, fr, _ = oracle.scan(sl(inp["x"]), sl(inp["dt"]), inp["A"][h:h + 1],
                                inp["B"][bi:bi + 1, :, g:g + 1], inp["C"][bi:bi + 1, :, g:g + 1],
                                inp["D"][h:h + 1], h0)
        yg = y[bi, :, h].double().cpu().numpy()
        fg = fin[bi, h].double().cpu().numpy()
        ey, ef = nerr(yg, yr[0, :, 0]), nerr(fg, fr[0, 0])
        print("  unit b=%d h=%d: y err %.3e final err %.3e" % (bi, h, ey, ef))
        assert ey < TOL[w.dtype] and ef < TOL[w.dtype]


@pytest.mark.parametrize("T", [64, 256])
def test_bf16_y_output_is_rounded_result(T):
    """A bf16 y is the fp32 result rounded once: per element within the bf16
    unit roundoff 2^-8 (8 significant bits) of |y| plus the fp32 path's own
    error, bounded here by 1e-3 rms(y)."""
    w = si.small(dtype="bf16", batch=2, seqlen=600, nheads=4, headdim=64, dstate=128, ngroups=1,
                 chunk_size=T, dt_mu=-2.0, init_std=0.1, seed=11)
    inp = si.generate(w)
    out = run(inp, "bf16", T, y_dtype="bf16")
    y_ref, fin_ref, _ = _oracle_all(inp, T)
    rms = np.sqrt(np.mean(y_ref ** 2))
    bound = 2.0 ** -8 * np.abs(y_ref) + 1e-3 * rms
    assert np.all(np.abs(out["y"] - y_ref) <= bound)
    assert np.all(np.abs(out["y"]) == np.abs(si.round_bf16(out["y"].astype(np.float32))))
    assert nerr(out["final"], fin_ref) < TOL["bf16"]


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _inputs(dtype="f32", **kw):
    d = dict(batch=1, seqlen=300, nheads=4, headdim=64, dstate=64, ngroups=2, chunk_size=64,
             init_std=0.1, seed=5)
    d.update(kw)
    w = si.small(dtype=dtype, **d)
    return w, si.generate(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dt_zero_keeps_state(dtype):
    w, inp = _inputs(dtype)
    inp["dt"] = np.zeros_like(inp["dt"])
    out = run(inp, dtype, 64)
    y_ref, fin_ref, _ = _oracle_all(inp, 64)
    assert np.array_equal(out["final"], inp["h0"].astype(np.float64))
    assert nerr(out["y"], y_ref) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_huge_decay_no_nan(dtype):
    w, inp = _inputs(dtype, chunk_size=128, seqlen=500)
    inp["A"] = np.full_like(inp["A"], -1e4)
    out = run(inp, dtype, 128)
    assert np.all(np.isfinite(out["y"])) and np.all(np.isfinite(out["final"]))
    y_ref, fin_ref, _ = _oracle_all(inp, 128)
    assert nerr(out["y"], y_ref) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("a_max", [0.0, 1e-3])
def test_slow_decay_long_carry(dtype, a_max):
    # many chunks with almost no decay: the carried state dominates y
    w, inp = _inputs(dtype, seqlen=2048, chunk_size=64, nheads=4, ngroups=1)
    inp["A"] = (-np.linspace(0.0, a_max, 4)).astype(np.float32)
    out = run(inp, dtype, 64)
    y_ref, fin_ref, _ = _oracle_all(inp, 64)
    assert nerr(out["y"], y_ref) < TOL[dtype]
    assert nerr(out["final"], fin_ref) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_chunk_size_same_inputs(dtype):
    w, inp = _inputs(dtype, seqlen=777)
    y_ref, fin_ref, _ = _oracle_all(inp, 64)
    for T in (64, 128, 256):
        out = run(inp, dtype, T)
        assert nerr(out["y"], y_ref) < TOL[dtype], T
        assert nerr(out["final"], fin_ref) < TOL[dtype], T


def test_initial_states_aliased_with_final():
    w, inp = _inputs("f32")
    t = to_device(inp, "f32")
    y_ref, fin_ref, _ = _oracle_all(inp, 64)
    h = t["h0"]
    y, fin = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=64,
                                initial_states=h, final_out=h, return_final_states=True)
    torch.cuda.synchronize()
    assert fin.data_ptr() == h.data_ptr()
    assert nerr(fin.double().cpu().numpy(), fin_ref) < TOL["f32"]
    assert nerr(y.double().cpu().numpy(), y_ref) < TOL["f32"]


def test_empty_sequence_returns_initial_state():
    w, inp = _inputs("f32", seqlen=0)
    out = run(inp, "f32", 64)
    assert out["y"].shape[1] == 0
    assert np.array_equal(out["final"], inp["h0"].astype(np.float64))


def test_no_initial_state_and_no_skip():
    w, inp = _inputs("bf16", init_std=0.0)
    inp["D"] = None
    out = run(inp, "bf16", 64)
    y_ref, fin_ref, _ = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"])
    assert nerr(out["y"], y_ref) < TOL["bf16"]
    assert nerr(out["final"], fin_ref) < TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_continuity(dtype):
    # run(0..L1) then run(L1..L, init = final) matches run(0..L)
    w, inp = _inputs(dtype, seqlen=640, chunk_size=128)
    full = run(inp, dtype, 128)
    L1 = 333
    tok = ("x", "dt", "B", "C")
    a = {k: (v[:, :L1] if k in tok else v) for k, v in inp.items()}
    b = {k: (v[:, L1:] if k in tok else v) for k, v in inp.items()}
    ra = run(a, dtype, 128)
    b["h0"] = ra["final"].astype(np.float32)
    rb = run(b, dtype, 128)
    y2 = np.concatenate([ra["y"], rb["y"]], axis=1)
    assert nerr(y2, full["y"]) < TOL[dtype]
    assert nerr(rb["final"], full["final"]) < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bitwise_deterministic(dtype):
    w, inp = _inputs(dtype, seqlen=1000, nheads=8, ngroups=2, chunk_size=256)
    outs = [run(inp, dtype, 256) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o["y"], outs[0]["y"]) and np.array_equal(o["final"], outs[0]["final"])


def test_group_expansion_matches():
    # ngroups = 2 equals ngroups = nheads with B/C repeated per head
    w, inp = _inputs("bf16", nheads=6, ngroups=2, seqlen=400)
    a = run(inp, "bf16", 64)
    ex = dict(inp)
    ex["B"] = np.repeat(inp["B"], 3, axis=2)
    ex["C"] = np.repeat(inp["C"], 3, axis=2)
    b = run(ex, "bf16", 64)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["final"], b["final"])


def test_invalid_arguments_raise_before_launch():
    w, inp = _inputs("f32")
    t = to_device(inp, "f32")
    flat = torch.empty(t["x"].numel() + 1, dtype=torch.float32, device="cuda")
    xm = flat[1:].view(t["x"].shape)  # 4-byte offset: misaligned for 16-byte loads
    with pytest.raises(ssd.SSDError) as ei:
        ssd.chunk_scan_fwd(xm, t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=64)
    assert ei.value.status == 3
    with pytest.raises(ssd.SSDError) as ei:
        ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=96)
    assert ei.value.status == 2
    with pytest.raises(ssd.SSDError) as ei:
        ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=64,
                           workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == 4

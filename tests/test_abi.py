"""The C ABI on the CPU: exports, workspace arithmetic and argument checks.

No kernel runs here.  The argument-check tests pass fake (never dereferenced)
device addresses to calls that validation must reject before any HIP call;
they are skipped when a GPU is visible, so that a validation bug can never turn
one of them into a real launch.
"""
import ctypes
import os
import re
import subprocess

import pytest

import mamba_chunked_ssd_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        from mamba_chunked_ssd_amd import build
        build.build()
    return ssd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert declared_functions() == sorted(ssd.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ssd_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        ssd.load_library(str(tmp_path / "libssd.so"))


def test_stage_launches(lib):
    # every stage launches its own kernel when there are tokens (split state
    # path); under the fused state path the chunk-state launch also carries
    # the state, and the state-passing stage launches nothing
    # (8 x 4096 tokens: the fused path is the default; the 2.7B-shaped
    # layer, one to two fused blocks per CU: the split path)
    s = ssd.make_shape(8, 4096, 80, 64, 128, 1, "bf16")
    assert ssd.default_plan(s, 256).state_path == ssd.SSD_STATE_FUSED
    assert ssd.stage_launches(s, 256) == ("chunk_cumsum", "chunk_state", "chunk_out")
    s = ssd.make_shape(2, 2048, 80, 64, 128, 1, "bf16")
    assert ssd.default_plan(s, 256).state_path == ssd.SSD_STATE_SPLIT
    assert ssd.stage_launches(s, 256) == ssd.STAGES
    assert ssd.stage_launches(s, 256, ssd.make_plan("split", 5, 5)) == ssd.STAGES
    assert ssd.stage_launches(s, 256, ssd.make_plan("fused", 5, 5, 32)) == (
        "chunk_cumsum", "chunk_state", "chunk_out")
    s = ssd.make_shape(4, 16384, 64, 128, 256, 8, "f32")
    assert ssd.stage_launches(s, 128) == ssd.STAGES
    s = ssd.make_shape(1, 65536, 32, 64, 256, 1, "bf16")
    assert ssd.stage_launches(s, 256) == ssd.STAGES
    # no tokens: only the state pass (initial state to final state) runs,
    # whichever the state path
    s = ssd.make_shape(2, 0, 4, 64, 128, 1, "bf16")
    assert ssd.stage_launches(s, 256) == ("state_pass",)
    assert ssd.stage_launches(s, 256, ssd.make_plan("fused", 1, 1, 64)) == ("state_pass",)
    s = ssd.make_shape(0, 100, 4, 64, 128, 1, "bf16")
    assert ssd.stage_launches(s, 256) == ()
    m = ctypes.c_uint32()
    assert lib.ssd_chunk_scan_fwd_stage_launches(ctypes.byref(s), 256, None, None) == 1
    assert lib.ssd_chunk_scan_fwd_stage_launches(ctypes.byref(s), 96, None, ctypes.byref(m)) != 0


def test_status_strings(lib):
    assert lib.ssd_status_string(0) == b"ok"
    for code in range(1, 7):
        assert len(lib.ssd_status_string(code)) > 10
    assert lib.ssd_version() == 200


def shape(**kw):
    d = dict(batch=2, seqlen=1000, nheads=8, headdim=64, dstate=128, ngroups=2, dtype="bf16",
             y_dtype="f32")
    d.update(kw)
    keep = d.pop("keep", False)
    return ssd.make_shape(d["batch"], d["seqlen"], d["nheads"], d["headdim"], d["dstate"],
                          d["ngroups"], d["dtype"], keep, d["y_dtype"])


def test_workspace_size_formula(lib):
    for T, keep, dt in [(T, k, d) for T in (64, 128, 256) for k in (False, True) for d in ("bf16", "f32")]:
        if True:
            s = shape(keep=keep, dtype=dt)
            nc = -(-1000 // T)
            seq = 4 * 2 * 8 * nc * T
            st = 4 * 2 * 8 * nc * 64 * 128
            up = lambda v: (v + 255) // 256 * 256  # noqa: E731
            own_h = keep or dt == "bf16"  # bf16 h_c is stored split, never over s_c
            # bf16 with headdim 64, dstate 128: C B^T tiles per (batch, chunk, group),
            # T/32 x (T/16 + 2) tiles of 1 KiB
            cb = 2 * nc * 2 * (T // 32) * (T // 16 + 2) * 1024 if dt == "bf16" else 0
            want = up(seq) * 4 + up(st) * (2 if own_h else 1) + up(cb)
            assert ssd.workspace_size(s, T) == want
            lay = ssd.workspace_layout(s, T)
            assert lay.total == want and lay.nchunks == nc and lay.padded_len == nc * T
            offs = [lay.g2_hi, lay.g2_lo, lay.dt, lay.w, lay.s, lay.h, lay.cb]
            assert all(o % 256 == 0 for o in offs)
            assert lay.g2_hi == 0 and lay.g2_lo == up(seq) and lay.dt == 2 * up(seq)
            assert lay.w == 3 * up(seq) and lay.s == 4 * up(seq)
            assert (lay.h == lay.s) != own_h
            assert lay.cb == want - up(cb)
    # no tiles for other head / state sizes; dstate 256 has them at chunk 256 only
    for kw, T in ((dict(headdim=32), 256), (dict(dstate=64), 256), (dict(dstate=256), 128),
                  (dict(dstate=256, dtype="f32"), 256)):
        lay = ssd.workspace_layout(shape(**kw), T)
        assert lay.cb == lay.total
    lay = ssd.workspace_layout(shape(dstate=256), 256)
    nc = -(-1000 // 256)
    assert lay.total - lay.cb == (2 * nc * 2 * 8 * 18 * 1024 + 255) // 256 * 256


@pytest.mark.parametrize("bad", [
    dict(nheads=6, ngroups=4),       # nheads % ngroups != 0
    dict(batch=-1), dict(seqlen=-5), dict(nheads=0), dict(ngroups=0),
])
def test_workspace_size_invalid_is_zero(lib, bad):
    assert ssd.workspace_size(shape(**bad), 256) == 0


def test_y_dtype_rules(lib):
    # y is fp32 or the input type; reserved must be 0
    assert ssd.workspace_size(shape(dtype="bf16", y_dtype="bf16"), 256) > 0
    assert ssd.workspace_size(shape(dtype="bf16", y_dtype="f32"), 256) > 0
    assert ssd.workspace_size(shape(dtype="f32", y_dtype="bf16"), 256) == 0
    s = shape()
    s.reserved = 1
    assert ssd.workspace_size(s, 256) == 0


@pytest.mark.parametrize("bad", [dict(headdim=48), dict(dstate=24), dict(dstate=272), dict(headdim=256)])
def test_unsupported_sizes(lib, bad):
    assert ssd.workspace_size(shape(**bad), 256) == 0
    lay = ssd.WorkspaceLayout()
    assert lib.ssd_chunk_scan_fwd_workspace_layout(ctypes.byref(shape(**bad)), 256, ctypes.byref(lay)) == 2


def test_y_chunk_offsets_must_fit_32_bits(lib):
    # one chunk's y rows of a head are addressed with 32-bit byte offsets
    # 256 x 16384 x 128 x 4 bytes = 2^31: one past the limit; half the chunk fits
    assert ssd.workspace_size(shape(nheads=8192, ngroups=1, headdim=128, seqlen=300), 256) > 0
    assert ssd.workspace_size(shape(nheads=16384, ngroups=1, headdim=128, seqlen=300), 256) == 0
    assert ssd.workspace_size(shape(nheads=16384, ngroups=1, headdim=128, seqlen=300), 128) > 0


def test_unsupported_chunk(lib):
    for T in (0, 32, 100, 512):
        assert ssd.workspace_size(shape(), T) == 0


# ---------------------------------------------------------------------------
# forward-call argument checks with fake device addresses (rejected before any
# HIP call)
# ---------------------------------------------------------------------------

GiB = 1 << 30


class Fake:
    """Disjoint, 256-byte aligned fake device addresses."""

    def __init__(self):
        self.base = 1 << 44

    def __call__(self, off=0):
        self.base += 64 * GiB
        return self.base + off


def call(lib, s, T=256, ws_bytes=None, **over):
    f = Fake()
    p = dict(x=f(), dt=f(), A=f(), B=f(), C=f(), D=f(), init=None, y=f(), fin=f(), ws=f())
    p.update(over)
    if ws_bytes is None:
        ws_bytes = max(ssd.workspace_size(s, T), 1)
    v = lambda a: None if a is None else ctypes.c_void_p(a)  # noqa: E731
    return lib.ssd_chunk_scan_fwd(ctypes.byref(s), v(p["x"]), v(p["dt"]), v(p["A"]), v(p["B"]),
                                  v(p["C"]), v(p["D"]), T, v(p["init"]), v(p["y"]), v(p["fin"]),
                                  v(p["ws"]), ws_bytes, None)


no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="fake device addresses are only passed where no GPU can be reached")


@no_gpu
def test_null_required_pointers(lib):
    for k in ("x", "dt", "A", "B", "C", "y"):
        assert call(lib, shape(), **{k: None}) == 1, k


@no_gpu
def test_null_shape_is_invalid(lib):
    assert lib.ssd_chunk_scan_fwd(None, *([None] * 6), 256, None, None, None, None, 0, None) == 1


@no_gpu
def test_bad_shapes(lib):
    assert call(lib, shape(nheads=6, ngroups=4)) == 1
    assert call(lib, shape(headdim=48)) == 2
    assert call(lib, shape(), T=100) == 2
    assert call(lib, shape(dtype="f32"), T=256, ws_bytes=1) == 4   # workspace too small


@no_gpu
def test_workspace_checks(lib):
    s = shape()
    need = ssd.workspace_size(s, 256)
    assert call(lib, s, ws_bytes=need - 1) == 4
    assert call(lib, s, ws=None) == 4


@no_gpu
def test_misaligned_pointers(lib):
    f = Fake()
    for k in ("x", "B", "C", "y"):
        assert call(lib, shape(), **{k: f() + 8}) == 3, k
    assert call(lib, shape(), fin=f() + 4) == 3
    assert call(lib, shape(), init=f() + 4) == 3
    assert call(lib, shape(), ws=f() + 128) == 3
    assert call(lib, shape(), A=f() + 2) == 3
    assert call(lib, shape(dtype="f32"), dt=f() + 2) == 3


@no_gpu
def test_aliasing_rejected(lib):
    f = Fake()
    x = f()
    assert call(lib, shape(), x=x, y=x) == 1                      # y over x
    assert call(lib, shape(), x=x, y=x + 1024 * 256) == 1         # partial overlap
    ws = f()
    assert call(lib, shape(), ws=ws, fin=ws) == 1                 # final over workspace
    assert call(lib, shape(), B=ws, ws=ws) == 1                   # workspace over input
    init = f()
    assert call(lib, shape(), init=init, fin=init + 256) == 1     # partial init/final overlap


def test_empty_batch_is_a_noop(lib):
    # batch == 0: nothing to compute, so no pointer is needed and nothing launches
    s = shape(batch=0)
    assert lib.ssd_chunk_scan_fwd(ctypes.byref(s), *([None] * 6), 256, None, None, None, None, 0, None) == 0


# ---------------------------------------------------------------------------
# launch plans (host only)
# ---------------------------------------------------------------------------

def test_default_plan_is_valid(lib):
    for s, T in [(ssd.make_shape(2, 2048, 80, 64, 128, 1, "bf16"), 256),
                 (ssd.make_shape(8, 4096, 80, 64, 128, 1, "bf16"), 256),
                 (ssd.make_shape(1, 65536, 32, 64, 256, 1, "bf16"), 256),
                 (ssd.make_shape(4, 16384, 64, 128, 256, 8, "f32"), 128),
                 (ssd.make_shape(1, 256, 4, 32, 16, 1, "f32"), 64)]:
        plan = ssd.default_plan(s, T)
        hpg = s.nheads // s.ngroups
        assert 1 <= plan.chunk_state_heads <= hpg and 1 <= plan.chunk_out_heads <= hpg
        assert plan.state_path in (ssd.SSD_STATE_SPLIT, ssd.SSD_STATE_FUSED)
        assert list(plan.reserved) == [0, 0, 0, 0]
        # the default plan and no plan launch the same stages
        assert ssd.stage_launches(s, T, plan) == ssd.stage_launches(s, T)


def test_default_plan_errors(lib):
    s = ssd.make_shape(2, 2048, 80, 64, 128, 1, "bf16")
    assert lib.ssd_chunk_scan_fwd_default_plan(ctypes.byref(s), 256, None) == 1
    plan = ssd.Plan()
    assert lib.ssd_chunk_scan_fwd_default_plan(ctypes.byref(s), 96, ctypes.byref(plan)) == 2
    assert lib.ssd_chunk_scan_fwd_default_plan(None, 256, ctypes.byref(plan)) == 1


@pytest.mark.parametrize("bad", [
    dict(chunk_state_heads=0), dict(chunk_out_heads=0), dict(chunk_state_heads=81),
    dict(chunk_out_heads=81), dict(state_path=2), dict(state_path=-1),
    dict(state_path=1, fused_cols=48), dict(state_path=1, fused_cols=256), dict(state_path=1, fused_cols=0),
])
def test_invalid_plans_rejected(lib, bad):
    s = ssd.make_shape(2, 2048, 80, 64, 128, 1, "bf16")
    plan = ssd.default_plan(s, 256)
    for k, v in bad.items():
        setattr(plan, k, v)
    m = ctypes.c_uint32()
    assert lib.ssd_chunk_scan_fwd_stage_launches(ctypes.byref(s), 256, ctypes.byref(plan),
                                                 ctypes.byref(m)) == 1


def test_plan_reserved_must_be_zero(lib):
    s = ssd.make_shape(2, 2048, 80, 64, 128, 1, "bf16")
    plan = ssd.default_plan(s, 256)
    plan.reserved[2] = 7
    m = ctypes.c_uint32()
    assert lib.ssd_chunk_scan_fwd_stage_launches(ctypes.byref(s), 256, ctypes.byref(plan),
                                                 ctypes.byref(m)) == 1


@no_gpu
def test_invalid_plan_rejected_before_launch(lib):
    s = shape()
    plan = ssd.default_plan(s, 256)
    plan.chunk_out_heads = 0
    f = Fake()
    v = lambda a: ctypes.c_void_p(a)  # noqa: E731
    st = lib.ssd_chunk_scan_fwd_ex(ctypes.byref(s), v(f()), v(f()), v(f()), v(f()), v(f()), v(f()), 256,
                                   None, v(f()), v(f()), v(f()), ssd.workspace_size(s, 256), None,
                                   ctypes.byref(plan), None)
    assert st == 1


@no_gpu
def test_noalloc_checks_before_any_device_access(lib):
    f = Fake()
    v = lambda a: ctypes.c_void_p(a)  # noqa: E731
    args = lambda: [v(f()), v(f()), v(f()), v(f()), v(f()), v(f())]  # noqa: E731
    # workspace beyond the 128 MiB scratch: rejected (the throughput workload needs ~0.7 GB)
    s = ssd.make_shape(8, 4096, 80, 64, 128, 1, "bf16")
    assert ssd.workspace_size(s, 256) > ssd.NOALLOC_SCRATCH_BYTES
    assert lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(s), *args(), 256, None, v(f()), v(f()), None) == 6
    # invalid and unsupported shapes report as the forward call does
    assert lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(shape(nheads=6, ngroups=4)), *args(), 256, None,
                                          v(f()), v(f()), None) == 1
    assert lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(shape()), *args(), 96, None, v(f()), v(f()),
                                          None) == 2
    assert lib.ssd_chunk_scan_fwd_noalloc(None, *args(), 256, None, v(f()), v(f()), None) == 1
    # the intermediates flag is refused (the scratch is not readable by the caller)
    assert lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(shape(keep=True)), *args(), 256, None, v(f()),
                                          v(f()), None) == 1
    # an empty batch touches no device
    assert lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(shape(batch=0)), *([None] * 6), 256, None, None,
                                          None, None) == 0


def test_fused_path_unsupported_for_fp32(lib):
    s = ssd.make_shape(4, 16384, 64, 128, 256, 8, "f32")
    m = ctypes.c_uint32()
    plan = ssd.make_plan("fused", 1, 1, 64)
    assert lib.ssd_chunk_scan_fwd_stage_launches(ctypes.byref(s), 128, ctypes.byref(plan),
                                                 ctypes.byref(m)) == 2


@no_gpu
def test_tune_rejects_before_any_device_work(lib):
    f = Fake()
    v = lambda a: ctypes.c_void_p(a)  # noqa: E731
    s = shape()
    plan = ssd.Plan()
    us = ctypes.c_float()

    def tune(T=256, init=None, fin=None, reps=5, best=True):
        fin = f() if fin is None else fin
        return lib.ssd_chunk_scan_fwd_tune(ctypes.byref(s), v(f()), v(f()), v(f()), v(f()), v(f()), v(f()), T,
                                           None if init is None else v(init), v(f()), v(fin), v(f()),
                                           ssd.workspace_size(s, 256), None, reps,
                                           ctypes.byref(plan) if best else None, ctypes.byref(us))
    assert tune(best=False) == 1
    assert tune(reps=0) == 1
    assert tune(reps=1001) == 1
    assert tune(T=96) == 2
    h = f()
    assert tune(init=h, fin=h) == 1   # the candidates would read each other's states


def bwd_call(lib, s, T=256, saved=True, fwd_bytes=None, ws_bytes=None, **over):
    """ssd_chunk_scan_bwd (saved=False) or ssd_chunk_scan_bwd_saved on fake
    addresses; returns the status."""
    f = Fake()
    p = dict(x=f(), dt=f(), A=f(), B=f(), C=f(), D=f(), init=None, dy=f(), dfin=None, fwd=f(),
             dx=f(), ddt=f(), dA=f(), dB=f(), dC=f(), dD=f(), dinit=None, ws=f())
    p.update(over)
    v = lambda k: None if p[k] is None else ctypes.c_void_p(p[k])  # noqa: E731
    keep = ssd.make_shape(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups,
                          "bf16" if s.dtype == 1 else "f32", True)
    fb = ssd.workspace_size(keep, T) if fwd_bytes is None else fwd_bytes
    wb = ssd.bwd_workspace_size(s, T) if ws_bytes is None else ws_bytes
    head = [ctypes.byref(s), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"), T, v("init"), v("dy"), v("dfin")]
    tail = [v("dx"), v("ddt"), v("dA"), v("dB"), v("dC"), v("dD"), v("dinit"), v("ws"), wb, None]
    if not saved:
        return lib.ssd_chunk_scan_bwd(*head, *tail)
    return lib.ssd_chunk_scan_bwd_saved(*head, v("fwd"), fb, *tail, None)


@no_gpu
def test_backward_rejects_before_launch(lib):
    s = shape()
    assert ssd.bwd_workspace_size(s, 256) > 0
    for k in ("x", "dt", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC"):
        assert bwd_call(lib, s, saved=False, **{k: None}) == 1, k
    assert bwd_call(lib, s, saved=False, ws_bytes=ssd.bwd_workspace_size(s, 256) - 1) == 4
    assert bwd_call(lib, s, saved=False, ws=None) == 4
    assert bwd_call(lib, s, saved=False, T=96) == 2
    assert bwd_call(lib, shape(keep=True), saved=False) == 1  # flags must be 0
    f = Fake()
    assert bwd_call(lib, s, saved=False, x=f(8)) == 3
    out = f()
    assert bwd_call(lib, s, saved=False, dB=out, dC=out) == 1  # outputs overlap


@no_gpu
def test_backward_with_saved_states_rejects_before_launch(lib):
    s = shape()
    keep = shape(keep=True)
    need = ssd.workspace_size(keep, 256)
    assert need > 0
    assert bwd_call(lib, s, fwd=None) == 1
    assert bwd_call(lib, s, fwd_bytes=need - 1) == 4
    # the size a forward call without the flag needs is not enough at fp32
    # (its H shares S's region there)
    s32, k32 = shape(dtype="f32"), shape(dtype="f32", keep=True)
    assert ssd.workspace_size(s32, 256) < ssd.workspace_size(k32, 256)
    assert bwd_call(lib, s32, fwd_bytes=ssd.workspace_size(s32, 256)) == 4
    f = Fake()
    assert bwd_call(lib, s, fwd=f(16)) == 3
    # the forward workspace is an input: it may not be an output or the workspace
    w = f()
    assert bwd_call(lib, s, fwd=w, ws=w) == 1
    # an output inside the forward workspace's H region
    h = f()
    assert bwd_call(lib, s, fwd=h, dx=h + ssd.workspace_layout(keep, 256).h) == 1
    assert bwd_call(lib, s, T=96) == 2
    assert bwd_call(lib, shape(nheads=6, ngroups=4)) == 1

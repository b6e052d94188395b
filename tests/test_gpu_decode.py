"""Parity of the recurrent decode step (ssd_decode_step, through the C ABI)
against the fp64 oracle: one step from a random state, chained steps against
the chunked forward pass and the oracle's scan, and the edge cases.

Bounds: max |gpu - oracle| / rms(oracle) <= 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs (fp32 state and arithmetic), as for the forward pass.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import mamba_chunked_ssd_amd as ssd
import oracle
import ssd_inputs as si
from tests.gpu_util import TOL, nerr, to_device

pytestmark = pytest.mark.gpu


def _step_inputs(dtype, b, nh, p, n, g, seed, state_std=0.5):
    # one token of a seeded workload, with a random state to start from
    w = si.small(dtype=dtype, batch=b, seqlen=1, nheads=nh, headdim=p, dstate=n, ngroups=g, chunk_size=64,
                 dt_mu=-1.0, init_std=state_std, seed=seed)
    inp = si.generate(w)
    return {"x": inp["x"][:, 0], "dt": inp["dt"][:, 0], "A": inp["A"], "B": inp["B"][:, 0],
            "C": inp["C"][:, 0], "D": inp["D"], "state": inp["h0"]}


def _dev(inp, dtype):
    t = to_device({k: v for k, v in inp.items() if k != "state"}, dtype)
    t["state"] = torch.from_numpy(np.ascontiguousarray(inp["state"], np.float32)).cuda()
    return t


# (batch, nheads, headdim, dstate, ngroups): every supported headdim, dstate
# from 16 to 256 including ones that are not powers of two, grouped heads,
# and the serving shape of the 2.7B-model layer (batch 128).
DECODE_SHAPES = [
    (4, 8, 64, 128, 1),
    (3, 6, 32, 48, 2),
    (2, 4, 128, 256, 4),
    (5, 3, 64, 16, 3),
    (1, 2, 32, 144, 1),
    (2, 16, 128, 80, 8),
    (128, 80, 64, 128, 1),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shp", DECODE_SHAPES, ids=lambda s: "b%d_h%d_p%d_n%d_g%d" % s)
def test_decode_step_parity(dtype, shp):
    b, nh, p, n, g = shp
    print("case", dtype, shp, flush=True)
    inp = _step_inputs(dtype, b, nh, p, n, g, seed=sum(shp))
    t = _dev(inp, dtype)
    y = ssd.decode_step(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["state"])
    torch.cuda.synchronize()
    yr, sr = oracle.decode_step(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["state"])
    ey = nerr(y.double().cpu().numpy(), yr)
    es = nerr(t["state"].double().cpu().numpy(), sr)
    print("  y err %.3e state err %.3e" % (ey, es))
    assert ey < TOL[dtype] and es < TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_chain_to_the_forward_pass(dtype):
    # K steps from an initial state reproduce the chunked forward pass over
    # the same K tokens (y per token and the final state), and the oracle
    w = si.small(dtype=dtype, batch=3, seqlen=40, nheads=6, headdim=64, dstate=64, ngroups=2, chunk_size=64,
                 dt_mu=-1.0, init_std=0.3, seed=91)
    inp = si.generate(w)
    t = to_device(inp, dtype)
    y_fwd, fin_fwd = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=64,
                                        initial_states=t["h0"], return_final_states=True)
    state = t["h0"].clone()
    ys = []
    for k in range(w.seqlen):
        ys.append(ssd.decode_step(t["x"][:, k].contiguous(), t["dt"][:, k].contiguous(), t["A"],
                                  t["B"][:, k].contiguous(), t["C"][:, k].contiguous(), t["D"], state))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=1).double().cpu().numpy()
    yr, fr, _ = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    assert nerr(y_dec, yr) < TOL[dtype] and nerr(state.double().cpu().numpy(), fr) < TOL[dtype]
    assert nerr(y_dec, y_fwd.double().cpu().numpy()) < TOL[dtype]
    assert nerr(state.double().cpu().numpy(), fin_fwd.double().cpu().numpy()) < TOL[dtype]


def test_decode_bf16_y_is_rounded_result():
    inp = _step_inputs("bf16", 8, 8, 64, 128, 1, seed=5)
    t = _dev(inp, "bf16")
    y = ssd.decode_step(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["state"], y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yr, _ = oracle.decode_step(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["state"])
    y = y.double().cpu().numpy()
    bound = 2.0 ** -8 * np.abs(yr) + 1e-4 * np.sqrt(np.mean(yr ** 2))
    assert np.all(np.abs(y - yr) <= bound)


def test_decode_without_skip_and_deterministic():
    inp = _step_inputs("f32", 4, 4, 32, 32, 2, seed=6)
    outs = []
    for _ in range(2):
        t = _dev(inp, "f32")
        y = ssd.decode_step(t["x"], t["dt"], t["A"], t["B"], t["C"], None, t["state"])
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), t["state"].cpu().numpy()))
    yr, sr = oracle.decode_step(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None, inp["state"])
    assert nerr(outs[0][0], yr) < TOL["f32"] and nerr(outs[0][1], sr) < TOL["f32"]
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_decode_rejects_before_launch():
    inp = _step_inputs("f32", 2, 4, 64, 64, 1, seed=7)
    t = _dev(inp, "f32")
    before = t["state"].clone()
    lib = ssd.load_library()
    y = torch.zeros((2, 4, 64), dtype=torch.float32, device="cuda")
    p = lambda v: ctypes.c_void_p(v.data_ptr())  # noqa: E731
    for shape, want in [(ssd.make_shape(2, 2, 4, 64, 64, 1, "f32"), 1),    # seqlen 2
                        (ssd.make_shape(2, 1, 4, 48, 64, 1, "f32"), 2),    # headdim 48
                        (ssd.make_shape(2, 1, 4, 64, 64, 1, "f32", keep=True), 1)]:
        st = lib.ssd_decode_step(ctypes.byref(shape), p(t["x"]), p(t["dt"]), p(t["A"]), p(t["B"]), p(t["C"]),
                                 None, p(t["state"]), p(y), None, None)
        assert st == want
    shape = ssd.make_shape(2, 1, 4, 64, 64, 1, "f32")
    st = lib.ssd_decode_step(ctypes.byref(shape), p(t["x"]), p(t["dt"]), p(t["A"]), p(t["B"]), p(t["C"]),
                             None, p(t["state"]), p(t["state"]), None, None)   # y inside the state
    assert st == 1
    torch.cuda.synchronize()
    assert torch.equal(t["state"], before) and not bool(y.any())
    # an empty batch is a no-op
    shape = ssd.make_shape(0, 1, 4, 64, 64, 1, "f32")
    assert lib.ssd_decode_step(ctypes.byref(shape), None, None, None, None, None, None, None, None, None,
                               None) == 0

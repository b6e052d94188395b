"""The per-shape autotuner (ssd_chunk_scan_fwd_tune) on the GPU: the plan it
returns is valid, the outputs it leaves hold the forward pass's result, and
that plan reproduces them bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_chunked_ssd_amd as ssd
import oracle
import ssd_inputs as si
from tests.gpu_util import TOL, nerr, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,shp", [
    ("bf16", (2, 700, 12, 64, 128, 2, 256)),
    ("f32", (1, 520, 8, 128, 256, 4, 128)),
    ("bf16", (1, 389, 6, 32, 96, 1, 64)),
], ids=lambda v: v if isinstance(v, str) else "b%d_L%d_h%d_p%d_n%d_g%d_T%d" % v)
def test_tuned_plan_is_valid_and_its_result_correct(dtype, shp):
    b, L, nh, p, n, g, T = shp
    w = si.small(dtype=dtype, batch=b, seqlen=L, nheads=nh, headdim=p, dstate=n, ngroups=g, chunk_size=T,
                 dt_mu=-1.0, init_std=0.1, seed=sum(shp))
    inp = si.generate(w)
    t = to_device(inp, dtype)
    y = torch.empty((b, L, nh, p), dtype=torch.float32, device="cuda")
    fin = torch.empty((b, nh, p, n), dtype=torch.float32, device="cuda")
    plan, us = ssd.tune(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], T, t["h0"], reps=3, out=y,
                        final_out=fin)
    torch.cuda.synchronize()
    print("case", dtype, shp, plan, "%.1f us" % us, flush=True)
    hpg = nh // g
    assert us > 0 and 1 <= plan.chunk_out_heads <= hpg and 1 <= plan.chunk_state_heads <= hpg
    shape = ssd.make_shape(b, L, nh, p, n, g, dtype)
    assert ssd.stage_launches(shape, T, plan)  # a plan the library accepts
    yr, fr, _ = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    assert nerr(y.double().cpu().numpy(), yr) < TOL[dtype]
    assert nerr(fin.double().cpu().numpy(), fr) < TOL[dtype]
    y2, f2 = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=T,
                                initial_states=t["h0"], return_final_states=True, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(y2, y) and torch.equal(f2, fin)

"""The backward pass at the five workload shapes (the configurations the
forward is measured on).

* Full size, every workload: the three scaling identities of the recurrence
  (tests/pins.py, ``bpin_scaling_invariants``) hold for the GPU's gradients as
  computed, to a tolerance derived from the dtype -- a property of any size
  that ties dx, ddt, dA, dB, dC, dD and the initial state's gradient
  together, including the sums over heads and tokens that no per-head
  comparison reaches.
* Full size, sampled heads (2.7B layer, throughput): dx, ddt, dA, dD and the
  initial state's gradient of two heads of a group against the oracle run on
  that head alone (a head's own gradients depend only on its inputs and the
  group's B, C).
* The long-sequence and grouped shapes at a shorter sequence (the oracle
  keeps every state of a head in memory): every gradient, every element.

Bound on max |gpu - oracle| / rms(oracle): 1e-4 for fp32 inputs, 2e-2 for bf16.
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

# relative residual of the identities: fp32 accumulation over the tensors
ID_TOL = {"f32": 1e-4, "bf16": 1e-3}


def _gpu_bwd(w, inp, cot):
    t = to_device(inp, w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dy = torch.from_numpy(cot["dy"]).cuda().to(tdt)
    dfin = torch.from_numpy(cot["dfinal"]).cuda()
    y, fin = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=w.chunk_size,
                                initial_states=t["h0"], return_final_states=True)
    g = ssd.chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dy, chunk_size=w.chunk_size,
                           initial_states=t["h0"], d_final_states=dfin)
    torch.cuda.synchronize()
    del y, t
    return g, fin


def _dot(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b), float(np.abs(a) @ np.abs(b))


@pytest.mark.parametrize("name", [w.name for w in si.WORKLOADS])
def test_backward_scaling_identities_full_size(name):
    w = si.BY_NAME[name]
    print("identities", name, flush=True)
    inp = si.generate(w)
    cot = si.cotangents(w)
    g, fin = _gpu_bwd(w, inp, cot)
    gd = {k: v.cpu().numpy() for k, v in g.items()}
    fin = fin.cpu().numpy()
    h0 = inp["h0"] if inp["h0"] is not None else np.zeros_like(cot["dfinal"])
    terms = {
        "dt-A-B": [_dot(inp["dt"], gd["ddt"]), _dot(inp["A"], gd["dA"]), _dot(inp["B"], gd["dB"])],
        "x-B-D": [_dot(inp["x"], gd["dx"]), _dot(inp["B"], gd["dB"]), _dot(inp["D"], gd["dD"])],
        "C-B-h0": [_dot(inp["C"], gd["dC"]), _dot(inp["B"], gd["dB"]), _dot(h0, gd["d_initial_states"]),
                   _dot(cot["dfinal"], fin)],
    }
    signs = {"dt-A-B": [1, -1, -1], "x-B-D": [1, -1, -1], "C-B-h0": [1, -1, -1, 1]}
    for k, ts in terms.items():
        val = sum(s * v for s, (v, _) in zip(signs[k], ts))
        scale = sum(m for _, m in ts)
        assert abs(val) <= ID_TOL[w.dtype] * scale, (name, k, val, scale)


@pytest.mark.parametrize("name", ["mamba2_2p7b_layer_bf16", "throughput_bf16"])
def test_backward_sampled_heads_full_size(name):
    w = si.BY_NAME[name]
    print("sampled heads", name, flush=True)
    inp = si.generate(w)
    cot = si.cotangents(w)
    g, _ = _gpu_bwd(w, inp, cot)
    hpg = w.nheads // w.ngroups
    for h in (0, hpg - 1):
        gi = h // hpg
        sl = slice(h, h + 1)
        ref = oracle.scan_bwd(inp["x"][:, :, sl], inp["dt"][:, :, sl], inp["A"][sl], inp["B"][:, :, gi:gi + 1],
                              inp["C"][:, :, gi:gi + 1], inp["D"][sl],
                              None if inp["h0"] is None else inp["h0"][:, sl], cot["dy"][:, :, sl],
                              cot["dfinal"][:, sl])
        pairs = {"dx": (g["dx"][:, :, sl], ref["dx"]), "ddt": (g["ddt"][:, :, sl], ref["ddt"]),
                 "dA": (g["dA"][sl], ref["dA"]), "dD": (g["dD"][sl], ref["dD"]),
                 "d_initial_states": (g["d_initial_states"][:, sl], ref["dh0"])}
        for k, (a, r) in pairs.items():
            a = a.double().cpu().numpy()
            if k in ("dA", "dD"):  # one number: relative error
                err = abs(float(a[0]) - float(r[0])) / max(abs(float(r[0])), 1e-30)
            else:
                err = nerr(a, r)
            assert err <= TOL[w.dtype], (name, h, k, err)


@pytest.mark.parametrize("name,seqlen,batch", [("long_seq_bf16", 4096, 1), ("grouped_f32", 1024, 2)])
def test_backward_workload_shapes_shortened(name, seqlen, batch):
    w = si.BY_NAME[name].replace(seqlen=seqlen, batch=batch)
    print("shortened", w, flush=True)
    inp = si.generate(w)
    cot = si.cotangents(w)
    g, _ = _gpu_bwd(w, inp, cot)
    ref = oracle.scan_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], cot["dy"],
                          cot["dfinal"])
    ref["d_initial_states"] = ref.pop("dh0")
    for k in ref:
        err = nerr(g[k].double().cpu().numpy(), ref[k])
        assert err <= TOL[w.dtype], (name, k, err)

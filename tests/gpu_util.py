"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
read its intermediates back.  Nothing here computes the method."""
from __future__ import annotations

import numpy as np
import torch

import mamba_chunked_ssd_amd as ssd

LOG2E = 1.4426950408889634
# spec tolerance on max |err| / rms(ref)
TOL = {"f32": 1e-4, "bf16": 2e-2}


def nerr(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    if a.size == 0:
        return 0.0
    if not np.all(np.isfinite(a)):
        return float("inf")
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0.0:
        return float(np.max(np.abs(a - ref)))
    return float(np.max(np.abs(a - ref)) / rms)


def to_device(inp: dict, dtype: str, dev="cuda"):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)
        out[k] = t.to(tdt) if k in ("x", "dt", "B", "C") else t
    return out


def run(inp: dict, dtype: str, chunk: int, keep: bool = False, final: bool = True,
        y_dtype: str = "f32", plan=None):
    """Forward pass (under ``plan``, None = the default plan); returns numpy
    fp64 dict with y, final and (keep) G2/DT/W/S/H (G2 = the stored hi + lo
    pair, summed in fp64).  S is absent when the plan fuses the state stages
    (the fused launch never writes s_c)."""
    t = to_device(inp, dtype)
    b, L, nh, p = t["x"].shape
    g, n = t["B"].shape[2], t["B"].shape[3]
    ws = None
    lay = None
    shape = ssd.make_shape(b, L, nh, p, n, g, dtype, keep=keep, y_dtype=y_dtype)
    eff = plan if plan is not None else ssd.default_plan(shape, chunk)
    if keep:
        lay = ssd.workspace_layout(shape, chunk)
        ws = torch.empty(max(lay.total, 1), dtype=torch.uint8, device="cuda")
    res = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=chunk,
                             initial_states=t["h0"], return_final_states=final, workspace=ws,
                             keep_intermediates=keep, plan=plan,
                             y_dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32)
    torch.cuda.synchronize()
    if final:
        y, fin = res
    else:
        y, fin = res, None
    out = {"y": y.double().cpu().numpy(), "final": None if fin is None else fin.double().cpu().numpy(),
           "plan": eff}
    if keep:
        nc, Lp = lay.nchunks, lay.padded_len

        def view(off, shape):
            cnt = int(np.prod(shape))
            return ws[off: off + 4 * cnt].view(torch.float32).reshape(shape).double().cpu().numpy()

        out["G2"] = view(lay.g2_hi, (b, nh, Lp)) + view(lay.g2_lo, (b, nh, Lp))
        out["DT"] = view(lay.dt, (b, nh, Lp))
        out["W"] = view(lay.w, (b, nh, Lp))
        if eff.state_path != ssd.SSD_STATE_FUSED:
            out["S"] = view(lay.s, (b, nh, nc, p, n))
        if dtype == "bf16":
            # h_c as hi and lo bf16 planes per (batch, head, chunk)
            cnt = b * nh * nc * 2 * p * n
            hl = ws[lay.h: lay.h + 2 * cnt].view(torch.bfloat16).reshape(b, nh, nc, 2, p, n)
            hl = hl.double().cpu().numpy()
            out["H"] = hl[:, :, :, 0] + hl[:, :, :, 1]
        else:
            out["H"] = view(lay.h, (b, nh, nc, p, n))
        if lay.cb < lay.total:
            out["CB"] = decode_cb(view(lay.cb, (b, nc, g, chunk // 32, chunk // 16 + 2, 64, 4)), chunk)
    return out


def decode_cb(raw, T):
    """Dense (b, nchunks, g, T, T) C B^T from the tile layout of include/ssd.h
    (tiles past the diagonal must be zero and are checked here)."""
    b, nc, g = raw.shape[:3]
    nt = T // 16
    out = np.zeros((b, nc, g, T, T))
    lane = np.arange(64)
    m, q = lane % 16, lane // 16
    for w in range(T // 32):
        base1 = (w + 2) & ~1
        for k in range(nt + 2):
            I, J = (w, k) if k < base1 else (nt - 1 - w, k - base1)
            tile = raw[:, :, :, w, k]
            if J > I:
                assert not np.any(tile), "C B^T tile above the diagonal is not zero"
                continue
            for r in range(4):
                out[:, :, :, 16 * I + m, 16 * J + 4 * q + r] = tile[..., r]
    return out

"""ssd_chunk_scan_fwd_noalloc: the forward pass with the library's own device
scratch (for callers that cannot allocate), through the C ABI.

Its output must equal ssd_chunk_scan_fwd's (same kernels, same default plan,
so bit for bit) on calls in a row -- a large problem, then smaller ones that
find the scratch holding the previous call's intermediates -- and stay within
the oracle tolerance.  A problem whose workspace exceeds the scratch is
rejected before anything is enqueued.
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


def _noalloc(t, w, y, fin):
    lib = ssd.load_library()
    shape = ssd.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype)
    p = lambda v: None if v is None else ctypes.c_void_p(v.data_ptr())  # noqa: E731
    s = torch.cuda.current_stream().cuda_stream
    return lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(shape), p(t["x"]), p(t["dt"]), p(t["A"]),
                                          p(t["B"]), p(t["C"]), p(t["D"]), w.chunk_size,
                                          p(t["h0"]), p(y), p(fin), ctypes.c_void_p(s))


# a large problem first (the 2.7B-shaped layer: 91.5 MB of workspace), then
# smaller ones of other shapes and types
CALLS = [
    si.WORKLOADS[1],
    si.small(dtype="bf16", batch=1, seqlen=700, nheads=6, headdim=64, dstate=128, ngroups=1,
             chunk_size=256, dt_mu=-1.0, init_std=0.1, seed=21),
    si.small(dtype="f32", batch=2, seqlen=300, nheads=4, headdim=32, dstate=48, ngroups=2,
             chunk_size=64, dt_mu=-1.0, init_std=0.1, seed=22),
]


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    for i, w in enumerate(CALLS):
        print("call", i, w.name, (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                  w.chunk_size), w.dtype, flush=True)
        inp = si.generate(w)
        t = to_device(inp, w.dtype)
        ref_y, ref_fin = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                            chunk_size=w.chunk_size, initial_states=t["h0"],
                                            return_final_states=True)
        y = torch.full_like(ref_y, float("nan"))
        fin = torch.full_like(ref_fin, float("nan"))
        st = _noalloc(t, w, y, fin)
        torch.cuda.synchronize()
        assert st == 0, ssd.status_string(st)
        assert torch.equal(y, ref_y) and torch.equal(fin, ref_fin)
        if w.tokens <= 4096:
            yr, fr, _ = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                    inp["h0"])
            ey = nerr(y.double().cpu().numpy(), yr)
            ef = nerr(fin.double().cpu().numpy(), fr)
            print("  y err %.3e final err %.3e" % (ey, ef), flush=True)
            assert ey < TOL[w.dtype] and ef < TOL[w.dtype]


def test_noalloc_rejects_problems_beyond_its_scratch():
    w = si.WORKLOADS[2]  # throughput workload: ~700 MB of workspace
    shape = ssd.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype)
    assert ssd.workspace_size(shape, w.chunk_size) > ssd.NOALLOC_SCRATCH_BYTES
    small = si.small(dtype="bf16", batch=1, seqlen=64, nheads=2, headdim=32, dstate=16,
                     chunk_size=64, seed=3)
    t = to_device(si.generate(small), "bf16")
    y = torch.zeros((1, 64, 2, 32), dtype=torch.float32, device="cuda")
    # the shape is checked before any pointer is used or anything is enqueued
    lib = ssd.load_library()
    p = lambda v: ctypes.c_void_p(v.data_ptr())  # noqa: E731
    st = lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(shape), p(t["x"]), p(t["dt"]), p(t["A"]),
                                        p(t["B"]), p(t["C"]), None, w.chunk_size, None, p(y), None,
                                        None)
    assert st == 6
    torch.cuda.synchronize()
    assert not bool(y.any())

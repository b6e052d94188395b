"""The seeded input generator: determinism, distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

import ssd_inputs as si


def test_workload_table():
    shapes = [(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size, w.dtype)
              for w in si.WORKLOADS]
    assert shapes == [
        (1, 256, 4, 32, 16, 1, 64, "f32"),
        (2, 2048, 80, 64, 128, 1, 256, "bf16"),
        (8, 4096, 80, 64, 128, 1, 256, "bf16"),
        (1, 65536, 32, 64, 256, 1, 256, "bf16"),
        (4, 16384, 64, 128, 256, 8, 128, "f32"),
    ]


def test_generation_is_deterministic():
    w = si.small(dtype="bf16", seqlen=50, init_std=0.1)
    a, b = si.generate(w), si.generate(w)
    for k in a:
        assert (a[k] is None) == (b[k] is None)
        if a[k] is not None:
            assert a[k].tobytes() == b[k].tobytes()
    c = si.generate(w, seed=w.seed + 1)
    assert c["x"].tobytes() != a["x"].tobytes()


def test_distributions_tiny():
    inp = si.generate(si.WORKLOADS[0])
    assert inp["h0"] is None
    assert np.all(inp["dt"] > 0)
    assert np.all((inp["A"] <= -1.0 + 1e-6) & (inp["A"] >= -16.0 - 1e-5))
    assert inp["x"].dtype == np.float32 and inp["x"].shape == (1, 256, 4, 32)


def test_dt_floor_mask_fraction():
    w = si.WORKLOADS[4].replace(batch=1, seqlen=2048)
    inp = si.generate(w)
    frac = np.mean(inp["dt"] == np.float32(1e-4))
    assert 0.08 < frac < 0.12


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0,
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-42], np.float32),
        # exact ties: bf16 value plus half an ulp, both parities
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ours = si.round_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    nan = si.round_bf16(np.array([np.nan], np.float32))
    assert np.isnan(nan[0])


def test_bf16_inputs_are_representable():
    w = si.small(dtype="bf16", seqlen=40)
    inp = si.generate(w)
    for k in ("x", "dt", "B", "C"):
        assert np.array_equal(si.round_bf16(inp[k]), inp[k])
        assert np.all((inp[k].view(np.uint32) & 0xFFFF) == 0)

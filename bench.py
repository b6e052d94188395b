#!/usr/bin/env python3
"""Benchmark of the Mamba-2 chunked SSD forward pass (libssd) on one MI355X.

A step is one full ``ssd_chunk_scan_fwd`` call -- all four stages (chunk
cumsum, chunk state, state passing, chunk output) -- over one batch of seeded
synthetic input already resident in HBM.  The default workload is the
Mamba-2 2.7B-shaped layer (batch 2, seqlen 2048, 80 heads, headdim 64,
dstate 128, 1 group, chunk 256, bf16 inputs, fp32 accumulation and fp32 y).

Prints ONE JSON line: tokens/s over K back-to-back steps (nothing else on the
stream), per-stage kernel times from a second run of K steps in which every
kernel's dispatch records a (start, stop) HIP event pair, the roofline of the
dominant kernel, and the fp64 CPU oracle timed on this host as a reference
baseline.  Beside the forward's figures the line carries the recurrent decode
step ("decode") and the backward pass ("backward": ssd_chunk_scan_bwd on the
same workload with seeded upstream gradients, its stages and the roofline of
its slowest stage, and the same calls reading one forward call's kept
chunk-start states instead of recomputing them).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/s at 1 MI355X + % of min(HBM,MFMA) roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA
STAGES = ["chunk_cumsum", "chunk_state", "state_pass", "chunk_out"]

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch), scaled by what the same counters read for a plain 1 GiB copy
# (fetch x 2.0, write x 1.0).  Valid only for the kernel sources they were
# taken on, identified by a hash; any change to those sources reports null.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
MEASURED_TRAFFIC = {
    # (workload, y dtype, stage, state path): (sources, sha256[:16], FETCH KiB, WRITE KiB)
    ("mamba2_2p7b_layer_bf16", "f32", "chunk_out", "fused"): (
        ('k4_chunk_out.h', 'k4_out_bf16_f32.hip', 'ssd_device.h'), 'a6a4318efe91604f', 45009.5, 81957.0),
    ("mamba2_2p7b_layer_bf16", "f32", "chunk_out", "split"): (
        ('k4_chunk_out.h', 'k4_out_bf16_f32.hip', 'ssd_device.h'), 'a6a4318efe91604f', 45009.5, 81958.0),
    ("mamba2_2p7b_layer_bf16", "f32", "chunk_state", "fused"): (
        ('k23_state_fused.hip', 'k_cb_tiles.h', 'ssd_device.h'), '9fcae62bce07bffa', 24185.4, 48387.9),
    ("grouped_f32", "f32", "chunk_out", "split"): (
        ('k4_chunk_out.h', 'k4_out_f32.hip', 'ssd_device.h'), '4ceaad19d8c20f43', 5792109.0, 2097153.0),
    ("long_seq_bf16", "f32", "chunk_out", "split"): (
        ('k4_chunk_out.h', 'k4_out_bf16_f32.hip', 'ssd_device.h'), 'a6a4318efe91604f', 453119.5, 596848.0),
    # backward (the y dtype and state path do not apply)
    ("mamba2_2p7b_layer_bf16", None, "bwd:dC_pass", None): (
        ('kb_pass.h', 'kb_pass_c.hip', 'kb_pass_inst.h', 'ssd_device.h', 'ssd_internal.h'), '6e517063a58e48e9', 85605.8, 50688.0),
}


def measured_traffic(workload: str, y_dtype: str, stage: str, plan: dict | None = None):
    """HBM bytes per launch of ``stage`` if counters exist for its current sources."""
    import hashlib
    key = (workload, None, stage, None) if stage.startswith("bwd:") else (
        workload, y_dtype, stage, (plan or {}).get("state_path", "split"))
    ent = MEASURED_TRAFFIC.get(key)
    if ent is None:
        return None
    files, digest, fetch_kib, write_kib = ent
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mamba_chunked_ssd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != digest:
        return None
    return int(round((fetch_kib * FETCH_SCALE + write_kib * WRITE_SCALE) * 1024))


# ---------------------------------------------------------------------------
# algorithmic bytes and MFMA flops per stage (what the method must move or
# compute; intermediates fp32; C B^T once per group; triangles with diagonal)
# ---------------------------------------------------------------------------
def stage_model(w, y_bytes: int, fused: bool = False) -> dict:
    e = 2 if w.dtype == "bf16" else 4
    B, L, NH, P, N, G, T = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    NC = -(-L // T)
    tok_h = B * L * NH
    states = 4 * B * NH * NC * P * N
    init = 4 * B * NH * P * N if w.init_std > 0 else 0
    final = 4 * B * NH * P * N
    # bf16, headdim 64, dstate 128 (or 256 at chunk 256): the state-passing
    # launch also reads B and C and writes the chunks' C B^T tiles (T/32 x
    # (T/16 + 2) tiles of 1 KiB per chunk and group), which the chunk output
    # reads in place of B
    cb_tiles = B * NC * G * (T // 32) * (T // 16 + 2) * 1024 if (
        w.dtype == "bf16" and P == 64 and (N == 128 or (N == 256 and T == 256))) else 0
    bc = B * L * G * N * e
    m = {
        "chunk_cumsum": (tok_h * (e + 4), 0.0),
        "chunk_state": (tok_h * P * e + bc + tok_h * (e + 4) + states,
                        2.0 * B * L * NH * N * P),
        "state_pass": (2 * states + 4 * B * NH * NC + init + final + (2 * bc + cb_tiles if cb_tiles else 0),
                       0.0),
        "chunk_out": (tok_h * P * (e + y_bytes) + tok_h * (e + 4) + (bc + cb_tiles if cb_tiles else 2 * bc)
                      + states,
                      float(B * NC * G * T * (T + 1) * N + B * NC * NH * T * (T + 1) * P
                            + 2 * B * L * NH * N * P)),
    }
    if fused:
        # one launch for the chunk states and the carry: x, B and the token
        # weights in, the chunk-start states (and the final state) out, s_c
        # never stored (+ B, C in and the C B^T tiles out, as the state pass)
        m["chunk_state"] = (tok_h * P * e + bc + tok_h * (e + 4) + states + init + final
                            + (2 * bc + cb_tiles if cb_tiles else 0), 2.0 * B * L * NH * N * P)
        m["state_pass"] = (0, 0.0)
    e2e_bytes = tok_h * P * (e + y_bytes) + tok_h * e + 2 * B * L * G * N * e + init + final
    m["e2e"] = (e2e_bytes, m["chunk_state"][1] + m["chunk_out"][1])
    return m


class Hip:
    """The few HIP runtime calls the benchmark needs (events, device sync)."""

    def __init__(self):
        import torch  # noqa: F401  (loads the HIP runtime)
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed (%d)" % rc)
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return float(out.value)

    def destroy(self, ev: int):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


def gpu_clocks():
    """Shader and memory clock levels of the first AMD GPU as the amdgpu
    driver lists them in sysfs (pp_dpm_sclk, pp_dpm_mclk): the highest level
    and the one marked current.  Read from files, not from a tool, so that no
    child process starts after the GPU is in use."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
        except OSError:
            continue
        out = {}
        for key in ("sclk", "mclk"):
            try:
                with open(os.path.join(dev, "pp_dpm_" + key)) as f:
                    lines = [ln.strip() for ln in f if ":" in ln]
            except OSError:
                continue
            mhz = []
            cur = None
            for ln in lines:
                v = ln.split(":", 1)[1].strip()
                num = "".join(ch for ch in v.split()[0] if ch.isdigit())
                if not num:
                    continue
                mhz.append(int(num))
                if v.endswith("*"):
                    cur = int(num)
            if mhz:
                out[key + "_max_MHz"] = max(mhz)
                out[key + "_current_MHz"] = cur
        if out:
            return out
    return None


def context(hip, dev) -> dict:
    """What this machine reaches beside the datasheet peaks: a device copy of
    1 GiB from a source that a second 1 GiB write has evicted from L2 and the
    Infinity Cache (bytes read plus written over the copy's own events,
    median of 5), and the GPU clock levels the driver lists (null if it
    cannot)."""
    import torch
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    flush = torch.empty(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream(dev).cuda_stream
    times = []
    for _ in range(5):
        flush.fill_(2.0)
        e0, e1 = hip.event(), hip.event()
        hip.lib.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(st))
        dst.copy_(src)
        hip.lib.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(st))
        hip.lib.hipEventSynchronize(ctypes.c_void_p(e1))
        times.append(hip.elapsed_ms(e0, e1) * 1e-3)
        hip.destroy(e0)
        hip.destroy(e1)
    del src, dst, flush
    t = sorted(times)[len(times) // 2]
    clocks = gpu_clocks()
    return {"copy_GB_s": round(2 * n * 4 / t / 1e9, 1), "copy_bytes": 2 * n * 4,
            "copy_note": "torch device copy, 1 GiB read + 1 GiB written, cold source",
            "gpu_clocks": clocks}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, reps: int, min_seconds: float = 10.0, single=None) -> dict:
    """The fp64 oracle, as it stands, on this host's cores: the whole workload,
    repeated (at least ``reps`` times) until ``min_seconds`` of CPU work.
    ``single``: the one-thread figures of single_thread_oracle, taken earlier."""
    import oracle
    ncores = len(os.sched_getaffinity(0))
    oracle.scan(inp["x"][:, :64], inp["dt"][:, :64], inp["A"], inp["B"][:, :64], inp["C"][:, :64])
    times = []
    t_start = time.perf_counter()
    while len(times) < reps or time.perf_counter() - t_start < min_seconds:
        t0 = time.perf_counter()
        oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
        times.append(time.perf_counter() - t0)
    med = float(sorted(times)[len(times) // 2])
    threads = int(os.environ.get("OMP_NUM_THREADS", ncores))
    return {
        "value": w.tokens / med,
        "unit": "tokens/s",
        "cores": min(threads, ncores),
        "cpu": cpu_model(),
        # the recurrence's fp64 flops: 4 B L NH N P (state update and readout)
        "fp64_GFLOP_s": round(4.0 * w.batch * w.seqlen * w.nheads * w.dstate * w.headdim / med / 1e9, 2),
        "kind": "oracle",
        "sample": "whole workload (%d tokens, all heads), fp64 sequential recurrence, median of %d runs "
                  "(%.3f s each, %.1f s in all); oracle built with gcc -O2 -fopenmp, no -march=native "
                  "(the same library runs on any x86-64 host)" % (w.tokens, len(times), med, sum(times)),
        "single_thread": single,
    }


def single_thread_oracle(w) -> dict:
    """The oracle on one thread (OMP_NUM_THREADS=1, in a child process so the
    OpenMP runtime starts with that setting) for the tiny workload and for
    ``w``: tokens/s of one run each.  Called before this process touches the
    GPU: no program is started after that."""
    import subprocess
    out = {}
    for name in dict.fromkeys(["tiny_f32", w.name]):
        code = ("import sys, time; sys.path.insert(0, %r); import oracle, ssd_inputs as si; "
                "w = si.BY_NAME[%r]; i = si.generate(w); oracle.scan(i['x'][:, :8], i['dt'][:, :8], i['A'], "
                "i['B'][:, :8], i['C'][:, :8]); t = time.perf_counter(); "
                "oracle.scan(i['x'], i['dt'], i['A'], i['B'], i['C'], i['D'], i['h0']); "
                "print(time.perf_counter() - t)" % (ROOT, name))
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
        if r.returncode != 0:
            out[name] = {"error": r.stderr[-300:]}
            continue
        sec = float(r.stdout.strip().splitlines()[-1])
        tok = si_tokens(name)
        out[name] = {"value": round(tok / sec, 1), "unit": "tokens/s", "seconds": round(sec, 4), "cores": 1}
    return out


def si_tokens(name: str) -> int:
    import ssd_inputs as si
    return si.BY_NAME[name].tokens


def decode_bench(hip, w, batch, dev, steps=20, warmup=5) -> dict:
    """The recurrent decode step (one token per sequence, fp32 state updated in
    place) at the layer shape of workload ``w`` with ``batch`` sequences:
    kernel time from the dispatch's own events, and its HBM roofline (the
    state read and written once, plus x, dt, B, C in and y out)."""
    import numpy as np
    import torch

    import mamba_chunked_ssd_amd as ssd
    import ssd_inputs as si

    dw = si.small(dtype=w.dtype, batch=batch, seqlen=1, nheads=w.nheads, headdim=w.headdim, dstate=w.dstate,
                  ngroups=w.ngroups, chunk_size=64, dt_mu=w.dt_mu, init_std=0.1, seed=w.seed + 100)
    inp = si.generate(dw)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k][:, 0] if k in ("x", "dt", "B", "C") else inp[k],
                                                  np.float32)).to(dev) for k in ("x", "dt", "A", "B", "C", "D")}
    for k in ("x", "dt", "B", "C"):
        t[k] = t[k].to(tdt)
    state = torch.from_numpy(inp["h0"]).to(dev)
    y = torch.empty((batch, w.nheads, w.headdim), dtype=torch.float32, device=dev)
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    for i in range(warmup + steps):
        ssd.decode_step(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], state, out=y,
                        events=evs[i - warmup] if i >= warmup else None)
    torch.cuda.synchronize()
    us = float(np.median([hip.elapsed_ms(a, b) for a, b in evs])) * 1e3
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    e = 2 if w.dtype == "bf16" else 4
    bh = batch * w.nheads
    byts = 2 * 4 * bh * w.headdim * w.dstate + bh * w.headdim * (e + 4) + bh * e + 2 * batch * w.ngroups * w.dstate * e
    gbs = byts / (us * 1e-6) / 1e9
    return {"workload": "decode_step_%s_batch%d" % (w.name, batch), "batch": batch, "us": round(us, 3),
            "tokens_per_s": round(batch / (us * 1e-6), 1), "GB_s": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": byts}}


def bwd_stage_model(w) -> dict:
    """Algorithmic (HBM bytes, flops) of each backward stage at workload ``w``:
    each input read once, each output and intermediate written once and read
    once by the stage that consumes it; MFMA flops of the contractions the
    method needs (the masked triangles counted as T (T + 16) / 2 of T x T, the
    16 x 16 blocks on the diagonal included), not of the bf16 term splits."""
    B, L, NH, P, N, G, T = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    e = 2 if w.dtype == "bf16" else 4
    NC = -(-L // T)
    Lp = NC * T
    tok_h = B * L * NH
    seq = 4 * B * NH * Lp
    states = 4 * B * NH * NC * P * N
    tri = T * (T + 16) / 2
    units = B * NC * NH
    bc = B * L * G * N * e
    x = tok_h * P * e
    init = 4 * B * NH * P * N if w.init_std > 0 else 0
    ntile = (T // 16) * (T // 16 + 1) // 2
    st = 4 * B * NC * G * ntile * 256
    m = {}
    m["chunk_cumsum"] = (tok_h * e + 5 * seq, 0.0)
    m["chunk_state"] = (x + bc + seq + states, 2.0 * B * L * NH * N * P)
    m["state_pass"] = (2 * states + seq / T + init, 0.0)
    m["adjoint_chunk_state"] = (x + bc + seq + states, 2.0 * B * L * NH * N * P)
    m["adjoint_carry"] = (3 * states + 4 * B * NH * P * N, 0.0)
    m["score_tiles"] = (2 * bc + st, 2.0 * B * NC * G * tri * N)
    if w.dtype != "bf16":
        # fp32 inputs: each head's decayed x . dy tiles are computed here once
        # (x and dy read, the tiles and their transposes written), and the dB,
        # dC and W passes read them instead of recomputing the scores
        ptiles = 2 * 4 * units * (T // 16) * (T // 16 + 1) // 2 * 256
        m["score_tiles"] = (2 * bc + st + 2 * x + ptiles, 2.0 * B * NC * G * tri * N + 2.0 * units * tri * P)
    m["dx_pass"] = (st + 2 * x + bc + states + 4 * tok_h * P + 3 * 4 * tok_h, 2.0 * units * (tri * P + T * N * P))
    bwd_bc = 2.0 * units * (tri * P + tri * N + T * P * N)
    m["dB_pass"] = (2 * x + bc + states + 4 * B * L * G * N, bwd_bc)
    m["dC_pass"] = (2 * x + 2 * bc + states + 4 * B * L * G * N + 4 * tok_h, bwd_bc)
    m["w_sums"] = (2 * x + st + 8 * tok_h, 2.0 * units * tri * P)
    if w.dtype != "bf16":
        ptile_one = 4 * units * (T // 16) * (T // 16 + 1) // 2 * 256
        no_scores = 2.0 * units * (tri * N + T * P * N)
        m["dB_pass"] = (x + ptile_one + bc + states + 4 * B * L * G * N, no_scores)
        m["dC_pass"] = (x + ptile_one + 2 * bc + states + 4 * B * L * G * N + 4 * tok_h, no_scores)
        m["w_sums"] = (ptile_one + st + 8 * tok_h, 0.0)
    m["token_finish"] = ((4 * 4 + 8 + 4) * tok_h, 0.0)
    m["reduce"] = (2 * 4 * B * L * G * N * 2, 0.0)
    return m


def backward_bench(hip, w, inp, t, dev, steps=10, warmup=3) -> dict:
    """ssd_chunk_scan_bwd at workload ``w`` with seeded upstream gradients:
    the whole call timed back to back (tokens/s), each stage from its kernel's
    own events (median over the steps), and the roofline of the slowest
    stage against the algorithmic model of ``bwd_stage_model``."""
    import numpy as np
    import torch

    import mamba_chunked_ssd_amd as ssd
    import ssd_inputs as si

    cot = si.cotangents(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dy = torch.from_numpy(cot["dy"]).to(dev).to(tdt)
    dfin = torch.from_numpy(cot["dfinal"]).to(dev)
    shape = ssd.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype)
    ws = torch.empty(ssd.bwd_workspace_size(shape, w.chunk_size), dtype=torch.uint8, device=dev)
    names = ssd.BWD_STAGES

    def call(events=None):
        return ssd.chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dy, chunk_size=w.chunk_size,
                                  initial_states=t["h0"], d_final_states=dfin, workspace=ws, events=events)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    for _ in range(steps):
        call()
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    hip.lib.hipEventSynchronize(ctypes.c_void_p(e1))
    total_us = hip.elapsed_ms(e0, e1) * 1e3 / steps

    # the same calls reading the chunk-start states that one forward call
    # kept in its workspace (ssd_chunk_scan_bwd_saved) instead of
    # recomputing them
    kshape = ssd.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype, True)
    fws = torch.empty(ssd.workspace_size(kshape, w.chunk_size), dtype=torch.uint8, device=dev)
    ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=w.chunk_size,
                       initial_states=t["h0"], workspace=fws, keep_intermediates=True)

    def call_saved():
        return ssd.chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dy, chunk_size=w.chunk_size,
                                  initial_states=t["h0"], d_final_states=dfin, workspace=ws,
                                  saved_workspace=fws)

    for _ in range(warmup):
        call_saved()
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    for _ in range(steps):
        call_saved()
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    hip.lib.hipEventSynchronize(ctypes.c_void_p(e1))
    saved_us = hip.elapsed_ms(e0, e1) * 1e3 / steps
    del fws
    hip.destroy(e0)
    hip.destroy(e1)
    evs = [[hip.event() for _ in range(2 * len(names))] for _ in range(steps)]
    for k in range(steps):
        call(evs[k])
    torch.cuda.synchronize()
    per = {n: float(np.median([hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for ev in evs])) * 1e3
           for i, n in enumerate(names)}
    for ev in evs:
        for e_ in ev:
            hip.destroy(e_)
    model = bwd_stage_model(w)
    peak_tf = PEAK_TFLOPS[w.dtype]
    stages = {}
    for n in names:
        byts, flops = model[n]
        us = per[n]
        floor = max(byts / (PEAK_HBM_GBS * 1e9), flops / (peak_tf * 1e12))
        stages[n] = {"us": round(us, 2), "roofline_frac": round(floor / (us * 1e-6), 4) if us > 0 else None}
    dom = max(names, key=lambda n: per[n])
    byts, flops = model[dom]
    hbm_t, mfma_t = byts / (PEAK_HBM_GBS * 1e9), flops / (peak_tf * 1e12)
    bound = "mfma" if mfma_t >= hbm_t else "hbm"
    t_dom = per[dom] * 1e-6
    achieved = flops / t_dom / 1e12 if bound == "mfma" else byts / t_dom / 1e9
    peak = peak_tf if bound == "mfma" else PEAK_HBM_GBS
    return {
        "workload": w.name,
        "metric": "SSD bwd tokens/s at 1 MI355X",
        "value": round(w.tokens / (total_us * 1e-6), 1),
        "unit": "tokens/s",
        "us_per_step": round(total_us, 2),
        "steps": steps,
        "saved_states": {"value": round(w.tokens / (saved_us * 1e-6), 1), "unit": "tokens/s",
                         "us_per_step": round(saved_us, 2),
                         "note": "ssd_chunk_scan_bwd_saved: the chunk-start states read from one forward "
                                 "call's workspace (SSD_FLAG_KEEP_INTERMEDIATES), not recomputed"},
        "stages": stages,
        "dominant": dom,
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(achieved / peak, 4),
                     "flops": flops, "bytes": byts, "traffic": measured_traffic(w.name, None, "bwd:" + dom),
                     "model": "bwd_stage_model: algorithmic HBM bytes and contraction flops of the dominant "
                              "stage; bound is the larger of the two floors"},
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 500 steps of the 2.7B layer take about 43 ms: enough that the timed
    # region's fixed start and finish (the first step's enqueue, the final
    # synchronisation; about 0.2 ms) stay under 0.5 % of it
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2_2p7b_layer_bf16")
    ap.add_argument("--y-dtype", choices=["f32", "input"], default="f32",
                    help="y element type: fp32 (default) or the input type")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3, help="least number of oracle runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle run until this much CPU time has passed")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed after a 1 GiB cache-flush write each (per-stage cold times; 0: skip)")
    ap.add_argument("--plan", choices=["default", "split", "fused", "tuned"], default="default",
                    help="launch plan: the library's default, the split / fused state path, or the "
                         "plan ssd_chunk_scan_fwd_tune picks (tuned before the warm-up, untimed)")
    ap.add_argument("--fused-cols", type=int, default=64,
                    help="dstate columns per fused-state block (32 or 64)")
    ap.add_argument("--bwd-steps", type=int, default=10,
                    help="timed steps of the backward pass (0: skip it)")
    ap.add_argument("--decode-batch", type=int, default=128,
                    help="batch of the recurrent decode-step measurement (0: skip it)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the measured copy bandwidth and the GPU clocks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy (for scaling rocprofv3 FETCH/WRITE counters)")
    a = ap.parse_args(argv)

    if a.gpus != 1:
        print("bench.py: this build measures one GPU; --gpus %d is not supported "
              "(run with --gpus 1)" % a.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mamba_chunked_ssd_amd as ssd
    import ssd_inputs as si

    w = si.BY_NAME[a.workload]
    # the one-thread oracle runs in child processes, started before the GPU
    # is initialised (torch.cuda.is_available() does that)
    single = None if a.no_cpu_baseline else single_thread_oracle(w)
    if not torch.cuda.is_available():
        print("bench.py: no ROCm GPU visible", file=sys.stderr)
        return 2
    inp = si.generate(w)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ydt = torch.float32 if a.y_dtype == "f32" else tdt
    t = {}
    for k, v in inp.items():
        if v is None:
            t[k] = None
            continue
        x = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)
        t[k] = x.to(tdt) if k in ("x", "dt", "B", "C") else x
    y = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), dtype=ydt, device=dev)
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    shape = ssd.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype,
                           y_dtype="bf16" if ydt == torch.bfloat16 else "f32")
    ws = torch.empty(ssd.workspace_size(shape, w.chunk_size), dtype=torch.uint8, device=dev)
    hip = Hip()
    stream = torch.cuda.current_stream(dev)
    plan = ssd.default_plan(shape, w.chunk_size)
    tuned_us = None
    if a.plan == "tuned":
        plan, tuned_us = ssd.tune(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], w.chunk_size, t["h0"],
                                  reps=5, y_dtype=ydt, out=y, final_out=fin, workspace=ws)
    elif a.plan != "default":
        plan = ssd.make_plan(a.plan, plan.chunk_state_heads, plan.chunk_out_heads,
                             a.fused_cols if a.plan == "fused" else 0)

    def step(events=None):
        ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk_size=w.chunk_size,
                           initial_states=t["h0"], y_dtype=ydt, out=y, final_out=fin, workspace=ws,
                           stream=stream.cuda_stream, events=events, plan=plan)

    if a.calibrate_copy:
        # a plain device copy of known size (1 GiB read + 1 GiB written) whose
        # FETCH_SIZE / WRITE_SIZE give the counters' scale.  The source is
        # written first (real data), then a second 1 GiB buffer is written so
        # that neither L2 nor the 256 MB Infinity Cache still holds the
        # source when the copy reads it.
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        src.fill_(1.0)
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        flush.fill_(2.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / a.steps

    # per-stage times: a second run of K steps in which every kernel's own
    # dispatch records a (start, stop) event pair (these records cost time of
    # their own, so this run is not the one the throughput comes from)
    ev_steps = min(a.steps, 50)
    evs = [[hip.event() for _ in range(8)] for _ in range(ev_steps)]
    torch.cuda.synchronize()
    for i in range(ev_steps):
        step(evs[i])
    torch.cuda.synchronize()
    per_stage = np.array([[hip.elapsed_ms(e[2 * j], e[2 * j + 1]) for j in range(4)] for e in evs])
    for e in evs:
        for ev in e:
            hip.destroy(ev)
    stage_ms = per_stage.mean(axis=0)

    model = stage_model(w, 4 if ydt == torch.float32 else (2 if w.dtype == "bf16" else 4),
                        fused=plan.state_path == ssd.SSD_STATE_FUSED)
    peak_tf = PEAK_TFLOPS[w.dtype]
    # Stages that launch no kernel for this problem (the library says which)
    # are reported as such and add no floor; their event pairs time nothing.
    launched = ssd.stage_launches(shape, w.chunk_size, plan)
    skipped = {name for name in STAGES if name not in launched}
    stages = {}
    for j, name in enumerate(STAGES):
        if name in skipped:
            stages[name] = {"us": 0.0, "launched": False}
            continue
        byts, flops = model[name]
        t_s = stage_ms[j] * 1e-3
        floor = max(byts / (PEAK_HBM_GBS * 1e9), flops / (peak_tf * 1e12))
        stages[name] = {"us": round(stage_ms[j] * 1e3, 3), "GB_s": round(byts / t_s / 1e9, 1),
                        "TFLOP_s": round(flops / t_s / 1e12, 2),
                        "roofline_frac": round(floor / t_s, 4)}
    dom = STAGES[int(np.argmax(stage_ms))]
    dj = STAGES.index(dom)
    dbytes, dflops = model[dom]
    t_dom = stage_ms[dj] * 1e-3
    hbm_t = dbytes / (PEAK_HBM_GBS * 1e9)
    mfma_t = dflops / (peak_tf * 1e12)
    if hbm_t >= mfma_t:
        roof = {"bound": "hbm", "achieved": round(dbytes / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(dbytes / t_dom / 1e9 / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(dflops / t_dom / 1e12, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(dflops / t_dom / 1e12 / peak_tf, 4)}
    roof["traffic"] = measured_traffic(w.name, "f32" if ydt == torch.float32 else w.dtype, dom,
                                       plan.as_dict())
    roof["kernel"] = dom
    # the byte model behind `achieved`: algorithmic bytes of one launch of the
    # dominant kernel (inputs in their dtype, fp32 intermediates, y at the
    # y dtype's size -- fp32 by default, whose floor is larger than a bf16 y's)
    roof["bytes"] = int(dbytes)
    roof["flops"] = float(dflops)
    roof["model"] = "algorithmic bytes per launch, y at %d bytes per element" % (
        4 if ydt == torch.float32 else 2)
    e2e_bytes, e2e_flops = model["e2e"]
    e2e_t = ms_per_step * 1e-3
    e2e_floor = max(e2e_bytes / (PEAK_HBM_GBS * 1e9), e2e_flops / (peak_tf * 1e12))
    sigma_floor = sum(max(model[s][0] / (PEAK_HBM_GBS * 1e9), model[s][1] / (peak_tf * 1e12))
                      for s in STAGES if s not in skipped)

    out = {
        "metric": METRIC,
        "value": round(w.tokens / e2e_t, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_size": w.chunk_size, "accumulate": "f32",
                   "y_dtype": "f32" if ydt == torch.float32 else w.dtype,
                   "initial_states": w.init_std > 0, "parallelism": "single_gpu",
                   "plan": plan.as_dict()},
        "roofline": roof,
        "stages": stages,
        "e2e_roofline_frac": round(e2e_floor / e2e_t, 4),
        "e2e_stage_sum_roofline_frac": round(sigma_floor / e2e_t, 4),
    }

    if a.cold_steps > 0:
        # per-stage times with cold caches: before each step a 1 GiB write
        # (more than L2 plus the 256 MB Infinity Cache) evicts the inputs and
        # the previous step's intermediates; the flush is outside the events
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold = []
        for _ in range(a.cold_steps):
            flush.fill_(1.0)
            e = [hip.event() for _ in range(8)]
            step(e)
            torch.cuda.synchronize()
            cold.append([hip.elapsed_ms(e[2 * j], e[2 * j + 1]) for j in range(4)])
            for ev in e:
                hip.destroy(ev)
        del flush
        cold_ms = np.median(np.array(cold), axis=0)
        cold_stages = {}
        for j, name in enumerate(STAGES):
            if name in skipped:
                continue
            byts, flops = model[name]
            t_s = cold_ms[j] * 1e-3
            floor = max(byts / (PEAK_HBM_GBS * 1e9), flops / (peak_tf * 1e12))
            cold_stages[name] = {"us": round(cold_ms[j] * 1e3, 3), "roofline_frac": round(floor / t_s, 4)}
        t_dom_c = cold_ms[dj] * 1e-3
        out["cold"] = {
            "steps": a.cold_steps,
            "stages": cold_stages,
            "stage_sum_us": round(sum(cold_ms[j] for j, n in enumerate(STAGES) if n not in skipped) * 1e3, 3),
            "roofline": dict(roof, achieved=round((dbytes if roof["bound"] == "hbm" else dflops / 1e3)
                                                  / t_dom_c / 1e9, 1),
                             frac=round((hbm_t if roof["bound"] == "hbm" else mfma_t) / t_dom_c, 4)),
        }

    if a.decode_batch > 0:
        out["decode"] = decode_bench(hip, w, a.decode_batch, dev)

    if not a.no_context:
        out["context"] = context(hip, dev)

    if a.bwd_steps > 0:
        out["backward"] = backward_bench(hip, w, inp, t, dev, steps=a.bwd_steps)

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_reps, a.cpu_seconds, single)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

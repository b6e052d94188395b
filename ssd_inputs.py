"""Seeded synthetic inputs for the Mamba-2 chunked SSD forward pass.

This module is shared by the tests, the smoke check and the benchmark.  It
holds only input distributions and storage rounding -- none of the method's
arithmetic -- so that the oracle and the HIP path can both consume the same
bits without sharing any code that computes the scan.

The five workload shapes are the Mamba-2 layer shapes the method is measured
on (tiny, a 2.7B-model layer, a throughput batch, a long sequence with a large
state, and grouped B/C with a large state).  Recipe for workload ``k`` (all
draws float32, in this order, from ``numpy.random.default_rng(1000 + k)``):

1. x ~ N(0, 1) (b, L, nh, p); B ~ N(0, 1) and C ~ N(0, 1) (b, L, g, n)
2. z ~ N(mu_k, 1) (b, L, nh); dt = softplus(z) = log1p(exp(z)), in fp64
3. u ~ U(0, ln 16) per head; A = -exp(u), so A is log-uniform in [-16, -1]
4. D ~ N(0, 1) per head
5. initial state ~ N(0, 0.1^2) (b, nh, p, n) when the workload has one
6. for the grouped workload: a Bernoulli(0.1) mask per (b, t, h), drawn as
   U(0, 1) < 0.1, sets dt = 1e-4 (near no update)

Workloads stored in bf16 round x, dt, B and C to bf16 with round-to-nearest-
even; the arrays stay float32 (exact bf16 values) so the fp64 oracle widens the
same bits the GPU reads.  A, D and states are always float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": storage of x, dt, B, C, y
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    dt_mu: float = 0.0
    init_std: float = 0.0       # 0 => zero initial state (None)
    dt_floor_frac: float = 0.0  # fraction of dt entries set to 1e-4
    seed: int = 1000

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = [
    Workload("tiny_f32", "f32", 1, 256, 4, 32, 16, 1, 64, dt_mu=0.0, seed=1000),
    Workload("mamba2_2p7b_layer_bf16", "bf16", 2, 2048, 80, 64, 128, 1, 256, dt_mu=-2.0, seed=1001),
    Workload("throughput_bf16", "bf16", 8, 4096, 80, 64, 128, 1, 256, dt_mu=-2.0,
             init_std=0.1, seed=1002),
    Workload("long_seq_bf16", "bf16", 1, 65536, 32, 64, 256, 1, 256, dt_mu=-3.0, seed=1003),
    Workload("grouped_f32", "f32", 4, 16384, 64, 128, 256, 8, 128, dt_mu=0.0,
             dt_floor_frac=0.1, seed=1004),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    NaN stays NaN; overflow rounds to +-inf as the RNE definition gives.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exact bf16 (as uint16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def softplus64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    return np.where(z > 30.0, z, np.log1p(np.exp(np.minimum(z, 30.0))))


def generate(w: Workload, seed: int | None = None) -> dict:
    """Inputs for workload ``w``: dict of float32 numpy arrays (h0 may be None)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b, L, nh, p, n, g = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    x = rng.standard_normal((b, L, nh, p), dtype=np.float32)
    Bm = rng.standard_normal((b, L, g, n), dtype=np.float32)
    Cm = rng.standard_normal((b, L, g, n), dtype=np.float32)
    z = rng.standard_normal((b, L, nh), dtype=np.float32) + np.float32(w.dt_mu)
    dt = softplus64(z).astype(np.float32)
    u = rng.uniform(0.0, np.log(16.0), size=nh).astype(np.float32)
    A = (-np.exp(u.astype(np.float64))).astype(np.float32)
    D = rng.standard_normal(nh, dtype=np.float32)
    h0 = None
    if w.init_std > 0:
        h0 = (rng.standard_normal((b, nh, p, n), dtype=np.float32) * np.float32(w.init_std))
    if w.dt_floor_frac > 0:
        mask = rng.uniform(0.0, 1.0, size=(b, L, nh)) < w.dt_floor_frac
        dt = np.where(mask, np.float32(1e-4), dt).astype(np.float32)
    if w.dtype == "bf16":
        x, Bm, Cm, dt = (round_bf16(v) for v in (x, Bm, Cm, dt))
    elif w.dtype != "f32":
        raise ValueError("unknown dtype %r" % w.dtype)
    return dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, h0=h0)


def small(name: str = "small", dtype: str = "f32", batch=1, seqlen=64, nheads=2, headdim=4,
          dstate=3, ngroups=1, chunk_size=16, dt_mu=0.0, init_std=0.0, seed=7) -> Workload:
    """A small workload for tests (same distributions, any shape)."""
    return Workload(name, dtype, batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size,
                    dt_mu=dt_mu, init_std=init_std, seed=seed)


def cotangents(w: Workload, seed: int | None = None, final: bool = True) -> dict:
    """Seeded upstream gradients for the backward pass of workload ``w``:
    dy ~ N(0, 1) (b, L, nh, p) in the workload's storage dtype (bf16-rounded
    for bf16 workloads) and, when ``final``, dfinal ~ N(0, 1) (b, nh, p, n)
    float32.  Drawn from ``default_rng(seed or w.seed + 500)`` in that order."""
    rng = np.random.default_rng(w.seed + 500 if seed is None else seed)
    b, L, nh, p, n = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate
    dy = rng.standard_normal((b, L, nh, p), dtype=np.float32)
    if w.dtype == "bf16":
        dy = round_bf16(dy)
    dfin = rng.standard_normal((b, nh, p, n), dtype=np.float32) if final else None
    return dict(dy=dy, dfinal=dfin)

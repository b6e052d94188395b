"""The oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct CPU definitions of what the Mamba-2 chunked SSD
forward pass computes, in fp64.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package; the HIP
product path never does, and the two share no code, headers or helpers.

Everything here follows "Accelerating Mamba-2 with High-Performance Forward
Pass Kernels in NVIDIA CUDA Tile":

* :func:`scan` -- the sequential recurrence of section "Mamba-2 architecture"
  (the first two displayed equations; readout with the post-update state, the
  reading that makes the chunked output formula of the same section with an
  inclusive causal mask exact).  Implemented in ``ssd_oracle.c`` (plain C,
  fp64, OpenMP over independent (batch, head, headdim-row) units).
* :func:`chunk_cumsum` -- the per-chunk inclusive cumulative sum of
  a_t = A dt_t (section "Kernel 1: Computing cumulative sums"), the G of the
  log-space equations, reset at each chunk start, zero-padded past seqlen.
* :func:`chunk_states` -- the state a chunk produces on its own from a zero
  state: the input term (exp(G_last - G) B) X^T of the state-jump equation
  (section "Mamba-2 architecture", the log-space jump), evaluated here by
  running the recurrence over that chunk alone.
* :func:`chunk_start_states` -- the state at the start of every chunk, the
  quantity the fwd_pass_state section stores per chunk.
* :func:`chunk_cb` -- the C B^T factor of the chunk output equation (section
  "Mamba-2 architecture"): every product C_i . B_j of two tokens of a chunk.
* :func:`decode_step` -- one step of the recurrence for one new token per
  sequence from a given state (the recurrent form the same section names for
  sequential inference): :func:`scan` over a sequence of length 1.
* :func:`scan_bwd` -- the gradients of <dy, y> + <dhT, h_final> with respect
  to every input of :func:`scan`: the adjoint of the same recurrence, run in
  reverse in fp64 (``ssd_oracle.c``).  The pages name the backward pass as
  what training depends on and derive none; this is the chain rule applied to
  each step of the recurrence, pinned by finite differences of :func:`scan`.

Inputs may be float32 or float64 numpy arrays; they are widened exactly to
fp64.  bf16 data is passed as float32 arrays holding bf16-representable values
(exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``ssd_oracle.c`` with gcc into ``oracle/libssd_oracle.so``.

    No ``-march=native``: the library is built on one machine and may run on
    another host CPU.
    """
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Open an oracle shared library and declare its C signature."""
    lib = ctypes.CDLL(path)
    f = lib.ssd_oracle_scan
    i64 = ctypes.c_int64
    dp = ctypes.c_void_p
    f.argtypes = [i64] * 6 + [dp] * 9 + [i64, dp]
    f.restype = ctypes.c_int
    g = lib.ssd_oracle_scan_bwd
    g.argtypes = [i64] * 6 + [dp] * 16
    g.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            _lib = load_library(_LIB_PATH)
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(x, dt, A, B, C, D=None, h0=None, ckpt_stride: int = 0):
    """Sequential fp64 recurrence over every (batch, head) (``ssd_oracle.c``).

    Shapes: x (b, L, nh, p), dt (b, L, nh), A (nh,), B/C (b, L, g, n),
    D (nh,) or None, h0 (b, nh, p, n) or None.

    Returns ``(y, h_final, ckpt)``: y (b, L, nh, p); h_final (b, nh, p, n), the
    state after the last token; ckpt (b, nh, ceil(L/stride), p, n), the state
    before token k*stride, or None when ``ckpt_stride`` is 0.
    """
    return scan_with(_load(), x, dt, A, B, C, D, h0, ckpt_stride)


def scan_with(lib, x, dt, A, B, C, D=None, h0=None, ckpt_stride: int = 0):
    """:func:`scan` through a given library handle (see :func:`load_library`)."""
    x, dt, A, B, C = (_f64(v) for v in (x, dt, A, B, C))
    D, h0 = _f64(D), _f64(h0)
    bsz, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    if dt.shape != (bsz, L, nh) or A.shape != (nh,):
        raise ValueError("dt/A shape mismatch")
    if B.shape != (bsz, L, g, n) or C.shape != B.shape:
        raise ValueError("B/C shape mismatch")
    if D is not None and D.shape != (nh,):
        raise ValueError("D shape mismatch")
    if h0 is not None and h0.shape != (bsz, nh, p, n):
        raise ValueError("h0 shape mismatch")
    y = np.zeros((bsz, L, nh, p), np.float64)
    hT = np.zeros((bsz, nh, p, n), np.float64)
    ckpt = None
    if ckpt_stride:
        nck = -(-L // ckpt_stride)
        ckpt = np.zeros((bsz, nh, nck, p, n), np.float64)
    rc = lib.ssd_oracle_scan(bsz, L, nh, p, n, g,
                             _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(h0), _ptr(y), _ptr(hT), int(ckpt_stride), _ptr(ckpt))
    if rc != 0:
        raise ValueError("ssd_oracle_scan rejected its arguments (rc=%d)" % rc)
    return y, hT, ckpt


def chunk_cumsum(dt, A, chunk_size: int):
    """Per-chunk inclusive cumsum of a_t = A[h] dt_t, natural-log units, fp64.

    Returns (b, nh, nchunks * chunk_size); positions past seqlen are padded with
    dt = 0, so the sum stays flat there and the last entry of every chunk is
    that chunk's G_last.
    """
    dt = _f64(dt)
    A = _f64(A)
    bsz, L, nh = dt.shape
    nc = -(-L // chunk_size)
    pad = np.zeros((bsz, nc * chunk_size, nh), np.float64)
    pad[:, :L] = dt
    a = pad * A[None, None, :]
    g = np.cumsum(a.reshape(bsz, nc, chunk_size, nh), axis=2)
    return np.ascontiguousarray(g.reshape(bsz, nc * chunk_size, nh).transpose(0, 2, 1))


def chunk_state_weights(dt, A, chunk_size: int):
    """Weight with which each token enters its chunk's state, (b, nh, Lp):
    exp(G_last - G_t) dt_t with G the per-chunk cumsum and G_last its value at
    the chunk's last token ("Accelerating Mamba-2 ...", section "Mamba-2
    architecture": the log-space state jump scales the chunk's B rows by the
    decay from each token to the chunk end; dt is the discretisation step
    that multiplies B).  Padding past seqlen has dt = 0, hence weight 0.
    """
    G = chunk_cumsum(dt, A, chunk_size)
    bsz, nh, Lp = G.shape
    Gc = G.reshape(bsz, nh, Lp // chunk_size, chunk_size)
    decay = np.exp(Gc[..., -1:] - Gc).reshape(bsz, nh, Lp)
    dtp = _pad_tokens(_f64(dt), Lp).transpose(0, 2, 1)
    return decay * dtp


def _pad_tokens(v, Lp):
    out = np.zeros((v.shape[0], Lp) + v.shape[2:], np.float64)
    out[:, : v.shape[1]] = v
    return out


def chunk_states(x, dt, A, B, C, chunk_size: int):
    """State each chunk produces from a zero state: (b, nh, nchunks, p, n)."""
    x, dt, B, C = (_f64(v) for v in (x, dt, B, C))
    bsz, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    nc = -(-L // chunk_size)
    Lp = nc * chunk_size
    T = chunk_size
    # Zero padding past seqlen: dt = 0 leaves the state unchanged.
    xs = _pad_tokens(x, Lp).reshape(bsz * nc, T, nh, p)
    dts = _pad_tokens(dt, Lp).reshape(bsz * nc, T, nh)
    Bs = _pad_tokens(B, Lp).reshape(bsz * nc, T, g, n)
    Cs = _pad_tokens(C, Lp).reshape(bsz * nc, T, g, n)
    _, hT, _ = scan(xs, dts, A, Bs, Cs)
    return np.ascontiguousarray(hT.reshape(bsz, nc, nh, p, n).transpose(0, 2, 1, 3, 4))


def chunk_start_states(x, dt, A, B, C, chunk_size: int, h0=None):
    """State at the start of every chunk: (b, nh, nchunks, p, n)."""
    _, _, ck = scan(x, dt, A, B, C, None, h0, ckpt_stride=chunk_size)
    return ck


def chunk_cb(B, C, chunk_size: int):
    """C B^T of every chunk, (b, nchunks, g, T, T), entry [..., i, j] = C_i . B_j
    for chunk-local tokens i, j ("Accelerating Mamba-2 ...", section "Mamba-2
    architecture": the C B^T factor of the chunk output, before the decay and
    the causal mask are applied).  Tokens past seqlen have zero B and C rows.
    """
    B, C = _f64(B), _f64(C)
    bsz, L, g, n = B.shape
    nc = -(-L // chunk_size)
    Lp = nc * chunk_size
    Bs = _pad_tokens(B, Lp).reshape(bsz, nc, chunk_size, g, n)
    Cs = _pad_tokens(C, Lp).reshape(bsz, nc, chunk_size, g, n)
    out = np.zeros((bsz, nc, g, chunk_size, chunk_size))
    for gi in range(g):
        out[:, :, gi] = np.matmul(Cs[:, :, :, gi, :], Bs[:, :, :, gi, :].transpose(0, 1, 3, 2))
    return out


def decode_step(x, dt, A, B, C, D, state):
    """One step of the recurrence from ``state``, for one token per sequence.

    Shapes: x (b, nh, p), dt (b, nh), B/C (b, g, n), A (nh,), D (nh,) or None,
    state (b, nh, p, n).  Returns ``(y, new_state)``: y (b, nh, p) fp64 with
    the readout after the update, new_state (b, nh, p, n) fp64.  This is
    :func:`scan` with seqlen 1 and initial state ``state``.
    """
    x, dt, B, C = (_f64(v) for v in (x, dt, B, C))
    y, hT, _ = scan(x[:, None], dt[:, None], A, B[:, None], C[:, None], D, state)
    return y[:, 0], hT


def scan_bwd(x, dt, A, B, C, D=None, h0=None, dy=None, dhT=None):
    """Gradients of ``<dy, y> + <dhT, h_final>`` through :func:`scan`, fp64.

    Same shapes as :func:`scan`; dy like y (None => 0), dhT like h_final
    (None => 0).  Returns a dict with ``dx`` (b, L, nh, p), ``ddt`` (b, L, nh),
    ``dA`` (nh,), ``dB`` and ``dC`` (b, L, g, n), ``dD`` (nh,) and ``dh0``
    (b, nh, p, n).  dB and dC sum over the heads that share a group; dA and dD
    over batch and tokens.
    """
    return scan_bwd_with(_load(), x, dt, A, B, C, D, h0, dy, dhT)


def scan_bwd_with(lib, x, dt, A, B, C, D=None, h0=None, dy=None, dhT=None):
    """:func:`scan_bwd` through a given library handle."""
    x, dt, A, B, C = (_f64(v) for v in (x, dt, A, B, C))
    D, h0, dy, dhT = _f64(D), _f64(h0), _f64(dy), _f64(dhT)
    bsz, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    if dt.shape != (bsz, L, nh) or A.shape != (nh,):
        raise ValueError("dt/A shape mismatch")
    if B.shape != (bsz, L, g, n) or C.shape != B.shape:
        raise ValueError("B/C shape mismatch")
    if D is not None and D.shape != (nh,):
        raise ValueError("D shape mismatch")
    if h0 is not None and h0.shape != (bsz, nh, p, n):
        raise ValueError("h0 shape mismatch")
    if dy is None:
        dy = np.zeros(x.shape, np.float64)
    if dy.shape != x.shape:
        raise ValueError("dy shape mismatch")
    if dhT is not None and dhT.shape != (bsz, nh, p, n):
        raise ValueError("dhT shape mismatch")
    out = {
        "dx": np.zeros(x.shape), "ddt": np.zeros(dt.shape), "dA": np.zeros(nh),
        "dB": np.zeros(B.shape), "dC": np.zeros(C.shape), "dD": np.zeros(nh),
        "dh0": np.zeros((bsz, nh, p, n)),
    }
    rc = lib.ssd_oracle_scan_bwd(bsz, L, nh, p, n, g,
                                 _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                 _ptr(h0), _ptr(dy), _ptr(dhT),
                                 _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
                                 _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                                 _ptr(out["dh0"]))
    if rc != 0:
        raise ValueError("ssd_oracle_scan_bwd rejected its arguments (rc=%d)" % rc)
    return out

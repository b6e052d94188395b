"""mamba_chunked_ssd_amd -- the Mamba-2 chunked SSD forward pass on MI355X (gfx950).

A thin ctypes binding over ``libssd.so`` (C ABI in ``include/ssd.h``).  It only
marshals arguments: torch provides device memory and the current stream, and
every step of the forward pass runs in the library's HIP kernels.  There is no
CPU fallback: if the library is missing, importing works but any call raises.

    y = chunk_scan_fwd(x, dt, A, B, C, D, chunk_size=256)
    y, final = chunk_scan_fwd(..., initial_states=h0, return_final_states=True)

The operation is the selective state-space recurrence of "Accelerating Mamba-2
with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile" (section
"Mamba-2 architecture"): h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t^T,
y_t = C_t^T h_t + D x_t, for every batch and head.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1
SSD_FLAG_KEEP_INTERMEDIATES = 1

STATUS = {
    0: "SSD_OK",
    1: "SSD_ERROR_INVALID_VALUE",
    2: "SSD_ERROR_UNSUPPORTED",
    3: "SSD_ERROR_MISALIGNED",
    4: "SSD_ERROR_WORKSPACE",
    5: "SSD_ERROR_LAUNCH",
    6: "SSD_ERROR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024

# Symbols include/ssd.h declares (checked by the CPU tests).
EXPORTS = [
    "ssd_chunk_scan_fwd_workspace_size",
    "ssd_chunk_scan_fwd_workspace_layout",
    "ssd_chunk_scan_fwd",
    "ssd_chunk_scan_fwd_profiled",
    "ssd_chunk_scan_fwd_stage_launches",
    "ssd_chunk_scan_fwd_default_plan",
    "ssd_chunk_scan_fwd_ex",
    "ssd_chunk_scan_fwd_noalloc",
    "ssd_decode_step",
    "ssd_chunk_scan_fwd_tune",
    "ssd_chunk_scan_bwd_workspace_size",
    "ssd_chunk_scan_bwd",
    "ssd_chunk_scan_bwd_profiled",
    "ssd_chunk_scan_bwd_saved",
    "ssd_status_string",
    "ssd_version",
]


class SSDError(RuntimeError):
    """A non-OK status from libssd."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s: %s (%s)" % (where, STATUS.get(status, "status %d" % status), status_string(status))
        super().__init__(msg)


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("ngroups", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("y_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [
        ("g2_hi", ctypes.c_size_t),
        ("g2_lo", ctypes.c_size_t),
        ("dt", ctypes.c_size_t),
        ("w", ctypes.c_size_t),
        ("s", ctypes.c_size_t),
        ("h", ctypes.c_size_t),
        ("cb", ctypes.c_size_t),
        ("total", ctypes.c_size_t),
        ("nchunks", ctypes.c_int64),
        ("padded_len", ctypes.c_int64),
    ]


SSD_STATE_SPLIT = 0
SSD_STATE_FUSED = 1


class Plan(ctypes.Structure):
    """ssd_plan: how the stages divide their work among thread blocks."""
    _fields_ = [
        ("state_path", ctypes.c_int32),
        ("chunk_state_heads", ctypes.c_int32),
        ("chunk_out_heads", ctypes.c_int32),
        ("fused_cols", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 4),
    ]

    def as_dict(self) -> dict:
        return {"state_path": "fused" if self.state_path == SSD_STATE_FUSED else "split",
                "chunk_state_heads": self.chunk_state_heads,
                "chunk_out_heads": self.chunk_out_heads, "fused_cols": self.fused_cols}

    def __repr__(self):
        return "Plan(%s)" % ", ".join("%s=%s" % kv for kv in self.as_dict().items())


def make_plan(state_path="split", chunk_state_heads=1, chunk_out_heads=1, fused_cols=0) -> Plan:
    sp = SSD_STATE_FUSED if state_path in ("fused", SSD_STATE_FUSED) else SSD_STATE_SPLIT
    return Plan(sp, chunk_state_heads, chunk_out_heads, fused_cols)


_lock = threading.Lock()
_lib = None


def load_library(path: str | None = None):
    """Load libssd.so (built in-tree by ``mamba_chunked_ssd_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                "libssd.so is not built (%s); run `python -m mamba_chunked_ssd_amd.build` "
                "or __graft_entry__.build()" % p)
        lib = ctypes.CDLL(p)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        sp = ctypes.POINTER(Shape)
        lib.ssd_chunk_scan_fwd_workspace_size.argtypes = [sp, i64]
        lib.ssd_chunk_scan_fwd_workspace_size.restype = sz
        lib.ssd_chunk_scan_fwd_workspace_layout.argtypes = [sp, i64, ctypes.POINTER(WorkspaceLayout)]
        lib.ssd_chunk_scan_fwd_workspace_layout.restype = ctypes.c_int
        fwd_args = [sp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
        lib.ssd_chunk_scan_fwd.argtypes = fwd_args
        lib.ssd_chunk_scan_fwd.restype = ctypes.c_int
        lib.ssd_chunk_scan_fwd_profiled.argtypes = fwd_args + [ctypes.POINTER(ctypes.c_void_p)]
        lib.ssd_chunk_scan_fwd_profiled.restype = ctypes.c_int
        pp = ctypes.POINTER(Plan)
        lib.ssd_chunk_scan_fwd_stage_launches.argtypes = [sp, i64, pp, ctypes.POINTER(ctypes.c_uint32)]
        lib.ssd_chunk_scan_fwd_stage_launches.restype = ctypes.c_int
        lib.ssd_chunk_scan_fwd_default_plan.argtypes = [sp, i64, pp]
        lib.ssd_chunk_scan_fwd_default_plan.restype = ctypes.c_int
        lib.ssd_chunk_scan_fwd_ex.argtypes = fwd_args + [pp, ctypes.POINTER(ctypes.c_void_p)]
        lib.ssd_chunk_scan_fwd_ex.restype = ctypes.c_int
        lib.ssd_chunk_scan_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp]
        lib.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
        lib.ssd_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_void_p)]
        lib.ssd_decode_step.restype = ctypes.c_int
        lib.ssd_chunk_scan_fwd_tune.argtypes = fwd_args + [ctypes.c_int, pp, ctypes.POINTER(ctypes.c_float)]
        lib.ssd_chunk_scan_fwd_tune.restype = ctypes.c_int
        lib.ssd_chunk_scan_bwd_workspace_size.argtypes = [sp, i64]
        lib.ssd_chunk_scan_bwd_workspace_size.restype = sz
        bwd_args = [sp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.ssd_chunk_scan_bwd.argtypes = bwd_args
        lib.ssd_chunk_scan_bwd.restype = ctypes.c_int
        lib.ssd_chunk_scan_bwd_profiled.argtypes = bwd_args + [ctypes.POINTER(ctypes.c_void_p)]
        lib.ssd_chunk_scan_bwd_profiled.restype = ctypes.c_int
        # as bwd_args, with the forward workspace and its size after d_final_states
        lib.ssd_chunk_scan_bwd_saved.argtypes = bwd_args[:11] + [vp, sz] + bwd_args[11:] + [
            ctypes.POINTER(ctypes.c_void_p)]
        lib.ssd_chunk_scan_bwd_saved.restype = ctypes.c_int
        lib.ssd_status_string.argtypes = [ctypes.c_int]
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_version.argtypes = []
        lib.ssd_version.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load_library().ssd_status_string(status).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


def _dtype_code(dtype) -> int:
    if dtype in ("bf16", SSD_DTYPE_BF16):
        return SSD_DTYPE_BF16
    if dtype in ("f32", SSD_DTYPE_F32):
        return SSD_DTYPE_F32
    raise ValueError("dtype must be 'f32' or 'bf16'")


def make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, keep=False,
               y_dtype="f32") -> Shape:
    return Shape(batch, seqlen, nheads, headdim, dstate, ngroups, _dtype_code(dtype),
                 SSD_FLAG_KEEP_INTERMEDIATES if keep else 0, _dtype_code(y_dtype), 0)


def workspace_size(shape: Shape, chunk_size: int) -> int:
    return int(load_library().ssd_chunk_scan_fwd_workspace_size(ctypes.byref(shape), chunk_size))


def workspace_layout(shape: Shape, chunk_size: int) -> WorkspaceLayout:
    lay = WorkspaceLayout()
    st = load_library().ssd_chunk_scan_fwd_workspace_layout(ctypes.byref(shape), chunk_size,
                                                            ctypes.byref(lay))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_workspace_layout")
    return lay


STAGES = ("chunk_cumsum", "chunk_state", "state_pass", "chunk_out")


def default_plan(shape: Shape, chunk_size: int) -> Plan:
    """The launch plan ``ssd_chunk_scan_fwd`` uses for this problem (host only)."""
    plan = Plan()
    st = load_library().ssd_chunk_scan_fwd_default_plan(ctypes.byref(shape), chunk_size,
                                                        ctypes.byref(plan))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_default_plan")
    return plan


def _plan_ref(plan):
    return None if plan is None else ctypes.byref(plan)


def stage_launches(shape: Shape, chunk_size: int, plan: Plan | None = None) -> tuple:
    """Names of the stages that launch a kernel of their own for this problem
    (under ``plan``; None = the default plan)."""
    mask = ctypes.c_uint32()
    st = load_library().ssd_chunk_scan_fwd_stage_launches(ctypes.byref(shape), chunk_size,
                                                          _plan_ref(plan), ctypes.byref(mask))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_stage_launches")
    return tuple(n for i, n in enumerate(STAGES) if mask.value >> i & 1)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _torch():
    import torch
    return torch


def _check(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def chunk_scan_fwd(x, dt, A, B, C, D=None, chunk_size: int = 256, initial_states=None,
                   return_final_states: bool = False, *, y_dtype=None, out=None,
                   final_out=None, workspace=None, keep_intermediates: bool = False,
                   stream=None, events=None, plan: Plan | None = None):
    """Run ``ssd_chunk_scan_fwd`` on the current (or given) stream.

    x (b, L, nh, p) and dt (b, L, nh), B/C (b, L, g, n): float32 or bfloat16,
    all the same dtype; A (nh,), D (nh,) or None, initial_states
    (b, nh, p, n) or None: float32.  ``y_dtype`` (torch dtype): float32 (the
    default) or the input dtype.  Returns y, or (y, final_states).
    ``workspace`` (uint8 device tensor) may be passed to reuse an allocation;
    with ``keep_intermediates`` its layout is :func:`workspace_layout` of the
    shape with the keep flag.  ``events``: 8 raw hipEvent_t handles (ints), a
    (start, stop) pair per stage recorded by each kernel's own dispatch
    (``ssd_chunk_scan_fwd_profiled``).  ``plan``: an explicit launch plan
    (:class:`Plan`; ``ssd_chunk_scan_fwd_ex``), None for the default one.
    """
    torch = _torch()
    lib = load_library()
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x and B must be 4-D")
    b, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    if x.dtype == torch.bfloat16:
        dname = "bf16"
    elif x.dtype == torch.float32:
        dname = "f32"
    else:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a ROCm device (got %s)" % dev)
    _check(x, "x", x.dtype, (b, L, nh, p), dev)
    _check(dt, "dt", x.dtype, (b, L, nh), dev)
    _check(A, "A", torch.float32, (nh,), dev)
    _check(B, "B", x.dtype, (b, L, g, n), dev)
    _check(C, "C", x.dtype, (b, L, g, n), dev)
    if D is not None:
        _check(D, "D", torch.float32, (nh,), dev)
    if initial_states is not None:
        _check(initial_states, "initial_states", torch.float32, (b, nh, p, n), dev)
    ytype = torch.float32 if y_dtype is None else y_dtype
    if ytype not in (torch.float32, x.dtype):
        raise TypeError("y_dtype must be float32 or the input dtype")
    shape = make_shape(b, L, nh, p, n, g, dname, keep_intermediates,
                       "bf16" if ytype == torch.bfloat16 else "f32")
    need = workspace_size(shape, chunk_size)  # 0 if invalid: the call reports why
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    y = out if out is not None else torch.empty((b, L, nh, p), dtype=ytype, device=dev)
    if out is not None:
        _check(out, "out", ytype, (b, L, nh, p), dev)
    fin = None
    if return_final_states or final_out is not None:
        fin = final_out if final_out is not None else torch.empty((b, nh, p, n), dtype=torch.float32, device=dev)
        _check(fin, "final_states", torch.float32, (b, nh, p, n), dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    args = [ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            int(chunk_size), _ptr(initial_states), _ptr(y), _ptr(fin), _ptr(workspace),
            workspace.numel() * workspace.element_size(), ctypes.c_void_p(s)]
    ev = None
    if events is not None:
        if len(events) != 8:
            raise ValueError("events: a (start, stop) pair for each of the 4 stages")
        ev = (ctypes.c_void_p * 8)(*[ctypes.c_void_p(e) for e in events])
    if plan is not None:
        st = lib.ssd_chunk_scan_fwd_ex(*args, ctypes.byref(plan), ev)
        where = "ssd_chunk_scan_fwd_ex"
    elif ev is None:
        st = lib.ssd_chunk_scan_fwd(*args)
        where = "ssd_chunk_scan_fwd"
    else:
        st = lib.ssd_chunk_scan_fwd_profiled(*args, ev)
        where = "ssd_chunk_scan_fwd_profiled"
    if st != 0:
        raise SSDError(st, where)
    if return_final_states:
        return y, fin
    return y


BWD_STAGES = ("chunk_cumsum", "chunk_state", "state_pass", "adjoint_chunk_state", "adjoint_carry",
              "score_tiles", "dx_pass", "dB_pass", "dC_pass", "w_sums", "token_finish", "reduce")


def bwd_workspace_size(shape: Shape, chunk_size: int) -> int:
    return int(load_library().ssd_chunk_scan_bwd_workspace_size(ctypes.byref(shape), chunk_size))


def chunk_scan_bwd(x, dt, A, B, C, D, dy, chunk_size: int = 256, initial_states=None,
                   d_final_states=None, *, want_dD: bool = True, want_d_initial: bool = True,
                   workspace=None, stream=None, events=None, saved_workspace=None):
    """Gradients through :func:`chunk_scan_fwd` (``ssd_chunk_scan_bwd``).

    Inputs as passed to :func:`chunk_scan_fwd`, plus ``dy`` (dL/dy, the input
    dtype), and optionally
    ``d_final_states`` (dL/dh_final, float32).  Returns a dict of float32
    tensors ``dx, ddt, dA, dB, dC`` and, when requested, ``dD`` and
    ``d_initial_states``.  ``events``: 24 raw hipEvent_t handles (a start and
    stop per stage of :data:`BWD_STAGES`).  ``saved_workspace``: the workspace
    of a :func:`chunk_scan_fwd` call on the same inputs made with
    ``keep_intermediates=True``; its chunk-start states are then read instead
    of recomputed (``ssd_chunk_scan_bwd_saved``).
    """
    torch = _torch()
    lib = load_library()
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x and B must be 4-D")
    b, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    if x.dtype == torch.bfloat16:
        dname = "bf16"
    elif x.dtype == torch.float32:
        dname = "f32"
    else:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a ROCm device (got %s)" % dev)
    _check(x, "x", x.dtype, (b, L, nh, p), dev)
    _check(dt, "dt", x.dtype, (b, L, nh), dev)
    _check(A, "A", torch.float32, (nh,), dev)
    _check(B, "B", x.dtype, (b, L, g, n), dev)
    _check(C, "C", x.dtype, (b, L, g, n), dev)
    if D is not None:
        _check(D, "D", torch.float32, (nh,), dev)
    if initial_states is not None:
        _check(initial_states, "initial_states", torch.float32, (b, nh, p, n), dev)
    _check(dy, "dy", x.dtype, (b, L, nh, p), dev)
    if d_final_states is not None:
        _check(d_final_states, "d_final_states", torch.float32, (b, nh, p, n), dev)
    shape = make_shape(b, L, nh, p, n, g, dname)
    need = bwd_workspace_size(shape, chunk_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {
        "dx": torch.empty((b, L, nh, p), **f32), "ddt": torch.empty((b, L, nh), **f32),
        "dA": torch.empty((nh,), **f32), "dB": torch.empty((b, L, g, n), **f32),
        "dC": torch.empty((b, L, g, n), **f32),
    }
    if want_dD:
        out["dD"] = torch.empty((nh,), **f32)
    if want_d_initial:
        out["d_initial_states"] = torch.empty((b, nh, p, n), **f32)
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    args = [ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), int(chunk_size),
            _ptr(initial_states), _ptr(dy), _ptr(d_final_states), _ptr(out["dx"]), _ptr(out["ddt"]),
            _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")),
            _ptr(out.get("d_initial_states")), _ptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(s)]
    ev = None
    if events is not None:
        if len(events) != 2 * len(BWD_STAGES):
            raise ValueError("events: a (start, stop) pair for each of the %d stages" % len(BWD_STAGES))
        ev = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e) for e in events])
    if saved_workspace is not None:
        if saved_workspace.device != dev:
            raise ValueError("saved_workspace must be on %s" % dev)
        saved = [_ptr(saved_workspace), saved_workspace.numel() * saved_workspace.element_size()]
        st = lib.ssd_chunk_scan_bwd_saved(*(args[:11] + saved + args[11:]), ev)
        where = "ssd_chunk_scan_bwd_saved"
    elif ev is None:
        st = lib.ssd_chunk_scan_bwd(*args)
        where = "ssd_chunk_scan_bwd"
    else:
        st = lib.ssd_chunk_scan_bwd_profiled(*args, ev)
        where = "ssd_chunk_scan_bwd_profiled"
    if st != 0:
        raise SSDError(st, where)
    return out


def decode_step(x, dt, A, B, C, D, state, *, y_dtype=None, out=None, stream=None, events=None):
    """One recurrent step for one new token per sequence (``ssd_decode_step``).

    x (b, nh, p) and dt (b, nh), B/C (b, g, n): float32 or bfloat16, all the
    same dtype; A (nh,), D (nh,) or None: float32; ``state`` (b, nh, p, n)
    float32 is updated in place.  Returns y (b, nh, p) (``y_dtype``: float32,
    the default, or the input dtype).  ``events``: 2 raw hipEvent_t handles
    (start, stop) recorded by the kernel's own dispatch.
    """
    torch = _torch()
    lib = load_library()
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be (batch, nheads, headdim) and B (batch, ngroups, dstate)")
    b, nh, p = x.shape
    g, n = B.shape[1], B.shape[2]
    if x.dtype == torch.bfloat16:
        dname = "bf16"
    elif x.dtype == torch.float32:
        dname = "f32"
    else:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    _check(x, "x", x.dtype, (b, nh, p), dev)
    _check(dt, "dt", x.dtype, (b, nh), dev)
    _check(A, "A", torch.float32, (nh,), dev)
    _check(B, "B", x.dtype, (b, g, n), dev)
    _check(C, "C", x.dtype, (b, g, n), dev)
    if D is not None:
        _check(D, "D", torch.float32, (nh,), dev)
    _check(state, "state", torch.float32, (b, nh, p, n), dev)
    ytype = torch.float32 if y_dtype is None else y_dtype
    if ytype not in (torch.float32, x.dtype):
        raise TypeError("y_dtype must be float32 or the input dtype")
    y = out if out is not None else torch.empty((b, nh, p), dtype=ytype, device=dev)
    _check(y, "out", ytype, (b, nh, p), dev)
    shape = make_shape(b, 1, nh, p, n, g, dname, False, "bf16" if ytype == torch.bfloat16 else "f32")
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    ev = None
    if events is not None:
        if len(events) != 2:
            raise ValueError("events: one (start, stop) pair")
        ev = (ctypes.c_void_p * 2)(*[ctypes.c_void_p(e) for e in events])
    st = lib.ssd_decode_step(ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(state), _ptr(y), ctypes.c_void_p(s), ev)
    if st != 0:
        raise SSDError(st, "ssd_decode_step")
    return y


def tune(x, dt, A, B, C, D=None, chunk_size: int = 256, initial_states=None, *, reps: int = 5,
         y_dtype=None, out=None, final_out=None, workspace=None, stream=None):
    """Run ``ssd_chunk_scan_fwd_tune`` on these inputs: returns ``(plan, us)``,
    the fastest launch plan found and its time in microseconds.  Pass the plan
    to :func:`chunk_scan_fwd` (``plan=``) for later calls of the same shape."""
    torch = _torch()
    lib = load_library()
    b, L, nh, p = x.shape
    g, n = B.shape[2], B.shape[3]
    dname = "bf16" if x.dtype == torch.bfloat16 else "f32"
    dev = x.device
    ytype = torch.float32 if y_dtype is None else y_dtype
    shape = make_shape(b, L, nh, p, n, g, dname, False, "bf16" if ytype == torch.bfloat16 else "f32")
    for name, t, dtp, shp in (("x", x, x.dtype, (b, L, nh, p)), ("dt", dt, x.dtype, (b, L, nh)),
                              ("A", A, torch.float32, (nh,)), ("B", B, x.dtype, (b, L, g, n)),
                              ("C", C, x.dtype, (b, L, g, n))):
        _check(t, name, dtp, shp, dev)
    if D is not None:
        _check(D, "D", torch.float32, (nh,), dev)
    if initial_states is not None:
        _check(initial_states, "initial_states", torch.float32, (b, nh, p, n), dev)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(shape, chunk_size), 1), dtype=torch.uint8, device=dev)
    y = out if out is not None else torch.empty((b, L, nh, p), dtype=ytype, device=dev)
    fin = final_out if final_out is not None else torch.empty((b, nh, p, n), dtype=torch.float32, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    plan = Plan()
    us = ctypes.c_float()
    st = lib.ssd_chunk_scan_fwd_tune(ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                     int(chunk_size), _ptr(initial_states), _ptr(y), _ptr(fin), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), ctypes.c_void_p(s), int(reps),
                                     ctypes.byref(plan), ctypes.byref(us))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_tune")
    return plan, float(us.value)

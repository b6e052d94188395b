"""Build libssd.so (gfx950) in-tree with hipcc.

Each translation unit under ``csrc/`` is compiled separately (in parallel) and
linked into ``mamba_chunked_ssd_amd/libssd.so``.  Usage:

    python -m mamba_chunked_ssd_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libssd.so")
SOURCES = ["ssd_api.cpp", "ssd_tune.cpp", "ssd_bwd.cpp", "k1_cumsum.hip", "k2_chunk_state.hip", "k3_state_pass.hip",
           "k23_state_fused.hip", "k5_decode_step.hip", "k4_out_bf16_f32.hip", "k4_out_bf16_bf16.hip",
           "k4_out_f32.hip", "ssd_noalloc.hip", "kb_aux.hip", "kb_pass_q.hip", "kb_pass_b.hip", "kb_pass_c.hip"]
HEADERS = ["ssd_device.h", "ssd_internal.h", "ssd_host.h", "ssd_launch.h", "k_cb_tiles.h", "k4_chunk_out.h",
           "kb_pass.h", "kb_pass_inst.h"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; libssd needs ROCm's hipcc to build")
    return path


def flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
        # no packed-fp32 VALU ops on this target
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
        "-I" + os.path.join(HERE, "..", "include"),
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + flags()
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libssd.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()

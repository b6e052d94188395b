"""Host logic of bench.py (CPU): the algorithmic byte model behind the
roofline fractions, the counter-measured traffic table, and the one-GPU
guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ssd_inputs as si  # noqa: E402

MB = 1e6


def test_chunk_output_bytes_from_its_tensors():
    # The 2.7B-shaped layer (batch 2, seqlen 2048, 80 heads, headdim 64,
    # dstate 128, chunk 256, bf16 in, fp32 y), tensor by tensor: x read, y
    # written, the per-token G2 pair / dt tables (2 + 4 bytes per token and
    # head as the model counts them), C read, the chunk's C B^T tiles read in
    # place of B (8 waves x 18 slots of 1 KiB per chunk), the chunk-start
    # states read.
    w = si.BY_NAME["mamba2_2p7b_layer_bf16"]
    tok_h = 2 * 2048 * 80
    x = tok_h * 64 * 2
    y = tok_h * 64 * 4
    tables = tok_h * (2 + 4)
    c_rows = 2 * 2048 * 1 * 128 * 2
    cb_tiles = 2 * 8 * 1 * 8 * 18 * 1024
    states = 4 * 2 * 80 * 8 * 64 * 128
    want = x + y + tables + c_rows + cb_tiles + states
    assert bench.stage_model(w, 4)["chunk_out"][0] == want


@pytest.mark.parametrize("name, stage, fused, mb", [
    ("mamba2_2p7b_layer_bf16", "chunk_state", False, 86.90),
    ("mamba2_2p7b_layer_bf16", "state_pass", False, 93.59),
    ("mamba2_2p7b_layer_bf16", "chunk_out", False, 173.15),
    ("mamba2_2p7b_layer_bf16", "chunk_state", True, 96.60),
    ("long_seq_bf16", "chunk_out", False, 1426.06),
    ("grouped_f32", "chunk_out", False, 9697.23),
])
def test_stage_model_matches_the_published_tables(name, stage, fused, mb):
    # the algorithmic megabytes the profile tables and the design notes quote
    w = si.BY_NAME[name]
    assert bench.stage_model(w, 4, fused=fused)[stage][0] / MB == pytest.approx(mb, abs=0.005)


def test_fused_model_drops_the_state_pass():
    w = si.BY_NAME["throughput_bf16"]
    m = bench.stage_model(w, 4, fused=True)
    assert m["state_pass"] == (0, 0.0)
    assert m["chunk_state"][1] == bench.stage_model(w, 4)["chunk_state"][1]


@pytest.mark.parametrize("key", sorted(bench.MEASURED_TRAFFIC, key=str))
def test_measured_traffic_belongs_to_the_current_sources(key):
    # every counter-measured entry was taken on the kernel sources in the
    # tree (else bench.py reports its traffic as null and the counters must
    # be taken again)
    workload, y_dtype, stage, path = key
    got = bench.measured_traffic(workload, y_dtype, stage, {"state_path": path} if path else None)
    assert got is not None and got > 0
    fetch_kib, write_kib = bench.MEASURED_TRAFFIC[key][2:]
    assert got == int(round((fetch_kib * bench.FETCH_SCALE + write_kib * bench.WRITE_SCALE) * 1024))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()

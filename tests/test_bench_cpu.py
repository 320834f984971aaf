"""Host-side checks of bench.py (no GPU): the algorithmic byte and FLOP
counts its rooflines divide by, the one-GPU contract, and that the recorded
HBM counters in profiles/ belong to the kernel sources as they stand."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_chunk_bytes_headline():
    """B=8, T=4096, H=16, d=128, bf16: 2,048 bytes per (token, head) -- q, k,
    b, v, w and o at 256 bytes each, alpha at 512 -- plus the FP32 state read
    and written once per (sequence, head)."""
    per_token_head = 5 * 128 * 2 + 128 * 4 + 128 * 2
    assert per_token_head == 2048
    expect = 8 * 4096 * 16 * per_token_head + 2 * 8 * 16 * 128 * 128 * 4
    assert expect == 1_090_519_040
    assert bench.chunk_bytes(8, 4096, 16, 128, 128, 8) == expect
    # at the 8 TB/s peak: 136.3 us per launch
    assert abs(expect / 8e12 * 1e6 - 136.3) < 0.1


@pytest.mark.parametrize("gates,per_token_head", [(0, 2048), (5, 1538), (13, 1030), (1, 1794), (8, 1540)])
def test_chunk_bytes_gate_layouts(gates, per_token_head):
    """Compact layouts: a scalar gate is one bf16 (erase, write) or FP32
    (decay) value per (token, head); a tied write gate is not read."""
    state = 2 * 1 * 1 * 128 * 128 * 4
    assert bench.chunk_bytes(1, 1, 1, 128, 128, 1, gates=gates) - state == per_token_head


def test_decode_step_bytes():
    """N=256, H=16, d=128: the 64 KiB FP32 state read and written, the bf16
    token vectors and the FP32 alpha read, o written: 133,120 bytes per
    (sequence, head) and step."""
    per = 2 * 128 * 128 * 4 + 3 * 128 * 2 + 2 * 128 * 2 + 128 * 4 + 128 * 2
    assert per == 133_120
    assert bench.step_bytes(256, 16, 128, 128) == 256 * 16 * per == 545_259_520


def test_chunk_flops_per_chunk():
    """Triangle-aware FLOPs of one 64-token chunk and head at d=128, counted
    term by term: A (64 x 63 products over 128 channels), P (64 x 65), the
    triangular inverse (64^3 / 3), T [Et | Z] (lower triangular, 256 wide),
    W S, Qt S and Kb^T U (three 64 x 128 x 128 products), P U."""
    L, d = 64, 128
    terms = [d * L * (L - 1), d * L * (L + 1), L ** 3 / 3, 2 * d * L * (L + 1), 3 * 2 * L * d * d, d * L * (L + 1)]
    assert abs(sum(terms) - 9.02e6) < 0.01e6
    assert abs(bench.chunk_flops([L], 1, d, d) - sum(terms)) < 1e-6
    # a ragged tail counts as a shorter chunk
    assert abs(bench.chunk_flops([L + 10], 1, d, d) - sum(terms) - bench.chunk_flops([10], 1, d, d)) < 1e-6


def test_more_than_one_gpu_is_refused():
    """The build measures one GPU: --gpus 2 exits with status 2 and says so,
    before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("part", ["chunk", "decode"])
def test_recorded_counters_match_the_sources(part):
    """profiles/pmc_traffic.json holds the FETCH_SIZE/WRITE_SIZE traffic of
    the chunk and decode kernels with a digest of the code it was taken on;
    it must be the current code, so that bench.py reports it, and the traffic
    must be within 0.1% of the algorithmic bytes (no wasted re-reads)."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "pmc_traffic.json")))["kernels"][part]
    assert rec["source_digest"] == bench.source_digest(part)
    assert bench.pmc_traffic(part) == rec["traffic_bytes"]
    ratio = rec["traffic_bytes"] / rec["algorithmic_bytes"]
    assert 1.0 <= ratio < 1.001
    algo = bench.chunk_bytes(8, 4096, 16, 128, 128, 8) if part == "chunk" else bench.step_bytes(256, 16, 128, 128)
    assert rec["algorithmic_bytes"] == algo

"""Host-side checks of bench.py (no GPU): the algorithmic work it divides by
is the count of the chunked method (restated here from its terms, not from
bench.py's code), and more than one GPU is refused with a message."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from test_learned_neural_amd import workloads as wl  # noqa: E402


def test_forward_work_of_the_headline_memory():
    # 2-layer d=64 h=256 memory, chunk 64: P = 2*64*256; per token the key
    # forward (P MACs), the backprop (P - d h), the two weighted reductions
    # (2P) and the read after write (2P + b * ((64 + 256) + (256 + 64))).
    cfg = wl.WORKLOADS["headline"]
    P, dh, b = 2 * 64 * 256, 64 * 256, 64
    macs = P + (P - dh) + 2 * P + 2 * P + b * 640
    flops, byts = bench.algorithmic_work(cfg)
    assert flops == 2 * macs == 442368
    # k, v, q, y in bf16, three fp32 gates, state read and written once over N
    assert byts == pytest.approx(4 * 64 * 2 + 12 + 4 * P * 4 / cfg.N)


def test_backward_work_of_the_headline_memory():
    # per token: state sweep 8P - 2dh, reverse products 32P - 6dh, and the
    # reads' [b x b] products b (2 (64 + 256 + 256) + 4 (320 + 320))
    cfg = wl.WORKLOADS["headline"].with_(N=1024)
    P, dh, b = 2 * 64 * 256, 64 * 256, 64
    expected = (8 * P - 2 * dh) + (32 * P - 6 * dh) + b * (2 * (64 + 256 + 256) + 4 * (320 + 320))
    assert bench.backward_flops_per_token(cfg) == expected == 1417216


def test_input_side_work():
    icfg = wl.INPUT_CONFIGS["headline"]
    R = icfg.B * icfg.N
    flops, _ = bench.input_side_work(icfg)
    assert flops == 2.0 * R * 1024 * 3 * (16 * 64 + 16)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr

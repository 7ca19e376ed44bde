"""GPU parity of titans_mem_retrieve on the matrix cores (2-layer d=64
hidden=256 bf16 memory) against the fp64 oracle's memory forward.

bf16 operands (the state rounded once, the activations once) and fp32 sums:
the bar is the bf16-io tolerance, 2e-2 norm-wise per stream (measured errors
are a few 1e-3).  Cases: ragged token counts around the 64-token tile and
the 1024-token workgroup range, several streams, a state of tiny magnitude
(bf16 keeps fp32's exponent range), the generic path on the same inputs,
and the headline shape (128 streams x 16,384 tokens) on sampled tokens.
"""
import numpy as np
import pytest

import oracle
from test_learned_neural_amd import workloads as wl
from parity_util import rel_err, to_device, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from test_learned_neural_amd import titans_mem as tmm
    assert tmm.select_path(tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16"), 64) == tmm.PATH_MLP2_D64_H256
    return torch


def _ref(W64, q64, tokens):
    return np.stack([oracle.memory_apply(W64, q64[t], 64, 256, 2) for t in tokens])


@pytest.mark.parametrize("B,H,N,scale", [(1, 1, 1, 1.0), (1, 3, 63, 1.0), (2, 2, 1030, 3.0), (1, 2, 2111, 1.0),
                                         (1, 1, 200, 1e-12)])
def test_retrieve_mfma(B, H, N, scale):
    """scale 1e-12: a state of tiny magnitude whose outputs (~1e-24) are
    still normal fp32 numbers, so the comparison is not vacuous."""
    from test_learned_neural_amd import titans_mem as tmm
    cfg = wl.WORKLOADS["headline"].with_(B=B, H=H, N=N)
    inp = wl.make_inputs(cfg)
    dev = to_device(cfg, inp)
    W = dev["W0"] * scale
    y = tmm.retrieve(dev["q"], W, hidden=256, n_layers=2)
    yg = y_to_f64(cfg, y)
    q64 = wl.io_to_f64(inp["q"], "bf16")
    W64 = W.reshape(-1, cfg.param_count).cpu().double().numpy()
    worst = 0.0
    for s in range(B * H):
        ref = _ref(W64[s], q64[s], range(N))
        e = rel_err(yg[s], ref, 1e-38)
        worst = max(worst, e)
        assert e < 2e-2, (s, e)
    print(f"retrieve B{B} H{H} N{N} scale {scale:g}: max error {worst:.2e}", flush=True)


def test_retrieve_mfma_matches_generic():
    import torch
    from test_learned_neural_amd import titans_mem as tmm
    cfg = wl.WORKLOADS["headline"].with_(B=2, H=2, N=333)
    inp = wl.make_inputs(cfg)
    dev = to_device(cfg, inp)
    a = tmm.retrieve(dev["q"], dev["W0"], hidden=256, n_layers=2).float()
    b = tmm.retrieve(dev["q"], dev["W0"], hidden=256, n_layers=2, force_generic=True).float()
    for s in range(2):
        for h in range(2):
            assert torch.linalg.norm(a[s, h] - b[s, h]) <= 2e-2 * torch.linalg.norm(b[s, h])


def test_retrieve_mfma_headline_sampled():
    """All 128 streams x 16,384 tokens on the GPU; the oracle checks 12
    tokens per stream (first, last, range and tile seams, and a spread)."""
    from test_learned_neural_amd import titans_mem as tmm
    cfg = wl.WORKLOADS["headline"]
    inp = wl.make_inputs(cfg, workers=8)
    dev = to_device(cfg, inp)
    y = tmm.retrieve(dev["q"], dev["W0"], hidden=256, n_layers=2)
    tokens = [0, 63, 64, 1023, 1024, 5000, 8191, 8192, 12345, 15359, 16320, 16383]
    yg = y[:, :, tokens].float().cpu().double().numpy().reshape(cfg.streams, len(tokens), 64)
    q64 = wl.io_to_f64(inp["q"], "bf16")
    W64 = inp["W0"].astype(np.float64)
    worst = 0.0
    for s in range(cfg.streams):
        ref = _ref(W64[s], q64[s], tokens)
        e = rel_err(yg[s], ref, 1e-38)
        worst = max(worst, e)
        assert e < 2e-2, (s, e)
    print(f"retrieve headline sampled: max error {worst:.2e}", flush=True)

"""The allocation-free forward (titans_mem_forward_noalloc) against the
forward call with a caller workspace, through the C ABI.

Two calls in a row on the same GPU share the library's scratch; the second
has fewer streams, fewer tokens and a smaller chunk, so it runs on fewer
pairs over scratch the first call left behind.  Each must give bitwise the
results of titans_mem_forward on the same inputs (same kernels, same
order of operations) and match the fp64 oracle to the bf16-io bar.
"""
import numpy as np
import pytest

from test_learned_neural_amd import workloads as wl
from parity_util import TOL, run_gpu, run_oracle, stream_errors, to_device, y_row_errors, y_to_f64

pytestmark = pytest.mark.gpu


def _noalloc(cfg, dev, read_mode=0):
    import torch
    from test_learned_neural_amd import titans_mem as tmm
    desc = tmm.make_desc(cfg.B, cfg.H, cfg.N, cfg.d, cfg.hidden, cfg.n_layers, cfg.io, read_mode=read_mode)
    y = torch.empty_like(dev["k"])
    W = torch.empty_like(dev["W0"])
    S = torch.empty_like(dev["S0"])
    p = lambda t: int(t.data_ptr())
    rc = tmm.raw_forward_noalloc(desc, p(dev["k"]), p(dev["v"]), p(dev["q"]), p(dev["alpha"]), p(dev["eta"]),
                                 p(dev["theta"]), p(dev["W0"]), p(dev["S0"]), cfg.chunk, p(y), p(W), p(S),
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == tmm.OK, tmm.status_string(rc)
    status = tmm.raw_workspace_status(desc, cfg.chunk, 0, 0, torch.cuda.current_stream().cuda_stream)
    assert status == tmm.OK, tmm.status_string(status)
    return y, W, S


@pytest.mark.parametrize("read_mode", [0, 1])
def test_forward_noalloc_matches_forward(read_mode):
    import torch
    first = wl.WORKLOADS["headline"].with_(N=640)                      # 128 streams: every resident pair
    second = wl.WORKLOADS["mlp2_short"].with_(B=2, H=3, N=150, chunk=40)  # 6 streams, ragged chunks
    for cfg in (first, second):
        inp = wl.make_inputs(cfg, workers=8)
        dev = to_device(cfg, inp)
        got = _noalloc(cfg, dev, read_mode)
        want = run_gpu(cfg, dev, read_mode=read_mode)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b)
        ref = run_oracle(cfg, inp, read_mode=read_mode, threads=16)
        yg = y_to_f64(cfg, got[0])
        Wg = got[1].reshape(-1, cfg.param_count).cpu().double().numpy()
        Sg = got[2].reshape(-1, cfg.param_count).cpu().double().numpy()
        e = stream_errors(cfg, inp, yg, Wg, Sg, *ref)
        ry, at = y_row_errors(cfg, inp, yg, ref[0])
        print(f"noalloc {cfg.name} N={cfg.N} chunk={cfg.chunk} read_mode={read_mode}: max e_y {e[:, 0].max():.2e} "
              f"e_W {e[:, 1].max():.2e} e_S {e[:, 2].max():.2e} per token y {ry:.2e}", flush=True)
        assert np.all(e < TOL["bf16"]) and ry < TOL["bf16"]


def test_forward_noalloc_reports_give_up():
    """The no-wait test hook makes the allocation-free call's pairs give up:
    NaN outputs and the give-up status through the NULL-workspace query; the
    next call on the shared scratch completes and reports OK."""
    import torch
    from test_learned_neural_amd import titans_mem as tmm
    cfg = wl.WORKLOADS["headline"].with_(B=1, H=6, N=100)
    dev = to_device(cfg, wl.make_inputs(cfg))
    desc = tmm.make_desc(cfg.B, cfg.H, cfg.N, cfg.d, cfg.hidden, cfg.n_layers, cfg.io, flags=tmm.FLAG_NO_WAIT)
    y = torch.empty_like(dev["k"])
    W = torch.empty_like(dev["W0"])
    S = torch.empty_like(dev["S0"])
    p = lambda t: int(t.data_ptr())
    st = torch.cuda.current_stream().cuda_stream
    args = [p(dev[n]) for n in ("k", "v", "q", "alpha", "eta", "theta", "W0", "S0")]
    assert tmm.raw_forward_noalloc(desc, *args, cfg.chunk, p(y), p(W), p(S), st) == tmm.OK
    assert tmm.raw_workspace_status(desc, cfg.chunk, 0, 0, st) == tmm.ERR_GAVE_UP
    assert bool(torch.isnan(W).all()) and bool(torch.isnan(y.float()).all())
    _noalloc(cfg, dev)

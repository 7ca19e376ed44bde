"""GPU parity of the deep-memory matrix-core path (TM_PATH_DEEP_BF16) against
the fp64 oracle.

The path serves MLP memories of any depth >= 2 with widths that are
multiples of 64, bf16 io and chunks up to 256 (the deep workload: 4 layers,
d = 128, hidden 512, chunk 128).  Its products take bf16 operands with fp32
sums and its state stays fp32, so y, W and S are all held to the bf16-io bar
(2e-2): norm-wise per stream, y per window and per token, W and S per row
and column of every layer.
"""
import numpy as np
import pytest

from test_learned_neural_amd import workloads as wl
from parity_util import (TOL, chunk_gate_inputs, live_lengths, prefix_inputs, run_gpu, run_oracle,
                         state_below_floor, state_row_errors, stream_errors, to_device, window_errors, y_errors,
                         y_row_errors, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from test_learned_neural_amd import titans_mem as tmm
    cfg = wl.WORKLOADS["deep"]
    d = tmm.make_desc(cfg.B, cfg.H, cfg.N, cfg.d, cfg.hidden, cfg.n_layers, cfg.io)
    assert tmm.select_path(d, cfg.chunk) == tmm.PATH_DEEP_BF16
    return torch


def _np(cfg, out):
    y, W, S = out
    return (y_to_f64(cfg, y), W.reshape(-1, cfg.param_count).cpu().double().numpy(),
            S.reshape(-1, cfg.param_count).cpu().double().numpy())


def _check(cfg, inp, out, ref, idx=None, label="", rows=True):
    tol = TOL["bf16"]
    yg, Wg, Sg = _np(cfg, out)
    e = stream_errors(cfg, inp, yg, Wg, Sg, *ref[:3], idx=idx)
    we = window_errors(cfg, inp, yg, ref[0], idx=idx)
    ry, at_y = y_row_errors(cfg, inp, yg, ref[0], idx=idx)
    rW, at_W = state_row_errors(cfg, inp, Wg, ref[1], idx=idx)
    rS, at_S = state_row_errors(cfg, inp, Sg, ref[2], idx=idx)
    print(f"{label or cfg.name} L={cfg.n_layers} d={cfg.d} h={cfg.hidden} N={cfg.N} chunk={cfg.chunk}: "
          f"max e_y {e[:, 0].max():.2e} e_W {e[:, 1].max():.2e} e_S {e[:, 2].max():.2e} window_y {we:.2e} | "
          f"per token y {ry:.2e} at {at_y}, per row W {rW:.2e} at {at_W}, S {rS:.2e} at {at_S}", flush=True)
    assert np.all(e < tol), e.max(axis=0)
    assert we < tol, we
    assert ry < tol, (ry, at_y)
    if rows:
        assert rW < tol and rS < tol, (rW, at_W, rS, at_S)
    return e


def _path(cfg, **kw):
    from test_learned_neural_amd import titans_mem as tmm
    flags = tmm.FLAG_CHUNK_GATES if kw.get("chunk_gates") else 0
    d = tmm.make_desc(cfg.B, cfg.H, cfg.N, cfg.d, cfg.hidden, cfg.n_layers, cfg.io, kw.get("read_mode", 0), flags)
    return tmm.select_path(d, cfg.chunk)


def test_deep_prefix_all_streams():
    """The deep workload's 32 streams over a 2048-token prefix (16 chunks)."""
    cfg = wl.WORKLOADS["deep"].with_(N=2048)
    inp = wl.make_inputs(cfg, workers=16)
    out = run_gpu(cfg, to_device(cfg, inp))
    _check(cfg, inp, out, run_oracle(cfg, inp, threads=16))


@pytest.mark.parametrize("L,d,h,N,chunk", [(2, 64, 128, 300, 100), (3, 64, 192, 130, 64), (2, 128, 256, 77, 256),
                                           (4, 64, 64, 50, 1), (2, 64, 256, 200, 128), (5, 128, 128, 90, 32),
                                           (4, 128, 512, 260, 128)])
def test_deep_shapes_and_ragged_chunks(L, d, h, N, chunk):
    """Depths 2-5, square and rectangular layers, one-token chunks, a single
    ragged chunk, tails of 1-63 tokens past a multiple of 64."""
    from test_learned_neural_amd import titans_mem as tmm
    cfg = wl.WORKLOADS["deep"].with_(B=1, H=3, N=N, d=d, hidden=h, n_layers=L, chunk=chunk)
    assert _path(cfg) == tmm.PATH_DEEP_BF16
    inp = wl.make_inputs(cfg)
    _check(cfg, inp, run_gpu(cfg, to_device(cfg, inp)), run_oracle(cfg, inp, threads=8))


@pytest.mark.parametrize("wname,BH,N,chunk", [("deep", (1, 3), 300, 128), ("deep", (2, 2), 190, 64)])
def test_deep_chunk_start_read(wname, BH, N, chunk):
    """y_j = M_{W_0}(q_j), the state at the chunk start, against the oracle in
    the same read mode."""
    cfg = wl.WORKLOADS[wname].with_(B=BH[0], H=BH[1], N=N, chunk=chunk)
    inp = wl.make_inputs(cfg)
    out = run_gpu(cfg, to_device(cfg, inp), read_mode=1)
    _check(cfg, inp, out, run_oracle(cfg, inp, read_mode=1, threads=8), label="deep chunk-start read")


@pytest.mark.parametrize("read_mode", [0, 1])
def test_deep_chunk_gates(read_mode):
    """One alpha, eta, theta per chunk (TM_FLAG_CHUNK_GATES), ragged tail."""
    cfg = wl.WORKLOADS["deep"].with_(B=1, H=2, N=250)
    inp = chunk_gate_inputs(wl.make_inputs(cfg), cfg.chunk)
    out = run_gpu(cfg, to_device(cfg, inp), read_mode=read_mode, chunk_gates=True)
    ref = run_oracle(cfg, inp, read_mode=read_mode, chunk_gates=True, threads=8)
    _check(cfg, inp, out, ref, label=f"deep chunk gates, read mode {read_mode}")


def _edge_gates(inp, case):
    out = dict(inp)
    if "eta0" in case:
        out["eta"] = np.zeros_like(inp["eta"])
    if "alpha1" in case:
        out["alpha"] = np.ones_like(inp["alpha"])
    return out


@pytest.mark.parametrize("case", ["eta0", "alpha1", "eta0_alpha1"])
def test_deep_gate_edges_against_oracle(case):
    """eta = 0 and alpha = 1, where the coefficients must come out exact
    (products of zeros), on y, W and S with a ragged tail."""
    cfg = wl.WORKLOADS["deep"].with_(B=1, H=2, N=140)
    inp = _edge_gates(wl.make_inputs(cfg), case)
    _check(cfg, inp, run_gpu(cfg, to_device(cfg, inp)), run_oracle(cfg, inp, threads=8), label=f"deep {case}")


def test_deep_theta_zero_keeps_memory():
    """theta = 0: no gradient enters, S stays at its zero start and W decays
    by the product of (1 - alpha) exactly as in fp32."""
    import torch
    cfg = wl.WORKLOADS["deep"].with_(B=1, H=2, N=300)
    dev = to_device(cfg, wl.make_inputs(cfg))
    dz = dev | {"theta": torch.zeros_like(dev["theta"])}
    y, W, S = run_gpu(cfg, dz)
    assert not S.any()
    decay = torch.prod(1 - dev["alpha"].double(), dim=-1, keepdim=True)
    assert torch.allclose(W.double(), decay * dev["W0"].double(), rtol=1e-5, atol=0)


def test_deep_inplace_deterministic_and_split_resume():
    """Two runs agree bit for bit; an in-place call (W_out = W_in, S_out =
    S_in) gives the same result; two calls split at a chunk boundary give
    the one call's outputs bit for bit."""
    import torch
    cfg = wl.WORKLOADS["deep"].with_(B=1, H=3, N=512)
    dev = to_device(cfg, wl.make_inputs(cfg))
    y1, W1, S1 = run_gpu(cfg, dev)
    y2, W2, S2 = run_gpu(cfg, dev)
    assert torch.equal(y1, y2) and torch.equal(W1, W2) and torch.equal(S1, S2)
    Wi, Si = dev["W0"].clone(), dev["S0"].clone()
    y3, W3, S3 = run_gpu(cfg, dev | {"W0": Wi, "S0": Si}, W_out=Wi, S_out=Si)
    assert W3.data_ptr() == Wi.data_ptr()
    assert torch.equal(y3, y1) and torch.equal(W3, W1) and torch.equal(S3, S1)
    cut = 256
    tok = ("k", "v", "q", "alpha", "eta", "theta")
    first = {k: (v[:, :, :cut].contiguous() if k in tok else v) for k, v in dev.items()}
    ya, Wa, Sa = run_gpu(cfg.with_(N=cut), first)
    second = {k: (v[:, :, cut:].contiguous() if k in tok else v) for k, v in dev.items()}
    second["W0"], second["S0"] = Wa, Sa
    yb, Wb, Sb = run_gpu(cfg.with_(N=cfg.N - cut), second)
    assert torch.equal(torch.cat([ya, yb], dim=2), y1)
    assert torch.equal(Wb, W1) and torch.equal(Sb, S1)


def test_deep_memory_full_length():
    """The deep workload (4 x 8 streams, 32768 tokens, chunk 128) at full
    size in one call; prefix inputs are drawn bit-identically and outputs are
    causal, so an oracle run over a prefix is the reference for it:

    * every stream over the first 4096 tokens, y per token and window, with
      each stream's live length (it must end inside that prefix);
    * four sampled streams over the first 8192 tokens and over a window of
      tokens 12288-12543 (a run of the oracle from the start), y per token;
    * past each stream's live length, to the end: every output row below the
      y floor, and the final W and S below the state floor.
    """
    import torch
    cfg = wl.WORKLOADS["deep"]
    inp = wl.make_inputs(cfg, workers=16)
    y, W, S = run_gpu(cfg, to_device(cfg, inp))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool(torch.isfinite(W).all()) and bool(torch.isfinite(S).all())
    n_pre = 4096
    pre = cfg.with_(N=n_pre)
    sub = prefix_inputs(inp, n_pre)
    y_ref, _, _, wn = run_oracle(pre, sub, threads=16, want_w_norm=True)
    live = live_lengths(pre, sub, wn)
    assert max(live) < n_pre, live
    yg = y_to_f64(pre, y[:, :, :n_pre].contiguous())
    ey = y_errors(pre, sub, yg, y_ref)
    we = window_errors(pre, sub, yg, y_ref)
    ry, at = y_row_errors(pre, sub, yg, y_ref)
    print(f"{cfg.name}: prefix {n_pre} max e_y {ey.max():.2e} window_y {we:.2e} per token {ry:.2e} at {at}; "
          f"live length min {min(live)} max {max(live)}", flush=True)
    assert np.all(ey < TOL["bf16"]) and we < TOL["bf16"] and ry < TOL["bf16"], (ey.max(), we, ry, at)
    worst = 0.0
    yall = y_to_f64(cfg, y)
    for s in range(cfg.streams):
        floor = 1e-30 * max(1.0, float(np.linalg.norm(wl.io_to_f64(inp["v"][s], "bf16"))))
        worst = max(worst, float(np.max(np.linalg.norm(yall[s, live[s]:], axis=-1))) / floor)
    ok, es = state_below_floor(cfg, inp, W.reshape(-1, cfg.param_count).cpu().double().numpy(),
                               S.reshape(-1, cfg.param_count).cpu().double().numpy(), TOL["bf16"])
    print(f"{cfg.name}: past the live length max ||y_t|| / floor {worst:.2e}; final state vs zero {es:.2e}", flush=True)
    assert worst < TOL["bf16"], worst
    assert ok, es

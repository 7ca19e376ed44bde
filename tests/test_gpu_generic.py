"""GPU parity of the shape-generic fp32 kernel against the fp64 oracle.

Forced onto the generic path (TM_FLAG_FORCE_GENERIC) so that it is checked
even for shapes that also have a specialised kernel.  fp32 arithmetic, so
the bar is the fp32-io tolerance (1e-3) on every case.
"""
import numpy as np
import pytest

from test_learned_neural_amd import workloads as wl
from parity_util import (TOL, chunk_gate_inputs, live_lengths, prefix_inputs, rel_err, run_gpu, run_oracle,
                         state_below_floor, state_row_errors, stream_errors, to_device, window_errors, y_errors,
                         y_row_errors, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch


def _check(cfg, inp, out, ref, tol, idx=None, windows=True, label=""):
    """y is held to its io dtype's bar (bf16 output rounding alone is ~2e-3);
    W and S, fp32 end to end on this path, to ``tol``: norm-wise per stream,
    y per window and per token, W and S per row and column of every layer."""
    y, W, S = out
    tol_y = max(tol, TOL[cfg.io])
    yg = y_to_f64(cfg, y)
    Wg = W.reshape(-1, cfg.param_count).cpu().double().numpy()
    Sg = S.reshape(-1, cfg.param_count).cpu().double().numpy()
    e = stream_errors(cfg, inp, yg, Wg, Sg, *ref[:3], idx=idx)
    ry, at_y = y_row_errors(cfg, inp, yg, ref[0], idx=idx)
    rW, at_W = state_row_errors(cfg, inp, Wg, ref[1], idx=idx)
    rS, at_S = state_row_errors(cfg, inp, Sg, ref[2], idx=idx)
    print(f"{label or cfg.name}: max e_y {e[:, 0].max():.2e} e_W {e[:, 1].max():.2e} e_S {e[:, 2].max():.2e} | "
          f"per token y {ry:.2e} at {at_y}, per row W {rW:.2e} at {at_W}, S {rS:.2e} at {at_S}", flush=True)
    assert np.all(e[:, 0] < tol_y) and np.all(e[:, 1:] < tol), e.max(axis=0)
    assert ry < tol_y, (ry, at_y)
    assert rW < tol and rS < tol, (rW, at_W, rS, at_S)   # fp32 end to end: at every length
    if windows:
        we = window_errors(cfg, inp, yg, ref[0], idx=idx)
        assert we < tol_y, we


def test_generic_linear_config1_full():
    cfg = wl.WORKLOADS["linear"]
    inp = wl.make_inputs(cfg)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True)
    _check(cfg, inp, out, run_oracle(cfg, inp), TOL["f32"])


@pytest.mark.parametrize("wname,n_tokens,BH", [("mlp2_short", 640, (2, 3)), ("headline", 300, (1, 5)), ("deep", 300, (1, 3))])
def test_generic_mlp_prefix(wname, n_tokens, BH):
    cfg = wl.WORKLOADS[wname].with_(B=BH[0], H=BH[1], N=n_tokens)
    inp = wl.make_inputs(cfg)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True)
    _check(cfg, inp, out, run_oracle(cfg, inp), TOL["f32"])


@pytest.mark.parametrize("L,d,h,N,chunk,io", [(1, 16, 0, 77, 5, "f32"), (2, 16, 48, 130, 64, "f32"),
                                              (3, 24, 40, 97, 16, "bf16"), (2, 32, 96, 65, 1, "bf16"),
                                              (2, 64, 256, 50, 64, "bf16"), (4, 8, 20, 33, 200, "f32")])
def test_generic_shapes_and_ragged_chunks(L, d, h, N, chunk, io):
    cfg = wl.WORKLOADS["mlp2_short"].with_(B=1, H=2, N=N, d=d, hidden=h, n_layers=L, chunk=chunk, io=io)
    inp = wl.make_inputs(cfg)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True)
    _check(cfg, inp, out, run_oracle(cfg, inp), TOL["f32"], windows=False)


def test_generic_deep_memory_prefix_all_streams():
    """Deep memory, 2048-token prefix, all 32 streams, y, W and S."""
    cfg = wl.WORKLOADS["deep"].with_(N=2048)
    inp = wl.make_inputs(cfg, workers=16)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True)
    _check(cfg, inp, out, run_oracle(cfg, inp, threads=16), TOL["f32"])


def test_generic_read_chunk_start():
    cfg = wl.WORKLOADS["mlp2_short"].with_(B=1, H=3, N=200)
    inp = wl.make_inputs(cfg)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True, read_mode=1)
    _check(cfg, inp, out, run_oracle(cfg, inp, read_mode=1), TOL["f32"])


def test_retrieve_matches_memory_forward():
    import oracle
    from test_learned_neural_amd import titans_mem as tmm
    import torch
    for L, d, h in ((1, 64, 0), (2, 64, 256), (4, 128, 512), (3, 20, 36)):
        cfg = wl.WORKLOADS["mlp2_short"].with_(B=2, H=2, N=37, d=d, hidden=h, n_layers=L, io="bf16")
        inp = wl.make_inputs(cfg)
        dev = to_device(cfg, inp)
        W = dev["W0"] * 3.0
        y = tmm.retrieve(dev["q"], W, hidden=h, n_layers=L)
        yg = y_to_f64(cfg, y)
        q64 = wl.io_to_f64(inp["q"], "bf16")
        W64 = W.reshape(-1, cfg.param_count).cpu().double().numpy()
        for s in range(4):
            ref = np.stack([oracle.memory_apply(W64[s], q64[s, t], d, h, L) for t in range(cfg.N)])
            assert rel_err(yg[s], ref, 1e-30) < 2e-2
        torch.cuda.synchronize()


def test_generic_empty_inplace_and_deterministic():
    import torch
    cfg = wl.WORKLOADS["mlp2_short"].with_(B=1, H=2, N=0)
    inp = wl.make_inputs(cfg)
    dev = to_device(cfg, inp)
    y, W, S = run_gpu(cfg, dev, force_generic=True)
    assert torch.equal(W, dev["W0"]) and torch.equal(S, dev["S0"])
    cfg = wl.WORKLOADS["mlp2_short"].with_(B=1, H=2, N=150)
    inp = wl.make_inputs(cfg)
    dev = to_device(cfg, inp)
    y1, W1, S1 = run_gpu(cfg, dev, force_generic=True)
    y2, W2, S2 = run_gpu(cfg, dev, force_generic=True)
    assert torch.equal(y1, y2) and torch.equal(W1, W2) and torch.equal(S1, S2)
    Wi, Si = dev["W0"].clone(), dev["S0"].clone()
    y3, W3, S3 = run_gpu(cfg, dev | {"W0": Wi, "S0": Si}, force_generic=True, W_out=Wi, S_out=Si)
    assert W3.data_ptr() == Wi.data_ptr()
    assert torch.equal(y3, y1) and torch.equal(W3, W1) and torch.equal(S3, S1)


def test_generic_split_resume():
    import torch
    cfg = wl.WORKLOADS["mlp2_short"].with_(B=1, H=2, N=256)
    inp = wl.make_inputs(cfg)
    dev = to_device(cfg, inp)
    y, W, S = run_gpu(cfg, dev, force_generic=True)
    cut = 128
    first = {k: (v[:, :, :cut].contiguous() if k in ("k", "v", "q", "alpha", "eta", "theta") else v)
             for k, v in dev.items()}
    ya, Wa, Sa = run_gpu(cfg, first, force_generic=True)
    second = {k: (v[:, :, cut:].contiguous() if k in ("k", "v", "q", "alpha", "eta", "theta") else v)
              for k, v in dev.items()}
    second["W0"], second["S0"] = Wa, Sa
    yb, Wb, Sb = run_gpu(cfg, second, force_generic=True)
    assert torch.equal(torch.cat([ya, yb], dim=2), y)
    assert torch.equal(Wb, W) and torch.equal(Sb, S)


def test_generic_gate_edge_cases():
    import torch
    cfg = wl.WORKLOADS["mlp2_short"].with_(B=1, H=2, N=130)
    inp = wl.make_inputs(cfg)
    dev = to_device(cfg, inp)
    # theta = 0: surprise stays zero, W decays by the product of (1 - alpha)
    dz = dev | {"theta": torch.zeros_like(dev["theta"])}
    y, W, S = run_gpu(cfg, dz, force_generic=True)
    assert not S.any()
    decay = torch.prod(1 - dev["alpha"].double(), dim=-1, keepdim=True)
    assert torch.allclose(W.double(), decay * dev["W0"].double(), rtol=1e-5, atol=0)
    # alpha = 1: the old memory is erased at every token, so W == S (up to the
    # rounding of A_n W_0 + F_n S_0 - G versus E_n S_0 - G with A_n = 0, F_n = E_n)
    d1 = dev | {"alpha": torch.ones_like(dev["alpha"])}
    y, W, S = run_gpu(cfg, d1, force_generic=True)
    # (norm-wise: single entries can cancel, E_n S_0 ~ G)
    rel = (torch.linalg.norm(W.double() - S.double()) / torch.linalg.norm(S.double())).item()
    assert rel < 1e-6, rel


@pytest.mark.parametrize("wname,n_tokens,BH,chunk,read_mode", [("linear", 1000, (1, 4), 16, 0), ("headline", 300, (1, 5), 64, 0),
                                                              ("deep", 250, (1, 2), 128, 1), ("mlp2_short", 97, (2, 3), 13, 0)])
def test_generic_chunk_gates(wname, n_tokens, BH, chunk, read_mode):
    """One alpha, eta, theta per chunk on the generic path, ragged tails
    included, against the oracle fed the same per-chunk gates."""
    cfg = wl.WORKLOADS[wname].with_(B=BH[0], H=BH[1], N=n_tokens, chunk=chunk)
    inp = chunk_gate_inputs(wl.make_inputs(cfg), chunk)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True, read_mode=read_mode, chunk_gates=True)
    _check(cfg, inp, out, run_oracle(cfg, inp, read_mode=read_mode, chunk_gates=True), TOL["f32"])


@pytest.mark.parametrize("n_chunks,H,read_mode,chunk_gates", [(2, 3, 0, False), (4, 3, 0, False), (5, 3, 0, False),
                                                           (4, 80, 0, False), (4, 3, 1, True), (5, 80, 1, True)])
def test_generic_split_launches_match_single_launch(n_chunks, H, read_mode, chunk_gates):
    """A state too large for LDS with chunks of 64 runs each chunk as two
    launches (sweep and reads on two streams), the chunk-start states
    rotating through three buffers of which W_out/S_out is one; an in-place
    call runs the single launch.  Both must agree bitwise, for every
    rotation phase (chunk counts 2, 4, 5 leave the outputs as buffer 2, 1,
    2 of the rotation; 3 chunks are covered above), ragged last chunk
    included, both read modes, per-token and per-chunk gates.  Few streams
    run every step as a launch of its own, tiles spread over workgroups; 80
    streams one launch per phase."""
    import torch
    cfg = wl.WORKLOADS["mlp2_short"].with_(B=1, H=H, N=64 * n_chunks - 9)
    inp = wl.make_inputs(cfg)
    if chunk_gates:
        inp = chunk_gate_inputs(inp, cfg.chunk)
    dev = to_device(cfg, inp)
    kw = dict(force_generic=True, read_mode=read_mode, chunk_gates=chunk_gates)
    y1, W1, S1 = run_gpu(cfg, dev, **kw)
    Wi, Si = dev["W0"].clone(), dev["S0"].clone()
    y2, W2, S2 = run_gpu(cfg, dev | {"W0": Wi, "S0": Si}, W_out=Wi, S_out=Si, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(W1, W2) and torch.equal(S1, S2)
    assert not torch.equal(W1, dev["W0"])


def test_generic_many_streams_split():
    """128 streams on the generic path with the state off chip: one launch
    per phase per chunk (sweep and reads on two streams), every stream
    against the oracle."""
    cfg = wl.WORKLOADS["headline"].with_(N=200)
    inp = wl.make_inputs(cfg, workers=16)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True)
    _check(cfg, inp, out, run_oracle(cfg, inp, threads=16), TOL["f32"])


def test_generic_split_calls_on_two_streams():
    """Two forward calls on the split path enqueued on two torch streams
    without a synchronisation between them (they share the library's side
    stream and its events) give bitwise the results of the calls run one
    after the other."""
    import torch
    cfg1 = wl.WORKLOADS["mlp2_short"].with_(B=1, H=3, N=64 * 4 - 9)
    cfg2 = wl.WORKLOADS["mlp2_short"].with_(B=1, H=2, N=64 * 5 - 3)
    d1, d2 = to_device(cfg1, wl.make_inputs(cfg1)), to_device(cfg2, wl.make_inputs(cfg2))
    ref1 = run_gpu(cfg1, d1, force_generic=True)
    torch.cuda.synchronize()
    ref2 = run_gpu(cfg2, d2, force_generic=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        out1 = run_gpu(cfg1, d1, force_generic=True)
    with torch.cuda.stream(s2):
        out2 = run_gpu(cfg2, d2, force_generic=True)
    torch.cuda.synchronize()
    for a, b in zip(out1 + out2, ref1 + ref2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,N,chunk,read_mode,io", [(64, 300, 64, 1, "bf16"), (32, 129, 1, 0, "f32"),
                                                    (8, 50, 7, 0, "bf16"), (64, 200, 16, 0, "f32")])
def test_linear_memory_kernel(d, N, chunk, read_mode, io):
    """The linear memory (d <= 64, chunk <= 64) runs on its own kernel within
    the generic path (four rows of W and S per workgroup): both read modes,
    both io dtypes, chunks of one token and ragged tails, d from 8 to 64; an
    in-place call agrees bitwise."""
    import torch
    cfg = wl.WORKLOADS["linear"].with_(B=2, H=2, N=N, d=d, chunk=chunk, io=io)
    inp = wl.make_inputs(cfg)
    dev = to_device(cfg, inp)
    out = run_gpu(cfg, dev, force_generic=True, read_mode=read_mode)
    _check(cfg, inp, out, run_oracle(cfg, inp, read_mode=read_mode), TOL["f32"], windows=False)
    Wi, Si = dev["W0"].clone(), dev["S0"].clone()
    y2, W2, S2 = run_gpu(cfg, dev | {"W0": Wi, "S0": Si}, force_generic=True, read_mode=read_mode, W_out=Wi,
                         S_out=Si)
    torch.cuda.synchronize()
    assert torch.equal(y2, out[0]) and torch.equal(W2, out[1]) and torch.equal(S2, out[2])


def _edge_gates(inp, case):
    out = dict(inp)
    if "eta0" in case:
        out["eta"] = np.zeros_like(inp["eta"])
    if "alpha1" in case:
        out["alpha"] = np.ones_like(inp["alpha"])
    return out


@pytest.mark.parametrize("case", ["eta0", "alpha1", "eta0_alpha1"])
@pytest.mark.parametrize("wname,BH,N,chunk", [("mlp2_short", (1, 3), 150, 64), ("linear", (1, 2), 200, 16),
                                              ("deep", (1, 2), 140, 128)])
def test_generic_gate_edges_against_oracle(case, wname, BH, N, chunk):
    """eta = 0 and alpha = 1 on the generic path (and the linear-memory
    kernel), where the coefficient recurrences must be exact, against the
    oracle on y, W and S."""
    cfg = wl.WORKLOADS[wname].with_(B=BH[0], H=BH[1], N=N, chunk=chunk)
    inp = _edge_gates(wl.make_inputs(cfg), case)
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True)
    _check(cfg, inp, out, run_oracle(cfg, inp), TOL["f32"], label=f"{cfg.name} {case}")


@pytest.mark.parametrize("N,chunk", [(64, 64), (300, 300), (45, 64)])
def test_generic_causal_linear_attention(N, chunk):
    """The linear memory with W_0 = S_0 = 0, alpha = eta = 0 and the whole
    sequence in one chunk is causal linear attention,
    y_t = sum_{i<=t} theta_i (k_i . q_t) v_i ("Titans", mer.dev notes,
    section 2.1: linear attention as a memory written with each key-value
    pair), computed here in fp64 from that formula.  Chunks up to 64 run on
    the linear-memory kernel, 300 on the generic kernel."""
    cfg = wl.WORKLOADS["linear"].with_(B=1, H=3, N=N, chunk=chunk)
    inp = wl.make_inputs(cfg)
    inp["alpha"][:] = 0.0
    inp["eta"][:] = 0.0
    assert not inp["W0"].any() and not inp["S0"].any()
    out = run_gpu(cfg, to_device(cfg, inp), force_generic=True)
    f = wl.inputs_f64(cfg, inp)
    ref = np.stack([np.tril(f["q"][s] @ f["k"][s].T) * f["theta"][s][None, :] @ f["v"][s] for s in range(cfg.streams)])
    yg = y_to_f64(cfg, out[0])
    ry, at = y_row_errors(cfg, inp, yg, ref)
    print(f"causal linear attention N={N} chunk={chunk}: per token y {ry:.2e} at {at}", flush=True)
    assert ry < TOL["f32"], (ry, at)
    _check(cfg, inp, out, run_oracle(cfg, inp), TOL["f32"], label="causal linear attention")


def test_generic_kernelised_linear_attention():
    """The 2-layer memory with W2_0 = 0, S_0 = 0, alpha = eta = 0 and one
    chunk on the generic path: y_t = sum_{i<=t} theta_i (phi(k_i) . phi(q_t))
    v_i with phi(x) = SiLU(W1_0 x), and W1 returned bitwise unchanged."""
    import torch
    cfg = wl.WORKLOADS["headline"].with_(B=1, H=2, N=100, chunk=128, io="f32")
    inp = wl.make_inputs(cfg)
    P1 = cfg.hidden * cfg.d
    inp["W0"][:, P1:] = 0.0
    inp["alpha"][:] = 0.0
    inp["eta"][:] = 0.0
    dev = to_device(cfg, inp)
    y, W, S = run_gpu(cfg, dev, force_generic=True)
    torch.cuda.synchronize()
    f = wl.inputs_f64(cfg, inp)
    refs = []
    for s in range(cfg.streams):
        W1 = f["W0"][s, :P1].reshape(cfg.hidden, cfg.d)
        zk, zq = f["k"][s] @ W1.T, f["q"][s] @ W1.T
        pk, pq = zk / (1 + np.exp(-zk)), zq / (1 + np.exp(-zq))
        refs.append((np.tril(pq @ pk.T) * f["theta"][s][None, :]) @ f["v"][s])
    ry, at = y_row_errors(cfg, inp, y_to_f64(cfg, y), np.stack(refs))
    print(f"generic kernelised linear attention: per token y {ry:.2e} at {at}", flush=True)
    assert ry < TOL["f32"], (ry, at)
    assert torch.equal(W[..., :P1], dev["W0"][..., :P1]) and not S[..., :P1].any()

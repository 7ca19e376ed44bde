"""Shared helpers for the GPU parity tests: input staging and the error norms.

Norm-wise criterion (per stream, max over streams):
    e(X) = ||X_gpu - X_ref||_F / max(||X_ref||_F, floor_X)
with floor_W = floor_S = 1e-30 * max(1, ||W_in||_F) and
floor_y = 1e-30 * max(1, ||v||_F).  The floor only matters once the
memory has decayed towards the W = 0 fixed point (the bias-free MLP's
state underflows fp32 late in the long workloads); a non-finite GPU value
where the reference is finite always fails.  Limits: 1e-3 for fp32 io,
2e-2 for bf16 io.

Local criteria, at the same limits, so that a few wrong tokens or state
entries cannot hide in a norm over many:
  * per token: ||y_gpu[t] - y_ref[t]|| / max(||y_ref[t]||, rms_t, floor_y), with
    rms_t the root-mean-square ||y_ref|| over the 64 tokens around t and floor_y
    the stream's y floor above.  A token's error is judged on the scale of its
    neighbourhood: y_t is a sum of terms of that scale computed with 16-bit
    operands, and where the terms nearly cancel in the reference itself
    (||y_t|| down to 1e-4 of its neighbours' in the workloads here) the
    rounding error cannot shrink with the result.  A wrong token still fails,
    its error being of its neighbours' size;
  * per row and per column of every layer matrix of W and S (a row is an
    output unit, a column an input unit, so every hidden unit is covered
    twice): ||X_gpu[r] - X_ref[r]|| / max(||X_ref[r]||, rms_r, floor_X), where
    rms_r is the root-mean-square row (column) norm of that layer.  The MFMA
    kernel scales its 16-bit operands per block, so its rounding error is
    bounded relative to the block, not to each row: a row far smaller than
    its layer's typical row is held to the typical row's scale.
"""
from __future__ import annotations

import numpy as np

from test_learned_neural_amd import workloads as wl

TOL = {"f32": 1e-3, "bf16": 2e-2}


def to_device(cfg, inp, n_streams_shape=None, device="cuda"):
    """numpy inputs -> torch device tensors shaped [B, H, N, ...]."""
    import torch
    S, N = inp["k"].shape[:2]
    G = inp["alpha"].shape[1]       # N per-token gates, or one per chunk
    B, H = n_streams_shape if n_streams_shape else (cfg.B, cfg.H)
    assert B * H == S

    def tok(a):
        if cfg.io == "bf16":
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        return t.reshape(B, H, N, cfg.d).to(device)

    def per(a, last):
        return torch.from_numpy(np.ascontiguousarray(a)).reshape(B, H, last).to(device)

    return dict(k=tok(inp["k"]), v=tok(inp["v"]), q=tok(inp["q"]),
                alpha=per(inp["alpha"], G), eta=per(inp["eta"], G), theta=per(inp["theta"], G),
                W0=per(inp["W0"], cfg.param_count), S0=per(inp["S0"], cfg.param_count))


def y_to_f64(cfg, y):
    """torch y [B,H,N,d] (io dtype) -> float64 numpy [S, N, d]."""
    import torch
    if y.dtype == torch.bfloat16:
        y = y.float()
    a = y.detach().cpu().numpy().astype(np.float64)
    return a.reshape(-1, a.shape[-2], a.shape[-1])


def run_gpu(cfg, dev, chunk=None, **kw):
    from test_learned_neural_amd import titans_mem as tmm
    return tmm.forward(dev["k"], dev["v"], dev["q"], dev["alpha"], dev["eta"], dev["theta"],
                       dev["W0"], dev["S0"], cfg.chunk if chunk is None else chunk,
                       hidden=cfg.hidden, n_layers=cfg.n_layers, **kw)


def run_oracle(cfg, inp, chunk=None, read_mode=0, threads=0, chunk_gates=False, want_w_norm=False):
    import oracle
    f = wl.inputs_f64(cfg, inp)
    return oracle.forward(f["k"], f["v"], f["q"], f["alpha"], f["eta"], f["theta"], f["W0"], f["S0"],
                          d=cfg.d, hidden=cfg.hidden, n_layers=cfg.n_layers,
                          chunk=cfg.chunk if chunk is None else chunk, read_mode=read_mode,
                          threads=threads, chunk_gates=chunk_gates, want_w_norm=want_w_norm)


def chunk_gate_inputs(inp, chunk):
    """The same inputs with one gate value per chunk (each chunk keeps the
    gates its first token drew): alpha, eta, theta become [S, ceil(N/chunk)]."""
    out = dict(inp)
    for g in ("alpha", "eta", "theta"):
        out[g] = np.ascontiguousarray(inp[g][:, ::chunk])
    return out


def rel_err(x, ref, floor):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if not np.all(np.isfinite(x[np.isfinite(ref)])):
        return np.inf
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), floor))


def stream_errors(cfg, inp, y_gpu, W_gpu, S_gpu, y_ref, W_ref, S_ref, idx=None):
    """Per-stream (e_y, e_W, e_S); idx maps rows of the refs to GPU streams."""
    idx = list(range(len(y_ref))) if idx is None else list(idx)
    vin = wl.io_to_f64(inp["v"], cfg.io)
    out = []
    for r, s in enumerate(idx):
        fw = 1e-30 * max(1.0, float(np.linalg.norm(inp["W0"][r].astype(np.float64))))
        fy = 1e-30 * max(1.0, float(np.linalg.norm(vin[r])))
        out.append((rel_err(y_gpu[s], y_ref[r], fy), rel_err(W_gpu[s], W_ref[r], fw),
                    rel_err(S_gpu[s], S_ref[r], fw)))
    return np.array(out)


def window_errors(cfg, inp, y_gpu, y_ref, idx=None, windows=8):
    """Relative y error per window of the sequence, for windows whose
    reference norm is above the floor; returns the max (0 if none)."""
    idx = list(range(len(y_ref))) if idx is None else list(idx)
    vin = wl.io_to_f64(inp["v"], cfg.io)
    worst = 0.0
    N = y_ref.shape[1]
    bounds = np.linspace(0, N, windows + 1).astype(int)
    for r, s in enumerate(idx):
        for a, b in zip(bounds[:-1], bounds[1:]):
            if b <= a:
                continue
            fy = 1e-30 * max(1.0, float(np.linalg.norm(vin[r, a:b])))
            if np.linalg.norm(y_ref[r, a:b]) < fy:
                continue
            worst = max(worst, rel_err(y_gpu[s, a:b], y_ref[r, a:b], fy))
    return worst


def live_length(w_norm_traj, chunk, floor):
    """Last token at which the reference ||W_t||_F stays above the floor."""
    alive = np.nonzero(w_norm_traj > floor)[0]
    return 0 if len(alive) == 0 else int((alive[-1] + 1) * chunk)


TOKEN_KEYS = ("k", "v", "q", "alpha", "eta", "theta")


def prefix_inputs(inp, n):
    """The first n tokens of every stream (the generator draws a prefix
    bit-identically, so this equals make_inputs(..., n_tokens=n))."""
    return {k: (np.ascontiguousarray(a[:, :n]) if k in TOKEN_KEYS else a) for k, a in inp.items()}


def y_errors(cfg, inp, y_gpu, y_ref):
    """Per-stream relative y error with the y floor."""
    vin = wl.io_to_f64(inp["v"], cfg.io)
    return np.array([rel_err(y_gpu[s], y_ref[s], 1e-30 * max(1.0, float(np.linalg.norm(vin[s]))))
                     for s in range(len(y_ref))])


def state_below_floor(cfg, inp, W_gpu, S_gpu, tol):
    """For a reference state that is exactly zero: the relative error against
    it, ||X_gpu|| / floor, per stream (W and S), must stay under tol."""
    worst = 0.0
    for s in range(len(W_gpu)):
        fw = 1e-30 * max(1.0, float(np.linalg.norm(inp["W0"][s].astype(np.float64))))
        worst = max(worst, rel_err(W_gpu[s], np.zeros_like(W_gpu[s]), fw),
                    rel_err(S_gpu[s], np.zeros_like(S_gpu[s]), fw))
    return worst < tol, worst


def _row_rel(diff, ref, floor):
    """Row-wise ||diff|| / max(||ref||, floor) (floor per row or scalar)."""
    return np.linalg.norm(diff, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), floor)


def local_rms(norms, half_window=32):
    """Root-mean-square of a sequence of row norms over the window
    [t - half_window, t + half_window) around every t (clipped at the ends).
    Each window is summed on its own (a direct convolution): differences of
    running sums would lose the windows of a decayed memory, whose squares
    are dozens of orders of magnitude below the early ones."""
    x2 = np.asarray(norms, np.float64) ** 2
    n = len(x2)
    full = np.convolve(x2, np.ones(2 * half_window))
    t = np.arange(n)
    lo, hi = np.maximum(t - half_window, 0), np.minimum(t + half_window, n)
    return np.sqrt(full[t + half_window - 1] / (hi - lo))


def y_row_errors(cfg, inp, y_gpu, y_ref, idx=None):
    """Worst per-token y error over every stream and token:
    ||y_gpu[t] - y_ref[t]|| / max(||y_ref[t]||, the local rms of ||y_ref|| over
    the 64 tokens around t, the stream's y floor 1e-30 max(1, ||v||_F)), as
    (worst, (stream, token)).  A non-finite GPU row where the reference is
    finite is an infinite error."""
    idx = list(range(len(y_ref))) if idx is None else list(idx)
    worst, where = 0.0, None
    for r, s in enumerate(idx):
        g = np.asarray(y_gpu[s], np.float64)
        ref = np.asarray(y_ref[r], np.float64)
        n = ref.shape[0]
        fy = 1e-30 * max(1.0, float(np.linalg.norm(wl.io_to_f64(inp["v"][r, :n], cfg.io))))
        rn = np.linalg.norm(ref, axis=-1)
        floor = np.maximum(local_rms(rn), fy)
        e = _row_rel(g - ref, ref, floor)
        bad = ~np.all(np.isfinite(g), axis=-1) & np.all(np.isfinite(ref), axis=-1)
        e[bad] = np.inf
        t = int(np.argmax(e))
        if e[t] > worst or where is None:
            worst, where = float(e[t]), (s, t)
    return worst, where


def state_row_errors(cfg, inp, X_gpu, X_ref, idx=None):
    """Worst per-row and per-column error of every layer matrix of a state
    (W or S) over every stream: ||X_gpu[r] - X_ref[r]|| / max(||X_ref[r]||,
    rms_r, floor), rms_r the layer's root-mean-square row (column) norm and
    floor = 1e-30 max(1, ||W_in||).  Returns (worst, (stream, layer, 'row' or
    'col', index))."""
    idx = list(range(len(X_ref))) if idx is None else list(idx)
    w = cfg.widths
    worst, where = 0.0, None
    for r, s in enumerate(idx):
        floor = 1e-30 * max(1.0, float(np.linalg.norm(inp["W0"][r].astype(np.float64))))
        g_all = np.asarray(X_gpu[s], np.float64)
        ref_all = np.asarray(X_ref[r], np.float64)
        off = 0
        for layer in range(cfg.n_layers):
            n_out, n_in = w[layer + 1], w[layer]
            g = g_all[off:off + n_out * n_in].reshape(n_out, n_in)
            ref = ref_all[off:off + n_out * n_in].reshape(n_out, n_in)
            off += n_out * n_in
            for kind, gg, rr in (("row", g, ref), ("col", g.T, ref.T)):
                rms = float(np.sqrt(np.mean(np.sum(rr * rr, axis=-1))))
                e = _row_rel(gg - rr, rr, max(rms, floor))
                bad = ~np.all(np.isfinite(gg), axis=-1) & np.all(np.isfinite(rr), axis=-1)
                e[bad] = np.inf
                i = int(np.argmax(e))
                if e[i] > worst or where is None:
                    worst, where = float(e[i]), (s, layer + 1, kind, i)
    return worst, where


def live_lengths(cfg, inp, w_norm):
    """Per stream: the live length (last token at which the reference
    ||W_t||_F, sampled at chunk ends, exceeds the floor 1e-30 max(1, ||W_in||))."""
    return [live_length(w_norm[r], cfg.chunk, 1e-30 * max(1.0, float(np.linalg.norm(inp["W0"][r].astype(np.float64)))))
            for r in range(len(w_norm))]

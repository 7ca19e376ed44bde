"""Rounding emulation of the deep-memory path against the fp64 oracle.

Evaluates the chunked closed form (mer.dev notes on "Titans: Learning to
Memorize at Test Time", section 3.2: gradients at the chunk-start weights)
in fp32 with the path's rounding points made explicit, each either rounded
to bf16 (round to nearest even) or kept in fp32:

    W, S   the chunk-start state as a product operand
    a      the key-side activations a^l
    d      the deltas delta^l
    h      the query-side activations
    P      the masked scores D o (h a^T)
    fw     the deltas scaled by the fold weights D[n-1, .] and U

and prints the worst per-token y error and the norm-wise W error of each
variant, with the criteria of the GPU parity tests.  Keeping every point in
fp32 stands for the split (hi + lo) operands of the kernels, whose products
carry about 2^-16.  This is the evidence for the deep path's operand choice:
with plain bf16 operands the alpha = 1 case lands at the 2e-2 bar.

Usage: python tests/emulate_deep_rounding.py [alpha1|eta0|default]
(a few minutes of CPU: two streams of the deep memory, 140 tokens).
Test infrastructure only, like the oracle it calls.
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from parity_util import stream_errors, y_row_errors  # noqa: E402
from test_learned_neural_amd import workloads as wl  # noqa: E402


def bf16(x):
    """fp32 -> bf16 -> fp32, round to nearest even."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def silu(z):
    return z / (1 + np.exp(-z))


def silu_prime(z):
    s = 1 / (1 + np.exp(-z))
    return s * (1 + z * (1 - s))


def coefficients(al, et, th):
    """A, E, F, U and D of one chunk (section 3.1's rules unrolled), fp32."""
    n = len(al)
    D = np.zeros((n, n), np.float32)
    U = np.zeros(n, np.float32)
    for i in range(n):
        di, pr = th[i], np.float32(1)
        D[i, i] = di
        for j in range(i + 1, n):
            pr = pr * et[j]
            di = (1 - al[j]) * di + th[i] * pr
            D[j, i] = di
        U[i] = th[i] * pr
    A = np.cumprod(1 - al).astype(np.float32)
    E = np.cumprod(et).astype(np.float32)
    F = np.zeros(n, np.float32)
    f = np.float32(0)
    for j in range(n):
        f = (1 - al[j]) * f + E[j]
        F[j] = f
    return A, E, F, U, D


def run(cfg, f, keep=()):
    """y, W, S of every stream with the rounding points not in `keep` rounded to bf16."""
    rnd = lambda name, x: np.asarray(x, np.float32) if name in keep else bf16(x)  # noqa: E731
    L, w, b, N = cfg.n_layers, cfg.widths, cfg.chunk, cfg.N
    ys = np.zeros((f["k"].shape[0], N, cfg.d))
    Ws, Ss = [], []
    for s in range(f["k"].shape[0]):
        W = f["W0"][s].astype(np.float32).copy()
        S = f["S0"][s].astype(np.float32).copy()

        def layer(X, l):
            o = sum(w[i + 1] * w[i] for i in range(l - 1))
            return X[o:o + w[l] * w[l - 1]].reshape(w[l], w[l - 1])

        for c0 in range(0, N, b):
            n = min(b, N - c0)
            K, V, Q = (f[x][s, c0:c0 + n].astype(np.float32) for x in ("k", "v", "q"))
            A, E, F, U, D = coefficients(*(f[g][s, c0:c0 + n].astype(np.float32) for g in ("alpha", "eta", "theta")))
            W16 = [None] + [rnd("W", layer(W, l)) for l in range(1, L + 1)]
            S16 = [None] + [rnd("S", layer(S, l)) for l in range(1, L + 1)]
            a, sp = [K], [None]
            for l in range(1, L + 1):
                z = a[l - 1] @ W16[l].T
                if l < L:
                    a.append(rnd("a", silu(z)))
                    sp.append(silu_prime(z))
                else:
                    dl = rnd("d", z - V)
            delta = {L: dl}
            for l in range(L, 1, -1):
                delta[l - 1] = rnd("d", (delta[l] @ W16[l]) * sp[l - 1])
            h = Q
            for l in range(1, L + 1):
                P = rnd("P", np.tril(D * (h @ a[l - 1].T)))
                zq = A[:, None] * (h @ W16[l].T) + F[:, None] * (h @ S16[l].T) - P @ delta[l]
                h = rnd("h", silu(zq)) if l < L else zq
            ys[s, c0:c0 + n] = h
            for l in range(1, L + 1):
                GD = rnd("fw", D[n - 1][:, None] * delta[l]).T @ a[l - 1]
                GU = rnd("fw", U[:, None] * delta[l]).T @ a[l - 1]
                Wl, Sl = layer(W, l), layer(S, l)
                Wn = A[n - 1] * Wl + F[n - 1] * Sl - GD
                Sl[...] = E[n - 1] * Sl - GU
                Wl[...] = Wn
        Ws.append(W)
        Ss.append(S)
    return ys, np.array(Ws), np.array(Ss)


VARIANTS = [(), ("W", "S"), ("W", "S", "d"), ("W", "S", "a", "d"), ("a", "d", "h", "P", "fw"),
            ("W", "S", "a", "d", "h", "P", "fw")]


def main(case="alpha1"):
    cfg = wl.WORKLOADS["deep"].with_(B=1, H=2, N=140)
    inp = wl.make_inputs(cfg)
    if "alpha1" in case:
        inp["alpha"] = np.ones_like(inp["alpha"])
    if "eta0" in case:
        inp["eta"] = np.zeros_like(inp["eta"])
    f = wl.inputs_f64(cfg, inp)
    ref = oracle.forward(f["k"], f["v"], f["q"], f["alpha"], f["eta"], f["theta"], f["W0"], f["S0"], d=cfg.d,
                         hidden=cfg.hidden, n_layers=cfg.n_layers, chunk=cfg.chunk, threads=4)
    print(f"deep memory, 2 streams x {cfg.N} tokens, gates: {case}")
    print(f"{'kept in fp32':40s} {'worst token y':>14s} {'norm e_W':>10s}")
    for keep in VARIANTS:
        y, W, S = run(cfg, f, keep)
        ry, _ = y_row_errors(cfg, inp, y, ref[0])
        e = stream_errors(cfg, inp, y, W, S, *ref[:3])
        print(f"{', '.join(keep) or '(all bf16)':40s} {ry:14.2e} {e[:, 1].max():10.2e}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "alpha1")

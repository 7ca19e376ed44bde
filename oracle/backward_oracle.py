"""fp64 oracle of the gradients through the memory (outer-loop training).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU library never does.

The memory's forward pass is written once more, token by token, with torch
float64 CPU ops ("Titans: Learning to Memorize at Test Time", mer.dev notes:
the loss of section 3.1 "Objective", the momentum of "Learning Process and
Surprise Metric", the forgetting of "Forgetting Mechanism", the read of
"Retrieving a Memory", gradients at the chunk-start weights as in section
3.2).  The per-token gradient of 0.5 ||M(k) - v||^2 is written as its
backpropagation (the memory's own inner gradient), so torch's reverse mode
differentiates through it, second-order terms included.  The scalar
differentiated is L = <y, dy> + <W_out, dW_out> + <S_out, dS_out>, so the
returned gradients are the vector-Jacobian products of the forward map with
(dy, dW_out, dS_out).

Pinned against the C oracle's forward (same values) and against central
finite differences of that C forward.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def _widths(d, hidden, n_layers):
    return [d, d] if n_layers == 1 else [d] + [hidden] * (n_layers - 1) + [d]


def _silu_parts(torch, z):
    s = torch.sigmoid(z)
    return z * s, s * (1 + z * (1 - s))


def forward_torch(torch, k, v, q, alpha, eta, theta, W_in, S_in, *, d, hidden, n_layers, chunk, read_mode=0):
    """Differentiable token loop over independent streams (leading axis).

    k, v, q: [S, N, d]; alpha, eta, theta: [S, N]; W_in, S_in: [S, P]
    (layers concatenated, layer l row-major [n_l, n_{l-1}]).  Returns
    (y [S, N, d], W_out [S, P], S_out [S, P])."""
    w = _widths(d, hidden, n_layers)
    L = n_layers
    Sn, N, _ = k.shape

    def split(flat):
        mats, off = [], 0
        for l in range(L):
            n_out, n_in = w[l + 1], w[l]
            mats.append(flat[:, off:off + n_out * n_in].reshape(Sn, n_out, n_in))
            off += n_out * n_in
        return mats

    def apply(mats, x):
        a = x
        for l in range(L):
            z = torch.einsum("soi,si->so", mats[l], a)
            a = _silu_parts(torch, z)[0] if l < L - 1 else z
        return a

    def grad(mats, x, target):
        """per-layer gradient of 0.5 ||M(x) - target||^2 (column convention)"""
        acts, zs = [x], []
        a = x
        for l in range(L):
            z = torch.einsum("soi,si->so", mats[l], a)
            zs.append(z)
            a = _silu_parts(torch, z)[0] if l < L - 1 else z
            acts.append(a)
        delta = acts[-1] - target
        gs = [None] * L
        for l in range(L - 1, -1, -1):
            gs[l] = delta[:, :, None] * acts[l][:, None, :]
            if l > 0:
                back = torch.einsum("soi,so->si", mats[l], delta)
                delta = back * _silu_parts(torch, zs[l - 1])[1]
        return gs

    Wm, Sm = split(W_in), split(S_in)
    ys = []
    Wc = Wm
    for t in range(N):
        if t % chunk == 0:
            Wc = Wm
        g = grad(Wc, k[:, t], v[:, t])
        a_t, e_t, th_t = alpha[:, t, None, None], eta[:, t, None, None], theta[:, t, None, None]
        Sm = [e_t * Sm[l] - th_t * g[l] for l in range(L)]
        Wm = [(1 - a_t) * Wm[l] + Sm[l] for l in range(L)]
        ys.append(apply(Wc if read_mode == 1 else Wm, q[:, t]))
    y = torch.stack(ys, dim=1)
    flat = lambda mats: torch.cat([m.reshape(Sn, -1) for m in mats], dim=1)
    return y, flat(Wm), flat(Sm)


def backward(k, v, q, alpha, eta, theta, W_in, S_in, dy, dW_out, dS_out, *, d: int, hidden: int,
             n_layers: int, chunk: int, read_mode: int = 0, chunk_gates: bool = False) -> Dict[str, np.ndarray]:
    """Gradients of <y, dy> + <W_out, dW_out> + <S_out, dS_out> with respect
    to every input of the forward call, as float64 numpy arrays keyed k, v,
    q, alpha, eta, theta, W_in, S_in.  dy / dW_out / dS_out may be None
    (zero).  With chunk_gates the gates (and their gradients) are per chunk,
    [S, ceil(N / chunk)]."""
    import torch
    t64 = lambda a: torch.tensor(np.asarray(a, np.float64), dtype=torch.float64, requires_grad=True)
    inp = {name: t64(a) for name, a in (("k", k), ("v", v), ("q", q), ("alpha", alpha), ("eta", eta),
                                         ("theta", theta), ("W_in", W_in), ("S_in", S_in))}
    N = inp["k"].shape[1]
    gates = []
    for name in ("alpha", "eta", "theta"):
        g = inp[name]
        if chunk_gates:
            g = torch.repeat_interleave(g, chunk, dim=1)[:, :N]
        gates.append(g)
    y, W, S = forward_torch(torch, inp["k"], inp["v"], inp["q"], *gates, inp["W_in"], inp["S_in"], d=d,
                            hidden=hidden, n_layers=n_layers, chunk=chunk, read_mode=read_mode)
    loss = torch.zeros((), dtype=torch.float64)
    for out, adj in ((y, dy), (W, dW_out), (S, dS_out)):
        if adj is not None:
            loss = loss + (out * torch.tensor(np.asarray(adj, np.float64))).sum()
    names = list(inp)
    if not loss.requires_grad:          # no adjoint given: every gradient is zero
        return {n: np.zeros(inp[n].shape) for n in names}
    grads = torch.autograd.grad(loss, [inp[n] for n in names], allow_unused=True)
    return {n: (np.zeros(inp[n].shape) if g is None else g.detach().numpy()) for n, g in zip(names, grads)}

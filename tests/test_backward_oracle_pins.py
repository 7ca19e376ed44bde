"""Pins of the gradient oracle (backward through the chunked memory).

The gradients come from torch's reverse mode over a token-by-token fp64
forward.  They are pinned to things other than that code: the C oracle's
forward (same values), central finite differences of the C forward along
random directions for every input, a closed form of the linear memory with
theta = 0, and the chunk-gate sums.  The pages ("Titans: Learning to
Memorize at Test Time", mer.dev notes) state that the memory is trained
inside an outer loop (section 3.1, "Objective") but print no gradient of
it, so no printed value exists to compare with.
"""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _problem(rng, S=2, N=23, d=4, h=6, L=2):
    P = oracle.param_count(d, h, L)
    unit = lambda a: a / np.linalg.norm(a, axis=-1, keepdims=True)
    return dict(k=unit(rng.standard_normal((S, N, d))), v=0.5 * rng.standard_normal((S, N, d)),
                q=unit(rng.standard_normal((S, N, d))), alpha=rng.uniform(0, .2, (S, N)),
                eta=rng.uniform(.5, .9, (S, N)), theta=rng.uniform(0, .15, (S, N)),
                W_in=rng.standard_normal((S, P)) * 0.3, S_in=rng.standard_normal((S, P)) * 0.05), P


def _loss_c(x, dy, dW, dS, **kw):
    y, W, S = oracle.forward(x["k"], x["v"], x["q"], x["alpha"], x["eta"], x["theta"], x["W_in"], x["S_in"], **kw)
    return float(np.sum(y * dy) + np.sum(W * dW) + np.sum(S * dS))


@pytest.mark.parametrize("L,h,read_mode,chunk", [(1, 0, 0, 5), (2, 6, 0, 5), (2, 6, 1, 4), (3, 5, 0, 7),
                                                 (2, 6, 0, 1), (2, 6, 0, 64)])
def test_gradients_match_finite_differences_of_the_c_forward(L, h, read_mode, chunk):
    rng = np.random.default_rng(10 + L + 3 * read_mode + chunk)
    d = 4
    x, P = _problem(rng, d=d, h=h, L=L)
    S, N = x["alpha"].shape
    dy, dW, dS = rng.standard_normal((S, N, d)), rng.standard_normal((S, P)), rng.standard_normal((S, P))
    kw = dict(d=d, hidden=h, n_layers=L, chunk=chunk, read_mode=read_mode)
    g = oracle.backward(**x, dy=dy, dW_out=dW, dS_out=dS, **kw)
    eps = 1e-6
    for name in x:
        u = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + eps * u
        xm = dict(x); xm[name] = x[name] - eps * u
        fd = (_loss_c(xp, dy, dW, dS, **kw) - _loss_c(xm, dy, dW, dS, **kw)) / (2 * eps)
        an = float(np.sum(g[name] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_linear_theta_zero_closed_form():
    """Linear memory, theta = 0, S0 = 0: S stays 0, W_t = A_t W0 and
    y_t = A_t W0 q_t with A_t = prod_{m<=t}(1 - alpha_m).  Then
    dq_t = A_t W0^T dy_t, dW0 = sum_t A_t dy_t q_t^T, dk = dv = deta = 0 and
    dalpha_m = -sum_{t>=m} (A_t / (1 - alpha_m)) dy_t . W0 q_t."""
    rng = np.random.default_rng(20)
    S, N, d = 1, 12, 3
    x, P = _problem(rng, S=S, N=N, d=d, L=1)
    x["theta"] = np.zeros((S, N))
    x["S_in"] = np.zeros((S, P))
    dy = rng.standard_normal((S, N, d))
    g = oracle.backward(**x, dy=dy, dW_out=None, dS_out=None, d=d, hidden=0, n_layers=1, chunk=4)
    W0 = x["W_in"][0].reshape(d, d)
    A = np.cumprod(1 - x["alpha"][0])
    for t in range(N):
        np.testing.assert_allclose(g["q"][0, t], A[t] * W0.T @ dy[0, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["W_in"][0].reshape(d, d),
                               sum(A[t] * np.outer(dy[0, t], x["q"][0, t]) for t in range(N)), rtol=1e-12)
    assert not np.any(g["k"]) and not np.any(g["v"]) and not np.any(g["eta"])
    for m in range(N):
        ref = -sum(A[t] / (1 - x["alpha"][0, m]) * dy[0, t] @ (W0 @ x["q"][0, t]) for t in range(m, N))
        assert g["alpha"][0, m] == pytest.approx(ref, rel=1e-11, abs=1e-14)


def test_chunk_gate_gradients_are_sums_over_the_chunk():
    rng = np.random.default_rng(21)
    x, P = _problem(rng, N=17)
    S, N = x["alpha"].shape
    chunk = 5
    nc = -(-N // chunk)
    xc = dict(x)
    for gname in ("alpha", "eta", "theta"):
        xc[gname] = x[gname][:, ::chunk].copy()
    xt = dict(xc)
    for gname in ("alpha", "eta", "theta"):
        xt[gname] = np.repeat(xc[gname], chunk, axis=1)[:, :N]
    dy = rng.standard_normal((S, N, 4))
    kw = dict(d=4, hidden=6, n_layers=2, chunk=chunk)
    gc = oracle.backward(**xc, dy=dy, dW_out=None, dS_out=None, chunk_gates=True, **kw)
    gt = oracle.backward(**xt, dy=dy, dW_out=None, dS_out=None, **kw)
    for gname in ("alpha", "eta", "theta"):
        assert gc[gname].shape == (S, nc)
        summed = np.add.reduceat(gt[gname], np.arange(0, N, chunk), axis=1)
        np.testing.assert_allclose(gc[gname], summed, rtol=1e-12, atol=1e-15)
    for name in ("k", "v", "q", "W_in", "S_in"):
        np.testing.assert_allclose(gc[name], gt[name], rtol=1e-12, atol=1e-15)


def test_zero_adjoints_give_zero_gradients():
    rng = np.random.default_rng(22)
    x, P = _problem(rng)
    g = oracle.backward(**x, dy=None, dW_out=None, dS_out=None, d=4, hidden=6, n_layers=2, chunk=5)
    assert all(not np.any(a) for a in g.values())


@pytest.mark.parametrize("L,h,read_mode", [(1, 0, 0), (2, 6, 0), (2, 6, 1), (4, 5, 0)])
def test_torch_forward_equals_the_c_forward(L, h, read_mode):
    rng = np.random.default_rng(30 + L + read_mode)
    x, P = _problem(rng, L=L, h=h)
    kw = dict(d=4, hidden=h, n_layers=L, chunk=5, read_mode=read_mode)
    yc, Wc, Sc = oracle.forward(*[x[n] for n in ("k", "v", "q", "alpha", "eta", "theta", "W_in", "S_in")], **kw)
    T = lambda a: torch.tensor(a, dtype=torch.float64)
    yt, Wt, St = oracle.forward_torch(torch, *[T(x[n]) for n in ("k", "v", "q", "alpha", "eta", "theta", "W_in",
                                                                 "S_in")], **kw)
    for a, b in ((yt, yc), (Wt, Wc), (St, Sc)):
        np.testing.assert_allclose(a.numpy(), b, rtol=1e-13, atol=1e-15)

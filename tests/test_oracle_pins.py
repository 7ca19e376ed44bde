"""Pins of the fp64 oracle against what the pages and the mathematics fix.

The oracle (oracle/titans_oracle.c) is the token-by-token recurrence of
"Titans: Learning to Memorize at Test Time" (mer.dev notes, sections 3.1 and
3.2).  Nothing here re-types that recurrence: each test checks it against an
independent statement of the result --

* library routines: torch's bias-free Linear/SiLU forward and autograd
  gradients in float64, and central finite differences;
* closed forms the pages print or imply: the delta rule (linear memory,
  no momentum), the pages' mini-batch form with forgetting products
  (section 3.2), causal linear attention and its kernelised form (section
  2.1, "kernel in place of softmax"), and the unrolled chunk closed form
  (decay products summed per token, gradients from autograd at the
  chunk-start weights);
* exact special cases: theta = 0 leaves the memory alone, alpha = 1 clears
  it, scaling linear inputs, split-and-resume.

Each docstring names the passage it follows.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from test_learned_neural_amd import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ----------------------------------------------------------------------------
# independent helpers (library routines, products written from the definition)
# ----------------------------------------------------------------------------
def widths_of(d, hidden, L):
    return [d, d] if L == 1 else [d] + [hidden] * (L - 1) + [d]


def split_layers(Wflat, widths):
    mats, off = [], 0
    for i in range(len(widths) - 1):
        n = widths[i + 1] * widths[i]
        mats.append(torch.as_tensor(Wflat[off:off + n], dtype=torch.float64).reshape(widths[i + 1], widths[i]))
        off += n
    return mats


def torch_forward(mats, x):
    """Bias-free MLP with SiLU between layers, via torch's own modules."""
    h = torch.as_tensor(x, dtype=torch.float64)
    for i, Wl in enumerate(mats):
        h = F.linear(h, Wl)
        if i < len(mats) - 1:
            h = F.silu(h)
    return h


def autograd_grad(Wflat, widths, k, v):
    """Gradient of 0.5 ||M_W(k) - v||^2 by torch autograd (flattened)."""
    mats = [m.clone().requires_grad_(True) for m in split_layers(Wflat, widths)]
    out = torch_forward(mats, k)
    loss = 0.5 * ((out - torch.as_tensor(v, dtype=torch.float64)) ** 2).sum()
    grads = torch.autograd.grad(loss, mats)
    return torch.cat([g.reshape(-1) for g in grads]).numpy()


def prod(xs):
    p = 1.0
    for x in xs:
        p *= x
    return p


def coeff_brute(alpha, eta, theta):
    """Chunk coefficients straight from unrolling S_t = eta S - theta g and
    W_t = (1 - alpha) W + S (section 3.1), as explicit products and sums:

    W_j = A_j W_0 + F_j S_0 - sum_{i<=j} D[j,i] g_i
    S_j = E_j S_0 - sum_{i<=j} C[j,i] g_i
    """
    n = len(alpha)
    A = np.array([prod(1 - alpha[m] for m in range(j + 1)) for j in range(n)])
    E = np.array([prod(eta[m] for m in range(j + 1)) for j in range(n)])
    Fc = np.array([sum(prod(1 - alpha[m] for m in range(l + 1, j + 1)) * prod(eta[m] for m in range(l + 1))
                       for l in range(j + 1)) for j in range(n)])
    C = np.zeros((n, n))
    D = np.zeros((n, n))
    for j in range(n):
        for i in range(j + 1):
            C[j, i] = theta[i] * prod(eta[m] for m in range(i + 1, j + 1))
            D[j, i] = theta[i] * sum(prod(1 - alpha[m] for m in range(l + 1, j + 1)) *
                                     prod(eta[m] for m in range(i + 1, l + 1)) for l in range(i, j + 1))
    return A, E, Fc, C, D


def run_oracle(oracle_mod, k, v, q, a, e, t, W0, S0, d, hidden, L, chunk, read_mode=0):
    return oracle_mod.forward(k[None], v[None], q[None], a[None], e[None], t[None], W0[None], S0[None],
                              d=d, hidden=hidden, n_layers=L, chunk=chunk, read_mode=read_mode)


def rand_stream(rng, N, d, P, unit=True):
    k = rng.standard_normal((N, d))
    q = rng.standard_normal((N, d))
    if unit:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = rng.standard_normal((N, d))
    return k, v, q


# ----------------------------------------------------------------------------
# input generator (storage rounding and counter-keyed streams)
# ----------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                        [0.0, -0.0, 1.0, -1.0, 3.0e38]])
    mine = wl.f64_to_bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = wl.bf16_bits_to_f64(mine)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_generator_prefix_and_subset_are_consistent():
    cfg = wl.WORKLOADS["mlp2_short"]
    full = wl.make_inputs(cfg, streams=[(0, 0), (1, 2), (3, 7)], n_tokens=256)
    sub = wl.make_inputs(cfg, streams=[(1, 2)], n_tokens=100)
    for name in ("k", "v", "q", "alpha", "eta", "theta"):
        assert np.array_equal(full[name][1, :100], sub[name][0]), name
    assert np.array_equal(full["W0"][1], sub["W0"][0])
    # unit-norm keys and queries (rounded once to bf16)
    kk = wl.io_to_f64(full["k"], "bf16")
    assert np.allclose(np.linalg.norm(kk, axis=-1), 1.0, atol=2 ** -7)


def test_generator_laws():
    c3 = wl.make_inputs(wl.WORKLOADS["headline"], streams=[(0, 0)], n_tokens=4096)
    assert c3["alpha"].max() <= 0.1 and c3["theta"].max() <= 0.1 and c3["alpha"].min() > 0
    assert 0 < c3["eta"].min() and c3["eta"].max() < 1
    c1 = wl.make_inputs(wl.WORKLOADS["linear"], n_tokens=512)
    assert c1["k"].dtype == np.float32 and not c1["W0"].any()
    assert 0.8 <= c1["eta"].min() and c1["alpha"].max() <= 0.1
    c2 = wl.make_inputs(wl.WORKLOADS["mlp2_short"], streams=[(0, 0)], n_tokens=8)
    bound = np.sqrt(6.0 / (64 + 256))
    assert np.abs(c2["W0"]).max() <= bound and np.abs(c2["W0"]).max() > 0.9 * bound


# ----------------------------------------------------------------------------
# P0/P1: forward and gradient against library routines and finite differences
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,d,h", [(1, 5, 0), (2, 3, 5), (2, 8, 32), (4, 3, 5), (4, 6, 9)])
def test_memory_forward_matches_torch(oracle_mod, L, d, h):
    """M(x) = W2 sigma(W1 x) with SiLU (blog, section 3.1; mer.dev 4.4 uses SiLU)."""
    rng = np.random.default_rng(L * 100 + d)
    widths = widths_of(d, h, L)
    P = oracle_mod.param_count(d, h, L)
    W = rng.standard_normal(P)
    for _ in range(3):
        x = rng.standard_normal(d)
        mine = oracle_mod.memory_apply(W, x, d, h, L)
        ref = torch_forward(split_layers(W, widths), x).numpy()
        np.testing.assert_allclose(mine, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("L,d,h", [(1, 3, 0), (2, 3, 5), (4, 3, 5), (2, 7, 11)])
def test_gradient_matches_autograd_and_finite_differences(oracle_mod, L, d, h):
    """Surprise = gradient of the associative loss (mer.dev 3.1 "Objective");
    scale 0.5 ||.||^2 as in the linear gradient printed in section 3.2."""
    rng = np.random.default_rng(7 + L)
    widths = widths_of(d, h, L)
    P = oracle_mod.param_count(d, h, L)
    W = rng.standard_normal(P) * 0.7
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    g, loss = oracle_mod.memory_grad(W, k, v, d, h, L)
    ref = autograd_grad(W, widths, k, v)
    np.testing.assert_allclose(g, ref, rtol=1e-12, atol=1e-12)
    out = oracle_mod.memory_apply(W, k, d, h, L)
    assert abs(loss - 0.5 * np.sum((out - v) ** 2)) < 1e-12 * max(1, loss)
    eps = 1e-6
    fd = np.empty(P)
    for p in range(P):
        Wp, Wm = W.copy(), W.copy()
        Wp[p] += eps
        Wm[p] -= eps
        lp = 0.5 * np.sum((oracle_mod.memory_apply(Wp, k, d, h, L) - v) ** 2)
        lm = 0.5 * np.sum((oracle_mod.memory_apply(Wm, k, d, h, L) - v) ** 2)
        fd[p] = (lp - lm) / (2 * eps)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_linear_gradient_is_printed_form(oracle_mod):
    """Linear memory: grad = (W k - v) k^T, the form printed in section 3.2."""
    rng = np.random.default_rng(3)
    d = 6
    W = rng.standard_normal(d * d)
    k, v = rng.standard_normal(d), rng.standard_normal(d)
    g, _ = oracle_mod.memory_grad(W, k, v, d, 0, 1)
    Wm = W.reshape(d, d)
    np.testing.assert_allclose(g.reshape(d, d), np.outer(Wm @ k - v, k), rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------------------------
# P2: chunk 1 is plain online gradient descent with momentum and forgetting
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,d,h", [(1, 4, 0), (2, 4, 6), (4, 3, 5)])
def test_chunk_one_is_online_momentum_gd(oracle_mod, L, d, h):
    """With b = 1 every token differentiates at the current weights
    (section 3.2 with t' = t), i.e. the per-token rules of section 3.1.
    Reference loop: torch autograd gradient at the current weights."""
    rng = np.random.default_rng(11 + L)
    N = 23
    widths = widths_of(d, h, L)
    P = oracle_mod.param_count(d, h, L)
    k, v, q = rand_stream(rng, N, d, P)
    a, e, t = rng.uniform(0, 0.3, N), rng.uniform(0.5, 1, N), rng.uniform(0, 0.5, N)
    W0, S0 = rng.standard_normal(P) * 0.5, rng.standard_normal(P) * 0.1
    y, Wo, So = run_oracle(oracle_mod, k, v, q, a, e, t, W0, S0, d, h, L, 1)
    W, S = W0.copy(), S0.copy()
    for i in range(N):
        g = autograd_grad(W, widths, k[i], v[i])
        S = e[i] * S - t[i] * g
        W = (1 - a[i]) * W + S
        np.testing.assert_allclose(y[0, i], torch_forward(split_layers(W, widths), q[i]).numpy(),
                                   rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Wo[0], W, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(So[0], S, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# P3: delta rule;  P4: the pages' mini-batch closed form
# ----------------------------------------------------------------------------
def test_delta_rule_closed_form(oracle_mod):
    """Linear memory, eta = 0, b = 1: W_t = W_{t-1}((1-a)I - th k k^T) + th v k^T."""
    rng = np.random.default_rng(5)
    d, N = 8, 40
    k, v, q = rand_stream(rng, N, d, d * d)
    a, t = rng.uniform(0, 0.2, N), rng.uniform(0, 1, N)
    e = np.zeros(N)
    W0 = rng.standard_normal(d * d)
    S0 = rng.standard_normal(d * d)      # eta = 0 wipes it at the first token
    y, Wo, So = run_oracle(oracle_mod, k, v, q, a, e, t, W0, S0, d, 0, 1, 1)
    W = W0.reshape(d, d).copy()
    for i in range(N):
        W = W @ ((1 - a[i]) * np.eye(d) - t[i] * np.outer(k[i], k[i])) + t[i] * np.outer(v[i], k[i])
        np.testing.assert_allclose(y[0, i], W @ q[i], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Wo[0].reshape(d, d), W, rtol=1e-12, atol=1e-12)


def test_delta_rule_writes_exactly(oracle_mod):
    """alpha = 0, theta = 1, ||k|| = 1: the write stores v at k and leaves the
    orthogonal complement untouched."""
    rng = np.random.default_rng(6)
    d, N = 7, 12
    k, v, q = rand_stream(rng, N, d, d * d)
    W0 = rng.standard_normal(d * d)
    W_prev = W0.reshape(d, d)
    for n in range(1, N + 1):
        _, Wo, _ = run_oracle(oracle_mod, k[:n], v[:n], q[:n], np.zeros(n), np.zeros(n), np.ones(n),
                              W0, np.zeros(d * d), d, 0, 1, 1)
        Wn = Wo[0].reshape(d, d)
        np.testing.assert_allclose(Wn @ k[n - 1], v[n - 1], atol=1e-12)
        x = rng.standard_normal(d)
        x -= (x @ k[n - 1]) * k[n - 1]
        np.testing.assert_allclose(Wn @ x, W_prev @ x, atol=1e-12)
        W_prev = Wn


@pytest.mark.parametrize("chunk", [5, 16, 64])
def test_minibatch_closed_form_with_forgetting(oracle_mod, chunk):
    """Section 3.2: within a chunk all gradients are taken at the chunk-start
    W_0, so with eta = 0, W_n = beta_n W_0 - sum_i theta_i (beta_n/beta_i)
    (W_0 k_i - v_i) k_i^T, beta the running product of (1 - alpha)."""
    rng = np.random.default_rng(chunk)
    d, N = 6, 50
    k, v, q = rand_stream(rng, N, d, d * d)
    a, t = rng.uniform(0, 0.3, N), rng.uniform(0, 0.6, N)
    e = np.zeros(N)
    W0 = rng.standard_normal(d * d)
    y, Wo, _ = run_oracle(oracle_mod, k, v, q, a, e, t, W0, np.zeros(d * d), d, 0, 1, chunk)
    W = W0.reshape(d, d).copy()
    for c0 in range(0, N, chunk):
        Wst = W.copy()
        idx = range(c0, min(c0 + chunk, N))
        for j in idx:
            bj = prod(1 - a[m] for m in range(c0, j + 1))
            Wj = bj * Wst
            for i in range(c0, j + 1):
                ratio = prod(1 - a[m] for m in range(i + 1, j + 1))
                Wj = Wj - t[i] * ratio * np.outer(Wst @ k[i] - v[i], k[i])
            np.testing.assert_allclose(y[0, j], Wj @ q[j], rtol=1e-11, atol=1e-12)
        W = Wj
    np.testing.assert_allclose(Wo[0].reshape(d, d), W, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# P5/P6: gate edge values
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,d,h", [(1, 5, 0), (2, 4, 8), (4, 3, 6)])
def test_theta_zero_leaves_memory(oracle_mod, L, d, h):
    rng = np.random.default_rng(21)
    N, chunk = 30, 7
    P = oracle_mod.param_count(d, h, L)
    k, v, q = rand_stream(rng, N, d, P)
    W0 = rng.standard_normal(P)
    a = rng.uniform(0, 0.2, N)
    e = rng.uniform(0, 1, N)
    y, Wo, So = run_oracle(oracle_mod, k, v, q, a, e, np.zeros(N), W0, np.zeros(P), d, h, L, chunk)
    assert not So.any()
    np.testing.assert_allclose(Wo[0], prod(1 - a) * W0, rtol=1e-13)
    y, Wo, So = run_oracle(oracle_mod, k, v, q, np.zeros(N), e, np.zeros(N), W0, np.zeros(P), d, h, L, chunk)
    assert np.array_equal(Wo[0], W0) and not So.any()
    mats = split_layers(W0, widths_of(d, h, L))
    for i in range(N):
        np.testing.assert_allclose(y[0, i], torch_forward(mats, q[i]).numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("L,d,h", [(1, 5, 0), (2, 4, 8)])
def test_alpha_one_clears_memory(oracle_mod, L, d, h):
    """alpha = 1 erases the old memory: W_t = S_t (mer.dev 3.1 "Forgetting")."""
    rng = np.random.default_rng(22)
    N, chunk = 20, 4
    P = oracle_mod.param_count(d, h, L)
    k, v, q = rand_stream(rng, N, d, P)
    W0, S0 = rng.standard_normal(P), rng.standard_normal(P)
    e, t = rng.uniform(0, 1, N), rng.uniform(0, 1, N)
    for n in (1, 5, 13, 20):
        _, Wo, So = run_oracle(oracle_mod, k[:n], v[:n], q[:n], np.ones(n), e[:n], t[:n], W0, S0, d, h, L, chunk)
        assert np.array_equal(Wo, So)
    y, Wo, So = run_oracle(oracle_mod, k, v, q, np.ones(N), e, np.zeros(N), W0, np.zeros(P), d, h, L, chunk)
    assert not Wo.any() and not So.any() and not y.any()


@pytest.mark.parametrize("L,d,h", [(2, 4, 8), (4, 3, 6)])
def test_zero_state_is_a_fixed_point_of_the_mlp(oracle_mod, L, d, h):
    """A bias-free MLP memory (mer.dev 3.1 "Memory Architecture", no biases)
    at W = S = 0 has zero gradient for any (k, v): every layer's gradient
    carries either an activation SiLU(0) = 0 or a delta back-propagated
    through a zero matrix (checked here with torch autograd).  So zero
    state stays exactly zero under any gates, and every read is zero --
    the state the long workloads decay into."""
    rng = np.random.default_rng(23)
    N, chunk = 40, 6
    P = oracle_mod.param_count(d, h, L)
    k, v, q = rand_stream(rng, N, d, P)
    assert not autograd_grad(np.zeros(P), widths_of(d, h, L), k[0], v[0]).any()
    a, e, t = rng.uniform(0, 1, N), rng.uniform(0, 1, N), rng.uniform(0, 1, N)
    y, Wo, So = run_oracle(oracle_mod, k, v, q, a, e, t, np.zeros(P), np.zeros(P), d, h, L, chunk)
    assert not Wo.any() and not So.any() and not y.any()


# ----------------------------------------------------------------------------
# gates shared within a chunk (mer.dev section 3.2, "Parameters as the
# Function of Chunks": the chunk is then a time-invariant system)
# ----------------------------------------------------------------------------
def test_chunk_gates_are_the_chunks_tokens_gates(oracle_mod):
    """One value per chunk means every token of the chunk uses it."""
    rng = np.random.default_rng(41)
    d, h, L, N, chunk = 4, 6, 2, 23, 5
    P = oracle_mod.param_count(d, h, L)
    k, v, q = rand_stream(rng, N, d, P)
    nc = -(-N // chunk)
    a, e, t = rng.uniform(0, .3, nc), rng.uniform(.5, 1, nc), rng.uniform(0, .3, nc)
    W0 = rng.standard_normal(P) * 0.3
    got = oracle_mod.forward(k[None], v[None], q[None], a[None], e[None], t[None], W0[None], np.zeros((1, P)),
                             d=d, hidden=h, n_layers=L, chunk=chunk, chunk_gates=True)
    rep = lambda g: np.repeat(g, chunk)[:N]
    ref = run_oracle(oracle_mod, k, v, q, rep(a), rep(e), rep(t), W0, np.zeros(P), d, h, L, chunk)
    for x, y in zip(got, ref):
        assert np.array_equal(x, y)


def test_chunk_gates_make_the_chunk_time_invariant():
    """With alpha, eta, theta constant over a chunk the unrolled coefficients
    depend on j - i only: A_j = a^(j+1), E_j = e^(j+1), U_i = theta e^(n-1-i)
    and D Toeplitz with D[j, i] = theta sum_{u=0}^{j-i} a^(j-i-u) e^u."""
    n, a_, e_, t_ = 9, 0.8, 0.6, 0.3
    A, E, Fc, C, D = coeff_brute(np.full(n, 1 - a_), np.full(n, e_), np.full(n, t_))
    jj = np.arange(n)
    np.testing.assert_allclose(A, a_ ** (jj + 1), rtol=1e-13)
    np.testing.assert_allclose(E, e_ ** (jj + 1), rtol=1e-13)
    np.testing.assert_allclose(C[n - 1], t_ * e_ ** (n - 1 - jj), rtol=1e-13)
    lag = lambda m: t_ * sum(a_ ** (m - u) * e_ ** u for u in range(m + 1))
    for j in range(n):
        for i in range(n):
            np.testing.assert_allclose(D[j, i], lag(j - i) if i <= j else 0.0, rtol=1e-13, atol=1e-15)


def test_chunk_gates_linear_memory_is_a_causal_convolution(oracle_mod):
    """Linear memory, zero start, one chunk with constant gates: retrieval is
    y_t = sum_{i<=t} D[t-i] (k_i . q_t) v_i with the Toeplitz lags above --
    the convolution the time-invariant form allows (section 3.2)."""
    rng = np.random.default_rng(42)
    d, N = 5, 12
    k, v, q = rand_stream(rng, N, d, d * d)
    a_, e_, t_ = 0.15, 0.7, 0.4
    y, _, _ = oracle_mod.forward(k[None], v[None], q[None], np.array([[a_]]), np.array([[e_]]),
                                 np.array([[t_]]), np.zeros((1, d * d)), np.zeros((1, d * d)),
                                 d=d, hidden=0, n_layers=1, chunk=N, chunk_gates=True)
    lag = lambda m: t_ * sum((1 - a_) ** (m - u) * e_ ** u for u in range(m + 1))
    for t in range(N):
        ref = sum(lag(t - i) * float(k[i] @ q[t]) * v[i] for i in range(t + 1))
        np.testing.assert_allclose(y[0, t], ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# P7/P8/P9: attention special cases (mer.dev section 2.1)
# ----------------------------------------------------------------------------
def test_causal_linear_attention(oracle_mod):
    """Linear memory from zero, alpha = eta = 0, one chunk: the memory is the
    linear-attention recurrence M_t = M_{t-1} + v k^T (identity kernel), so
    y_t = sum_{i<=t} theta_i (k_i . q_t) v_i."""
    rng = np.random.default_rng(31)
    d, N = 8, 37
    k, v, q = rand_stream(rng, N, d, d * d)
    t = rng.uniform(0, 1, N)
    y, _, _ = run_oracle(oracle_mod, k, v, q, np.zeros(N), np.zeros(N), t,
                         np.zeros(d * d), np.zeros(d * d), d, 0, 1, N)
    for j in range(N):
        ref = sum(t[i] * (k[i] @ q[j]) * v[i] for i in range(j + 1))
        np.testing.assert_allclose(y[0, j], ref, rtol=1e-12, atol=1e-13)


def test_decayed_linear_attention(oracle_mod):
    """As above with momentum and forgetting: y_t = sum_i D[t,i] (k_i.q_t) v_i,
    D from the explicit products of the unrolled rules."""
    rng = np.random.default_rng(32)
    d, N = 6, 19
    k, v, q = rand_stream(rng, N, d, d * d)
    a, e, t = rng.uniform(0, 0.5, N), rng.uniform(0, 1, N), rng.uniform(0, 1, N)
    y, _, _ = run_oracle(oracle_mod, k, v, q, a, e, t, np.zeros(d * d), np.zeros(d * d), d, 0, 1, N + 3)
    _, _, _, _, D = coeff_brute(a, e, t)
    for j in range(N):
        ref = sum(D[j, i] * (k[i] @ q[j]) * v[i] for i in range(j + 1))
        np.testing.assert_allclose(y[0, j], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("decay", [False, True])
def test_kernelised_linear_attention(oracle_mod, decay):
    """2-layer memory with W2_0 = 0, S_0 = 0, one chunk: the first layer never
    moves (its gradient carries a factor W2_0 = 0), so retrieval is linear
    attention with feature map phi(x) = SiLU(W1_0 x) (section 2.1, kernel
    form): y_t = sum_i D[t,i] (phi(k_i).phi_t(q_t)) v_i, where forgetting
    scales the query-side first layer to A_t W1_0."""
    rng = np.random.default_rng(33 + decay)
    d, h, N = 5, 9, 21
    P = oracle_mod.param_count(d, h, 2)
    k, v, q = rand_stream(rng, N, d, P)
    W0 = np.concatenate([rng.standard_normal(h * d), np.zeros(d * h)])
    if decay:
        a, e, t = rng.uniform(0, 0.4, N), rng.uniform(0, 1, N), rng.uniform(0, 1, N)
    else:
        a, e, t = np.zeros(N), np.zeros(N), rng.uniform(0, 1, N)
    y, Wo, _ = run_oracle(oracle_mod, k, v, q, a, e, t, W0, np.zeros(P), d, h, 2, N)
    W1 = torch.as_tensor(W0[:h * d]).reshape(h, d)
    phi = lambda x, s=1.0: F.silu(F.linear(torch.as_tensor(x), s * W1)).numpy()
    A, _, _, _, D = coeff_brute(a, e, t)
    for j in range(N):
        # forgetting also shrinks the (gradient-free) first layer: W1_j = A_j W1_0
        ref = sum(D[j, i] * (phi(k[i]) @ phi(q[j], A[j])) * v[i] for i in range(j + 1))
        np.testing.assert_allclose(y[0, j], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Wo[0, :h * d], prod(1 - a) * W0[:h * d], rtol=1e-13)


# ----------------------------------------------------------------------------
# P12: unrolled chunk closed form for MLP memories (gradients by autograd)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,d,h,N,chunk", [(2, 4, 8, 29, 8), (2, 6, 10, 40, 16), (4, 3, 6, 23, 5), (1, 5, 0, 33, 7)])
@pytest.mark.parametrize("read_mode", [0, 1])
def test_unrolled_chunk_closed_form(oracle_mod, L, d, h, N, chunk, read_mode):
    """Per chunk (section 3.2: gradients at the chunk-start state), the
    per-token rules of section 3.1 unroll to
        W_j = A_j W_0 + F_j S_0 - sum_i D[j,i] g_i(W_0),
        S_j = E_j S_0 - sum_i C[j,i] g_i(W_0),
    with explicit decay products; g from autograd; y_j = M_{W_j}(q_j)
    (read_mode 0) or M_{W_0}(q_j) (read_mode 1).  Ragged last chunk."""
    rng = np.random.default_rng(L * 1000 + N)
    widths = widths_of(d, h, L)
    P = oracle_mod.param_count(d, h, L)
    k, v, q = rand_stream(rng, N, d, P)
    a, e, t = rng.uniform(0, 0.3, N), rng.uniform(0.3, 1, N), rng.uniform(0, 0.4, N)
    W0, S0 = rng.standard_normal(P) * 0.6, rng.standard_normal(P) * 0.05
    y, Wo, So = run_oracle(oracle_mod, k, v, q, a, e, t, W0, S0, d, h, L, chunk, read_mode)
    W, S = W0.copy(), S0.copy()
    for c0 in range(0, N, chunk):
        idx = list(range(c0, min(c0 + chunk, N)))
        A, E, Fc, C, D = coeff_brute(a[idx], e[idx], t[idx])
        g = [autograd_grad(W, widths, k[i], v[i]) for i in idx]
        Wj = Sj = None
        for jj, j in enumerate(idx):
            Wj = A[jj] * W + Fc[jj] * S - sum(D[jj, ii] * g[ii] for ii in range(jj + 1))
            Sj = E[jj] * S - sum(C[jj, ii] * g[ii] for ii in range(jj + 1))
            Wread = Wj if read_mode == 0 else W
            np.testing.assert_allclose(y[0, j], torch_forward(split_layers(Wread, widths), q[j]).numpy(),
                                       rtol=1e-10, atol=1e-12)
        W, S = Wj, Sj
    np.testing.assert_allclose(Wo[0], W, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(So[0], S, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# P10/P11: linearity, split-and-resume, empty input, stream independence
# ----------------------------------------------------------------------------
def test_linear_memory_is_linear_in_state_and_values(oracle_mod):
    rng = np.random.default_rng(41)
    d, N, chunk = 6, 45, 8
    k, v, q = rand_stream(rng, N, d, d * d)
    a, e, t = rng.uniform(0, 0.2, N), rng.uniform(0.5, 1, N), rng.uniform(0, 0.3, N)
    W0, S0 = rng.standard_normal(d * d), rng.standard_normal(d * d)
    y1, W1, S1 = run_oracle(oracle_mod, k, v, q, a, e, t, W0, S0, d, 0, 1, chunk)
    y2, W2, S2 = run_oracle(oracle_mod, k, 2 * v, q, a, e, t, 2 * W0, 2 * S0, d, 0, 1, chunk)
    assert np.array_equal(y2, 2 * y1) and np.array_equal(W2, 2 * W1) and np.array_equal(S2, 2 * S1)
    y3, W3, S3 = run_oracle(oracle_mod, k, -3 * v, q, a, e, t, -3 * W0, -3 * S0, d, 0, 1, chunk)
    np.testing.assert_allclose(y3, -3 * y1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(W3, -3 * W1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("L,d,h", [(1, 6, 0), (2, 4, 8), (4, 3, 5)])
def test_split_and_resume_is_bitwise(oracle_mod, L, d, h):
    """The state (W, S) is the whole carry between chunks (section 3.2 keeps
    only per-chunk coefficients), so a split on a chunk boundary resumes
    exactly."""
    rng = np.random.default_rng(51)
    N, chunk, N1 = 48, 8, 24
    P = oracle_mod.param_count(d, h, L)
    k, v, q = rand_stream(rng, N, d, P)
    a, e, t = rng.uniform(0, 0.2, N), rng.uniform(0.5, 1, N), rng.uniform(0, 0.3, N)
    W0, S0 = rng.standard_normal(P) * 0.5, np.zeros(P)
    y, Wo, So = run_oracle(oracle_mod, k, v, q, a, e, t, W0, S0, d, h, L, chunk)
    ya, Wa, Sa = run_oracle(oracle_mod, k[:N1], v[:N1], q[:N1], a[:N1], e[:N1], t[:N1], W0, S0, d, h, L, chunk)
    yb, Wb, Sb = run_oracle(oracle_mod, k[N1:], v[N1:], q[N1:], a[N1:], e[N1:], t[N1:], Wa[0], Sa[0],
                            d, h, L, chunk)
    assert np.array_equal(np.concatenate([ya[0], yb[0]]), y[0])
    assert np.array_equal(Wb, Wo) and np.array_equal(Sb, So)


def test_empty_sequence_and_stream_independence(oracle_mod):
    rng = np.random.default_rng(61)
    d, h, L, N = 4, 8, 2, 10
    P = oracle_mod.param_count(d, h, L)
    W0 = rng.standard_normal((3, P))
    S0 = rng.standard_normal((3, P))
    z = np.zeros((3, 0, d))
    y, Wo, So = oracle_mod.forward(z, z, z, np.zeros((3, 0)), np.zeros((3, 0)), np.zeros((3, 0)), W0, S0,
                                   d=d, hidden=h, n_layers=L, chunk=4)
    assert y.shape == (3, 0, d) and np.array_equal(Wo, W0) and np.array_equal(So, S0)
    k = rng.standard_normal((3, N, d))
    gates = [rng.uniform(0, 0.5, (3, N)) for _ in range(3)]
    y, Wo, So = oracle_mod.forward(k, k[::-1].copy(), k[:, ::-1].copy(), *gates, W0, S0,
                                   d=d, hidden=h, n_layers=L, chunk=4, threads=3)
    for s in range(3):
        y1, W1, S1 = oracle_mod.forward(k[s:s + 1], k[::-1][s:s + 1].copy(), k[:, ::-1][s:s + 1].copy(),
                                        *[g[s:s + 1] for g in gates], W0[s:s + 1], S0[s:s + 1],
                                        d=d, hidden=h, n_layers=L, chunk=4, threads=1)
        assert np.array_equal(y1[0], y[s]) and np.array_equal(W1[0], Wo[s]) and np.array_equal(S1[0], So[s])


def test_oracle_rejects_bad_arguments(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.param_count(0, 4, 2)
    z = np.zeros((1, 4, 3))
    g = np.zeros((1, 4))
    W = np.zeros((1, 9))
    with pytest.raises(RuntimeError):
        oracle_mod.forward(z, z, z, g, g, g, W, W, d=3, hidden=0, n_layers=1, chunk=0)

"""The fold weights from scans, as the few-stream key side computes them.

The chunked update of "Titans: Learning to Memorize at Test Time" (section
3.2, the tensorised mini-batch form, with the momentum and forgetting of
section 3.1) folds a chunk of n tokens into the state with two weight
vectors: U_i = theta_i prod_{i<m} eta_m for the surprise and the last row
D[n-1, i] of the matrix D[j, i] = (1 - alpha_j) D[j-1, i] + theta_i
prod_{i<m<=j} eta_m (D[i-1, i] = 0) for the weights.  The reads need all of
D; a key side that does not read gets D's last row from a scan over the
tokens in reverse order instead,

    D[n-1, i] = theta_i R_i,   R_i = a_i + eta_{i+1} R_{i+1},   R_n = 0,
    a_i = prod_{i<m<=n-1} (1 - alpha_m),

run over a 64-token tile whose padding tokens carry alpha = 0, eta = 1,
theta = 0 (so products may run to token 63, and a_i is cut to 0 past n-1).
These tests check that identity in float64 against the recurrence written
out, on random gates and the degenerate ones (eta = 0, alpha = 1, theta = 0,
one-token and ragged chunks).  CPU only.
"""
import numpy as np
import pytest

TILE = 64


def d_last_row_by_recurrence(alpha, eta, theta):
    n = len(alpha)
    d = np.zeros((n, n))
    for i in range(n):
        t = 0.0
        for j in range(n):
            if j < i:
                continue
            t = theta[i] if j == i else t * eta[j]
            prev = d[j - 1, i] if j > i else 0.0
            d[j, i] = (1.0 - alpha[j]) * prev + t
    return d[n - 1]


def u_by_definition(eta, theta):
    n = len(eta)
    return np.array([theta[i] * np.prod(eta[i + 1:n]) for i in range(n)])


def weights_by_scans(alpha, eta, theta):
    """The kernel's reading: a 64-token tile with identity padding, lane l
    holding token i = 63 - l, prefix products and an affine prefix scan over
    the lanes (written here as plain loops over l)."""
    n = len(alpha)
    a = np.zeros(TILE)
    e = np.ones(TILE)
    th = np.zeros(TILE)
    a[:n], e[:n], th[:n] = alpha, eta, theta
    one_minus_a = 1.0 - a
    # lane l's inputs: token i + 1's (1 - alpha, eta), identity at i = 63
    gx = np.array([1.0 if l == 0 else one_minus_a[TILE - l] for l in range(TILE)])
    gy = np.array([1.0 if l == 0 else e[TILE - l] for l in range(TILE)])
    pa = np.cumprod(gx)          # prod_{i<m<=63} (1 - alpha_m)
    pe = np.cumprod(gy)          # prod_{i<m<=63} eta_m
    u = np.zeros(TILE)
    dl = np.zeros(TILE)
    r = 0.0
    for l in range(TILE):
        i = TILE - 1 - l
        ai = pa[l] if i <= n - 1 else 0.0
        r = gy[l] * r + ai       # R_i = a_i + eta_{i+1} R_{i+1}
        u[i] = th[i] * pe[l]
        dl[i] = th[i] * r
    return u[:n], dl[:n]


def _gates(rng, n, case):
    alpha = rng.uniform(0.0, 0.1, n)
    eta = rng.uniform(0.8, 1.0, n)
    theta = rng.uniform(0.0, 0.1, n)
    if case == "eta0":
        eta[:] = 0.0
    elif case == "alpha1":
        alpha[:] = 1.0
    elif case == "eta0_alpha1":
        eta[:] = 0.0
        alpha[:] = 1.0
    elif case == "theta0":
        theta[:] = 0.0
    elif case == "wide":
        alpha = rng.uniform(0.0, 1.0, n)
        eta = rng.uniform(0.0, 1.0, n)
        theta = rng.uniform(0.0, 2.0, n)
    return alpha, eta, theta


@pytest.mark.parametrize("n", [1, 2, 17, 33, 63, 64])
@pytest.mark.parametrize("case", ["random", "eta0", "alpha1", "eta0_alpha1", "theta0", "wide"])
def test_fold_weights_from_scans_match_d_recurrence(n, case):
    rng = np.random.default_rng([7, n, len(case)])
    alpha, eta, theta = _gates(rng, n, case)
    u, dl = weights_by_scans(alpha, eta, theta)
    np.testing.assert_allclose(dl, d_last_row_by_recurrence(alpha, eta, theta), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(u, u_by_definition(eta, theta), rtol=1e-12, atol=1e-300)


def test_fold_weights_closed_forms():
    """Special cases with a closed form: alpha = 1 leaves only the newest
    write (D[n-1, i] = theta_i prod_{i<m<=n-1} eta_m = U_i); eta = 0 keeps
    no earlier surprise (D[n-1, i] = theta_i prod_{i<m<=n-1} (1 - alpha_m));
    one token gives D = U = theta."""
    rng = np.random.default_rng(11)
    n = 40
    alpha, eta, theta = _gates(rng, n, "random")
    u, dl = weights_by_scans(np.ones(n), eta, theta)
    np.testing.assert_allclose(dl, u, rtol=1e-12)
    _, dl = weights_by_scans(alpha, np.zeros(n), theta)
    want = np.array([theta[i] * np.prod(1.0 - alpha[i + 1:]) for i in range(n)])
    np.testing.assert_allclose(dl, want, rtol=1e-12)
    u, dl = weights_by_scans(alpha[:1], eta[:1], theta[:1])
    np.testing.assert_allclose(u, theta[:1], rtol=0)
    np.testing.assert_allclose(dl, theta[:1], rtol=0)

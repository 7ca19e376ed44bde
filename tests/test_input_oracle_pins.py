"""Pins of the input-side oracle (x -> k, v, q and the gates).

Each test checks the fp64 oracle against something other than itself: a
hand-worked example, an impulse response, the receptive field of a causal
width-w convolution, invariants of the l2 norm and the gates, and torch's
own convolution / SiLU / normalisation routines.  The pages ("Titans:
Learning to Memorize at Test Time", mer.dev notes, sections 3.1 and 4.4)
print no numbers for this step.
"""
import math

import numpy as np
import pytest

import oracle
from test_learned_neural_amd import workloads as wl


def _run(f, H, d):
    return oracle.input_side(f["x"], f["w_proj"], f["conv_w"], f["w_gate"], f["b_gate"], f["gate_scale"], H=H, d=d)


def _rand(rng, B=2, N=11, D=8, H=2, d=4, w=3):
    C = H * d
    return {"x": rng.standard_normal((B, N, D)), "w_proj": rng.standard_normal((3, C, D)) / math.sqrt(D),
            "conv_w": rng.standard_normal((3, C, w)), "w_gate": rng.standard_normal((3, H, D)),
            "b_gate": rng.standard_normal((3, H)), "gate_scale": np.array([0.1, 1.0, 0.1])}


def _silu(z):
    return z / (1.0 + math.exp(-z))


def test_hand_worked_example():
    """D = 2, one head of width 2, width-2 convolution, two tokens.

    Rows of W are output channels: channel 0 weighs x by (1, 2), channel 1
    by (3, 4).  x_0 = (1, 0), x_1 = (1, 1) give projections p_0 = (1, 3),
    p_1 = (3, 7).  Taps (current, previous) = (1, 0.5) for channel 0 and
    (2, -1) for channel 1 give u_0 = (1, 6), u_1 = (3.5, 11)."""
    W = np.array([[1.0, 2.0], [3.0, 4.0]])
    taps = np.array([[1.0, 0.5], [2.0, -1.0]])
    f = {"x": np.array([[[1.0, 0.0], [1.0, 1.0]]]), "w_proj": np.stack([W, W, W]),
         "conv_w": np.stack([taps, taps, taps]), "w_gate": np.zeros((3, 1, 2)),
         "b_gate": np.zeros((3, 1)), "gate_scale": np.array([1.0, 1.0, 1.0])}
    k, v, q, a, e, t = _run(f, 1, 2)
    u = [(1.0, 6.0), (3.5, 11.0)]
    for tok in range(2):
        s = np.array([_silu(u[tok][0]), _silu(u[tok][1])])
        np.testing.assert_allclose(v[0, 0, tok], s, rtol=1e-15)
        np.testing.assert_allclose(k[0, 0, tok], s / np.linalg.norm(s), rtol=1e-15)
        np.testing.assert_allclose(q[0, 0, tok], s / np.linalg.norm(s), rtol=1e-15)
    np.testing.assert_array_equal(a, 0.5)     # sigmoid(0) with unit scale


def test_impulse_response_gives_the_taps():
    """Identity projection and one nonzero input element: channel j of
    token t0 + tau sees a * tap[j, tau]; every other element is SiLU(0) = 0."""
    H, d, w, N = 2, 4, 4, 12
    C = H * d
    rng = np.random.default_rng(3)
    taps = rng.standard_normal((3, C, w))
    eye = np.stack([np.eye(C)] * 3)
    t0, j, amp = 5, 6, 1.7
    x = np.zeros((1, N, C))
    x[0, t0, j] = amp
    f = {"x": x, "w_proj": eye, "conv_w": taps, "w_gate": np.zeros((3, H, C)), "b_gate": np.zeros((3, H)),
         "gate_scale": np.ones(3)}
    k, v, q, *_ = _run(f, H, d)
    h, c = divmod(j, d)
    for i, out in enumerate((k, v, q)):
        expect = np.zeros((1, H, N, d))
        for tau in range(w):
            s = _silu(amp * taps[i, j, tau])
            expect[0, h, t0 + tau, c] = s if i == 1 else math.copysign(1.0, s)
        np.testing.assert_allclose(out, expect, rtol=1e-14, atol=0)


def test_causal_receptive_field():
    """Changing x at token t1 changes the k, v, q of tokens t1 .. t1 + w - 1
    only, and the gates of token t1 only."""
    rng = np.random.default_rng(4)
    f = _rand(rng, w=3)
    base = _run(f, 2, 4)
    t1 = 5
    g = dict(f)
    g["x"] = f["x"].copy()
    g["x"][1, t1] += rng.standard_normal(f["x"].shape[2])
    pert = _run(g, 2, 4)
    for i in range(3):
        np.testing.assert_array_equal(pert[i][0], base[i][0])                  # other sequence
        np.testing.assert_array_equal(pert[i][1, :, :t1], base[i][1, :, :t1])  # the past
        np.testing.assert_array_equal(pert[i][1, :, t1 + 3:], base[i][1, :, t1 + 3:])
        assert np.all(np.abs(pert[i][1, :, t1:t1 + 3] - base[i][1, :, t1:t1 + 3]).max(axis=(0, 2)) > 0)
    for i in range(3, 6):
        changed = np.nonzero(np.any(pert[i] != base[i], axis=(0, 1)))[0]
        assert list(changed) == [t1]


def test_window_reproduces_the_full_sequence():
    """Running on tokens [t0 - w + 1, t0 + n) reproduces tokens [t0, t0 + n)
    of the full run (the sampled full-size parity checks rely on this)."""
    rng = np.random.default_rng(5)
    f = _rand(rng, N=30, w=4)
    full = _run(f, 2, 4)
    t0, n = 17, 9
    g = dict(f)
    g["x"] = f["x"][:, t0 - 3:t0 + n]
    win = _run(g, 2, 4)
    for i in range(3):
        np.testing.assert_allclose(win[i][:, :, 3:], full[i][:, :, t0:t0 + n], rtol=1e-14, atol=1e-15)
    for i in range(3, 6):
        np.testing.assert_allclose(win[i][:, :, 3:], full[i][:, :, t0:t0 + n], rtol=1e-15)


def test_norms_and_zero_input():
    rng = np.random.default_rng(6)
    f = _rand(rng)
    k, v, q, *_ = _run(f, 2, 4)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-14)
    assert np.abs(np.linalg.norm(v, axis=-1) - 1.0).max() > 0.1   # v is not normalised
    f["x"] = np.zeros_like(f["x"])                                # SiLU(0) = 0 everywhere: the floor keeps 0
    k, v, q, *_ = _run(f, 2, 4)
    assert not np.any(k) and not np.any(v) and not np.any(q)


def test_gate_closed_forms():
    rng = np.random.default_rng(7)
    f = _rand(rng)
    f["w_gate"] = np.zeros_like(f["w_gate"])
    f["b_gate"] = np.array([[0.0, 2.0], [-1.0, 0.0], [0.0, 40.0]])
    f["gate_scale"] = np.array([0.1, 1.0, 0.25])
    _, _, _, a, e, t = _run(f, 2, 4)
    np.testing.assert_array_equal(a[:, 0], 0.05)
    np.testing.assert_allclose(a[:, 1], 0.1 / (1 + math.exp(-2.0)), rtol=1e-15)
    np.testing.assert_allclose(e[:, 0], 1 / (1 + math.e), rtol=1e-15)
    np.testing.assert_allclose(t[:, 1], 0.25, rtol=1e-15)
    # logits are per head: x . w_gate[g, h]
    f = _rand(rng)
    _, _, _, a, e, t = _run(f, 2, 4)
    for g, out in enumerate((a, e, t)):
        z = f["x"][1, 3] @ f["w_gate"][g, 1] + f["b_gate"][g, 1]
        assert out[1, 1, 3] == pytest.approx(f["gate_scale"][g] / (1 + math.exp(-z)), rel=1e-14)


def test_against_torch_routines():
    """torch's grouped conv1d (a cross-correlation, hence the flipped taps and
    left padding), SiLU and normalize in float64 on the CPU."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(8)
    H, d, w = 3, 8, 4
    f = _rand(rng, B=2, N=19, D=16, H=H, d=d, w=w)
    mine = _run(f, H, d)
    x = torch.from_numpy(f["x"])
    C = H * d
    for i in range(3):
        p = x @ torch.from_numpy(f["w_proj"][i]).T                        # [B, N, C]
        ker = torch.from_numpy(f["conv_w"][i][:, ::-1].copy()).unsqueeze(1)   # [C, 1, w], oldest tap first
        u = F.conv1d(F.pad(p.transpose(1, 2), (w - 1, 0)), ker, groups=C).transpose(1, 2)
        s = F.silu(u).reshape(2, 19, H, d)
        if i != 1:
            s = F.normalize(s, dim=-1, eps=1e-6)
        np.testing.assert_allclose(mine[i], s.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-14)
    for g in range(3):
        z = x @ torch.from_numpy(f["w_gate"][g]).T + torch.from_numpy(f["b_gate"][g])
        ref = (f["gate_scale"][g] * torch.sigmoid(z)).permute(0, 2, 1).numpy()
        np.testing.assert_allclose(mine[3 + g], ref, rtol=1e-13)


def test_generator_prefix_and_law():
    cfg = wl.INPUT_CONFIGS["small"]
    full = wl.make_input_side(cfg)
    pre = wl.make_input_side(cfg, n_tokens=100)
    np.testing.assert_array_equal(pre["x"], full["x"][:, :100])
    for key in ("w_proj", "conv_w", "w_gate", "b_gate"):
        np.testing.assert_array_equal(pre[key], full[key])
    f = wl.input_side_f64(full)
    assert abs(f["x"].std() - 1) < 0.02
    assert abs(f["w_proj"].std() * math.sqrt(cfg.D) - 1) < 0.02

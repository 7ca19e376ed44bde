"""CPU checks of the parity criteria themselves (no GPU): the per-token y
error and the per-row state error catch one wrong token or one wrong row,
and tolerate rounding-sized errors at a token whose reference nearly
cancels."""
import numpy as np

from test_learned_neural_amd import workloads as wl
from parity_util import local_rms, state_row_errors, y_row_errors


def _case(N=256):
    cfg = wl.WORKLOADS["headline"].with_(B=1, H=2, N=N)
    inp = wl.make_inputs(cfg)
    rng = np.random.default_rng(5)
    y_ref = rng.standard_normal((2, N, cfg.d))
    return cfg, inp, y_ref, rng


def test_local_rms_is_the_windowed_rms():
    x = np.arange(1.0, 101.0)
    r = local_rms(x, half_window=3)
    for t in (0, 1, 50, 99):
        lo, hi = max(0, t - 3), min(100, t + 3)
        assert np.isclose(r[t], np.sqrt(np.mean(x[lo:hi] ** 2)))


def test_local_rms_keeps_decayed_windows():
    # a memory that has decayed by 1e-30 late in the sequence: the late
    # windows must come out at their own scale, not as zero
    x = np.concatenate([np.ones(500), np.full(500, 1e-30)])
    r = local_rms(x)
    assert np.allclose(r[700:], 1e-30) and np.allclose(r[:460], 1.0)


def test_y_row_errors_catch_one_wrong_token():
    cfg, inp, y_ref, rng = _case()
    y = y_ref * (1 + 1e-3 * rng.standard_normal(y_ref.shape))
    worst, _ = y_row_errors(cfg, inp, y, y_ref)
    assert worst < 1e-2
    bad = y.copy()
    bad[1, 77] *= 1.5                       # one token off by 50 %
    worst, where = y_row_errors(cfg, inp, bad, y_ref)
    assert worst > 0.3 and where == (1, 77)
    bad = y.copy()
    bad[0, 200] = rng.standard_normal(cfg.d)   # one token entirely wrong
    worst, where = y_row_errors(cfg, inp, bad, y_ref)
    assert worst > 0.5 and where == (0, 200)
    bad = y.copy()
    bad[0, 3, 0] = np.nan
    assert y_row_errors(cfg, inp, bad, y_ref)[0] == np.inf


def test_y_row_errors_judge_a_cancelling_token_on_its_neighbourhood():
    cfg, inp, y_ref, rng = _case()
    y_ref[0, 100] *= 1e-4                   # the reference nearly cancels at token 100
    y = y_ref.copy()
    y[0, 100] += 1e-3 * rng.standard_normal(cfg.d)   # rounding-sized absolute error
    worst, where = y_row_errors(cfg, inp, y, y_ref)
    assert worst < 2e-2, (worst, where)


def test_state_row_errors_catch_one_wrong_row_and_column():
    cfg = wl.WORKLOADS["headline"].with_(B=1, H=1, N=8)
    inp = wl.make_inputs(cfg)
    ref = inp["W0"].astype(np.float64)
    ok = ref * (1 + 1e-3 * np.random.default_rng(1).standard_normal(ref.shape))
    assert state_row_errors(cfg, inp, ok, ref)[0] < 1e-2
    d, h = cfg.d, cfg.hidden
    bad = ok.copy()
    bad[0, 5 * d:(5 + 1) * d] *= 1.3        # row 5 of W1 (hidden unit 5) 30 % off
    worst, where = state_row_errors(cfg, inp, bad, ref)
    assert worst > 0.2 and where[1:3] == (1, "row") and where[3] == 5
    bad = ok.copy()
    W2 = bad[0, h * d:].reshape(d, h)
    W2[:, 9] = 0.0                          # column 9 of W2 (hidden unit 9) lost
    worst, where = state_row_errors(cfg, inp, bad, ref)
    assert worst > 0.9 and where[1:] == (2, "col", 9)

"""GPU parity of the input-side kernel (x -> k, v, q and the gates).

Compared with the fp64 oracle fed the same bf16 x and weights.  The kernel
sums bf16 x bf16 products in fp32 (about 1e-6 relative error over D = 1024
terms) and rounds k, v, q once to bf16, so the bar per element is one bf16
ulp of the reference (a rounding boundary may fall either side of the fp32
value) plus 2e-5 absolute for values near zero, and a norm-wise error per
(token, head) row below 4e-3 (half an ulp is at most 2^-8 relative).  Gates
stay fp32: 1e-5 relative plus 1e-7 absolute.  Sizes: a small workload over
every element (several token tiles, a sequence boundary inside a tile, a
ragged last tile), head widths 16..128, convolution widths 1..4, sequences
shorter than the convolution, and the full headline input side checked on
token windows at sequence starts, tile seams and the end.
"""
import math

import numpy as np
import pytest

import oracle
from test_learned_neural_amd import workloads as wl

pytestmark = pytest.mark.gpu

BF16_ULP_REL = 2.0 ** -7


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch


def _device(inp):
    import torch

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    return dict(x=bf(inp["x"]), w_proj=bf(inp["w_proj"]), conv_w=torch.from_numpy(inp["conv_w"]).cuda(),
                w_gate=bf(inp["w_gate"]), b_gate=torch.from_numpy(inp["b_gate"]).cuda())


def _run_gpu_dev(cfg, inp):
    from test_learned_neural_amd import titans_mem as tmm
    dev = _device(inp)
    return tmm.input_side(dev["x"], dev["w_proj"], dev["conv_w"], dev["w_gate"], dev["b_gate"],
                          tuple(inp["gate_scale"]), H=cfg.H, d=cfg.d)


def _host(ts):
    return [o.float().cpu().double().numpy() for o in ts]


def _run_gpu(cfg, inp):
    return _host(_run_gpu_dev(cfg, inp))


def _run_oracle(cfg, inp, x=None):
    f = wl.input_side_f64(inp)
    if x is not None:
        f["x"] = x
    return oracle.input_side(f["x"], f["w_proj"], f["conv_w"], f["w_gate"], f["b_gate"], f["gate_scale"],
                             H=cfg.H, d=cfg.d)


def _compare(got, ref, label):
    worst = []
    for i, name in enumerate(("k", "v", "q")):
        g, r = got[i], ref[i]
        assert np.all(np.isfinite(g)), name
        err = np.abs(g - r)
        bound = 1.01 * BF16_ULP_REL * np.abs(r) + 2e-5
        assert np.all(err <= bound), (name, float((err - bound).max()), np.unravel_index(np.argmax(err - bound),
                                                                                       err.shape))
        rn = np.linalg.norm(r, axis=-1)
        rows = np.linalg.norm(g - r, axis=-1) / np.maximum(rn, 1e-6)
        assert rows.max() < 4e-3, (name, float(rows.max()))
        worst.append(float(rows.max()))
    for i, name in enumerate(("alpha", "eta", "theta")):
        g, r = got[3 + i], ref[3 + i]
        err = np.abs(g - r)
        assert np.all(err <= 1e-5 * np.abs(r) + 1e-7), (name, float(err.max()))
        worst.append(float((err / np.maximum(np.abs(r), 1e-30)).max()))
    print(f"{label}: row errors k {worst[0]:.2e} v {worst[1]:.2e} q {worst[2]:.2e}; "
          f"gate rel {max(worst[3:]):.2e}", flush=True)


def test_input_small_all_elements():
    cfg = wl.INPUT_CONFIGS["small"]
    inp = wl.make_input_side(cfg)
    _compare(_run_gpu(cfg, inp), _run_oracle(cfg, inp), cfg.name)


@pytest.mark.parametrize("B,N,D,H,d,w", [(1, 300, 64, 8, 16, 4), (2, 257, 128, 4, 32, 3), (1, 400, 96, 1, 128, 2),
                                         (3, 5, 32, 2, 64, 4), (2, 254, 160, 2, 64, 1), (4, 1, 64, 4, 32, 4),
                                         (1, 520, 64, 6, 64, 4), (5, 61, 64, 2, 64, 3)])
def test_input_shapes(B, N, D, H, d, w):
    cfg = wl.INPUT_CONFIGS["small"].with_(B=B, N=N, D=D, H=H, d=d, conv_width=w)
    inp = wl.make_input_side(cfg)
    _compare(_run_gpu(cfg, inp), _run_oracle(cfg, inp), f"B{B} N{N} D{D} H{H} d{d} w{w}")


def test_input_gate_edges():
    """Saturated logits: scale * sigmoid reaches scale and 0 without overflow."""
    cfg = wl.INPUT_CONFIGS["small"].with_(B=1, N=64)
    inp = wl.make_input_side(cfg)
    inp["b_gate"] = np.array([[200.0, -200.0, 0.0, 30.0]] * 3, np.float32)
    got = _run_gpu(cfg, inp)
    ref = _run_oracle(cfg, inp)
    _compare(got, ref, "saturated gates")
    assert np.all(got[3][:, 0] == np.float32(0.1)) and np.all(got[4][:, 1] == 0.0)


def test_input_headline_sampled_windows():
    """The full input side of the headline workload (8 x 16,384 tokens,
    D = 1024, 16 heads of 64), checked on token windows: each window is
    recomputed by the oracle from its tokens and the w - 1 before it."""
    import torch
    cfg = wl.INPUT_CONFIGS["headline"]
    inp = wl.make_input_side(cfg, workers=8)
    out = _run_gpu_dev(cfg, inp)
    torch.cuda.synchronize()
    f = wl.input_side_f64(inp)
    mo = 256 - (cfg.conv_width - 1)
    halo = cfg.conv_width - 1
    # (sequence, first token): sequence starts, a tile seam, a seam that is
    # also a sequence boundary in the flattened rows, the end
    starts = [(0, 0), (3, 0), (0, 5 * mo - 10), (1, (mo * 65) - cfg.N - 8), (5, 8000), (7, cfg.N - 40)]
    n = 40
    for b, t0 in starts:
        lo = max(0, t0 - halo)
        ref = oracle.input_side(f["x"][b:b + 1, lo:t0 + n], f["w_proj"], f["conv_w"], f["w_gate"], f["b_gate"],
                                f["gate_scale"], H=cfg.H, d=cfg.d)
        sub = _host([g[b:b + 1, :, t0:t0 + n] for g in out])
        _compare(sub, [r[:, :, t0 - lo:] for r in ref], f"{cfg.name} seq {b} tokens {t0}..{t0 + n}")
    # the whole output: finite, k and q rows unit vectors, gates inside (0, scale]
    for i in range(3):
        assert bool(torch.isfinite(out[i]).all())
    for i in (0, 2):
        nrm = torch.linalg.vector_norm(out[i].float(), dim=-1)
        assert float((nrm - 1).abs().max()) < 1e-2
    for i in range(3):
        assert bool((out[3 + i] > 0).all()) and bool((out[3 + i] <= cfg.gate_scale[i]).all())


def test_input_feeds_the_memory():
    """x -> (k, v, q, gates) -> memory on the GPU, against the input oracle
    -> bf16 / fp32 storage rounding -> memory oracle on the CPU."""
    import torch
    from test_learned_neural_amd import titans_mem as tmm
    cfg = wl.INPUT_CONFIGS["small"].with_(B=2, N=256)
    inp = wl.make_input_side(cfg)
    k, v, q, a, e, t = _run_gpu_dev(cfg, inp)
    mcfg = wl.WORKLOADS["mlp2_short"].with_(B=cfg.B, H=cfg.H, N=cfg.N)
    W0n = wl.make_inputs(mcfg)["W0"].astype(np.float64)
    W0 = torch.from_numpy(W0n.astype(np.float32)).reshape(cfg.B, cfg.H, -1).cuda()
    y, W, S = tmm.forward(k, v, q, a, e, t, W0, torch.zeros_like(W0), 64, hidden=256, n_layers=2)

    ref = _run_oracle(cfg, inp)
    S_ = cfg.B * cfg.H
    kk, vv, qq = (wl.bf16_bits_to_f64(wl.f64_to_bf16_bits(r)).reshape(S_, cfg.N, cfg.d) for r in ref[:3])
    gg = [r.astype(np.float32).astype(np.float64).reshape(S_, cfg.N) for r in ref[3:]]
    yr, Wr, Sr = oracle.forward(kk, vv, qq, *gg, W0n, np.zeros_like(W0n), d=64, hidden=256, n_layers=2, chunk=64)
    yg = y.float().cpu().double().numpy().reshape(yr.shape)
    Wg = W.cpu().double().numpy().reshape(Wr.shape)
    Sg = S.cpu().double().numpy().reshape(Sr.shape)
    errs = []
    for s in range(S_):
        ey = np.linalg.norm(yg[s] - yr[s]) / np.linalg.norm(yr[s])
        eW = np.linalg.norm(Wg[s] - Wr[s]) / np.linalg.norm(Wr[s])
        eS = np.linalg.norm(Sg[s] - Sr[s]) / np.linalg.norm(Sr[s])
        errs.append(max(ey, eW, eS))
        assert ey < 2e-2 and eW < 2e-2 and eS < 2e-2, (s, ey, eW, eS)
    print(f"x -> memory: max error over y, W, S {max(errs):.2e}")

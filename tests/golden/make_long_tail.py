"""Writes long_tail.json: how the fp64 oracle's memory decays on the
million-token workload (2-layer MLP, d = 64, hidden 256, 16 streams of
1,048,576 tokens, chunk 64, uniform gates alpha ~ U(0, .05), eta ~ U(.85, 1),
theta ~ U(0, .05)).

For four sampled streams it runs the oracle alone (nothing else) over the
first 262,144 tokens and records, per stream, the live length (the last
token at which ||W_t||_F exceeds the floor 1e-30 max(1, ||W_in||_F)), the
largest |y| the reference produces past it, and the largest |W|, |S| at the
end.  The GPU parity test of that workload uses these figures to judge the
outputs past the live length.  Run:  python tests/golden/make_long_tail.py
(about 13 minutes on 4 threads: the fp64 state reaches denormals near token
90,000, where the arithmetic slows down).
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from test_learned_neural_amd import workloads as wl  # noqa: E402

N_TOKENS = 262144
STREAMS = [(0, 0), (0, 5), (0, 10), (0, 15)]


def main():
    cfg = wl.WORKLOADS["long"]
    inp = wl.make_inputs(cfg, streams=STREAMS, n_tokens=N_TOKENS, workers=4)
    f = wl.inputs_f64(cfg, inp)
    y, W, S, wn = oracle.forward(f["k"], f["v"], f["q"], f["alpha"], f["eta"], f["theta"], f["W0"], f["S0"],
                                 d=cfg.d, hidden=cfg.hidden, n_layers=cfg.n_layers, chunk=cfg.chunk,
                                 threads=len(STREAMS), want_w_norm=True)
    rows = []
    for i, (b, h) in enumerate(STREAMS):
        floor = 1e-30 * max(1.0, float(np.linalg.norm(f["W0"][i])))
        alive = np.nonzero(wn[i] > floor)[0]
        live = 0 if len(alive) == 0 else int((alive[-1] + 1) * cfg.chunk)
        rows.append({"b": b, "h": h, "live_length": live,
                     "max_abs_y_past_live": float(np.abs(y[i, live:]).max()),
                     "max_abs_W_end": float(np.abs(W[i]).max()), "max_abs_S_end": float(np.abs(S[i]).max())})
    out = {"workload": cfg.name, "tokens": N_TOKENS, "chunk": cfg.chunk, "streams": rows}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_tail.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()

"""Seeded synthetic workloads for the Titans neural-memory hot path.

This module only draws inputs: random keys/values/queries, gates and initial
memory weights, rounded once to the storage dtype.  It holds none of the
memory's arithmetic (no forward pass, gradient, momentum or forgetting), so
the fp64 oracle and the HIP path can both be fed from it without sharing any
of the method's code.

Workload shapes follow the five memory configurations this project is
measured on (a linear matrix memory and 2- and 4-layer MLP memories).  The
pages behind the method ("Titans: Learning to Memorize at Test Time",
mer.dev notes, section 3.1 "Memory Architecture") fix the memory as a
matrix W or an MLP trained at test time on key/value pairs; they print no
dataset for the memory itself, so everything here is synthetic:

* k, q ~ N(0, 1) per element, each token's row L2-normalised in fp64;
  v ~ N(0, 1) (not normalised).
* gates alpha (forgetting), eta (surprise decay) and theta (surprise weight)
  are per (batch, head, token) fp32 scalars drawn from the law of the
  configuration.
* W0 is either zero or Xavier-uniform per layer; S0 is zero.

Every tensor of every (batch, head) stream comes from its own counter-keyed
generator ``numpy.random.default_rng([seed, b, h, tag])``, so a prefix of
the sequence or a subset of the streams is drawn bit-identically to the
full workload (prefix runs and sampled-stream parity rely on this).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

# tags of the per-tensor generators
_TAG_W0, _TAG_K, _TAG_V, _TAG_Q, _TAG_ALPHA, _TAG_ETA, _TAG_THETA = range(7)


@dataclasses.dataclass(frozen=True)
class MemoryConfig:
    """Shape and input law of one workload.

    n_layers == 1 is the linear matrix memory W (d x d); n_layers >= 2 is a
    bias-free MLP d -> hidden -> ... -> hidden -> d with SiLU between layers.
    """
    name: str
    seed: int
    B: int
    H: int
    N: int
    d: int
    hidden: int
    n_layers: int
    chunk: int
    io: str                       # "f32" or "bf16": dtype of k, v, q and y
    gate_law: str                 # "uniform" or "sigmoid"
    alpha_range: Tuple[float, float] = (0.0, 0.05)
    eta_range: Tuple[float, float] = (0.85, 1.0)
    theta_range: Tuple[float, float] = (0.0, 0.05)
    w0: str = "xavier"            # "xavier" or "zero"

    @property
    def streams(self) -> int:
        return self.B * self.H

    @property
    def widths(self) -> List[int]:
        if self.n_layers == 1:
            return [self.d, self.d]
        return [self.d] + [self.hidden] * (self.n_layers - 1) + [self.d]

    @property
    def param_count(self) -> int:
        w = self.widths
        return sum(w[i] * w[i + 1] for i in range(self.n_layers))

    def with_(self, **kw) -> "MemoryConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  Index 1 is the small linear case, 3 the headline
# throughput case, 4 the million-token streaming case, 5 the deep memory.
WORKLOADS: Dict[str, MemoryConfig] = {
    "linear": MemoryConfig("linear_d64_b1h1_n1024_c16_f32", 1001, B=1, H=1, N=1024, d=64,
                    hidden=0, n_layers=1, chunk=16, io="f32", gate_law="uniform",
                    alpha_range=(0.0, 0.1), eta_range=(0.8, 1.0),
                    theta_range=(0.0, 0.1), w0="zero"),
    "mlp2_short": MemoryConfig("mlp2_d64_h256_b4h8_n4096_c64_bf16", 1002, B=4, H=8, N=4096, d=64,
                    hidden=256, n_layers=2, chunk=64, io="bf16", gate_law="uniform"),
    "headline": MemoryConfig("mlp2_d64_h256_b8h16_n16384_c64_bf16", 1003, B=8, H=16, N=16384,
                    d=64, hidden=256, n_layers=2, chunk=64, io="bf16",
                    gate_law="sigmoid"),
    "long": MemoryConfig("mlp2_d64_h256_b1h16_n1048576_c64_bf16", 1004, B=1, H=16,
                    N=1048576, d=64, hidden=256, n_layers=2, chunk=64, io="bf16",
                    gate_law="uniform"),
    "deep": MemoryConfig("mlp4_d128_h512_b4h8_n32768_c128_bf16", 1005, B=4, H=8, N=32768,
                    d=128, hidden=512, n_layers=4, chunk=128, io="bf16",
                    gate_law="uniform"),
}


# ----------------------------------------------------------------------------
# rounding helpers (storage formats only)
# ----------------------------------------------------------------------------
def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (via fp32, round-to-nearest-even at both steps).

    Returns the raw 16-bit patterns as uint16.  Inputs here are finite.
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def io_to_f64(arr: np.ndarray, io: str) -> np.ndarray:
    """Exact widening of a stored io tensor to float64."""
    if io == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


def round_io(x64: np.ndarray, io: str) -> np.ndarray:
    if io == "bf16":
        return f64_to_bf16_bits(x64)
    return np.asarray(x64, dtype=np.float32)


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------
def _rng(seed: int, b: int, h: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([seed, b, h, tag])


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _draw_stream(cfg: MemoryConfig, b: int, h: int, n_tokens: int):
    s, d = cfg.seed, cfg.d
    k = _unit_rows(_rng(s, b, h, _TAG_K).standard_normal((n_tokens, d)))
    v = _rng(s, b, h, _TAG_V).standard_normal((n_tokens, d))
    q = _unit_rows(_rng(s, b, h, _TAG_Q).standard_normal((n_tokens, d)))
    if cfg.gate_law == "uniform":
        a = _rng(s, b, h, _TAG_ALPHA).uniform(*cfg.alpha_range, size=n_tokens)
        e = _rng(s, b, h, _TAG_ETA).uniform(*cfg.eta_range, size=n_tokens)
        t = _rng(s, b, h, _TAG_THETA).uniform(*cfg.theta_range, size=n_tokens)
    elif cfg.gate_law == "sigmoid":
        # per-token sigmoid of N(0,1) logits; forgetting and surprise weight
        # scaled so that alpha <= 0.1 and theta <= 0.1
        a = 0.1 * _sigmoid(_rng(s, b, h, _TAG_ALPHA).standard_normal(n_tokens))
        e = _sigmoid(_rng(s, b, h, _TAG_ETA).standard_normal(n_tokens))
        t = 0.1 * _sigmoid(_rng(s, b, h, _TAG_THETA).standard_normal(n_tokens))
    else:
        raise ValueError(f"unknown gate law {cfg.gate_law!r}")
    widths = cfg.widths
    g = _rng(s, b, h, _TAG_W0)
    layers = []
    for li in range(cfg.n_layers):
        fan_in, fan_out = widths[li], widths[li + 1]
        if cfg.w0 == "zero":
            layers.append(np.zeros(fan_out * fan_in))
        else:
            bound = math.sqrt(6.0 / (fan_in + fan_out))
            layers.append(g.uniform(-bound, bound, size=fan_out * fan_in))
    w0 = np.concatenate(layers)
    return k, v, q, a, e, t, w0


def stream_ids(cfg: MemoryConfig) -> List[Tuple[int, int]]:
    return [(b, h) for b in range(cfg.B) for h in range(cfg.H)]


def make_inputs(cfg: MemoryConfig, streams: Optional[Sequence[Tuple[int, int]]] = None,
                n_tokens: Optional[int] = None, workers: int = 1) -> Dict[str, np.ndarray]:
    """Draw the inputs of ``cfg`` for the selected (b, h) streams.

    Returns numpy arrays with a leading stream axis (in the order given, by
    default row-major over (b, h)):

    * ``k``, ``v``, ``q``: [S, n, d] in storage form (float32, or uint16
      bfloat16 bit patterns when ``cfg.io == "bf16"``),
    * ``alpha``, ``eta``, ``theta``: [S, n] float32,
    * ``W0``, ``S0``: [S, P] float32 (S0 is zero).
    """
    ids = list(streams) if streams is not None else stream_ids(cfg)
    n = cfg.N if n_tokens is None else int(n_tokens)
    S, d, P = len(ids), cfg.d, cfg.param_count
    kdt = np.uint16 if cfg.io == "bf16" else np.float32
    out = {
        "k": np.empty((S, n, d), kdt), "v": np.empty((S, n, d), kdt),
        "q": np.empty((S, n, d), kdt),
        "alpha": np.empty((S, n), np.float32), "eta": np.empty((S, n), np.float32),
        "theta": np.empty((S, n), np.float32),
        "W0": np.empty((S, P), np.float32), "S0": np.zeros((S, P), np.float32),
    }
    def fill(i):
        b, h = ids[i]
        k, v, q, a, e, t, w0 = _draw_stream(cfg, b, h, n)
        out["k"][i] = round_io(k, cfg.io)
        out["v"][i] = round_io(v, cfg.io)
        out["q"][i] = round_io(q, cfg.io)
        out["alpha"][i] = a
        out["eta"][i] = e
        out["theta"][i] = t
        out["W0"][i] = w0

    if workers > 1 and S > 1:
        # each stream has its own generators, so the fill order is irrelevant
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(S)))
    else:
        for i in range(S):
            fill(i)
    return out


def inputs_f64(cfg: MemoryConfig, inp: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Exact float64 views of stored inputs (what the oracle consumes)."""
    return {
        "k": io_to_f64(inp["k"], cfg.io), "v": io_to_f64(inp["v"], cfg.io),
        "q": io_to_f64(inp["q"], cfg.io),
        "alpha": inp["alpha"].astype(np.float64), "eta": inp["eta"].astype(np.float64),
        "theta": inp["theta"].astype(np.float64),
        "W0": inp["W0"].astype(np.float64), "S0": inp["S0"].astype(np.float64),
    }


# ----------------------------------------------------------------------------
# input side: model activations and projection / convolution / gate weights
# ----------------------------------------------------------------------------
_TAG_X, _TAG_WPROJ, _TAG_CONV, _TAG_WGATE, _TAG_BGATE = range(16, 21)


@dataclasses.dataclass(frozen=True)
class InputConfig:
    """Shape and input law of the input side (x -> k, v, q and the gates).

    x [B, N, D] ~ N(0, 1) rounded to bf16; projection and gate weights
    ~ N(0, 1/D) rounded to bf16 (so each projected channel is ~N(0, 1));
    depthwise taps ~ N(0, 1/w) fp32; gate biases ~ N(0, 0.25) fp32.  The
    gate scales put alpha and theta in (0, 0.1) and eta in (0, 1), the law
    of the sigmoid memory workload.
    """
    name: str
    seed: int
    B: int
    N: int
    D: int
    H: int
    d: int
    conv_width: int = 4
    gate_scale: Tuple[float, float, float] = (0.1, 1.0, 0.1)

    @property
    def channels(self) -> int:
        return self.H * self.d

    def with_(self, **kw) -> "InputConfig":
        return dataclasses.replace(self, **kw)


# the input side of the headline memory workload: 16 heads of width 64 over a
# model width of 1024, 8 sequences of 16,384 tokens
INPUT_CONFIGS: Dict[str, InputConfig] = {
    "headline": InputConfig("input_D1024_h16_d64_b8_n16384_w4_bf16", 2003, B=8, N=16384, D=1024, H=16, d=64),
    "small": InputConfig("input_D256_h4_d64_b2_n700_w4_bf16", 2001, B=2, N=700, D=256, H=4, d=64),
}


def make_input_side(cfg: InputConfig, n_tokens: Optional[int] = None, workers: int = 1) -> Dict[str, np.ndarray]:
    """Draw x and the weights of ``cfg`` (x for the first n_tokens of each
    sequence; a prefix is drawn bit-identically to the full sequence).

    Returns bf16 bit patterns (uint16) for x [B, n, D], w_proj [3, H*d, D]
    and w_gate [3, H, D]; float32 conv_w [3, H*d, w] and b_gate [3, H]; and
    the gate scales as a float64 array of 3.
    """
    n = cfg.N if n_tokens is None else n_tokens
    C, D = cfg.channels, cfg.D
    out = {"x": np.empty((cfg.B, n, D), np.uint16)}

    def fill(b):
        out["x"][b] = f64_to_bf16_bits(_rng(cfg.seed, b, 0, _TAG_X).standard_normal((n, D)))

    if workers > 1 and cfg.B > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(cfg.B)))
    else:
        for b in range(cfg.B):
            fill(b)
    sd = 1.0 / math.sqrt(D)
    out["w_proj"] = f64_to_bf16_bits(_rng(cfg.seed, 0, 0, _TAG_WPROJ).standard_normal((3, C, D)) * sd)
    out["conv_w"] = (_rng(cfg.seed, 0, 0, _TAG_CONV).standard_normal((3, C, cfg.conv_width))
                     / math.sqrt(cfg.conv_width)).astype(np.float32)
    out["w_gate"] = f64_to_bf16_bits(_rng(cfg.seed, 0, 0, _TAG_WGATE).standard_normal((3, cfg.H, D)) * sd)
    out["b_gate"] = (0.5 * _rng(cfg.seed, 0, 0, _TAG_BGATE).standard_normal((3, cfg.H))).astype(np.float32)
    out["gate_scale"] = np.array(cfg.gate_scale, np.float64)
    return out


def input_side_f64(inp: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Exact float64 views of stored input-side tensors (what the oracle consumes)."""
    return {"x": bf16_bits_to_f64(inp["x"]), "w_proj": bf16_bits_to_f64(inp["w_proj"]),
            "conv_w": inp["conv_w"].astype(np.float64), "w_gate": bf16_bits_to_f64(inp["w_gate"]),
            "b_gate": inp["b_gate"].astype(np.float64), "gate_scale": inp["gate_scale"]}

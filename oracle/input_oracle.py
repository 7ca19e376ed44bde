"""fp64 oracle of the memory's input side: x -> k, v, q and the gates.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU library never does.

What it computes, per sequence b, token t and head h ("Titans: Learning to
Memorize at Test Time", mer.dev notes):

* projections k = x W_K, v = x W_V (section 3.1, "Objective") and
  q = x W_Q (section 3.1, "Retrieving a Memory"), without biases;
* a causal depthwise 1-D convolution over time after each of the three
  projections (section 4.4, "Convolution"): channel j of token t mixes the
  projections of tokens t, t-1, ..., t-w+1 with its own w weights, tokens
  before the sequence start counting as zero;
* SiLU on the convolved q, k, v and an l2 normalisation of q and k over each
  head's d channels (section 4.4, "Architectural Details");
* input-dependent gates (section 3.1, "Learning Process and Surprise Metric"
  calls eta_t input dependent, and the forgetting gate alpha_t and the
  surprise weight theta_t are per token too): per head a linear map of x_t
  and a logistic sigmoid, scaled into (0, scale).

The pages leave the order of these steps, the convolution width, the norm's
floor and the gate parameterisation open; the readings taken are:
projection -> convolution -> SiLU -> l2 norm; width w (1..4; the separable
convolution's pointwise half is the projection that precedes it);
k = s / max(||s||, 1e-6); gate = scale * sigmoid(x . w_g + b_g).

Every step below is written as its definition in float64; numpy's matmul is
the only library primitive.
"""
from __future__ import annotations

import numpy as np

NORM_FLOOR = 1e-6


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def causal_depthwise_conv(p: np.ndarray, taps: np.ndarray) -> np.ndarray:
    """u[b, t, j] = sum_{tau < w} taps[j, tau] * p[b, t - tau, j], with
    p[b, t', j] = 0 for t' < 0 (section 4.4, "Convolution").

    p: [B, N, C]; taps: [C, w] (tap tau weighs the token tau steps back)."""
    B, N, C = p.shape
    w = taps.shape[1]
    u = np.zeros_like(p)
    for tau in range(w):
        if tau >= N:
            break
        u[:, tau:, :] += taps[None, None, :, tau] * p[:, :N - tau, :]
    return u


def silu(u: np.ndarray) -> np.ndarray:
    """SiLU(u) = u * sigmoid(u) (section 4.4, "Architectural Details")."""
    return u * _sigmoid(u)


def l2_normalize_heads(s: np.ndarray, H: int, d: int) -> np.ndarray:
    """Each head's d channels divided by their l2 norm (floored at NORM_FLOOR).

    s: [B, N, H*d] -> [B, N, H*d]."""
    B, N, _ = s.shape
    sh = s.reshape(B, N, H, d)
    nrm = np.sqrt(np.sum(sh * sh, axis=-1, keepdims=True))
    return (sh / np.maximum(nrm, NORM_FLOOR)).reshape(B, N, H * d)


def input_side(x, w_proj, conv_w, w_gate, b_gate, gate_scale, *, H: int, d: int):
    """The input side of the memory for whole sequences.

    x:       [B, N, D]       model activations
    w_proj:  [3, H*d, D]     rows of W_K, W_V, W_Q (channel c of head h is
                             row h*d + c; output = x @ w_proj[i].T)
    conv_w:  [3, H*d, w]     causal depthwise taps (tap tau weighs token t - tau)
    w_gate:  [3, H, D]       gate logit weights for alpha, eta, theta
    b_gate:  [3, H]          gate logit biases
    gate_scale: 3 numbers    alpha, eta, theta = scale * sigmoid(logit)

    Returns k, v, q as [B, H, N, d] and alpha, eta, theta as [B, H, N], all
    float64 (no storage rounding).
    """
    x = np.asarray(x, np.float64)
    w_proj = np.asarray(w_proj, np.float64)
    conv_w = np.asarray(conv_w, np.float64)
    w_gate = np.asarray(w_gate, np.float64)
    b_gate = np.asarray(b_gate, np.float64)
    B, N, D = x.shape
    C = H * d
    if w_proj.shape != (3, C, D) or conv_w.shape[:2] != (3, C) or w_gate.shape != (3, H, D) \
            or b_gate.shape != (3, H) or len(gate_scale) != 3:
        raise ValueError("shape mismatch")

    outs = []
    for i in range(3):                         # k, v, q
        p = x @ w_proj[i].T                    # projection [B, N, C]
        u = causal_depthwise_conv(p, conv_w[i])
        s = silu(u)
        if i != 1:                             # k and q are normalised, v is not
            s = l2_normalize_heads(s, H, d)
        outs.append(s.reshape(B, N, H, d).transpose(0, 2, 1, 3).copy())

    gates = []
    for g in range(3):                         # alpha, eta, theta
        z = x @ w_gate[g].T + b_gate[g][None, None, :]      # [B, N, H]
        gates.append((float(gate_scale[g]) * _sigmoid(z)).transpose(0, 2, 1).copy())
    return outs[0], outs[1], outs[2], gates[0], gates[1], gates[2]

"""fp64 CPU oracle for the steps either side of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module; the product path never imports, links or calls it and shares no code
with it.

What the pages define (jianyuh.github.io reading notes "Qwen3.8-Next: GDN, QSA, Gated
Residual", section 2.1 "Gated DeltaNet", "Feature parameterization", "Gating dynamics" and the
output equation after them; ta-paperlens "Designing Qwen3.8-Next", section "Inside GDN: erase
before you write", the paragraph on the actual parameterization):

* features: each projection passes a short causal depthwise convolution, then SiLU; q and k
  are then L2-normalised (per head), v is not;
* gates: beta_t = sigmoid(b_t); alpha_t = exp(-exp(A) * softplus(a_t + b_alpha)) with a per-head
  time constant A and bias b_alpha;
* output: sigmoid(z_t) (.) RMSNorm(y_t), with a zero-centred RMSNorm, before the output
  projection.

Readings where the pages are silent:

* the convolution width is not given: any width W >= 1 is accepted here; tests use W = 4;
  out[t, c] = sum_j w[c, j] x[t - (W-1) + j, c] (w[c, W-1] weighs the current token), with
  the W-1 inputs before a sequence's first token taken from a carried convolution state
  [N, C, W-1] (oldest first) or zero;
* L2Norm(x) = x / sqrt(sum x^2 + eps) over one head's channels, eps = 1e-6;
* "zero-centred RMSNorm": the learnable scale is stored as an offset from one,
  RMSNorm(y) = y / sqrt(mean(y^2) + eps) * (1 + w), eps = 1e-6, over one head's d_v values;
* softplus(x) = log(1 + exp(x)).

Everything is plain numpy in float64, token by token where the definition is sequential; the
only library primitives are exp, log1p, sqrt and sums.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

EPS = 1e-6


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def short_conv_silu(x: np.ndarray, w: np.ndarray, cu_seqlens: Sequence[int],
                    head_dim: int = 0, state_in: Optional[np.ndarray] = None,
                    eps: float = EPS) -> Tuple[np.ndarray, np.ndarray]:
    """Causal depthwise convolution, SiLU and (head_dim > 0) a per-head L2 normalisation.

    x: [T, C] (tokens of all sequences packed); w: [C, W]; cu_seqlens: [N+1] row offsets;
    state_in: [N, C, W-1] or None (zeros).  Returns (out [T, C], state_out [N, C, W-1]):
    state_out[n] holds the W-1 inputs that end sequence n, oldest first, reaching back into
    state_in[n] when the sequence is shorter than W-1."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    N = len(cu_seqlens) - 1
    out = np.zeros((T, C))
    state_out = np.zeros((N, C, W - 1))
    for n in range(N):
        s, e = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        prev = np.zeros((C, W - 1)) if state_in is None else np.asarray(state_in[n], np.float64)
        # ext row i (0 <= i < W-1 + L) is the input W-1 rows before row i of the sequence
        ext = np.concatenate([prev.T, x[s:e]], axis=0)
        for t in range(e - s):
            acc = np.zeros(C)
            for j in range(W):
                acc += w[:, j] * ext[t + j]
            out[s + t] = acc
        state_out[n] = ext[e - s:e - s + W - 1].T
    out = silu(out)
    if head_dim:
        H = C // head_dim
        o = out.reshape(T, H, head_dim)
        o = o / np.sqrt((o * o).sum(axis=-1, keepdims=True) + eps)
        out = o.reshape(T, C)
    return out, state_out


def gates(a: np.ndarray, b: np.ndarray, A: np.ndarray,
          b_alpha: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """a, b: [T, H] pre-activations; A, b_alpha: [H].  Returns (alpha, beta, log alpha)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    log_alpha = -np.exp(np.asarray(A, np.float64))[None, :] * softplus(a + np.asarray(b_alpha, np.float64)[None, :])
    return np.exp(log_alpha), sigmoid(b), log_alpha


def output_gate(y: np.ndarray, z: np.ndarray, w: np.ndarray, eps: float = EPS) -> np.ndarray:
    """y, z: [..., d_v]; w: [d_v] (the zero-centred scale).  Returns
    sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w) over the last axis."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    r = y / np.sqrt((y * y).mean(axis=-1, keepdims=True) + eps)
    return sigmoid(z) * r * (1.0 + w)

"""Independent fp64 checkers used to pin the oracle (test code only).

Nothing here imports the oracle or the HIP path.

* :func:`transition_bruteforce` -- the boxed "equivalent transition matrix" form from the
  jianyuh.github.io reading notes on Qwen3.8-Next, section 2.1:
  S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, with every transition
  written as an explicit d_k x d_k matrix and the state after t tokens formed as the product
  A_t ... A_1 S_0 + sum_i A_t ... A_{i+1} B_i.  Meant for T <= 8.
* :func:`chunked_fp64` -- the chunked (WY / UT) form of the same recurrence, derived from the
  transition form: within a chunk that starts at state S0, with g_t the within-chunk prefix
  sum of log alpha, gamma_t = e^{g_t} and Gamma_ti = e^{g_t - g_i} (i <= t),
    T  = (I + diag(beta) strictlower(K K^T o Gamma))^{-1}
    U  = T diag(beta) (V - diag(gamma) K S0)
    Y  = diag(gamma) Q S0 + tril(Q K^T o Gamma) U
    S' = gamma_c S0 + (diag(gamma_c / gamma) K)^T U.
  This is the algebra the GPU kernels implement; here it is checked against the oracle.
* mutants -- plausible mistakes in the recurrence, each of which must fail one pin.
"""
from __future__ import annotations

import numpy as np


def transition_bruteforce(q, k, v, alpha, beta, s0):
    """Explicit transition-matrix products (boxed form).  Returns (y [T, dv], S_T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, dk = k.shape
    I = np.eye(dk)
    A = [alpha[t] * (I - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    Bm = [beta[t] * np.outer(k[t], v[t]) for t in range(T)]
    y = np.zeros((T, v.shape[1]))
    S_t = None
    for t in range(T):
        # S_t = (A_t ... A_1) S_0 + sum_{i<=t} (A_t ... A_{i+1}) B_i
        prod = I.copy()
        for j in range(t, -1, -1):
            prod = prod @ A[j]
        S_t = prod @ s0
        for i in range(t + 1):
            P = I.copy()
            for j in range(t, i, -1):
                P = P @ A[j]
            S_t = S_t + P @ Bm[i]
        y[t] = S_t.T @ q[t]
    return y, (np.array(s0, np.float64) if S_t is None else S_t)


def chunked_fp64(q, k, v, alpha, beta, s0, C):
    """Chunked form with chunk size C (any C >= 1).  Returns (y [T, dv], S_T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    T = k.shape[0]
    S = np.array(s0, np.float64)
    y = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        Kc, Qc, Vc = k[c0:c1], q[c0:c1], v[c0:c1]
        bc = beta[c0:c1]
        g = np.cumsum(np.log(alpha[c0:c1]))
        n = c1 - c0
        diff = g[:, None] - g[None, :]
        lower_incl = np.tril(np.ones((n, n), bool))
        Gam = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
        gam = np.exp(g)
        A = np.diag(bc) @ np.tril(Kc @ Kc.T * Gam, -1)
        Tm = np.linalg.inv(np.eye(n) + A)
        U = Tm @ np.diag(bc) @ (Vc - np.diag(gam) @ Kc @ S)
        y[c0:c1] = np.diag(gam) @ Qc @ S + np.tril(Qc @ Kc.T * Gam) @ U
        S = gam[-1] * S + (np.diag(np.exp(g[-1] - g)) @ Kc).T @ U
    return y, S


# ---------------------------------------------------------------------------------------
# Mutants: plausible mistakes.  Same signature as the oracle's single-chain functions.
# ---------------------------------------------------------------------------------------

def _mutant(step):
    def run(q, k, v, alpha, beta, s0=None):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        T, dk = k.shape
        S = np.zeros((dk, v.shape[1])) if s0 is None else np.array(s0, np.float64)
        y = np.zeros((T, v.shape[1]))
        for t in range(T):
            S, y[t] = step(S, q, k, v, alpha, beta, t)
        return y, S
    return run


def _placed_step(residual_against: str, decay_at: str):
    """One delta-rule step with the decay placed by the arguments.  The rule (Gated DeltaNet,
    section 2.1; the paper-lens walkthrough's section "Inside GDN: erase before you write")
    erases against the decayed state and decays before writing: residual_against="decayed",
    decay_at="before".  The other settings are the plausible misplacements: the residual taken
    against the state before its decay, and/or the decay applied after the write."""
    assert residual_against in ("decayed", "undecayed") and decay_at in ("before", "after")

    def step(S, q, k, v, a, b, t):
        R = a[t] * S if residual_against == "decayed" else S
        e = v[t] - R.T @ k[t]
        if decay_at == "before":
            S = a[t] * S + b[t] * np.outer(k[t], e)
        else:
            S = a[t] * (S + b[t] * np.outer(k[t], e))
        return S, S.T @ q[t]
    return step


# residual against the undecayed state, while the kept part of the state is decayed
_undecayed_residual = _placed_step("undecayed", "before")


def _additive(S, q, k, v, a, b, t):
    # plain gated linear attention: no erase term
    S = a[t] * S + b[t] * np.outer(k[t], v[t])
    return S, S.T @ q[t]


def _read_before_write(S, q, k, v, a, b, t):
    Sd = a[t] * S
    y = Sd.T @ q[t]
    e = v[t] - Sd.T @ k[t]
    return Sd + b[t] * np.outer(k[t], e), y


# the whole update, write included, decayed afterwards
_decay_after_write = _placed_step("undecayed", "after")


def _residual_sign(S, q, k, v, a, b, t):
    Sd = a[t] * S
    e = v[t] + Sd.T @ k[t]
    S = Sd + b[t] * np.outer(k[t], e)
    return S, S.T @ q[t]


def _erase_without_beta(S, q, k, v, a, b, t):
    # S = alpha S + beta k v^T - alpha k k^T S   (beta dropped from the erase)
    S = a[t] * S + b[t] * np.outer(k[t], v[t]) - a[t] * np.outer(k[t], k[t]) @ S
    return S, S.T @ q[t]


def _erase_without_alpha(S, q, k, v, a, b, t):
    # S = alpha S + beta k v^T - beta k k^T S   (alpha dropped from the erase)
    S = a[t] * S + b[t] * np.outer(k[t], v[t]) - b[t] * np.outer(k[t], k[t]) @ S
    return S, S.T @ q[t]


def _shifted_gate(S, q, k, v, a, b, t):
    at = a[t - 1] if t > 0 else 1.0
    Sd = at * S
    e = v[t] - Sd.T @ k[t]
    S = Sd + b[t] * np.outer(k[t], e)
    return S, S.T @ q[t]


def _query_is_key(S, q, k, v, a, b, t):
    Sd = a[t] * S
    e = v[t] - Sd.T @ k[t]
    S = Sd + b[t] * np.outer(k[t], e)
    return S, S.T @ k[t]


def _transposed_state(S, q, k, v, a, b, t):
    # uses S k / S q instead of S^T k / S^T q (only shape-compatible when d_k == d_v)
    Sd = a[t] * S
    e = v[t] - Sd @ k[t]
    S = Sd + b[t] * np.outer(k[t], e)
    return S, S @ q[t]


def _write_outer_swapped(S, q, k, v, a, b, t):
    # S + beta e k^T  instead of  S + beta k e^T
    Sd = a[t] * S
    e = v[t] - Sd.T @ k[t]
    S = Sd + b[t] * np.outer(e, k[t])
    return S, S.T @ q[t]


def _beta_squared(S, q, k, v, a, b, t):
    Sd = a[t] * S
    e = v[t] - Sd.T @ k[t]
    S = Sd + b[t] * b[t] * np.outer(k[t], e)
    return S, S.T @ q[t]


def _no_initial_state(S, q, k, v, a, b, t):
    if t == 0:
        S = np.zeros_like(S)
    Sd = a[t] * S
    e = v[t] - Sd.T @ k[t]
    S = Sd + b[t] * np.outer(k[t], e)
    return S, S.T @ q[t]


MUTANTS = {
    "undecayed_residual": _mutant(_undecayed_residual),
    "additive_linear_attention": _mutant(_additive),
    "read_before_write": _mutant(_read_before_write),
    "decay_after_write": _mutant(_decay_after_write),
    "residual_sign": _mutant(_residual_sign),
    "erase_without_beta": _mutant(_erase_without_beta),
    "erase_without_alpha": _mutant(_erase_without_alpha),
    "shifted_gate": _mutant(_shifted_gate),
    "query_is_key": _mutant(_query_is_key),
    "transposed_state": _mutant(_transposed_state),
    "write_outer_swapped": _mutant(_write_outer_swapped),
    "beta_squared": _mutant(_beta_squared),
    "ignores_initial_state": _mutant(_no_initial_state),
}

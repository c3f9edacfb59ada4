"""Pins for a single-chain implementation of the gated delta rule (test code only).

Each ``pin_*`` takes ``impl(q, k, v, alpha, beta, s0) -> (y [T, d_v], S_T [d_k, d_v])`` and
raises ``AssertionError`` when the implementation disagrees with something the pages or the
mathematics fix independently of it.  The recurrence is the one in the jianyuh.github.io
reading notes on Qwen3.8-Next, section 2.1 "Gated DeltaNet"; each pin names what fixes it.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from checkers import chunked_fp64, transition_bruteforce

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, "%s: max |diff| %.3e > %.1e * %.3e" % (what, err, rtol, scale)


def _rand_chain(rng, T, dk, dv, a_lo=0.3, a_hi=1.0, unit_keys=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = rng.uniform(a_lo, a_hi, T)
    b = rng.uniform(0.0, 1.0, T)
    s0 = rng.standard_normal((dk, dv))
    return q, k, v, a, b, s0


def pin_hand_worked(impl):
    """Hand-worked three-token example in exact rationals (tests/golden)."""
    with open(os.path.join(GOLDEN, "hand_worked_d2_T3.json")) as f:
        g = json.load(f)
    fr = lambda s: float(Fraction(s))
    s0 = np.array([[fr(x) for x in r] for r in g["S0"]])
    toks = g["tokens"]
    q = np.array([[fr(x) for x in t["q"]] for t in toks])
    k = np.array([[fr(x) for x in t["k"]] for t in toks])
    v = np.array([[fr(x) for x in t["v"]] for t in toks])
    a = np.array([fr(t["alpha"]) for t in toks])
    b = np.array([fr(t["beta"]) for t in toks])
    y, S = impl(q, k, v, a, b, s0)
    ey = np.array([[fr(x) for x in r] for r in g["expected"]["y"]])
    eS = np.array([[fr(x) for x in r] for r in g["expected"]["S_final"]])
    _close(y, ey, 1e-14, "hand-worked y")
    _close(S, eS, 1e-14, "hand-worked S_final")


def pin_bruteforce(impl):
    """Explicit transition-matrix products (the page's boxed form) for T = 1..8."""
    rng = np.random.default_rng(11)
    for T in range(1, 9):
        q, k, v, a, b, s0 = _rand_chain(rng, T, 4, 3, unit_keys=(T % 2 == 0))
        y, S = impl(q, k, v, a, b, s0)
        ey, eS = transition_bruteforce(q, k, v, a, b, s0)
        _close(y, ey, 1e-12, "bruteforce y T=%d" % T)
        _close(S, eS, 1e-12, "bruteforce S T=%d" % T)


def pin_identity_gates(impl):
    """alpha = 1, beta = 0: the state never changes (bit for bit); y_t = S0^T q_t."""
    rng = np.random.default_rng(12)
    q, k, v, _, _, s0 = _rand_chain(rng, 9, 5, 3)
    T = q.shape[0]
    y, S = impl(q, k, v, np.ones(T), np.zeros(T), s0)
    assert np.array_equal(S, s0), "alpha=1, beta=0 changed the state"
    _close(y, q @ s0, 1e-14, "alpha=1, beta=0 read-out")


def pin_beta_zero(impl):
    """beta = 0: S_T = (prod alpha) S0 and y_t = gamma_t S0^T q_t (pure decay)."""
    rng = np.random.default_rng(13)
    q, k, v, a, _, s0 = _rand_chain(rng, 12, 5, 4)
    T = q.shape[0]
    y, S = impl(q, k, v, a, np.zeros(T), s0)
    gam = np.cumprod(a)
    _close(S, gam[-1] * s0, 1e-13, "beta=0 state")
    _close(y, gam[:, None] * (q @ s0), 1e-13, "beta=0 read-out")


def pin_orthonormal_recall(impl):
    """beta = 1 with orthonormal keys: S_T^T k_i = (prod_{j>i} alpha_j) v_i for every i,
    whatever S0 ("targeted erase-and-write": the write replaces what k_i retrieves)."""
    rng = np.random.default_rng(14)
    dk, dv, T = 6, 4, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm.T[:T]                      # orthonormal rows
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    s0 = rng.standard_normal((dk, dv))
    for a in (np.ones(T), rng.uniform(0.4, 0.95, T)):
        _, S = impl(q, k, v, a, np.ones(T), s0)
        for i in range(T):
            expect = np.prod(a[i + 1:]) * v[i]
            _close(S.T @ k[i], expect, 1e-13, "orthonormal recall i=%d" % i)


def pin_repeated_key(impl):
    """Writing (k, v1) then (k, v2) with beta = 1, alpha = 1 leaves S^T k = v2 (replace,
    not accumulate; additive linear attention would give v1 + v2 + S0^T k)."""
    rng = np.random.default_rng(15)
    dk, dv = 5, 3
    kk = rng.standard_normal(dk)
    kk /= np.linalg.norm(kk)
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    s0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((2, dk))
    _, S = impl(q, np.stack([kk, kk]), np.stack([v1, v2]), np.ones(2), np.ones(2), s0)
    _close(S.T @ kk, v2, 1e-13, "repeated key")


def pin_scalar(impl):
    """d_k = d_v = 1 with constant coefficients: s_t = a s_{t-1} + c with
    a = alpha (1 - beta k^2), c = beta k v, whose closed form is
    s_T = a^T s_0 + c (1 - a^T) / (1 - a)."""
    T = 50
    alpha, beta, kk, vv, qq, s0 = 0.9, 0.6, 0.8, 1.7, -1.3, 0.25
    y, S = impl(np.full((T, 1), qq), np.full((T, 1), kk), np.full((T, 1), vv),
                np.full(T, alpha), np.full(T, beta), np.array([[s0]]))
    a = alpha * (1.0 - beta * kk * kk)
    c = beta * kk * vv
    t = np.arange(1, T + 1)
    s_t = a ** t * s0 + c * (1.0 - a ** t) / (1.0 - a)
    _close(S[0, 0], s_t[-1], 1e-13, "scalar closed form S")
    _close(y[:, 0], qq * s_t, 1e-13, "scalar closed form y")


def pin_superposition(impl):
    """For fixed q, k, alpha, beta the outputs are jointly linear in (V, S0)."""
    rng = np.random.default_rng(16)
    q, k, v1, a, b, s01 = _rand_chain(rng, 10, 5, 4)
    v2 = rng.standard_normal(v1.shape)
    s02 = rng.standard_normal(s01.shape)
    y1, S1 = impl(q, k, v1, a, b, s01)
    y2, S2 = impl(q, k, v2, a, b, s02)
    y3, S3 = impl(q, k, v1 - 2.5 * v2, a, b, s01 - 2.5 * s02)
    _close(y3, y1 - 2.5 * y2, 1e-12, "superposition y")
    _close(S3, S1 - 2.5 * S2, 1e-12, "superposition S")


def pin_contraction(impl):
    """||S_t||_2 <= alpha_t ||S_{t-1}||_2 + beta_t ||k_t|| ||v_t|| when beta_t ||k_t||^2 <= 2
    (I - beta k k^T has spectral norm <= 1 then)."""
    rng = np.random.default_rng(17)
    q, k, v, a, b, s0 = _rand_chain(rng, 12, 5, 4, unit_keys=False)
    k *= 1.2 / np.linalg.norm(k, axis=1, keepdims=True)   # ||k||^2 = 1.44, beta <= 1
    prev = np.linalg.norm(s0, 2)
    for t in range(1, q.shape[0] + 1):
        _, S = impl(q[:t], k[:t], v[:t], a[:t], b[:t], s0)
        cur = np.linalg.norm(S, 2)
        bound = a[t - 1] * prev + b[t - 1] * np.linalg.norm(k[t - 1]) * np.linalg.norm(v[t - 1])
        assert cur <= bound * (1 + 1e-12), "contraction bound broken at t=%d" % t
        prev = cur


def pin_chunked(impl):
    """The chunked WY/UT form reaches the same result for every chunk size."""
    rng = np.random.default_rng(18)
    T, dk, dv = 40, 8, 6
    q, k, v, _, b, s0 = _rand_chain(rng, T, dk, dv)
    a = 1.0 / (1.0 + np.exp(-(1.0 + 2.0 * rng.standard_normal(T))))   # strong decay mix
    y, S = impl(q, k, v, a, b, s0)
    for C in (1, 3, 7, 16, T, T + 5):
        cy, cS = chunked_fp64(q, k, v, a, b, s0, C)
        _close(y, cy, 1e-12, "chunked y C=%d" % C)
        _close(S, cS, 1e-12, "chunked S C=%d" % C)


def pin_affine(impl):
    """S_T(S0, V) = M S0 + B with M = S_T(I, 0) and B = S_T(0, V); ||M||_2 <= prod alpha
    (composition of segments, and the decay bound on the segment transition)."""
    rng = np.random.default_rng(19)
    T, dk, dv = 14, 5, 3
    q, k, v, a, b, s0 = _rand_chain(rng, T, dk, dv)
    _, S = impl(q, k, v, a, b, s0)
    _, M = impl(q, k, np.zeros((T, dk)), a, b, np.eye(dk))
    _, Bm = impl(q, k, v, a, b, np.zeros((dk, dv)))
    _close(S, M @ s0 + Bm, 1e-12, "affine composition")
    assert np.linalg.norm(M, 2) <= np.prod(a) * (1 + 1e-12), "||M|| exceeds prod alpha"


def pin_resume(impl):
    """Running T tokens equals running T1 tokens, then the rest from the returned state."""
    rng = np.random.default_rng(20)
    q, k, v, a, b, s0 = _rand_chain(rng, 17, 4, 5)
    y, S = impl(q, k, v, a, b, s0)
    for t1 in (1, 6, 16):
        y1, S1 = impl(q[:t1], k[:t1], v[:t1], a[:t1], b[:t1], s0)
        y2, S2 = impl(q[t1:], k[t1:], v[t1:], a[t1:], b[t1:], S1)
        _close(np.concatenate([y1, y2]), y, 1e-13, "resume y t1=%d" % t1)
        _close(S2, S, 1e-13, "resume S t1=%d" % t1)


PINS = [pin_hand_worked, pin_bruteforce, pin_identity_gates, pin_beta_zero,
        pin_orthonormal_recall, pin_repeated_key, pin_scalar, pin_superposition,
        pin_contraction, pin_chunked, pin_affine, pin_resume]

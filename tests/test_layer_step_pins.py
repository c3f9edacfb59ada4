"""The layer-step oracle (oracle/layer_steps.py) against what the pages and the mathematics
fix (CPU only): the hand-worked fixture, a library convolution, closed forms and invariants.
A mutation test checks that each plausible mistake fails at least one pin."""
import json
import math
import os

import numpy as np
import pytest

from oracle import layer_steps as ls

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "hand_worked_layer_steps.json")))


def _silu_ref(x):
    # x / (1 + e^-x), written independently of the oracle's tanh form
    return np.array([[v / (1.0 + math.exp(-v)) for v in row] for row in x])


# ---- pins, each taking the three oracle functions so that mutants can stand in ----------

def pin_conv_fixture(conv, gates, gate_out):
    g = GOLD["conv"]
    out, st = conv(np.array(g["x"]), np.array(g["w"]), g["cu_seqlens"], 0,
                   np.array(g["state_in"]))
    np.testing.assert_allclose(out, _silu_ref(g["pre_activation"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(st, np.array(g["state_out"]), rtol=0, atol=0)


def pin_gates_fixture(conv, gates, gate_out):
    g = GOLD["gates"]
    al, be, la = gates(np.array(g["a"]), np.array(g["b"]), np.array(g["A"]),
                       np.array(g["b_alpha"]))
    np.testing.assert_allclose(al, np.array(g["alpha"]), rtol=1e-14)
    np.testing.assert_allclose(be, np.array(g["beta"]), rtol=1e-14)
    np.testing.assert_allclose(la, np.log(np.array(g["alpha"])), rtol=1e-14)


def pin_output_gate_fixture(conv, gates, gate_out):
    g = GOLD["output_gate"]
    o = gate_out(np.array(g["y"]), np.array(g["z"]), np.array(g["w"]), g["eps"])
    np.testing.assert_allclose(o, np.array(g["expected"]), rtol=1e-14)


def pin_conv_matches_library(conv, gates, gate_out):
    """With zero state, each sequence is torch's grouped conv1d over the left-padded input
    (a library routine, fp64 on the CPU), followed by x * sigmoid(x)."""
    import torch
    rng = np.random.default_rng(11)
    cu = [0, 5, 5, 37, 40]
    C, W = 6, 4
    x = rng.standard_normal((40, C))
    w = rng.standard_normal((C, W))
    out, _ = conv(x, w, cu, 0, None)
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        if e == s:
            continue
        xt = torch.from_numpy(x[s:e].T.copy())[None]                   # [1, C, L]
        xt = torch.nn.functional.pad(xt, (W - 1, 0))
        ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w[:, None, :].copy()), groups=C)
        ref = ref[0].numpy().T
        np.testing.assert_allclose(out[s:e], ref / (1.0 + np.exp(-ref)), rtol=1e-12, atol=1e-14)


def pin_conv_state_chains(conv, gates, gate_out):
    """One call over a sequence equals two calls over its halves with the state carried, for
    every split, including splits shorter than the window."""
    rng = np.random.default_rng(12)
    C, W, L = 5, 4, 11
    x = rng.standard_normal((L, C))
    w = rng.standard_normal((C, W))
    s0 = rng.standard_normal((1, C, W - 1))
    full, sf = conv(x, w, [0, L], 0, s0)
    for cut in range(0, L + 1):
        a, sa = conv(x[:cut], w, [0, cut], 0, s0)
        b, sb = conv(x[cut:], w, [0, L - cut], 0, sa)
        np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(sb, sf, rtol=0, atol=0)


def pin_conv_state_layout(conv, gates, gate_out):
    """The carried state is the W-1 inputs before the next token, oldest first: for a long
    sequence its last W-1 rows; for a short one, the tail of the incoming state followed by
    the sequence's rows."""
    rng = np.random.default_rng(16)
    C, W = 3, 4
    x = rng.standard_normal((9, C))
    s0 = rng.standard_normal((2, C, W - 1))
    w = rng.standard_normal((C, W))
    _, st = conv(x, w, [0, 7, 9], 0, s0)
    np.testing.assert_array_equal(st[0], x[4:7].T)
    np.testing.assert_array_equal(st[1], np.concatenate([s0[1][:, 2:], x[7:9].T], axis=1))


def pin_conv_delta_weight_is_identity(conv, gates, gate_out):
    """A weight that keeps only the current token turns the block into SiLU."""
    rng = np.random.default_rng(13)
    C, W = 4, 3
    x = rng.standard_normal((9, C))
    w = np.zeros((C, W)); w[:, W - 1] = 1.0
    out, _ = conv(x, w, [0, 4, 9], 0, rng.standard_normal((2, C, W - 1)))
    np.testing.assert_allclose(out, _silu_ref(x), rtol=1e-13, atol=1e-15)


def pin_l2norm_unit_heads(conv, gates, gate_out):
    """With head_dim set, every head of every token has unit norm (up to eps) and points the
    way the un-normalised output does."""
    rng = np.random.default_rng(14)
    C, W, d = 8, 4, 4
    x = rng.standard_normal((12, C)) * 3
    w = rng.standard_normal((C, W))
    raw, _ = conv(x, w, [0, 12], 0, None)
    out, _ = conv(x, w, [0, 12], d, None, 0.0)
    o = out.reshape(12, C // d, d); r = raw.reshape(12, C // d, d)
    np.testing.assert_allclose(np.linalg.norm(o, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(o * np.linalg.norm(r, axis=-1, keepdims=True), r, rtol=1e-12, atol=1e-14)


def pin_gates_closed_forms(conv, gates, gate_out):
    """alpha in (0, 1) and decreasing in a and in A; beta = 1 - beta(-b); A -> -inf gives 1;
    large a gives alpha ~ exp(-e^A (a + b_alpha))."""
    a = np.linspace(-30, 30, 61)[:, None] * np.ones((1, 3))
    b = np.linspace(-8, 8, 61)[:, None] * np.ones((1, 3))
    A = np.array([-1.0, 0.0, 0.5]); ba = np.array([0.3, -0.2, 0.0])
    al, be, la = gates(a, b, A, ba)
    assert np.all(al > 0) and np.all(al <= 1)
    assert np.all(np.diff(al, axis=0) <= 0)
    _, be2, _ = gates(a, -b, A, ba)
    np.testing.assert_allclose(be + be2, 1.0, rtol=1e-15)
    np.testing.assert_allclose(la[-1], -np.exp(A) * (30 + ba), rtol=1e-12)
    al_inf, _, _ = gates(a, b, np.array([-800.0, -800.0, -800.0]), ba)
    np.testing.assert_allclose(al_inf, 1.0, rtol=0, atol=0)


def pin_output_gate_invariants(conv, gates, gate_out):
    """With w = 0 and eps = 0: a positive rescale of y changes nothing, the ungated output has
    RMS one, and z = 0 halves it."""
    rng = np.random.default_rng(15)
    y = rng.standard_normal((7, 3, 16))
    w = np.zeros(16)
    big = np.full_like(y, 60.0)
    o1 = gate_out(y, big, w, 0.0)
    np.testing.assert_allclose(np.sqrt((o1 * o1).mean(axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(gate_out(5.5 * y, big, w, 0.0), o1, rtol=1e-13)
    np.testing.assert_allclose(gate_out(y, np.zeros_like(y), w, 0.0), 0.5 * o1, rtol=1e-13)
    w2 = rng.standard_normal(16)
    np.testing.assert_allclose(gate_out(y, big, w2, 0.0), o1 * (1 + w2), rtol=1e-13)


PINS = [pin_conv_fixture, pin_gates_fixture, pin_output_gate_fixture, pin_conv_matches_library,
        pin_conv_state_chains, pin_conv_state_layout, pin_conv_delta_weight_is_identity, pin_l2norm_unit_heads,
        pin_gates_closed_forms, pin_output_gate_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ls.short_conv_silu, ls.gates, ls.output_gate)


# ---- mutants: plausible mistakes, each must fail a pin --------------------------------------

def _conv_flipped(x, w, cu, head_dim=0, state_in=None, eps=ls.EPS):
    return ls.short_conv_silu(x, w[:, ::-1], cu, head_dim, state_in, eps)


def _conv_no_state(x, w, cu, head_dim=0, state_in=None, eps=ls.EPS):
    return ls.short_conv_silu(x, w, cu, head_dim, None, eps)


def _conv_state_newest_first(x, w, cu, head_dim=0, state_in=None, eps=ls.EPS):
    s = None if state_in is None else np.asarray(state_in)[..., ::-1]
    out, st = ls.short_conv_silu(x, w, cu, head_dim, s, eps)
    return out, st[..., ::-1]


def _conv_across_sequences(x, w, cu, head_dim=0, state_in=None, eps=ls.EPS):
    out, st = ls.short_conv_silu(x, w, [0, cu[-1]], head_dim, None if state_in is None else state_in[:1], eps)
    return out, np.repeat(st, len(cu) - 1, axis=0)


def _conv_relu(x, w, cu, head_dim=0, state_in=None, eps=ls.EPS):
    out, st = ls.short_conv_silu(x, w, cu, 0, state_in, eps)
    pre = np.where(out != 0, out, 0.0)
    return np.maximum(pre, 0), st


def _conv_norm_all(x, w, cu, head_dim=0, state_in=None, eps=ls.EPS):
    out, st = ls.short_conv_silu(x, w, cu, x.shape[1] if head_dim else 0, state_in, eps)
    return out, st


def _gates_no_exp_A(a, b, A, ba):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    la = -np.asarray(A, np.float64)[None, :] * ls.softplus(a + np.asarray(ba)[None, :])
    return np.exp(la), ls.sigmoid(b), la


def _gates_relu_softplus(a, b, A, ba):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    la = -np.exp(A)[None, :] * np.maximum(a + np.asarray(ba)[None, :], 0.0)
    return np.exp(la), ls.sigmoid(b), la


def _gates_bias_on_beta(a, b, A, ba):
    return ls.gates(a - np.asarray(ba)[None, :] * 0, np.asarray(b) + np.asarray(ba)[None, :] + 0.1, A, ba)


def _out_no_center(y, z, w, eps=ls.EPS):
    return ls.sigmoid(z) * (y / np.sqrt((np.asarray(y) ** 2).mean(axis=-1, keepdims=True) + eps)) * np.asarray(w)


def _out_silu_gate(y, z, w, eps=ls.EPS):
    return ls.output_gate(y, z, w, eps) / ls.sigmoid(z) * ls.silu(z)


def _out_mean_centered(y, z, w, eps=ls.EPS):
    y = np.asarray(y, np.float64)
    return ls.output_gate(y - y.mean(axis=-1, keepdims=True), z, w, eps)


MUTANTS = {
    "conv_weights_reversed": (_conv_flipped, ls.gates, ls.output_gate),
    "conv_state_ignored": (_conv_no_state, ls.gates, ls.output_gate),
    "conv_state_newest_first": (_conv_state_newest_first, ls.gates, ls.output_gate),
    "conv_runs_across_sequences": (_conv_across_sequences, ls.gates, ls.output_gate),
    "conv_relu_instead_of_silu": (_conv_relu, ls.gates, ls.output_gate),
    "l2norm_over_all_heads": (_conv_norm_all, ls.gates, ls.output_gate),
    "gates_A_without_exp": (ls.short_conv_silu, _gates_no_exp_A, ls.output_gate),
    "gates_relu_for_softplus": (ls.short_conv_silu, _gates_relu_softplus, ls.output_gate),
    "gates_bias_on_beta": (ls.short_conv_silu, _gates_bias_on_beta, ls.output_gate),
    "rmsnorm_scale_not_zero_centred": (ls.short_conv_silu, ls.gates, _out_no_center),
    "output_gate_silu": (ls.short_conv_silu, ls.gates, _out_silu_gate),
    "rmsnorm_subtracts_mean": (ls.short_conv_silu, ls.gates, _out_mean_centered),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_fails_a_pin(name):
    caught = []
    for pin in PINS:
        try:
            pin(*MUTANTS[name])
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passes every pin" % name

"""Pins of the fp64 oracle of the channel-wise gated variants (oracle.channel_prefill,
oracle.channel_chain_numpy).

The reading (per token: decay every key channel by a_t, retrieve with k_t, write the gated
value minus the gated retrieval along k_t, read with q_t) is pinned to things other than
itself:

* uniform gates reduce it to the gated delta rule, whose oracle the forward pins hold;
* with the erase gate at zero it is linear attention with a per-channel decay, a closed sum;
* with one-hot keys every (key channel, value channel) entry is its own scalar recurrence;
* for short chains the state is a product of explicit d_k x d_k transition matrices, one per
  value column;
* with both gates at zero only the per-channel decay remains.

Mutants (plausible mistakes) must each fail at least one pin.
"""
import numpy as np
import pytest

import oracle


def _chain(rng, T, dk, dv, a_lo=0.4):
    q = rng.normal(size=(T, dk))
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.normal(size=(T, dv))
    a = rng.uniform(a_lo, 1.0, size=(T, dk))
    b = rng.uniform(0.0, 1.0, size=(T, dv))
    w = rng.uniform(0.0, 1.0, size=(T, dv))
    s0 = rng.normal(size=(dk, dv))
    return q, k, v, a, b, w, s0


def _close(got, want, tol, what):
    err = np.abs(np.asarray(got) - np.asarray(want)).max() / max(np.abs(want).max(), 1e-300)
    assert err <= tol, "%s: relative error %.3e > %.1e" % (what, err, tol)


def pin_uniform_gates_are_the_rule(run):
    rng = np.random.default_rng(11)
    q, k, v, _, _, _, s0 = _chain(rng, 40, 5, 3)
    alpha = rng.uniform(0.3, 1.0, 40)
    beta = rng.uniform(0.0, 1.0, 40)
    beta[3] = 0.0
    beta[4] = 1.0
    y, S = run(q, k, v, np.repeat(alpha[:, None], 5, 1), np.repeat(beta[:, None], 3, 1),
               np.repeat(beta[:, None], 3, 1), s0)
    ry, rS = oracle.chain_numpy(q, k, v, alpha, beta, s0)
    _close(y, ry, 1e-12, "uniform gates: y")
    _close(S, rS, 1e-12, "uniform gates: state")


def pin_write_only_is_decayed_linear_attention(run):
    # b = 0:  S_t = Diag(prod_{s<=t} a_s) S0 + sum_{i<=t} Diag(prod_{i<s<=t} a_s) k_i (w_i v_i)^T
    rng = np.random.default_rng(12)
    T, dk, dv = 12, 4, 3
    q, k, v, a, _, w, s0 = _chain(rng, T, dk, dv)
    b = np.zeros((T, dv))
    y, S = run(q, k, v, a, b, w, s0)
    for t in range(T):
        St = np.prod(a[:t + 1], axis=0)[:, None] * s0
        for i in range(t + 1):
            St = St + np.prod(a[i + 1:t + 1], axis=0)[:, None] * np.outer(k[i], w[i] * v[i])
        _close(y[t], St.T @ q[t], 1e-12, "write only: y_%d" % t)
    _close(S, St, 1e-12, "write only: state")


def pin_one_hot_keys_are_scalar_recurrences(run):
    # k_t = e_{c_t}: entry (c, j) decays by a_t[c] and, when c = c_t, becomes
    # (1 - b_t[j]) * (decayed entry) + w_t[j] v_t[j]
    rng = np.random.default_rng(13)
    T, dk, dv = 30, 4, 3
    q, _, v, a, b, w, s0 = _chain(rng, T, dk, dv)
    ch = rng.integers(0, dk, size=T)
    k = np.zeros((T, dk))
    k[np.arange(T), ch] = 1.0
    y, S = run(q, k, v, a, b, w, s0)
    ref = s0.copy()
    for t in range(T):
        for c in range(dk):
            for j in range(dv):
                x = a[t, c] * ref[c, j]
                if c == ch[t]:
                    x = (1.0 - b[t, j]) * x + w[t, j] * v[t, j]
                ref[c, j] = x
        _close(y[t], ref.T @ q[t], 1e-12, "one-hot keys: y_%d" % t)
    _close(S, ref, 1e-12, "one-hot keys: state")


def pin_transition_matrices(run):
    # column j of the state: S[:, j] <- (I - b_t[j] k k^T) Diag(a_t) S[:, j] + w_t[j] v_t[j] k
    rng = np.random.default_rng(14)
    T, dk, dv = 6, 4, 4
    q, k, v, a, b, w, s0 = _chain(rng, T, dk, dv)
    y, S = run(q, k, v, a, b, w, s0)
    ref = np.zeros((dk, dv))
    for j in range(dv):
        col = s0[:, j].copy()
        for t in range(T):
            M = (np.eye(dk) - b[t, j] * np.outer(k[t], k[t])) @ np.diag(a[t])
            col = M @ col + w[t, j] * v[t, j] * k[t]
        ref[:, j] = col
    _close(S, ref, 1e-12, "transition matrices")


def pin_decay_only(run):
    rng = np.random.default_rng(15)
    T, dk, dv = 9, 4, 4
    q, k, v, a, _, _, s0 = _chain(rng, T, dk, dv)
    z = np.zeros((T, dv))
    y, S = run(q, k, v, a, z, z, s0)
    _close(S, np.prod(a, axis=0)[:, None] * s0, 1e-13, "decay only")


PINS = [pin_uniform_gates_are_the_rule, pin_write_only_is_decayed_linear_attention,
        pin_one_hot_keys_are_scalar_recurrences, pin_transition_matrices, pin_decay_only]


@pytest.fixture(params=["c", "numpy"])
def run(request, oracle_lib):
    return oracle.channel_chain_c if request.param == "c" else oracle.channel_chain_numpy


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(run, pin):
    pin(run)


def test_packed_heads_and_decode_stack(oracle_lib):
    """Packed sequences and heads equal per-chain runs; a stack of one-token steps (rows
    strided by the batch) equals the packed prefill of the same tokens."""
    rng = np.random.default_rng(16)
    lens = [5, 0, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    R, H, dk, dv = int(cu[-1]), 2, 4, 3
    q = rng.normal(size=(R, H, dk))
    k = rng.normal(size=(R, H, dk)) / 2
    v = rng.normal(size=(R, H, dv))
    a = rng.uniform(0.5, 1, (R, H, dk))
    b = rng.uniform(0, 1, (R, H, dv))
    w = rng.uniform(0, 1, (R, H, dv))
    s0 = rng.normal(size=(3, H, dk, dv))
    y, S = oracle.channel_prefill(q, k, v, a, b, w, cu_seqlens=cu, s0=s0)
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        for h in range(H):
            ry, rS = oracle.channel_chain_numpy(q[s:e, h], k[s:e, h], v[s:e, h], a[s:e, h],
                                                b[s:e, h], w[s:e, h], s0[n, h])
            np.testing.assert_allclose(y[s:e, h], ry, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S[n, h], rS, rtol=1e-12, atol=1e-12)
    # decode stack: B = 2 chains of 6 steps, row = step * B + b
    B, T = 2, 6
    qq = rng.normal(size=(T * B, H, dk))
    kk = rng.normal(size=(T * B, H, dk)) / 2
    vv = rng.normal(size=(T * B, H, dv))
    aa = rng.uniform(0.5, 1, (T * B, H, dk))
    bb = rng.uniform(0, 1, (T * B, H, dv))
    ww = rng.uniform(0, 1, (T * B, H, dv))
    s0 = rng.normal(size=(B, H, dk, dv))
    y1, S1 = oracle.channel_prefill(qq, kk, vv, aa, bb, ww, s0=s0, seq_row0=np.arange(B),
                                    seq_len=np.full(B, T), row_step=B)
    for bi in range(B):
        idx = np.arange(T) * B + bi
        y2, S2 = oracle.channel_prefill(qq[idx], kk[idx], vv[idx], aa[idx], bb[idx], ww[idx],
                                        s0=s0[bi:bi + 1])
        np.testing.assert_allclose(y1[idx], y2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S1[bi], S2[0], rtol=1e-12, atol=1e-12)


# ---- mutants ----------------------------------------------------------------------------

def _mutant(mut):
    def run(q, k, v, a, b, w, s0=None):
        T, dk = k.shape
        dv = v.shape[1]
        S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
        y = np.zeros((T, dv))
        for t in range(T):
            if mut == "decay_on_value_axis":
                St = S * a[t][None, :dv] if dv <= dk else S
            elif mut == "decay_after_write":
                St = S
            else:
                St = a[t][:, None] * S
            base = S if mut == "erase_against_undecayed" else St
            wt, bt = (b[t], w[t]) if mut == "gates_swapped" else (w[t], b[t])
            if mut == "write_gate_ignored":
                wt = np.ones_like(wt)
            e = wt * v[t] - bt * (base.T @ k[t])
            Sn = St + np.outer(k[t], e)
            if mut == "decay_after_write":
                Sn = a[t][:, None] * Sn
            y[t] = (St if mut == "read_before_write" else Sn).T @ q[t]
            S = Sn
        return y, S
    return run


MUTANTS = ["decay_on_value_axis", "decay_after_write", "erase_against_undecayed",
           "gates_swapped", "write_gate_ignored", "read_before_write"]


def test_unmutated_copy_passes_every_pin(oracle_lib):
    for pin in PINS:
        pin(_mutant(None))


@pytest.mark.parametrize("name", MUTANTS)
def test_every_channel_mutant_fails_a_pin(oracle_lib, name):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant(name))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passes every pin" % name

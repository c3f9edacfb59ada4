"""Pins of the fp64 oracle of the sparse-attention indexer (oracle/qsa.py).

Each step is checked against a property or a hand-worked value rather than against itself:
RoPE by its defining relative-position property, norm preservation and untouched dimensions;
RMSNorm by its unit mean square; pooling by constant blocks; the scores by a brute-force loop
on a tiny case and the abstention of negative heads; the selection by a hand-worked example
(ties, causality, the tail and the padding).  Planted mistakes must each fail a pin.
"""
import numpy as np
import pytest

from oracle import qsa


def _rand(rng, n, H=4, D=128):
    return rng.normal(size=(n, H, D)), rng.normal(size=(n, D))


# ---- pins: each takes a module-like namespace of the oracle's functions --------------------

def pin_rope_relative_position(m):
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=128), rng.normal(size=128)
    # rotated dims: <R_i q, R_j k> depends on i - j only; the others are untouched
    a = np.dot(m.rope(q, 7.0)[:64], m.rope(k, 3.0)[:64])
    b = np.dot(m.rope(q, 104.0)[:64], m.rope(k, 100.0)[:64])
    assert abs(a - b) < 1e-9 * (1 + abs(a)), (a, b)
    x = m.rope(q, 12345.0)
    np.testing.assert_allclose(x[64:], q[64:], rtol=0, atol=0)
    assert abs(np.linalg.norm(x) - np.linalg.norm(q)) < 1e-9
    np.testing.assert_allclose(m.rope(q, 0.0), q, rtol=0, atol=1e-15)
    # the first pair turns by pos radians (base^0 = 1), pairing dims 0 and 32
    e = np.zeros(128)
    e[0] = 1.0
    y = m.rope(e, 0.5)
    assert abs(y[0] - np.cos(0.5)) < 1e-12 and abs(y[32] - np.sin(0.5)) < 1e-12


def pin_rmsnorm_unit_mean_square(m):
    rng = np.random.default_rng(2)
    x = rng.normal(size=(5, 128)) * 3.0
    y = m.rmsnorm(x)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-6)


def pin_pooling_of_constant_blocks(m):
    rng = np.random.default_rng(3)
    base = rng.normal(size=(3, 128))
    k = np.repeat(base, 4, axis=0)                      # every block holds one key 4 times
    q = rng.normal(size=(12, 4, 128))
    _, kb = m.prepare(q, k)
    for b in range(3):
        np.testing.assert_allclose(kb[b], m.rope(m.rmsnorm(base[b]), 4.0 * b), atol=1e-12)


def pin_scores_brute_force(m):
    rng = np.random.default_rng(4)
    n, H, D = 10, 4, 128
    q, k = _rand(rng, n, H, D)
    qr, kb = m.prepare(q, k)
    I = m.scores(qr, kb)
    for i in range(n):
        for b in range(n // 4):
            if 4 * b + 3 <= i:
                want = 0.0
                for h in range(H):
                    d = sum(qr[i, h, x] * kb[b, x] for x in range(D))
                    want += d if d > 0 else 0.0
                assert abs(I[i, b] - want) < 1e-9 * (1 + abs(want))
            else:
                assert I[i, b] == -np.inf


def pin_negative_heads_abstain(m):
    # one head aligned with the block key, the others anti-aligned: only the first counts
    kb = np.zeros((1, 128))
    kb[0, 100] = 1.0
    qr = np.zeros((4, 4, 128))
    qr[3, 0, 100] = 2.0
    qr[3, 1:, 100] = -5.0
    I = m.scores(qr, kb)
    assert I[3, 0] == 2.0


def pin_selection_hand_worked(m):
    # n = 14 queries, 3 complete blocks at the end; budget 2 blocks
    I = np.full((14, 3), -np.inf)
    I[13] = [5.0, 1.0, 5.0]          # tie between blocks 0 and 2 at the top: both taken
    I[12] = [0.0, 0.0, 0.0]          # three-way tie at zero: blocks 0 and 1
    I[7] = [3.0, 4.0, -np.inf]       # only two complete blocks (0, 1): both
    I[5] = [7.0, -np.inf, -np.inf]   # one complete block
    blocks, tokens = m.select(I, kb_budget=2)
    assert list(blocks[13]) == [0, 2]
    # query 13: blocks 0, 2 -> tokens 0..3, 8..11; tail = {12, 13}
    assert list(tokens[13]) == [0, 1, 2, 3, 8, 9, 10, 11, 12, 13, -1]
    assert list(blocks[12]) == [0, 1]
    assert list(tokens[12]) == [0, 1, 2, 3, 4, 5, 6, 7, 12, -1, -1]
    assert list(blocks[7]) == [0, 1]
    assert list(tokens[7]) == [0, 1, 2, 3, 4, 5, 6, 7, -1, -1, -1]       # i = 7: no tail
    assert list(blocks[5]) == [0, -1]
    assert list(tokens[5]) == [0, 1, 2, 3, 4, 5, -1, -1, -1, -1, -1]
    assert list(blocks[2]) == [-1, -1]
    assert list(tokens[2]) == [0, 1, 2, -1, -1, -1, -1, -1, -1, -1, -1]


PINS = [pin_rope_relative_position, pin_rmsnorm_unit_mean_square,
        pin_pooling_of_constant_blocks, pin_scores_brute_force, pin_negative_heads_abstain,
        pin_selection_hand_worked]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(qsa)


def test_indexer_end_to_end_small():
    rng = np.random.default_rng(5)
    q, k = _rand(rng, 64)
    I, blocks, tokens = qsa.indexer(q, k, kb_budget=4)
    for i in range(64):
        nvalid = (i + 1) // 4
        sel = blocks[i][blocks[i] >= 0]
        assert len(sel) == min(4, nvalid)
        if nvalid > len(sel):
            rest = np.setdiff1d(np.arange(nvalid), sel)
            assert I[i, sel].min() >= I[i, rest].max()
        assert tokens[i][tokens[i] >= 0][-1] == i or nvalid == 0 or (i + 1) % 4 == 0


def test_prepare_rows_matches_prepare():
    """The row-subset preparation gives prepare()'s values at those rows (positions taken from
    the row indices, block keys over the whole sequence)."""
    rng = np.random.default_rng(6)
    q, k = _rand(rng, 203)
    qr, kb = qsa.prepare(q, k)
    rows = np.array([0, 3, 4, 77, 202])
    qr_s, kb_s = qsa.prepare_rows(q[rows], rows, k)
    assert np.array_equal(qr_s, qr[rows])
    assert np.array_equal(kb_s, kb)


# ---- mutants ------------------------------------------------------------------------------

class _Mut:
    def __init__(self, name):
        self.name = name
        self.rmsnorm = qsa.rmsnorm

    def rope(self, x, pos, dims=qsa.ROPE_DIMS, base=qsa.ROPE_BASE):
        if self.name == "rope_adjacent_pairs":
            x = np.array(x, dtype=np.float64)
            half = dims // 2
            ang = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * np.arange(half) / dims)
            a, b = x[..., 0:dims:2].copy(), x[..., 1:dims:2].copy()
            x[..., 0:dims:2] = a * np.cos(ang) - b * np.sin(ang)
            x[..., 1:dims:2] = a * np.sin(ang) + b * np.cos(ang)
            return x
        if self.name == "rope_last_dims":
            x = np.array(x, dtype=np.float64)
            y = qsa.rope(x[..., ::-1], pos, dims, base)
            return y[..., ::-1].copy()
        return qsa.rope(x, pos, dims, base)

    def prepare(self, q, k, r=qsa.R):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        n = q.shape[0]
        nb = n // r
        qr = self.rope(self.rmsnorm(q), np.arange(n)[:, None] * np.ones(q.shape[1]))
        if self.name == "rope_before_pooling":
            kr = self.rope(k, np.arange(n))
            kb = self.rmsnorm(kr[:nb * r].reshape(nb, r, -1).mean(axis=1))
            return qr, kb
        pooled = k[:nb * r].reshape(nb, r, -1).mean(axis=1)
        pos = np.arange(nb) * r + (r - 1 if self.name == "block_position_last_token" else 0)
        return qr, self.rope(self.rmsnorm(pooled), pos)

    def scores(self, qr, kb, r=qsa.R):
        n, nb = qr.shape[0], kb.shape[0]
        dots = np.einsum("nhd,bd->nhb", qr, kb)
        I = dots.sum(axis=1) if self.name == "relu_after_head_sum" else np.maximum(dots, 0).sum(axis=1)
        if self.name == "relu_after_head_sum":
            I = np.maximum(I, 0)
        i = np.arange(n)[:, None]
        b = np.arange(nb)[None, :]
        lim = b * r if self.name == "causal_on_block_start" else b * r + r - 1
        return np.where(lim <= i, I, -np.inf)

    def select(self, I, kb_budget=qsa.KB, r=qsa.R):
        if self.name == "ties_to_higher_index":
            n, nb = I.shape
            blocks = np.full((n, kb_budget), -1, dtype=np.int64)
            for i in range(n):
                nvalid = min((i + 1) // r, nb)
                row = I[i, :nvalid]
                order = np.lexsort((-np.arange(nvalid), -row))
                ch = np.sort(order[:kb_budget])
                blocks[i, :len(ch)] = ch
            return blocks, self._tokens(blocks, n, kb_budget, r)
        blocks, tokens = qsa.select(I, kb_budget, r)
        if self.name == "tail_dropped":
            tokens = self._tokens(blocks, I.shape[0], kb_budget, r, tail=False)
        return blocks, tokens

    def _tokens(self, blocks, n, kb_budget, r, tail=True):
        width = kb_budget * r + r - 1
        tokens = np.full((n, width), -1, dtype=np.int64)
        for i in range(n):
            ch = blocks[i][blocks[i] >= 0]
            t = (ch[:, None] * r + np.arange(r)[None, :]).reshape(-1)
            if tail:
                t = np.concatenate([t, np.arange(((i + 1) // r) * r, i + 1)])
            tokens[i, :len(t)] = t
        return tokens


MUTANTS = ["rope_adjacent_pairs", "rope_last_dims", "rope_before_pooling",
           "block_position_last_token", "relu_after_head_sum", "causal_on_block_start",
           "ties_to_higher_index", "tail_dropped"]


def test_unmutated_copy_passes_every_pin():
    for pin in PINS:
        pin(_Mut(None))


@pytest.mark.parametrize("name", MUTANTS)
def test_every_qsa_mutant_fails_a_pin(name):
    caught = []
    for pin in PINS:
        try:
            pin(_Mut(name))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passes every pin" % name

"""fp64 CPU oracle of the sparse-attention indexer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module; the product path never imports, links or calls it and shares no code
with it.

What the pages define (jianyuh.github.io reading notes "Qwen3.8-Next: GDN, QSA, Gated
Residual", section "The compressed lightweight indexer"; ta-paperlens "Designing Qwen3.8-Next",
"Component 2: QSA"): an MQA indexer with H = 4 query heads and one shared key head of 128
dimensions;

1. q^h_i = RMSNorm(projected query), k_i = projected key (the projections are inputs here);
2. keys pooled in non-overlapping blocks of r = 4 tokens, then RMSNorm:
   kb_b = RMSNorm(mean(k_{4b} .. k_{4b+3}));
3. partial RoPE on 64 of the 128 dimensions, after pooling: queries at their own position i,
   block keys at the position of their first token p_b = 4b;
4. block-causal scores I_ib = sum_h ReLU(<q^h_i, kb_b>) for p_b + r - 1 <= i, else excluded;
5. the top K_B = ceil(K / r) = 512 blocks (token budget K = 2048) per query, expanded to their
   tokens and joined with the tail of the current incomplete block, {floor((i+1)/r) r .. i}.

Readings where the pages are silent:

* RMSNorm(x) = x / sqrt(mean(x^2) + 1e-6), no learnable scale;
* the rotated dimensions are the first 64; they are rotated in pairs (m, m + 32),
  m = 0..31, by angle pos * base^(-2m/64) with base 10000; dimensions 64..127 are left alone;
* ties in the top-K go to the lower block index; a query with fewer complete blocks than
  K_B selects all of them;
* output: per query the selected token indices in ascending order (the blocks' tokens, then
  the tail), padded with -1 to K_B r + r - 1 entries.

Plain numpy in float64; the top-K is a stable sort on (-score, block index).
"""
from __future__ import annotations

import numpy as np

R = 4               # tokens per key block
K_TOKENS = 2048     # token budget
KB = -(-K_TOKENS // R)   # block budget, 512
ROPE_DIMS = 64
ROPE_BASE = 10000.0
EPS = 1e-6


def rmsnorm(x, eps=EPS):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, pos, dims=ROPE_DIMS, base=ROPE_BASE):
    """Rotate dims (m, m + dims/2), m < dims/2, of x[..., D] by pos * base^(-2m/dims).
    pos broadcasts against x[..., 0]."""
    x = np.array(x, dtype=np.float64)
    half = dims // 2
    m = np.arange(half)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * m / dims)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half].copy(), x[..., half:dims].copy()
    x[..., :half] = a * c - b * s
    x[..., half:dims] = a * s + b * c
    return x


def prepare(q, k, r=R):
    """q: [n, H, D] projected queries; k: [n, D] projected keys.  Returns (qr [n, H, D],
    kb [n // r, D]): normalised and rotated queries, pooled, normalised, rotated block keys."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    nb = n // r
    qr = rope(rmsnorm(q), np.arange(n)[:, None] * np.ones(q.shape[1]))
    if nb == 0:                      # no complete block: nothing to pool
        return qr, np.zeros((0, k.shape[1]))
    pooled = k[:nb * r].reshape(nb, r, -1).mean(axis=1)
    kb = rope(rmsnorm(pooled), np.arange(nb) * r)
    return qr, kb


def prepare_rows(q_rows, rows, k, r=R):
    """prepare() for a subset of the queries: q_rows [m, H, D] are the projected queries at
    token positions rows [m]; returns (qr [m, H, D], kb [n // r, D]), the same values that
    prepare(q, k) gives at those rows (used where the whole query tensor is too large to
    normalise in fp64)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    qr = rope(rmsnorm(q_rows), rows[:, None] * np.ones(q_rows.shape[1]))
    nb = k.shape[0] // r
    if nb == 0:
        return qr, np.zeros((0, k.shape[1]))
    pooled = k[:nb * r].reshape(nb, r, -1).mean(axis=1)
    return qr, rope(rmsnorm(pooled), np.arange(nb) * r)


def scores(qr, kb, r=R):
    """I [n, nb]: sum over heads of ReLU(<q^h_i, kb_b>); -inf where block b is not complete
    before query i (p_b + r - 1 > i)."""
    n = qr.shape[0]
    nb = kb.shape[0]
    dots = np.einsum("nhd,bd->nhb", qr, kb)
    I = np.maximum(dots, 0.0).sum(axis=1)
    i = np.arange(n)[:, None]
    b = np.arange(nb)[None, :]
    return np.where(b * r + r - 1 <= i, I, -np.inf)


def select(I, kb_budget=KB, r=R):
    """Per query: the selected blocks (ascending) and the token list (ascending, -1 padded
    to kb_budget * r + r - 1)."""
    n, nb = I.shape
    width = kb_budget * r + r - 1
    blocks = np.full((n, kb_budget), -1, dtype=np.int64)
    tokens = np.full((n, width), -1, dtype=np.int64)
    for i in range(n):
        nvalid = min((i + 1) // r, nb)
        if nvalid > 0:
            row = I[i, :nvalid]
            order = np.lexsort((np.arange(nvalid), -row))   # score descending, index ascending
            chosen = np.sort(order[:kb_budget])
            blocks[i, :len(chosen)] = chosen
        else:
            chosen = np.zeros(0, dtype=np.int64)
        toks = (chosen[:, None] * r + np.arange(r)[None, :]).reshape(-1)
        tail = np.arange(((i + 1) // r) * r, i + 1)
        allt = np.concatenate([toks, tail])
        tokens[i, :len(allt)] = allt
    return blocks, tokens


def indexer(q, k, r=R, kb_budget=KB):
    """The whole indexer: returns (I, blocks, tokens)."""
    qr, kb = prepare(q, k, r)
    I = scores(qr, kb, r)
    blocks, tokens = select(I, kb_budget, r)
    return I, blocks, tokens

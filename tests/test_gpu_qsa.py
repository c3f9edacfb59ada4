"""GPU parity of gdn_qsa_index (the sparse-attention block indexer) against the fp64 oracle.

The selection is integer output decided by floating-point scores.  The kernel scores with
bf16 products of the normalised, rotated vectors, the oracle in fp64, so near the selection
threshold the two may order blocks differently.  The checks: everything that is unique is
exact (the count, order, range and padding of the blocks, their expansion to tokens and the
tail); the selection is a valid top-K under the oracle's scores within the kernel's rounding
bound E_ib = 2^-8 sum_h |q_i^h| . |kb_b| (both operands rounded to bf16, each by at most
2^-9 relative); and where all scores are exactly equal (zero keys) the tie-break is exact.
"""
import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def run(inp, dev, kb, rows=None):
    """The indexer on the GPU; returns the blocks and tokens of the given rows (all rows by
    default), selected on the device so that only they are copied back."""
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    q = wl.to_torch(inp["q"], dev, inp["dtype"])
    k = wl.to_torch(inp["k"], dev, inp["dtype"])
    b, t = gdn.gdn_qsa_index(q, k, block_budget=kb)
    torch.cuda.synchronize()
    if rows is not None:
        idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=dev)
        b, t = b[idx], t[idx]
    return b.cpu().numpy().astype(np.int64), t.cpu().numpy().astype(np.int64)


def check_rows(inp, blocks, tokens, kb, rows, label):
    """blocks[j], tokens[j] are the outputs of row rows[j]."""
    from oracle import qsa
    from linear_attention_recurrence_chunked_amd import workloads as wl
    n = inp["n"]
    rows = np.asarray(list(rows), dtype=np.int64)
    q = wl.as_f64(inp["q"][rows], inp["dtype"])
    k = wl.as_f64(inp["k"], inp["dtype"])
    qr, kbk = qsa.prepare_rows(q, rows, k)
    nb = n // 4
    W = 4 * kb + 3
    exact = 0
    worst_margin = np.inf
    for j, i in enumerate(rows):
        i = int(i)
        nvalid = min((i + 1) // 4, nb)
        sel = blocks[j][blocks[j] >= 0]
        nsel = min(kb, nvalid)
        assert len(sel) == nsel, (label, i, len(sel), nsel)
        assert np.all(blocks[j][nsel:] == -1)
        assert np.all(np.diff(sel) > 0) and (nsel == 0 or sel[-1] < nvalid)
        toks = (sel[:, None] * 4 + np.arange(4)[None, :]).reshape(-1)
        want = np.concatenate([toks, np.arange(((i + 1) // 4) * 4, i + 1)])
        assert np.array_equal(tokens[j][:len(want)], want), (label, i)
        assert np.all(tokens[j][len(want):W] == -1)
        if nvalid > kb:
            d = np.einsum("hd,bd->hb", qr[j], kbk[:nvalid])
            I = np.maximum(d, 0).sum(axis=0)
            E = 2.0 ** -8 * np.einsum("hd,bd->b", np.abs(qr[j]), np.abs(kbk[:nvalid]))
            rest = np.setdiff1d(np.arange(nvalid), sel)
            margin = (I[sel] + E[sel]).min() - (I[rest] - E[rest]).max()
            worst_margin = min(worst_margin, margin)
            assert margin >= 0, (label, i, margin)
            order = np.lexsort((np.arange(nvalid), -I))
            exact += np.array_equal(np.sort(order[:kb]), sel)
        else:
            exact += 1
    say("    %s: %d rows, %d equal to the oracle's selection, worst margin %.3g" % (
        label, len(rows), exact, worst_margin))


@pytest.mark.parametrize("n,kb,dtype", [(1000, 16, "bf16"), (1027, 64, "f32"), (3, 4, "bf16"),
                                        (258, 1000, "bf16"), (513, 1, "bf16")])
def test_qsa_against_oracle(dev, n, kb, dtype):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.qsa_inputs(n, dtype, seed=n)
    say("[gpu] qsa n=%d budget=%d %s" % (n, kb, dtype))
    blocks, tokens = run(inp, dev, kb)
    check_rows(inp, blocks, tokens, kb, range(n), "n=%d" % n)


def test_qsa_zero_keys_take_the_lowest_blocks(dev):
    """Zero keys make every score exactly 0 on both sides: the budget goes to blocks 0..
    (rows of up to 500 blocks: one crowded threshold bin of equal scores)."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.qsa_inputs(2000, "bf16", seed=7)
    inp["k"][:] = 0
    blocks, tokens = run(inp, dev, 8)
    for i in range(2000):
        nvalid = (i + 1) // 4
        want = np.arange(min(8, nvalid))
        assert np.array_equal(blocks[i][:len(want)], want), i


def test_qsa_tie_classes_break_ties_by_index(dev):
    """Keys zero in the rotated half and equal to one of three vectors within each block give
    identical block keys, so each query sees three exactly tied score levels (two of them
    closer than the bf16 rounding bound, so their order may differ from the oracle's).  Every
    row must be a valid top-K, and within each class of identical keys the selected blocks
    must be the class's lowest indices (ties to the lower index), through both the small
    and the crowded threshold-bin paths."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    n = 3000
    inp = wl.qsa_inputs(n, "bf16", seed=9)
    rng = np.random.default_rng(9)
    cls = rng.integers(0, 3, n // 4 + 1)
    vecs = wl.qsa_inputs(3, "bf16", seed=10)["k"]          # three bf16 rows
    k = np.zeros_like(inp["k"])
    for t in range(n):
        k[t, 64:] = vecs[cls[t // 4], 64:]
    inp["k"] = k
    say("[gpu] qsa tie classes n=%d budget=64" % n)
    blocks, tokens = run(inp, dev, 64)
    check_rows(inp, blocks, tokens, 64, range(n), "tie classes")
    for i in range(n):
        nvalid = min((i + 1) // 4, n // 4)
        sel = set(blocks[i][blocks[i] >= 0].tolist())
        for c in range(3):
            members = [b for b in range(nvalid) if cls[b] == c]
            m = sum(b in sel for b in members)
            assert all(b in sel for b in members[:m]), (i, c)


def test_qsa_budget_65536_tokens(dev):
    """n = 65,536 tokens (16,384 blocks), the notes' budget of 512 blocks: sampled rows."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    n = 65536
    inp = wl.qsa_inputs(n, "bf16", seed=11)
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 3, 2047, 2048, 2051, n - 1] + list(rng.integers(0, n, 60))))
    say("[gpu] qsa n=%d budget=512" % n)
    blocks, tokens = run(inp, dev, 512, rows)
    check_rows(inp, blocks, tokens, 512, rows, "n=65536 sampled")


@pytest.mark.parametrize("kb", [1000, 2048])
def test_qsa_large_budgets(dev, kb):
    """Budgets of 1,000 and 2,048 blocks (workgroups of 8 and 4 queries, lists of 2,048 and
    4,096 entries) over 2,250 blocks: every row."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    n = 9000
    inp = wl.qsa_inputs(n, "bf16", seed=kb)
    say("[gpu] qsa n=%d budget=%d" % (n, kb))
    blocks, tokens = run(inp, dev, kb)
    check_rows(inp, blocks, tokens, kb, range(n), "budget %d" % kb)


@pytest.mark.parametrize("kb,n", [(512, 2200), (1000, 4200), (2048, 8400)])
def test_qsa_budget_just_below_the_visible_blocks(dev, kb, n):
    """Rows with a few more visible blocks than the budget: about one block in 16 scores
    exactly 0 (all four heads negative), so the budget's last place falls among many exactly
    tied zeros and is decided by block index (each workgroup size: 16, 8 and 4 queries).
    Every row."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.qsa_inputs(n, "bf16", seed=kb + 5)
    say("[gpu] qsa n=%d budget=%d (ties at zero)" % (n, kb))
    blocks, tokens = run(inp, dev, kb)
    check_rows(inp, blocks, tokens, kb, range(n), "budget %d, n %d" % (kb, n))
    # the zero-score ties are taken lowest block first: blocks whose four head products are
    # all below minus their rounding bound score exactly 0 on both sides, and the taken ones
    # among them must be the lowest (a block the kernel rounds to 0 may join its zeros, but
    # never ahead of a lower zero)
    from oracle import qsa
    q = wl.as_f64(inp["q"], "bf16")
    k = wl.as_f64(inp["k"], "bf16")
    qr, kbk = qsa.prepare(q, k)
    for i in range(n - 40, n):
        nvalid = min((i + 1) // 4, n // 4)
        if nvalid <= kb:
            continue
        sel = blocks[i][blocks[i] >= 0]
        d = np.einsum("hd,bd->hb", qr[i], kbk[:nvalid])
        E = 2.0 ** -8 * np.einsum("hd,bd->hb", np.abs(qr[i]), np.abs(kbk[:nvalid]))
        zeros = np.flatnonzero(np.all(d + E < 0, axis=0))
        taken = np.isin(zeros, sel)
        assert np.all(taken[:taken.sum()]), i


def test_qsa_rising_scores_trim_every_step(dev):
    """Keys zero in the rotated half, pointing ever closer to the queries' shared direction
    as the block index grows: each block scores above the ones before it, so every visible
    block passes the running threshold and the lists are trimmed every few steps."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    n = 24000
    nb = n // 4
    inp = wl.qsa_inputs(n, "f32", seed=21)
    rng = np.random.default_rng(21)
    u = np.zeros(128)
    u[64:] = rng.standard_normal(64)
    u /= np.linalg.norm(u)
    w = np.zeros(128)
    w[64:] = rng.standard_normal(64)
    w -= (w @ u) * u
    w /= np.linalg.norm(w)
    theta = np.linspace(1.4, 0.05, nb)                   # falling angle to u
    kb_dir = np.cos(theta)[:, None] * u + np.sin(theta)[:, None] * w
    inp["k"] = np.repeat(kb_dir, 4, axis=0).astype(np.float32)
    q = np.repeat(u[None, None, :], n, axis=0).repeat(4, axis=1)
    inp["q"] = (q + 0.01 * rng.standard_normal(q.shape)).astype(np.float32)
    say("[gpu] qsa rising scores n=%d budget=64" % n)
    rows = sorted(set([300, 1023, 5000, 12000, n - 1] + list(rng.integers(0, n, 20))))
    blocks, tokens = run(inp, dev, 64, rows)
    check_rows(inp, blocks, tokens, 64, rows, "rising scores")


def test_qsa_longest_sequence(dev):
    """n = 2^20 tokens (262,144 blocks, the largest supported; the notes time the indexer at
    this length), budget 512: sampled rows, the last one included."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    n = 1 << 20
    inp = wl.qsa_inputs(n, "bf16", seed=13)
    rng = np.random.default_rng(1)
    rows = sorted(set([2047, 2048, 65535, 65536, 524291, n - 2, n - 1] +
                      list(rng.integers(0, n, 16))))
    say("[gpu] qsa n=%d budget=512" % n)
    blocks, tokens = run(inp, dev, 512, rows)
    check_rows(inp, blocks, tokens, 512, rows, "n=2^20 sampled")

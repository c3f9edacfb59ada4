"""GPU parity of gdn_channel_gated (channel-wise decay, erase and write gates) against the
fp64 oracle of the variants: per-(sequence, head) max relative error of y and the final
state, 1e-4 for fp32 inputs and 2e-2 for bf16."""
import numpy as np
import pytest

from gpu_util import TOL, cu_of, say, slice_rel_err, state_rel_err, torch_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _inp(lengths, H=2, d=(128, 128), dtype="bf16", s0=0.02, seed=0, varlen=True):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    return wl.make_inputs(lengths, H, d[0], d[1], dtype, s0_sd=s0, seed=seed, varlen=varlen)


def run_gpu(inp, gates, dev, want_state=True, state_in_place=False):
    from linear_attention_recurrence_chunked_amd import gdn
    t = torch_inputs(inp, dev)
    g = {n: torch.from_numpy(gates[n]).to(dev) for n in ("decay", "erase", "write")}
    fs = t["s0"] if state_in_place else None
    y, sf = gdn.gdn_channel_gated(t["q"], t["k"], t["v"], g["decay"], g["erase"], g["write"],
                                  initial_state=t["s0"], cu_seqlens=t["cu"],
                                  num_seqs=inp["num_seqs"], final_state=fs,
                                  want_final_state=want_state)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), None if sf is None else sf.cpu().numpy()


def check(inp, gates, dev, oracle, label, heads=None):
    say("[gpu] channel %s lengths=%s H=%d dk=%d dv=%d %s" % (
        label, list(inp["lengths"][:8]), inp["H"], inp["dk"], inp["dv"], inp["dtype"]))
    gy, gs = run_gpu(inp, gates, dev)
    ry, rs = oracle.channel_prefill(inp["q"], inp["k"], inp["v"], gates["decay"],
                                    gates["erase"], gates["write"], cu_seqlens=cu_of(inp),
                                    s0=inp["s0"], heads=heads, threads=16)
    h0, h1 = (0, inp["H"]) if heads is None else heads
    ey = slice_rel_err(gy[:, h0:h1], ry, cu_of(inp))
    es = state_rel_err(gs[:, h0:h1], rs)
    say("    err y %.3e  state %.3e" % (ey, es))
    tol = TOL[inp["dtype"]]
    assert np.all(np.isfinite(gy)) and np.all(np.isfinite(gs))
    assert ey <= tol and es <= tol, (ey, es)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_channel_ragged(dev, oracle_lib, dtype, d):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([1, 63, 0, 130, 7], H=3, d=d, dtype=dtype, seed=31)
    check(inp, wl.channel_gates(inp, seed=31), dev, oracle_lib, "ragged")


def test_channel_strong_decay_and_gate_edges(dev, oracle_lib):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([300, 41], H=2, seed=32)
    g = wl.channel_gates(inp, a=(1.0, 2.0), b=(0.0, 2.0), seed=32)
    g["decay"][::3] = 1.0
    g["erase"][::5] = 0.0
    g["write"][1::7] = 1.0
    g["erase"][2::7] = 1.0
    check(inp, g, dev, oracle_lib, "strong-decay-edges")


def test_channel_without_states(dev, oracle_lib):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([96] * 3, H=2, s0=None, seed=33, varlen=False)
    check(inp, wl.channel_gates(inp, seed=33), dev, oracle_lib, "no-state")


def test_uniform_gates_match_the_chunked_rule(dev):
    """a = alpha, b = w = beta reproduce gdn_prefill (chunked, bf16 MFMA) within its bound."""
    from linear_attention_recurrence_chunked_amd import gdn
    inp = _inp([200, 64, 333], H=2, seed=34)
    H, dk, dv = inp["H"], inp["dk"], inp["dv"]
    gates = dict(decay=np.repeat(inp["alpha"][:, :, None], dk, 2),
                 erase=np.repeat(inp["beta"][:, :, None], dv, 2),
                 write=np.repeat(inp["beta"][:, :, None], dv, 2))
    gy, gs = run_gpu(inp, gates, dev)
    t = torch_inputs(inp, dev)
    y, sf = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                            initial_state=t["s0"], cu_seqlens=t["cu"])
    ey = slice_rel_err(gy, y.float().cpu().numpy().astype(np.float64), cu_of(inp))
    es = state_rel_err(gs, sf.cpu().numpy())
    say("    channel vs chunked rule: y %.3e state %.3e" % (ey, es))
    assert ey <= 2e-2 and es <= 2e-2


def test_decode_steps_in_place(dev, oracle_lib):
    """T one-token calls (the decode kernel) carrying the state in place agree with one call
    over the T tokens and with the oracle."""
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    for dtype, d in (("bf16", (128, 128)), ("f32", (64, 128)), ("bf16", (128, 64))):
        B, T, H = 3, 9, 2
        inp = _inp([T] * B, H=H, d=d, dtype=dtype, seed=35, varlen=False)
        g = wl.channel_gates(inp, seed=35)
        gy, gs = run_gpu(inp, g, dev)
        t = torch_inputs(inp, dev)
        gt = {n: torch.from_numpy(g[n]).to(dev) for n in ("decay", "erase", "write")}
        state = t["s0"].clone()
        ys = torch.empty_like(t["v"])
        for s in range(T):
            idx = torch.arange(B, device=dev) * T + s
            y, _ = gdn.gdn_channel_gated(t["q"][idx].contiguous(), t["k"][idx].contiguous(),
                                         t["v"][idx].contiguous(), gt["decay"][idx].contiguous(),
                                         gt["erase"][idx].contiguous(),
                                         gt["write"][idx].contiguous(), initial_state=state,
                                         num_seqs=B, final_state=state)
            ys[idx] = y
        torch.cuda.synchronize()
        dy = ys.float().cpu().numpy()
        ds = state.cpu().numpy()
        tol = 1e-5 if dtype == "f32" else 2e-2
        assert slice_rel_err(dy, gy, cu_of(inp)) <= tol
        assert state_rel_err(ds, gs) <= 1e-5
        ry, rs = oracle_lib.channel_prefill(inp["q"], inp["k"], inp["v"], g["decay"],
                                            g["erase"], g["write"], cu_seqlens=cu_of(inp),
                                            s0=inp["s0"])
        ey, es = slice_rel_err(dy, ry, cu_of(inp)), state_rel_err(ds, rs)
        say("    decode %s d=%s: err y %.3e state %.3e" % (dtype, d, ey, es))
        assert ey <= TOL[dtype] and es <= TOL[dtype]


def test_channel_full_prefill_shape(dev, oracle_lib):
    """4 x 4096 tokens, 16 heads of 128, bf16: every head against the oracle."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.workload_inputs(wl.PREFILL)
    g = wl.channel_gates(inp, seed=36)
    check(inp, g, dev, oracle_lib, "full-size, all heads")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_channel_short_sequences(dev, oracle_lib, dtype):
    """Sequences of a few tokens (the one-token-ahead kernel) against the oracle."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([1, 3, 7, 2, 0, 5, 1, 1], H=2, dtype=dtype, seed=37)
    check(inp, wl.channel_gates(inp, seed=37), dev, oracle_lib, "short")


def test_staged_and_step_kernels_agree(dev):
    """The same four 40-token sequences through the staged kernel and, padded with empty
    sequences so that the average length falls below one block, through the step kernel."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([40] * 4, H=2, d=(128, 64), dtype="f32", seed=38)
    g = wl.channel_gates(inp, seed=38)
    ya, sa = run_gpu(inp, g, dev)
    pad = dict(inp)
    pad["lengths"] = np.array([40] * 4 + [0] * 12)
    pad["num_seqs"] = 16
    pad["cu_seqlens"] = np.concatenate([[0], np.cumsum(pad["lengths"])]).astype(np.int32)
    pad["s0"] = np.concatenate([inp["s0"], np.zeros((12,) + inp["s0"].shape[1:], np.float32)])
    yb, sb = run_gpu(pad, g, dev)
    np.testing.assert_allclose(ya, yb, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(sa, sb[:4], rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(sb[4:], 0.0)

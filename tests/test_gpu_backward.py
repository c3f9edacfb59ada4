"""GPU parity of gdn_prefill_backward against the fp64 backward oracle.

Every gradient (dq, dk, dv, dalpha, dbeta, dS0) is compared element by element; the error is
the per-(sequence, head) max relative error, bound 2e-2 for bf16 activations (the forward's
bound).  The full-size prefill workload is checked on every head against the oracle and
through the adjoint identity <dq, q> = <dy, y>.
"""
import numpy as np
import pytest

from gpu_util import say, slice_rel_err, state_rel_err, torch_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 2e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _inp(lengths, H=2, d=(128, 128), s0=0.02, seed=0, alpha=(3.0, 1.0), beta=(0.0, 1.0),
         varlen=True):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    return wl.make_inputs(lengths, H, d[0], d[1], "bf16", alpha=alpha, beta=beta, s0_sd=s0,
                          seed=seed, varlen=varlen)


def gpu_backward(inp, adj, dev, want_ds0=True):
    """Run the library's backward on NaN-filled outputs; returns numpy float64 arrays."""
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    t = torch_inputs(inp, dev)
    dy = wl.to_torch(adj["dy"], dev, "bf16")
    dsf = None if adj["ds_final"] is None else torch.from_numpy(adj["ds_final"]).to(dev)
    rows, H, dk, dv, N = inp["q"].shape[0], inp["H"], inp["dk"], inp["dv"], inp["num_seqs"]
    nan = float("nan")
    out = (torch.full((rows, H, dk), nan, dtype=torch.bfloat16, device=dev),
           torch.full((rows, H, dk), nan, dtype=torch.bfloat16, device=dev),
           torch.full((rows, H, dv), nan, dtype=torch.bfloat16, device=dev),
           torch.full((rows, H), nan, dtype=torch.float32, device=dev),
           torch.full((rows, H), nan, dtype=torch.float32, device=dev),
           torch.full((N, H, dk, dv), nan, dtype=torch.float32, device=dev)
           if want_ds0 else None)
    res = gdn.gdn_prefill_backward(t["q"], t["k"], t["v"], t["alpha"], t["beta"], dy,
                                   initial_state=t["s0"], d_final_state=dsf,
                                   cu_seqlens=t["cu"], num_seqs=N, out=out)
    torch.cuda.synchronize()
    return [None if x is None else x.float().cpu().numpy().astype(np.float64) for x in res]


def oracle_backward(inp, adj, oracle, heads=None, threads=16):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    cu = np.concatenate([[0], np.cumsum(inp["lengths"])]).astype(np.int64)
    return oracle.prefill_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                   wl.as_f64(adj["dy"], "bf16"), cu_seqlens=cu,
                                   s0=inp["s0"], ds_final=adj["ds_final"], heads=heads,
                                   threads=threads)


def compare(got, ref, cu, label, heads=None, tol=TOL):
    dq, dk, dv, da, db, ds0 = got
    h0, h1 = (0, ref["dq"].shape[1]) if heads is None else heads
    errs = {}
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        g = g[:, h0:h1]
        assert np.all(np.isfinite(g)), "%s: %s has non-finite values" % (label, name)
        errs[name] = slice_rel_err(g, ref[name], cu)
    for name, g in (("dalpha", da), ("dbeta", db)):
        g = g[:, h0:h1]
        assert np.all(np.isfinite(g)), "%s: %s has non-finite values" % (label, name)
        errs[name] = slice_rel_err(g[:, :, None], ref[name][:, :, None], cu)
    if ds0 is not None:
        g = ds0[:, h0:h1]
        assert np.all(np.isfinite(g)), "%s: dS0 has non-finite values" % label
        errs["ds0"] = state_rel_err(g, ref["ds0"])
    say("    %s errors: %s" % (label, "  ".join("%s %.2e" % kv for kv in errs.items())))
    for name, e in errs.items():
        assert e <= tol, "%s: %s error %.3e > %.1e" % (label, name, e, tol)
    return errs


def check(inp, adj, dev, oracle, label, want_ds0=True):
    say("[gpu] backward %s lengths=%s H=%d dk=%d dv=%d s0=%s dsT=%s" % (
        label, list(inp["lengths"][:8]), inp["H"], inp["dk"], inp["dv"],
        inp["s0"] is not None, adj["ds_final"] is not None))
    got = gpu_backward(inp, adj, dev, want_ds0)
    ref = oracle_backward(inp, adj, oracle)
    cu = np.concatenate([[0], np.cumsum(inp["lengths"])]).astype(np.int64)
    return compare(got, ref, cu, label)


@pytest.mark.parametrize("d", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_backward_ragged_lengths(dev, oracle_lib, d):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([1, 63, 64, 65, 0, 130], H=2, d=d, seed=21)
    check(inp, wl.backward_inputs(inp, 0.02, seed=21), dev, oracle_lib, "ragged")


def test_backward_strong_decay(dev, oracle_lib):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([200, 77], H=2, seed=22, alpha=(1.0, 2.0), beta=(0.0, 1.5))
    check(inp, wl.backward_inputs(inp, 0.02, seed=22), dev, oracle_lib, "strong-decay")


def test_backward_gate_edges(dev, oracle_lib):
    """alpha = 1 and beta in {0, 1} exactly."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([150, 40], H=2, seed=23)
    inp["alpha"][::3] = 1.0
    inp["beta"][::5] = 0.0
    inp["beta"][1::7] = 1.0
    check(inp, wl.backward_inputs(inp, 0.02, seed=23), dev, oracle_lib, "gate-edges")


def test_backward_without_states(dev, oracle_lib):
    """No initial state, no final-state adjoint, no dS0 output; equal lengths, no cu_seqlens."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([192] * 3, H=3, s0=None, seed=24, varlen=False)
    check(inp, wl.backward_inputs(inp, None, seed=24), dev, oracle_lib, "no-states",
          want_ds0=False)


def test_backward_all_sequences_empty(dev, oracle_lib):
    """Zero tokens: dS0 is the final-state adjoint passed through."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([0, 0], H=2, seed=25)
    adj = wl.backward_inputs(inp, 0.02, seed=25)
    got = gpu_backward(inp, adj, dev)
    np.testing.assert_array_equal(got[5], adj["ds_final"].astype(np.float64))


def test_backward_matches_forward_adjoint_identities(dev):
    """<dq, q> = <dy, y> and <dv, v> + <dS0, S0> = <dy, y> + <dS_T, S_T> with the library's
    own forward (bf16 y), on a mid-size batch."""
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([700, 333, 64], H=4, seed=26)
    adj = wl.backward_inputs(inp, 0.02, seed=26)
    t = torch_inputs(inp, dev)
    y, sT = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                            initial_state=t["s0"], cu_seqlens=t["cu"])
    torch.cuda.synchronize()
    got = gpu_backward(inp, adj, dev)
    dy = wl.as_f64(adj["dy"], "bf16")
    yy = y.float().cpu().numpy().astype(np.float64)
    q = wl.as_f64(inp["q"], "bf16")
    v = wl.as_f64(inp["v"], "bf16")
    lhs_q = np.sum(got[0] * q)
    rhs = np.sum(dy * yy)
    scale = np.sum(np.abs(dy * yy))
    say("    <dq,q> %.6e  <dy,y> %.6e  scale %.3e" % (lhs_q, rhs, scale))
    assert abs(lhs_q - rhs) <= 5e-3 * scale
    lhs_v = np.sum(got[2] * v) + np.sum(got[5] * inp["s0"])
    rhs_v = rhs + np.sum(adj["ds_final"] * sT.cpu().numpy())
    say("    <dv,v>+<dS0,S0> %.6e  <dy,y>+<dST,ST> %.6e" % (lhs_v, rhs_v))
    assert abs(lhs_v - rhs_v) <= 5e-3 * scale


def test_backward_full_prefill_workload(dev, oracle_lib):
    """The 4 x 4096-token, 16-head, d = 128 bf16 prefill at full size, in the launch
    configuration the benchmark times: every gradient of every head and sequence against the
    oracle, every output finite."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.workload_inputs(wl.PREFILL)
    adj = wl.backward_inputs(inp, 0.02, seed=27)
    say("[gpu] backward full prefill workload")
    got = gpu_backward(inp, adj, dev)
    for i, x in enumerate(got):
        assert np.all(np.isfinite(x)), "output %d has non-finite values" % i
    cu = np.concatenate([[0], np.cumsum(inp["lengths"])]).astype(np.int64)
    say("[gpu] backward full prefill workload: oracle over all %d heads" % inp["H"])
    ref = oracle_backward(inp, adj, oracle_lib)
    compare(got, ref, cu, "full-size, all heads")


def test_backward_deterministic(dev):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([300, 129], H=2, seed=28)
    adj = wl.backward_inputs(inp, 0.02, seed=28)
    a = gpu_backward(inp, adj, dev)
    b = gpu_backward(inp, adj, dev)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)

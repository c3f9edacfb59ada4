"""GPU parity of gdn_prefill_output_gated, the prefill followed by the layer's output gate
(sigmoid(z) * RMSNorm(y) * (1 + w) per (token, head) row), against the oracle's prefill and
output gate in fp64; both the fused path (the one-launch scan gates each row as it leaves) and
the composed path (other plans: prefill, then the output-gate kernel in place)."""
import numpy as np
import pytest

from gpu_util import TOL, cu_of, say, slice_rel_err, state_rel_err, torch_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _inputs(lengths, H, dtype, seed, alpha=(3.0, 1.0), beta=(0.0, 1.0), d=128):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.make_inputs(lengths, H, d, d, dtype, alpha=alpha, beta=beta, s0_sd=0.02, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    T = int(sum(lengths))
    z = rng.standard_normal((T, H, d)) * 2.0
    inp["z"] = wl.bf16_bits(z) if dtype == "bf16" else z.astype(np.float32)
    inp["norm_w"] = (0.1 * rng.standard_normal(d)).astype(np.float32)
    return inp


def _gated(inp, dev, dv_tile, seg, eps):
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    t = torch_inputs(inp, dev)
    z = wl.to_torch(inp["z"], dev, inp["dtype"])
    w = torch.from_numpy(inp["norm_w"]).to(dev)
    out, sf = gdn.gdn_prefill_output_gated(t["q"], t["k"], t["v"], t["alpha"], t["beta"], z, w,
                                           eps, initial_state=t["s0"], cu_seqlens=t["cu"],
                                           num_seqs=inp["num_seqs"], dv_tile=dv_tile,
                                           segment_chunks=seg)
    return out, sf, z, w


def _check(inp, dev, oracle_lib, dv_tile, seg, label, eps=1e-6):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    from oracle import layer_steps as ls
    say("[gpu] prefill+output gate %s tile=%s seg=%s lengths=%s H=%d %s" % (
        label, dv_tile, seg, list(inp["lengths"][:8]), inp["H"], inp["dtype"]))
    out, sf, _, _ = _gated(inp, dev, dv_tile, seg, eps)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    gs = sf.cpu().numpy()
    ry, rs = oracle_lib.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                cu_of(inp), s0=inp["s0"], threads=16)
    ref = ls.output_gate(ry, wl.as_f64(inp["z"], inp["dtype"]), inp["norm_w"], eps)
    err = slice_rel_err(got, ref, cu_of(inp))
    es = state_rel_err(gs, rs)
    say("    err out %.3e  state %.3e" % (err, es))
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(gs))
    tol = TOL[inp["dtype"]]
    assert err <= tol, "output error %.3e > %.1e" % (err, tol)
    assert es <= tol, "state error %.3e > %.1e" % (es, tol)


@pytest.mark.parametrize("seg", [-1, 3])
def test_fused_gate_one_launch_scan(dev, oracle_lib, seg):
    """bf16 d = 128 with dv_tile 128: the gate runs inside the scan's y store (ragged and
    empty sequences; with segments, later segments warm up or wait for their predecessor)."""
    inp = _inputs([300, 64, 1, 129, 0, 700], 3, "bf16", seed=71 + seg)
    _check(inp, dev, oracle_lib, 128, seg, "fused")


@pytest.mark.parametrize("d,seg", [(128, -1), (128, 2), (64, -1), (64, 3)])
def test_composed_gate_pipelined_scan(dev, oracle_lib, d, seg):
    """bf16 with 32-column tiles (the default plan of short work), whose rows are gated after
    the prefill: four tiles per head at d = 128, two at d = 64; ragged, single-token and empty
    sequences, and segments whose final pass starts from combined segment states."""
    inp = _inputs([300, 64, 1, 129, 0, 700, 65], 3, "bf16", seed=81 + d + seg, d=d)
    _check(inp, dev, oracle_lib, 32, seg, "composed, pipelined scan")


def test_gate_prefill_workload_full_size(dev, oracle_lib):
    """The prefill workload (B = 4, H = 16, T = 4096, d = 128, bf16, S0 = 0) on the library's
    own plan (32-column tiles, 256 workgroups), gated: every token of every head."""
    from linear_attention_recurrence_chunked_amd import gdn
    assert gdn.gdn_prefill_plan(4, 4 * 4096, 16, 128, 128, gdn.GDN_DTYPE_BF16)[0] == 32
    inp = _inputs([4096] * 4, 16, "bf16", seed=85)
    inp["s0"] = None
    _check(inp, dev, oracle_lib, 0, 0, "prefill workload")


@pytest.mark.parametrize("dtype,tile", [("bf16", 16), ("bf16", 64), ("f32", 0)])
def test_composed_gate_other_plans(dev, oracle_lib, dtype, tile):
    """The other column-split plans: prefill, then the output-gate kernel over the output in
    place."""
    inp = _inputs([300, 64, 1, 129, 0, 200], 2, dtype, seed=75)
    _check(inp, dev, oracle_lib, tile, 0, "composed")


def test_fused_equals_gate_of_prefill(dev):
    """The fused path against gdn_output_gate applied to gdn_prefill's own bf16 y on the same
    plan: the same inputs to the gate, so the two agree to within a bf16 rounding of the
    output (each row compared on its own scale)."""
    from linear_attention_recurrence_chunked_amd import gdn
    inp = _inputs([513, 70, 1000], 4, "bf16", seed=77, alpha=(1.0, 2.0), beta=(0.0, 1.5))
    t = torch_inputs(inp, dev)
    out, sf, z, w = _gated(inp, dev, 128, 4, 1e-5)
    y, sf2 = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                             initial_state=t["s0"], cu_seqlens=t["cu"],
                             num_seqs=inp["num_seqs"], dv_tile=128, segment_chunks=4)
    og = gdn.gdn_output_gate(y, z, w, eps=1e-5)
    torch.cuda.synchronize()
    a = out.float().cpu().numpy()
    b = og.float().cpu().numpy()
    row = np.maximum(np.abs(b).max(axis=-1, keepdims=True), 1e-30)
    err = float(np.max(np.abs(a - b) / row))
    say("[gpu] fused vs composed on the same y: per-row rel err %.3e" % err)
    assert np.array_equal(sf.cpu().numpy(), sf2.cpu().numpy())
    assert err <= 2.0 ** -7

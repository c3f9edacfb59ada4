"""GPU parity of the layer steps (short conv + SiLU + L2Norm, gates, output gate) against the
fp64 oracle in oracle/layer_steps.py, through the C ABI."""
import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# fp32 kernels use the hardware exp and reciprocal square root (about 1e-6 relative); bf16
# outputs round to 8 significant bits
TOL = {"f32": 2e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _t(arr, dev, dt):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    return None if arr is None else wl.to_torch(arr, dev, dt)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _rel(got, ref):
    scale = np.max(np.abs(ref)) if ref.size else 1.0
    return float(np.max(np.abs(got - ref)) / max(scale, 1e-30)) if ref.size else 0.0


CONV_CASES = [
    # lengths, H, d, W, dtype, head_dim, with_state
    ([37, 0, 5, 130, 2, 64], 3, 64, 4, "f32", 64, True),       # ragged, empty, shorter than W
    ([37, 0, 5, 130, 2, 64], 3, 64, 4, "bf16", 0, True),
    ([200, 1, 77], 4, 128, 4, "bf16", 128, True),
    ([200, 1, 77], 4, 128, 2, "f32", 128, False),
    ([50, 50], 2, 128, 1, "bf16", 128, True),                   # width 1: no state
    ([64] * 8, 16, 128, 3, "bf16", 128, True),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "L%d_H%d_d%d_W%d_%s_hd%d_%s" % (
    len(c[0]), c[1], c[2], c[3], c[4], c[5], "state" if c[6] else "zero"))
def test_short_conv_parity(dev, case):
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    from oracle import layer_steps as ls
    lengths, H, d, W, dt, hd, with_state = case
    say("short_conv %s" % (case,))
    inp = wl.layer_step_inputs(lengths, H, d, W, dt, seed=len(lengths) * 7 + W, with_state=with_state)
    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
    x = _t(inp["x_q"], dev, dt)
    w = torch.from_numpy(inp["w_q"]).to(dev)
    sin = None if inp["s_q"] is None else torch.from_numpy(inp["s_q"]).to(dev)
    sout = torch.full((inp["N"], inp["C"], max(W - 1, 1)), 7.0, device=dev) if W > 1 else None
    out = gdn.gdn_short_conv(x, w, cu_seqlens=cu, head_dim=hd, state_in=sin, state_out=sout)
    torch.cuda.synchronize()
    ref, ref_state = ls.short_conv_silu(wl.as_f64(inp["x_q"], dt), inp["w_q"], inp["cu_seqlens"],
                                        hd, inp["s_q"])
    err = _rel(_host(out), ref)
    say("  rel err %.3e" % err)
    assert err <= TOL[dt]
    if W > 1:
        # the carried state is a copy of inputs: exact
        np.testing.assert_array_equal(_host(sout), ref_state)


def test_short_conv_state_chains_and_decode(dev):
    """A sequence run in one call equals the same tokens run as a prefill of its first part
    and then token by token as decode steps (num_seqs = B, one token each), with the state
    carried in place."""
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    B, H, d, W, L, cut = 3, 2, 128, 4, 12, 5
    inp = wl.layer_step_inputs([L] * B, H, d, W, "f32", seed=5)
    x = torch.from_numpy(inp["x_k"]).to(dev).view(B, L, -1)          # [B, L, C] by sequence
    w = torch.from_numpy(inp["w_k"]).to(dev)
    s0 = torch.from_numpy(inp["s_k"]).to(dev)
    full = gdn.gdn_short_conv(x.reshape(B * L, -1), w, num_seqs=B, head_dim=d,
                              state_in=s0, state_out=torch.empty_like(s0))
    st = s0.clone()
    pre = gdn.gdn_short_conv(x[:, :cut].reshape(B * cut, -1).contiguous(), w, num_seqs=B,
                             head_dim=d, state_in=st, state_out=st)
    steps = []
    for t in range(cut, L):
        steps.append(gdn.gdn_short_conv(x[:, t].contiguous(), w, num_seqs=B, head_dim=d,
                                        state_in=st, state_out=st))
    torch.cuda.synchronize()
    got = torch.cat([pre.view(B, cut, -1)] + [s.view(B, 1, -1) for s in steps], dim=1)
    np.testing.assert_allclose(_host(got), _host(full.view(B, L, -1)), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("T,H", [(1000, 16), (37, 3), (1, 1)])
def test_gates_parity(dev, T, H):
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    from oracle import layer_steps as ls
    inp = wl.layer_step_inputs([T], H, 64, 4, "f32", seed=T + H)
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("a", "b", "A", "b_alpha")}
    al, be = gdn.gdn_gates(t["a"], t["b"], t["A"], t["b_alpha"])
    torch.cuda.synchronize()
    ral, rbe, _ = ls.gates(inp["a"], inp["b"], inp["A"], inp["b_alpha"])
    np.testing.assert_allclose(_host(be), rbe, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(_host(al), ral, rtol=2e-5, atol=1e-37)
    assert np.all(_host(al) <= 1.0) and np.all(_host(al) >= 0.0)


OG_CASES = [(1000, 4, 128, "bf16"), (333, 3, 64, "f32"), (257, 16, 128, "f32"), (5, 1, 64, "bf16")]


@pytest.mark.parametrize("T,H,d,dt", OG_CASES)
@pytest.mark.parametrize("in_place", [False, True])
def test_output_gate_parity(dev, T, H, d, dt, in_place):
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    from oracle import layer_steps as ls
    inp = wl.layer_step_inputs([T], H, d, 4, dt, seed=3 * T + d)
    y = _t(inp["y"], dev, dt)
    z = _t(inp["z"], dev, dt)
    w = torch.from_numpy(inp["norm_w"]).to(dev)
    out = gdn.gdn_output_gate(y, z, w, eps=1e-6, out=y if in_place else None)
    torch.cuda.synchronize()
    ref = ls.output_gate(wl.as_f64(inp["y"], dt), wl.as_f64(inp["z"], dt), inp["norm_w"], 1e-6)
    got = _host(out)
    # per row relative error (each row is normalised on its own)
    err = np.max(np.abs(got - ref) / np.maximum(np.abs(ref).max(axis=-1, keepdims=True), 1e-30))
    say("output gate %s in_place=%s rel err %.3e" % ((T, H, d, dt), in_place, err))
    assert err <= TOL[dt]


def test_layer_steps_full_size(dev):
    """The config-2 shape (T = 16384 packed tokens, H = 16, d = 128, bf16): the convolution
    with its carried states and the output gate at full size, every token and every (token,
    head) row against the oracle (each compared on its own scale)."""
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    from oracle import layer_steps as ls
    lengths = [4096] * 4
    inp = wl.layer_step_inputs(lengths, 16, 128, 4, "bf16", seed=77)
    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
    x = _t(inp["x_q"], dev, "bf16")
    out = gdn.gdn_short_conv(x, torch.from_numpy(inp["w_q"]).to(dev), cu_seqlens=cu,
                             head_dim=128, state_in=torch.from_numpy(inp["s_q"]).to(dev))
    y = _t(inp["y"], dev, "bf16")
    og = gdn.gdn_output_gate(y, _t(inp["z"], dev, "bf16"), torch.from_numpy(inp["norm_w"]).to(dev))
    torch.cuda.synchronize()
    got = _host(out)
    assert np.all(np.isfinite(got))
    ref, _ = ls.short_conv_silu(wl.as_f64(inp["x_q"], "bf16"), inp["w_q"], inp["cu_seqlens"],
                                128, inp["s_q"])
    err = np.max(np.abs(got - ref).max(axis=-1) /
                 np.maximum(np.abs(ref).max(axis=-1), 1e-30))
    say("layer steps full size: convolution rel err %.3e over %d tokens" % (err, got.shape[0]))
    assert err <= TOL["bf16"]
    ref = ls.output_gate(wl.as_f64(inp["y"], "bf16"), wl.as_f64(inp["z"], "bf16"),
                         inp["norm_w"])
    got = _host(og)
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - ref).max(axis=-1) /
                 np.maximum(np.abs(ref).max(axis=-1), 1e-30))
    say("layer steps full size: output gate rel err %.3e over %d rows" % (
        err, got.shape[0] * got.shape[1]))
    assert err <= TOL["bf16"]

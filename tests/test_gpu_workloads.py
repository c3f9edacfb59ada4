"""The workloads at full size, in the launch configuration the benchmark uses (the library's
own plan), against the fp64 oracle: element by element where the oracle can cover the whole
run, and on exact sub-problems where it cannot (the 2^20-token sequence).

Tolerances: per (sequence, head) slice max relative error 2e-2 for bf16 inputs."""
import numpy as np
import pytest

from gpu_util import TOL, check_prefill, gpu_prefill, say, slice_rel_err, state_rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def test_workload_prefill_b4_h16_t4096(dev, oracle_lib):
    """B=4, H=16, T=4096, d=128 bf16: every token of every head against the oracle."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.workload_inputs(wl.PREFILL)
    check_prefill(inp, dev, oracle_lib, label="prefill B4 H16 T4096")


def test_workload_packed_varlen(dev, oracle_lib):
    """32 packed sequences of 512..16384 tokens, per-sequence initial states, strong decay:
    every token of every head and every final state against the oracle."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.workload_inputs(wl.VARLEN)
    check_prefill(inp, dev, oracle_lib, label="packed varlen 32 seqs")


def test_workload_long_sequence(dev, oracle_lib):
    """One sequence of 2^20 tokens, H=16 (the segment-parallel plan).

    The oracle cannot run whole 2^20-token chains inside a test, so three exact checks:
      * the first 65,536 tokens of two heads against the oracle from the true start (zero);
      * fading memory: the decay gates of this workload multiply to below 2^-1300 over any
        32,768 tokens (checked on the data below), so the oracle started from zero 65,536
        tokens before the end reproduces the final state and the last 32,768 outputs to
        fp64 rounding;
      * the unsegmented plan gives the same result as the segmented one.
    """
    from linear_attention_recurrence_chunked_amd import workloads as wl
    from linear_attention_recurrence_chunked_amd import gdn
    inp = wl.workload_inputs(wl.LONG)
    T = inp["q"].shape[0]
    H = inp["H"]
    tile, seg = gdn.gdn_prefill_plan(1, T, H, 128, 128, gdn.GDN_DTYPE_BF16)
    say("[gpu] long sequence T=%d plan tile=%d seg=%d" % (T, tile, seg))
    assert seg > 0, "the long sequence is expected to use the segment-parallel plan"
    y, sf = gpu_prefill(inp, dev)
    torch.cuda.synchronize()
    heads = (0, 2)
    W = 65536
    # fading memory over the last window: log2 of the decay product over 32,768 tokens
    la = np.log2(inp["alpha"][T - W: T - W + 32768, heads[0]:heads[1]].astype(np.float64))
    assert la.sum(axis=0).max() < -1300.0

    # (1) exact prefix
    ry, _ = oracle_lib.prefill(inp["q"][:W], inp["k"][:W], inp["v"][:W], inp["alpha"][:W],
                               inp["beta"][:W], None, heads=heads, threads=2, want_state=False)
    gy = y[:W, heads[0]:heads[1]].float().cpu().numpy()
    e1 = slice_rel_err(gy, ry, np.array([0, W]))
    # (2) last window from zero
    sl = slice(T - W, T)
    ry2, rs2 = oracle_lib.prefill(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["alpha"][sl],
                                  inp["beta"][sl], None, heads=heads, threads=2)
    gy2 = y[T - 32768:, heads[0]:heads[1]].float().cpu().numpy()
    e2 = slice_rel_err(gy2, ry2[W - 32768:], np.array([0, 32768]))
    es = state_rel_err(sf[:, heads[0]:heads[1]].cpu().numpy(), rs2)
    say("    prefix y %.3e  tail y %.3e  final state %.3e" % (e1, e2, es))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"] and es <= TOL["bf16"]
    # (3) plan independence at full size
    y_flat, sf_flat = gpu_prefill(inp, dev, segment_chunks=-1)
    torch.cuda.synchronize()
    worst_y = 0.0
    for h in range(H):
        a, b = y[:, h].float(), y_flat[:, h].float()
        worst_y = max(worst_y, ((a - b).abs().max() / b.abs().max()).item())
    ds = ((sf - sf_flat).abs().amax(dim=(2, 3)) / sf_flat.abs().amax(dim=(2, 3))).max().item()
    say("    segmented vs unsegmented: y %.3e  state %.3e" % (worst_y, ds))
    assert worst_y <= TOL["bf16"] and ds <= TOL["bf16"]

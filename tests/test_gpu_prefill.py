"""GPU parity of gdn_prefill against the fp64 oracle (element by element, per-slice max
relative error: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs)."""
import numpy as np
import pytest

from gpu_util import TOL, check_prefill, cu_of, gpu_prefill, say, slice_rel_err, state_rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _inp(lengths, H=2, d=(128, 128), dtype="bf16", s0=0.02, seed=0, alpha=(3.0, 1.0),
         beta=(0.0, 1.0)):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    return wl.make_inputs(lengths, H, d[0], d[1], dtype, alpha=alpha, beta=beta, s0_sd=s0,
                          seed=seed)


# ---- the tiny fp32 workload, every column tile --------------------------------------------

@pytest.mark.parametrize("tile", [0, 16, 32, 64])
def test_tiny_fp32_workload(dev, oracle_lib, tile):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.workload_inputs(wl.TINY)
    check_prefill(inp, dev, oracle_lib, tol=1e-4, dv_tile=tile, label="tiny-fp32")


# ---- ragged lengths, both dtypes and head sizes -------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_ragged_lengths(dev, oracle_lib, dtype, d):
    lengths = [1, 63, 64, 65, 0, 127, 200]
    inp = _inp(lengths, H=3, d=d, dtype=dtype, seed=11)
    check_prefill(inp, dev, oracle_lib, label="ragged")


@pytest.mark.parametrize("tile", [16, 32, 64, 128])
def test_bf16_tiles(dev, oracle_lib, tile):
    inp = _inp([130, 7, 300], H=2, seed=12, alpha=(1.0, 2.0), beta=(0.0, 1.5))
    check_prefill(inp, dev, oracle_lib, dv_tile=tile, label="tiles")


def test_no_initial_state_equal_lengths(dev, oracle_lib):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = wl.make_inputs([192] * 3, 4, 128, 128, "bf16", s0_sd=None, seed=13, varlen=False)
    check_prefill(inp, dev, oracle_lib, label="equal-lengths-no-s0")


def test_gate_edges(dev, oracle_lib):
    """alpha = 1 and beta in {0, 1} exactly (closed ends of the gate ranges)."""
    inp = _inp([150], H=2, seed=14)
    inp["alpha"][::3] = 1.0
    inp["beta"][::5] = 0.0
    inp["beta"][1::5] = 1.0
    check_prefill(inp, dev, oracle_lib, label="gate-edges")


def test_strong_decay_fp32(dev, oracle_lib):
    """alpha = sigmoid(N(1, 2)): per-chunk decay products far below fp32 range."""
    inp = _inp([256, 129], H=2, d=(64, 64), dtype="f32", seed=15, alpha=(1.0, 2.0),
               beta=(0.0, 1.5))
    check_prefill(inp, dev, oracle_lib, tol=1e-4, label="strong-decay-fp32")


# ---- the segment-parallel scan ------------------------------------------------------------

@pytest.mark.parametrize("seg", [1, 2, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segmented_scan(dev, oracle_lib, seg, dtype):
    lengths = [500, 64, 0, 129, 1000, 65]
    inp = _inp(lengths, H=2, dtype=dtype, seed=16 + seg, alpha=(3.0, 1.0))
    tile = 16 if dtype == "f32" else 64
    check_prefill(inp, dev, oracle_lib, dv_tile=tile, segment_chunks=seg, label="segmented")


def test_segmented_slow_decay(dev, oracle_lib):
    """alpha close to 1: the segment transition matrices stay large, so phase B matters."""
    inp = _inp([2000, 700], H=2, seed=20, alpha=(8.0, 0.5))
    check_prefill(inp, dev, oracle_lib, dv_tile=128, segment_chunks=2, label="seg-slow-decay")


@pytest.mark.parametrize("seg", [1, 2, 3])
@pytest.mark.parametrize("tile", [16, 32])
def test_segmented_pipelined_scan_slow_decay(dev, oracle_lib, tile, seg):
    """The pipelined scan (16- and 32-column tiles) in segmented mode: every segment but a
    sequence's first starts from the state phases A and B composed, and with alpha close to
    1 (sigmoid(N(8, 0.5))) that state is far from negligible at every segment boundary."""
    lengths = [700, 1, 64, 0, 129, 450, 65]
    inp = _inp(lengths, H=2, seed=40 + 3 * tile + seg, alpha=(8.0, 0.5))
    check_prefill(inp, dev, oracle_lib, dv_tile=tile, segment_chunks=seg,
                  label="segmented-pipe")


# ---- the one-launch scan (bf16, d = 128, the whole state per workgroup) -------------------
# Segments after a sequence's first start from a warm-up over the chunks before them when the
# transition norm over those chunks provably falls below 2^-48, and otherwise wait for the
# previous segment's exact end state; these cases force each of the four starts.

@pytest.mark.parametrize("seg", [2, 4])
def test_wide_segments_warm_up(dev, oracle_lib, seg):
    """Strong decay (sigmoid(N(1, 2))): every later segment starts from a verified warm-up."""
    inp = _inp([3000, 1100, 64, 65, 0, 700], H=2, seed=50 + seg, alpha=(1.0, 2.0),
               beta=(0.0, 1.5))
    check_prefill(inp, dev, oracle_lib, dv_tile=128, segment_chunks=seg, label="wide-warm")


def test_wide_segments_chained(dev, oracle_lib):
    """Slow decay (sigmoid(N(8, 0.5))): no window within a segment reaches the bound, so
    every segment takes its predecessor's published end state (and the second segment of a
    sequence warms up from the sequence start instead)."""
    inp = _inp([2500, 900, 130], H=3, seed=56, alpha=(8.0, 0.5))
    check_prefill(inp, dev, oracle_lib, dv_tile=128, segment_chunks=3, label="wide-chain")


def test_wide_segments_mixed(dev, oracle_lib):
    """sigmoid(N(3, 1)) with segments of 8 chunks: windows of about 7-8 chunks, so some
    segments warm up and others wait for their predecessor."""
    inp = _inp([5000, 2000], H=4, seed=57, alpha=(3.0, 1.0))
    check_prefill(inp, dev, oracle_lib, dv_tile=128, segment_chunks=8, label="wide-mixed")


def test_wide_segments_unnormalised_keys(dev, oracle_lib):
    """Keys of norm 1.5: |1 - beta ||k||^2| exceeds 1 for large beta, so the key terms of the
    bound count and some warm-ups fail verification and fall back to the exact chain."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    inp = _inp([2600, 800], H=2, seed=58, alpha=(1.0, 2.0), beta=(0.0, 1.5))
    inp["k"] = wl.bf16_bits(wl.bf16_to_f64(inp["k"]) * 1.5)
    check_prefill(inp, dev, oracle_lib, dv_tile=128, segment_chunks=2, label="wide-keys")


def test_wide_unsegmented_many_chains(dev, oracle_lib):
    """1024 chains and more: no segments, one workgroup per (sequence, head)."""
    rng = np.random.default_rng(59)
    lengths = rng.integers(0, 300, size=130)
    inp = _inp(lengths, H=8, seed=59)
    check_prefill(inp, dev, oracle_lib, label="wide-unsegmented")


def test_many_sequences_segment_table(dev, oracle_lib):
    """More sequences than one table-building pass (1024) with segments and empties."""
    rng = np.random.default_rng(21)
    lengths = rng.integers(0, 140, size=1500)
    inp = _inp(lengths, H=1, d=(64, 64), seed=21)
    check_prefill(inp, dev, oracle_lib, dv_tile=64, segment_chunks=1, label="many-seqs")


# ---- outputs, resume, hygiene ---------------------------------------------------------------

def test_resume_split_equals_whole(dev, oracle_lib):
    from linear_attention_recurrence_chunked_amd import gdn
    from gpu_util import torch_inputs
    inp = _inp([300], H=2, seed=22)
    t = torch_inputs(inp, dev)
    y_all, s_all = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                                   initial_state=t["s0"])
    t1 = 130
    y1, s1 = gdn.gdn_prefill(t["q"][:t1], t["k"][:t1], t["v"][:t1], t["alpha"][:t1],
                             t["beta"][:t1], initial_state=t["s0"].clone())
    # in-place resume: the final state overwrites the initial one
    y2, s2 = gdn.gdn_prefill(t["q"][t1:], t["k"][t1:], t["v"][t1:], t["alpha"][t1:],
                             t["beta"][t1:], initial_state=s1, final_state=s1)
    torch.cuda.synchronize()
    assert s2.data_ptr() == s1.data_ptr()
    ry, rs = oracle_lib.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                cu_of(inp), s0=inp["s0"])
    gy = torch.cat([y1, y2]).float().cpu().numpy()
    assert slice_rel_err(gy, ry, cu_of(inp)) <= TOL["bf16"]
    assert state_rel_err(s2.cpu().numpy(), rs) <= TOL["bf16"]
    assert slice_rel_err(y_all.float().cpu().numpy(), ry, cu_of(inp)) <= TOL["bf16"]


def test_without_final_state(dev):
    from linear_attention_recurrence_chunked_amd import gdn
    from gpu_util import torch_inputs
    inp = _inp([100, 50], H=2, seed=23)
    t = torch_inputs(inp, dev)
    y, sf = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                            initial_state=t["s0"], cu_seqlens=t["cu"], want_final_state=False)
    y2, _ = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                            initial_state=t["s0"], cu_seqlens=t["cu"])
    torch.cuda.synchronize()
    assert sf is None
    assert torch.equal(y, y2)


@pytest.mark.parametrize("seg", [-1, 2])
def test_deterministic_and_every_output_written(dev, seg):
    """Bitwise-identical repeats; NaN-poisoned y and state are fully overwritten."""
    from linear_attention_recurrence_chunked_amd import gdn
    from gpu_util import torch_inputs
    inp = _inp([333, 0, 64, 77], H=3, seed=24)
    t = torch_inputs(inp, dev)
    outs = []
    for rep in range(2):
        y = torch.full((inp["q"].shape[0], 3, 128), float("nan"), dtype=torch.bfloat16,
                       device=dev)
        sf = torch.full((4, 3, 128, 128), float("nan"), dtype=torch.float32, device=dev)
        need = gdn.gdn_prefill_workspace_bytes(4, inp["q"].shape[0], 3, 128, 128, 1, 64, seg)
        ws = None
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            ws.view(torch.float32)[: need // 4].fill_(float("nan"))
        gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"], initial_state=t["s0"],
                        cu_seqlens=t["cu"], y=y, final_state=sf, workspace=ws, dv_tile=64,
                        segment_chunks=seg)
        torch.cuda.synchronize()
        assert not torch.isnan(y.float()).any()
        assert not torch.isnan(sf).any()
        outs.append((y.clone(), sf.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # the zero-length sequence returns its initial state unchanged
    assert torch.equal(outs[0][1][1], t["s0"][1])


def test_plan_independence(dev):
    """Every column tile and segmentation gives the same result up to rounding."""
    inp = _inp([700, 260], H=2, seed=25)
    ref_y, ref_s = gpu_prefill(inp, dev, dv_tile=32, segment_chunks=-1)
    for tile, seg in [(64, -1), (128, -1), (64, 3), (128, 1), (16, 2)]:
        y, s = gpu_prefill(inp, dev, dv_tile=tile, segment_chunks=seg)
        torch.cuda.synchronize()
        dy = (y.float() - ref_y.float()).abs().max().item() / ref_y.float().abs().max().item()
        ds = (s - ref_s).abs().max().item() / ref_s.abs().max().item()
        say("    tile %d seg %d: dy %.2e ds %.2e" % (tile, seg, dy, ds))
        assert dy <= 2e-2 and ds <= 2e-2

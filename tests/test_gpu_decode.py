"""GPU parity of gdn_decode_step against the fp64 oracle."""
import numpy as np
import pytest

from gpu_util import TOL, gpu_prefill, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _decode_inputs(steps, B, H, dk, dv, dtype, seed):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    w = wl.Workload("decode-test", "decode", H=H, dk=dk, dv=dv, dtype=dtype,
                    alpha=(3.0, 1.0), beta=(0.0, 1.0), seed=seed, B=B, s0_sd=0.5,
                    steps=steps)
    return wl.decode_inputs(w)


def _run_gpu(d, dev, steps=None):
    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl
    dt = d["dtype"]
    steps = d["steps"] if steps is None else steps
    q = wl.to_torch(d["q"], dev, dt)
    k = wl.to_torch(d["k"], dev, dt)
    v = wl.to_torch(d["v"], dev, dt)
    a = torch.from_numpy(d["alpha"]).to(dev)
    b = torch.from_numpy(d["beta"]).to(dev)
    state = torch.from_numpy(d["s0"]).to(dev)
    y = torch.empty((steps,) + tuple(v.shape[1:]), dtype=v.dtype, device=dev)
    for s in range(steps):
        gdn.gdn_decode_step(q[s], k[s], v[s], a[s], b[s], state, y=y[s])
    torch.cuda.synchronize()
    return y, state


def _rel(got, ref, axis_slices):
    """Max over the slices of ||got - ref||_inf / ||ref||_inf; a NaN anywhere is kept."""
    worst = 0.0
    for sl in axis_slices:
        r = ref[sl]
        den = float(np.max(np.abs(r)))
        e = float(np.max(np.abs(got[sl] - r))) / (den if den > 0 else 1.0)
        worst = _worse(worst, e)
    return worst


def _worse(a, b):
    """max(a, b) that keeps a NaN (Python's max(0.0, nan) is 0.0)."""
    if a != a or b != b:
        return float("nan")
    return a if a >= b else b


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_decode_steps(dev, oracle_lib, dtype, d):
    steps, B, H = 12, 5, 3
    inp = _decode_inputs(steps, B, H, d[0], d[1], dtype, seed=31)
    say("[gpu] decode %s d=%s B=%d H=%d steps=%d" % (dtype, d, B, H, steps))
    y, state = _run_gpu(inp, dev)
    ry, rs = oracle_lib.decode(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                               inp["s0"])
    gy = y.float().cpu().numpy()
    gs = state.cpu().numpy()
    assert np.all(np.isfinite(gy)) and np.all(np.isfinite(gs))
    slices = [(slice(None), b, h) for b in range(B) for h in range(H)]
    ey = _rel(gy, ry, slices)
    es = _rel(gs, rs, [(b, h) for b in range(B) for h in range(H)])
    say("    err y %.3e state %.3e" % (ey, es))
    assert ey <= TOL[dtype] and es <= TOL[dtype]


def test_decode_steps_equal_prefill(dev):
    """T decode steps of one sequence reproduce a T-token prefill of it."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    steps, B, H = 70, 1, 2
    inp = _decode_inputs(steps, B, H, 128, 128, "bf16", seed=32)
    y, state = _run_gpu(inp, dev)
    pre = dict(q=inp["q"][:, 0], k=inp["k"][:, 0], v=inp["v"][:, 0],
               alpha=inp["alpha"][:, 0], beta=inp["beta"][:, 0], s0=inp["s0"],
               cu_seqlens=np.array([0, steps], np.int32), lengths=np.array([steps]),
               num_seqs=1, H=H, dk=128, dv=128, dtype="bf16")
    py, ps = gpu_prefill(pre, dev)
    torch.cuda.synchronize()
    dy = (y[:, 0].float() - py.float()).abs().max().item() / py.float().abs().max().item()
    ds = (state - ps).abs().max().item() / ps.abs().max().item()
    say("    decode vs prefill: dy %.2e ds %.2e" % (dy, ds))
    assert dy <= 2e-2 and ds <= 2e-2


def test_decode_workload_full_size(dev, oracle_lib):
    """B=128, H=16, d=128, 1024 steps exactly as the benchmark launches them; the oracle
    follows every one of the 2,048 (sequence, head) pairs through all 1024 steps and every
    output and final state is compared."""
    from linear_attention_recurrence_chunked_amd import workloads as wl
    w = wl.DECODE
    say("[gpu] decode workload full size: generating inputs")
    d = wl.decode_inputs(w)
    y, state = _run_gpu(d, dev)
    gy = y.float().cpu().numpy()          # [steps, B, H, dv]
    gs = state.cpu().numpy()              # [B, H, dk, dv]
    assert np.all(np.isfinite(gy)) and np.all(np.isfinite(gs))
    say("[gpu] decode workload full size: oracle over all %d pairs" % (w.B * w.H))
    ry, rs = oracle_lib.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["s0"])
    # per (sequence, head): ||dy||_inf over all 1024 steps / ||y||_inf, and the final state
    dy = np.abs(gy - ry).max(axis=(0, 3))
    ny = np.abs(ry).max(axis=(0, 3))
    ds = np.abs(gs - rs).max(axis=(2, 3))
    ns = np.abs(rs).max(axis=(2, 3))
    ey = dy / np.where(ny > 0, ny, 1.0)
    es = ds / np.where(ns > 0, ns, 1.0)
    worst_y = float("nan") if np.isnan(ey).any() else float(ey.max())
    worst_s = float("nan") if np.isnan(es).any() else float(es.max())
    say("    err y %.3e state %.3e over %d pairs" % (worst_y, worst_s, ey.size))
    assert worst_y <= 2e-2 and worst_s <= 2e-2

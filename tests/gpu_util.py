"""Helpers for the GPU parity tests: run the HIP path on generated inputs and measure the
error against the fp64 oracle (test code only)."""
from __future__ import annotations

import sys
import time

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_inputs(inp: dict, dev):
    import torch
    from linear_attention_recurrence_chunked_amd import workloads as wl
    dt = inp["dtype"]
    out = {n: wl.to_torch(inp[n], dev, dt) for n in ("q", "k", "v")}
    out["alpha"] = torch.from_numpy(inp["alpha"]).to(dev)
    out["beta"] = torch.from_numpy(inp["beta"]).to(dev)
    out["s0"] = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).to(dev)
    out["cu"] = None if inp["cu_seqlens"] is None else torch.from_numpy(
        inp["cu_seqlens"]).to(dev)
    return out


def gpu_prefill(inp: dict, dev, dv_tile=0, segment_chunks=0, want_state=True):
    """Run gdn_prefill on the inputs; returns torch (y, final_state) on the device."""
    from linear_attention_recurrence_chunked_amd import gdn
    t = torch_inputs(inp, dev)
    y, sf = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                            initial_state=t["s0"], cu_seqlens=t["cu"],
                            num_seqs=inp["num_seqs"], dv_tile=dv_tile,
                            segment_chunks=segment_chunks, want_final_state=want_state)
    return y, sf


def cu_of(inp: dict) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(inp["lengths"])]).astype(np.int64)


def slice_rel_err(got_y, ref_y, cu, heads=None):
    """Max over (sequence, head) slices of ||got - ref||_inf / ||ref||_inf (y arrays
    [rows, nh, dv]).  Empty slices are skipped."""
    worst = 0.0
    nh = ref_y.shape[1]
    for n in range(len(cu) - 1):
        r0, r1 = int(cu[n]), int(cu[n + 1])
        if r1 == r0:
            continue
        for h in range(nh):
            ref = ref_y[r0:r1, h]
            den = float(np.max(np.abs(ref)))
            err = float(np.max(np.abs(got_y[r0:r1, h] - ref)))
            e = err / den if den > 0 else err
            if e != e or (worst == worst and e > worst):   # a NaN stays (max() would drop it)
                worst = e
    return worst


def state_rel_err(got_s, ref_s):
    """Max over (sequence, head) of ||got - ref||_inf / ||ref||_inf for [N, nh, dk, dv]."""
    worst = 0.0
    for n in range(ref_s.shape[0]):
        for h in range(ref_s.shape[1]):
            ref = ref_s[n, h]
            den = float(np.max(np.abs(ref)))
            err = float(np.max(np.abs(got_s[n, h] - ref)))
            e = err / den if den > 0 else err
            if e != e or (worst == worst and e > worst):   # a NaN stays (max() would drop it)
                worst = e
    return worst


def check_prefill(inp: dict, dev, oracle, tol=None, dv_tile=0, segment_chunks=0,
                  label="", threads=16):
    """GPU prefill vs the oracle on every (sequence, head); returns (err_y, err_state)."""
    import torch
    tol = TOL[inp["dtype"]] if tol is None else tol
    say("[gpu] prefill %s tile=%s seg=%s lengths=%s H=%d dk=%d dv=%d %s" % (
        label, dv_tile, segment_chunks, list(inp["lengths"][:8]), inp["H"], inp["dk"],
        inp["dv"], inp["dtype"]))
    y, sf = gpu_prefill(inp, dev, dv_tile, segment_chunks)
    torch.cuda.synchronize()
    gy = y.float().cpu().numpy()
    gs = sf.cpu().numpy()
    t0 = time.time()
    ry, rs = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                            cu_of(inp), s0=inp["s0"], threads=threads)
    cu = cu_of(inp)
    ey = slice_rel_err(gy, ry, cu)
    es = state_rel_err(gs, rs)
    say("    err y %.3e  state %.3e  (oracle %.1fs)" % (ey, es, time.time() - t0))
    assert np.all(np.isfinite(gy)) and np.all(np.isfinite(gs))
    assert ey <= tol, "y error %.3e > %.1e" % (ey, tol)
    assert es <= tol, "state error %.3e > %.1e" % (es, tol)
    return ey, es

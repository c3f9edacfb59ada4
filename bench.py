"""Benchmark of the gated delta rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  ``value`` is prefill throughput (tokens/s) on the B=4, H=16,
T=4096, d=128 bf16 workload with inputs resident in HBM; the decode step on B=128, H=16,
d=128 (1024 successive steps) is reported in the ``decode`` object.  Timing uses HIP events
on the stream the library launches on.  The fp64 oracle is timed on the host cores as a
baseline (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s (MFMA %) + decode steps/s at B=128 (HBM GB/s %)"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
# fp32 vector peak without packed instructions (every HIP file is built with packed fp32 off):
# 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP per FMA x 2.4 GHz = 78.6 TFLOP/s (the packed rate,
# 157.3 TFLOP/s, is out of reach of this build)
PEAK_FP32_VALU_TFLOPS = 78.6
CHUNK = 64


def prefill_flops_per_token_head(d: int, C: int = CHUNK) -> int:
    # dense-tile count of the chunked form: K K^T, Q K^T, the solve-side products T.K, T.V,
    # P.U (five C-sized products) and W.S, Q.S, K^T.U (three d-sized products)
    return 2 * d * (5 * C + 3 * d)


def backward_flops_per_token_head(d: int, C: int = CHUNK) -> int:
    """Dense-tile FLOPs of the chunked backward per token-head, each distinct product once:
    K K^T and Q K^T (4Cd); the forward state pass K S, T' R, K^T U (4d^2 + 2Cd); the adjoint
    pass P^T dY, K D, T'^T dU, L^T Z, Q^T dY, K^T Z (6d^2 + 6Cd); dY U^T and E U^T (4Cd);
    dY S^T, Z S^T, U D^T (6d^2); the four c x c by c x d products of dQ and dK (8Cd)."""
    return 24 * C * d + 16 * d * d


def backward_bytes(T: int, H: int, d: int, nseq: int) -> int:
    """Algorithmic HBM bytes of one backward call (bf16 activations): q, k, v, dy read and dq,
    dk, dv written (2 bytes each), alpha and beta read and dalpha, dbeta written (fp32), dS0
    written (fp32)."""
    return 7 * T * H * d * 2 + 4 * T * H * 4 + nseq * H * d * d * 4


def prefill_bytes(T: int, H: int, d: int, nseq: int) -> int:
    # q, k, v, y (bf16), alpha, beta (fp32), final state (fp32)
    return T * H * (4 * d * 2 + 2 * 4) + nseq * H * d * d * 4


def decode_bytes_per_head_step(d: int) -> int:
    # state read + write (fp32), q, k, v (bf16), alpha, beta (fp32), y (bf16)
    return 2 * d * d * 4 + 3 * d * 2 + 2 * 4 + d * 2


CSRC = os.path.join(ROOT, "linear_attention_recurrence_chunked_amd", "csrc")
PREFILL_SOURCES = ["gdn_device.hpp", "gdn_internal.hpp", "gdn_prefill_common.hpp",
                   "gdn_split_bf16.hpp", "gdn_prefill_ops.hpp", "gdn_prefill.hip",
                   "gdn_prefill_split.hip", "gdn_prefill_wide.hip"]
DECODE_SOURCES = ["gdn_device.hpp", "gdn_decode.hip"]
CHANNEL_SOURCES = ["gdn_device.hpp", "gdn_internal.hpp", "gdn_channel.hip"]
QSA_SOURCES = ["gdn_device.hpp", "gdn_internal.hpp", "gdn_qsa.hip"]
BACKWARD_SOURCES = ["gdn_device.hpp", "gdn_internal.hpp", "gdn_split_bf16.hpp",
                    "gdn_backward.hip"]


def sha_of(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_sha") != sha_of(sources):
        return None
    return ent


def profile_run(torch, gdn, wl, dev):
    """Three prefill launches, three decode steps, three backward calls, three channel-gated
    prefills and decode steps, three indexer calls, two prefills of each of the long and the
    mixed-length workloads and a 1 GiB elementwise pass, untimed."""
    import numpy as np
    inp = wl.workload_inputs(wl.PREFILL)
    q, k, v = (wl.to_torch(inp[n], dev, "bf16") for n in ("q", "k", "v"))
    a = torch.from_numpy(inp["alpha"]).to(dev)
    b = torch.from_numpy(inp["beta"]).to(dev)
    for _ in range(3):
        gdn.gdn_prefill(q, k, v, a, b, num_seqs=wl.PREFILL.B)
    d = wl.decode_inputs(wl.DECODE, steps=3)
    state = torch.from_numpy(d["s0"]).to(dev)
    for s in range(3):
        gdn.gdn_decode_step(wl.to_torch(d["q"][s], dev, "bf16"), wl.to_torch(d["k"][s], dev, "bf16"),
                            wl.to_torch(d["v"][s], dev, "bf16"), torch.from_numpy(d["alpha"][s]).to(dev),
                            torch.from_numpy(d["beta"][s]).to(dev), state)
    adj = wl.backward_inputs(inp, None, seed=2)
    dy = wl.to_torch(adj["dy"], dev, "bf16")
    for _ in range(3):
        gdn.gdn_prefill_backward(q, k, v, a, b, dy, num_seqs=wl.PREFILL.B)
    del dy
    # the channel-gated variant at the prefill shape, and three of its decode steps
    cg = wl.channel_gates(inp, seed=2)
    ca, cb, cw = (torch.from_numpy(cg[n]).to(dev) for n in ("decay", "erase", "write"))
    for _ in range(3):
        gdn.gdn_channel_gated(q, k, v, ca, cb, cw, num_seqs=wl.PREFILL.B)
    del ca, cb, cw, cg
    B, H, dh = wl.DECODE.B, wl.DECODE.H, wl.DECODE.dk
    dg = wl.channel_gates({"q": np.empty((B, 1, 1)), "H": H, "dk": dh, "dv": dh}, seed=3)
    dga, dgb, dgw = (torch.from_numpy(dg[n]).to(dev) for n in ("decay", "erase", "write"))
    for s in range(3):
        gdn.gdn_channel_gated(wl.to_torch(d["q"][s], dev, "bf16"), wl.to_torch(d["k"][s], dev, "bf16"),
                              wl.to_torch(d["v"][s], dev, "bf16"), dga, dgb, dgw,
                              initial_state=state, num_seqs=B, final_state=state)
    del dga, dgb, dgw
    # the sparse-attention indexer over one sequence of 65,536 tokens, budget 512 blocks
    qi = wl.qsa_inputs(65536, "bf16", seed=2)
    iq, ik = wl.to_torch(qi["q"], dev, "bf16"), wl.to_torch(qi["k"], dev, "bf16")
    for _ in range(3):
        gdn.gdn_qsa_index(iq, ik, block_budget=512, want_blocks=False)
    del iq, ik, qi
    # the 2^20-token sequence and the 32 mixed-length sequences, two prefills each (in that
    # order: the one-launch scan's dispatches of the long workload come first)
    for wobj in (wl.LONG, wl.VARLEN):
        wi = wl.workload_inputs(wobj)
        tq, tk, tv = (wl.to_torch(wi[n], dev, "bf16") for n in ("q", "k", "v"))
        ta, tb = (torch.from_numpy(wi[n]).to(dev) for n in ("alpha", "beta"))
        ts0 = None if wi["s0"] is None else torch.from_numpy(wi["s0"]).to(dev)
        tcu = None if wi["cu_seqlens"] is None else torch.from_numpy(wi["cu_seqlens"]).to(dev)
        n_s = wi["num_seqs"]
        del wi
        for _ in range(2):
            gdn.gdn_prefill(tq, tk, tv, ta, tb, initial_state=ts0, cu_seqlens=tcu, num_seqs=n_s)
        torch.cuda.synchronize()
        del tq, tk, tv, ta, tb, ts0, tcu
        torch.cuda.empty_cache()
    torch.cuda.synchronize()
    # calibration: an elementwise kernel that reads 1 GiB and writes 1 GiB
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print("profile run done", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-layer-steps", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-channel", action="store_true")
    ap.add_argument("--no-qsa", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 2^20-token single-sequence prefill")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the 32-sequence packed prefill")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3 counter passes: 3 prefill launches, 3 decode "
                         "steps and an elementwise kernel over 1 GiB (the calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_recurrence_chunked_amd import gdn
    from linear_attention_recurrence_chunked_amd import workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    gdn.load()
    if args.profile:
        profile_run(torch, gdn, wl, dev)
        return

    # ------------------------------------------------------------------ prefill
    w = wl.PREFILL
    t0 = time.time()
    inp = wl.workload_inputs(w)
    print("[bench] prefill inputs generated in %.1fs" % (time.time() - t0), file=sys.stderr,
          flush=True)
    q = wl.to_torch(inp["q"], dev, "bf16")
    k = wl.to_torch(inp["k"], dev, "bf16")
    v = wl.to_torch(inp["v"], dev, "bf16")
    alpha = torch.from_numpy(inp["alpha"]).to(dev)
    beta = torch.from_numpy(inp["beta"]).to(dev)
    T, H, d = q.shape
    nseq = w.B
    y = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    sf = torch.empty((nseq, H, d, d), dtype=torch.float32, device=dev)
    tile, seg = gdn.gdn_prefill_plan(nseq, T, H, d, d, gdn.GDN_DTYPE_BF16)
    need = gdn.gdn_prefill_workspace_bytes(nseq, T, H, d, d, gdn.GDN_DTYPE_BF16)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush_r = torch.ones(128 << 20, dtype=torch.float32, device=dev)     # 512 MiB

    def cache_flush():
        # write 512 MiB, then read another 512 MiB: the read evicts the dirty lines the write
        # left in L2 and the MALL, so the timed call starts with cold caches and no pending
        # write-back of unrelated data
        flush.fill_(1)
        flush_r.sum()

    def run_prefill():
        gdn.gdn_prefill(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None,
                        num_seqs=nseq, y=y, final_state=sf, workspace=ws if need else None)

    def time_output_gated(tq, tk, tv, ta, tb, ts0, tcu, n_s, ty, tsf, reps):
        """The prefill with the layer's output gate: the fused entry point against the prefill
        followed by the output-gate kernel, each call timed after a cache flush (z: seeded
        N(0, 4) bf16, weight: seeded N(0, 0.01))."""
        TT, HH, dd_ = tq.shape
        g = torch.Generator(device=dev)
        g.manual_seed(1234)
        tz = (2.0 * torch.randn((TT, HH, dd_), generator=g, device=dev)).to(torch.bfloat16)
        tw = 0.1 * torch.randn((dd_,), generator=g, device=dev)
        ptile, pseg = gdn.gdn_prefill_plan(n_s, TT, HH, dd_, dd_, gdn.GDN_DTYPE_BF16)
        wneed = gdn.gdn_prefill_workspace_bytes(n_s, TT, HH, dd_, dd_, gdn.GDN_DTYPE_BF16)
        tws = torch.empty(max(wneed, 16), dtype=torch.uint8, device=dev)

        def fused():
            gdn.gdn_prefill_output_gated(tq, tk, tv, ta, tb, tz, tw, 1e-6, initial_state=ts0,
                                         cu_seqlens=tcu, num_seqs=n_s, out=ty, final_state=tsf,
                                         workspace=tws if wneed else None)

        def composed():
            gdn.gdn_prefill(tq, tk, tv, ta, tb, initial_state=ts0, cu_seqlens=tcu,
                            num_seqs=n_s, y=ty, final_state=tsf,
                            workspace=tws if wneed else None)
            gdn.gdn_output_gate(ty, tz, tw, eps=1e-6, out=ty)

        res = {}
        for name, f in (("ms_fused_call", fused), ("ms_prefill_then_output_gate", composed)):
            f()
            torch.cuda.synchronize()
            ts_ = []
            for _ in range(reps):
                cache_flush()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                f()
                e1.record(stream)
                torch.cuda.synchronize()
                ts_.append(e0.elapsed_time(e1))
            res[name] = round(float(np.median(ts_)), 4)
        res["gate_applied"] = ("as each row of y leaves the one-launch scan" if ptile == 128
                               else "by the output-gate kernel after the prefill")
        del tz, tw, tws
        return res

    for _ in range(args.warmup):
        run_prefill()
    torch.cuda.synchronize()

    # cold-cache timing: the caches are flushed between launches, outside the events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for e0, e1 in evs:
        if not args.no_flush:
            cache_flush()
        e0.record(stream)
        run_prefill()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    times_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    pre_ms = float(np.mean(times_ms))
    pre_med = float(np.median(times_ms))

    # warm back-to-back timing
    ew0, ew1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ew0.record(stream)
    for _ in range(args.steps):
        run_prefill()
    ew1.record(stream)
    torch.cuda.synchronize()
    warm_ms = ew0.elapsed_time(ew1) / args.steps

    # the same calls after a write-only flush, whose dirty lines are written back during the
    # timed call (for comparison with the flush above)
    wo = []
    for _ in range(args.steps):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_prefill()
        e1.record(stream)
        torch.cuda.synchronize()
        wo.append(e0.elapsed_time(e1))
    wo_med = float(np.median(wo))

    # bf16 prefill = two launches: chunk records, then the state scan; the roofline covers
    # the pair (HIP events around the library call); rocprofv3 splits it per kernel
    if tile == 128 and d == 128:
        kernel_name = "wide_scan_kernel<128,128>"
        if seg >= 0:
            kernel_name = "segment_table_kernel + " + kernel_name
    elif tile <= 32:
        kernel_name = "chunk_prep_kernel<128> + scan_pipe_kernel<128,%d>" % tile
    elif tile <= 64:
        kernel_name = "chunk_prep_kernel<128> + scan_split_kernel<128,%d,scan>" % tile
    else:
        kernel_name = "prefill_kernel<128,%d,bf16,scan>" % tile
    if seg >= 0 and tile != 128:
        kernel_name += " (+ segment phases)"
    tok_s = T / (pre_ms * 1e-3)
    flops = prefill_flops_per_token_head(d) * T * H
    achieved_tflops = flops / (pre_ms * 1e-3) / 1e12
    pbytes = prefill_bytes(T, H, d, nseq)
    tr = load_traffic("prefill_bf16_B4_H16_T4096_d128", PREFILL_SOURCES)
    roofline = {
        "bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": None if tr is None else tr["bytes_per_launch"],
        "kernel": kernel_name,
        "flops_per_launch": flops,
        "algorithmic_bytes_per_launch": pbytes,
        "hbm_frac_of_algorithmic_bytes": round(pbytes / (pre_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
    }

    og_main = time_output_gated(q, k, v, alpha, beta, None, None, nseq, y, sf, args.steps)

    # ------------------------------------------------------------------ other prefill shapes
    # the 2^20-token single sequence and the 32 packed sequences, each in the library's own
    # plan, timed call by call after a cache flush
    def time_workload(wobj, reps):
        t0 = time.time()
        wi = wl.workload_inputs(wobj)
        print("[bench] %s inputs generated in %.1fs" % (wobj.name, time.time() - t0),
              file=sys.stderr, flush=True)
        tq = wl.to_torch(wi["q"], dev, "bf16")
        tk = wl.to_torch(wi["k"], dev, "bf16")
        tv = wl.to_torch(wi["v"], dev, "bf16")
        ta = torch.from_numpy(wi["alpha"]).to(dev)
        tb = torch.from_numpy(wi["beta"]).to(dev)
        ts0 = None if wi["s0"] is None else torch.from_numpy(wi["s0"]).to(dev)
        tcu = None if wi["cu_seqlens"] is None else torch.from_numpy(wi["cu_seqlens"]).to(dev)
        n_s = wi["num_seqs"]
        TT, HH, dd_ = tq.shape
        del wi
        ty = torch.empty((TT, HH, dd_), dtype=torch.bfloat16, device=dev)
        tsf = torch.empty((n_s, HH, dd_, dd_), dtype=torch.float32, device=dev)
        ptile, pseg = gdn.gdn_prefill_plan(n_s, TT, HH, dd_, dd_, gdn.GDN_DTYPE_BF16)
        wneed = gdn.gdn_prefill_workspace_bytes(n_s, TT, HH, dd_, dd_, gdn.GDN_DTYPE_BF16)
        tws = torch.empty(max(wneed, 16), dtype=torch.uint8, device=dev)

        def call():
            gdn.gdn_prefill(tq, tk, tv, ta, tb, initial_state=ts0, cu_seqlens=tcu,
                            num_seqs=n_s, y=ty, final_state=tsf,
                            workspace=tws if wneed else None)

        # three untimed calls first: the clock of a GPU that has been idle or running short
        # kernels takes a few milliseconds of this load to rise
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            cache_flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        fl = prefill_flops_per_token_head(dd_) * TT * HH
        tf = fl / (ms * 1e-3) / 1e12
        nb = prefill_bytes(TT, HH, dd_, n_s) + (0 if ts0 is None else n_s * HH * dd_ * dd_ * 4)
        trk = load_traffic(wobj.name, PREFILL_SOURCES)
        res = {"workload": wobj.name, "tokens": TT, "sequences": n_s,
               "dv_tile": ptile, "segment_chunks": pseg, "ms_median": round(ms, 4),
               "ms_all": [round(x, 4) for x in times],
               "tokens_per_s": round(TT / (ms * 1e-3), 1),
               "flops_per_launch": fl,
               "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                            "traffic": None if trk is None else trk["bytes_per_launch"]},
               "algorithmic_bytes_per_launch": nb,
               "hbm_frac_of_algorithmic_bytes": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del tws
        res["output_gated"] = time_output_gated(tq, tk, tv, ta, tb, ts0, tcu, n_s, ty, tsf,
                                                reps)
        del tq, tk, tv, ta, tb, ts0, tcu, ty, tsf
        torch.cuda.empty_cache()
        return res

    long_obj = None if args.no_long else time_workload(wl.LONG, 5)
    varlen_obj = None if args.no_varlen else time_workload(wl.VARLEN, 10)

    # ------------------------------------------------------------------ decode
    wd = wl.DECODE
    nsteps = args.decode_steps
    t0 = time.time()
    dd = wl.decode_inputs(wd, steps=nsteps)
    print("[bench] decode inputs generated in %.1fs" % (time.time() - t0), file=sys.stderr,
          flush=True)
    dq = wl.to_torch(dd["q"], dev, "bf16")
    dk_ = wl.to_torch(dd["k"], dev, "bf16")
    dv_ = wl.to_torch(dd["v"], dev, "bf16")
    da = torch.from_numpy(dd["alpha"]).to(dev)
    db = torch.from_numpy(dd["beta"]).to(dev)
    s0 = torch.from_numpy(dd["s0"]).to(dev)
    B, Hd, dh = wd.B, wd.H, wd.dk
    dy = torch.empty((nsteps, B, Hd, dh), dtype=torch.bfloat16, device=dev)
    state = s0.clone()

    def run_decode(states):
        for s in range(nsteps):
            gdn.gdn_decode_step(dq[s], dk_[s], dv_[s], da[s], db[s], states[s % len(states)],
                                y=dy[s])

    run_decode([state])          # warm-up pass over all steps
    state.copy_(s0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run_decode([state])
    e1.record(stream)
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) * 1e3 / nsteps
    # cache-defeating variant: four independent state sets (512 MiB) in rotation
    states4 = [s0.clone() for _ in range(4)]
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    run_decode(states4)
    e3.record(stream)
    torch.cuda.synchronize()
    dec4_us = e2.elapsed_time(e3) * 1e3 / nsteps
    dbytes = decode_bytes_per_head_step(dh) * B * Hd
    gbs = dbytes / (dec_us * 1e-6) / 1e9
    gbs4 = dbytes / (dec4_us * 1e-6) / 1e9
    # what a plain device copy reaches on the same traffic: torch's copy of one state set's
    # bytes (read once, written once), four source / destination pairs in rotation as above
    csrc = [torch.empty_like(s0).uniform_() for _ in range(4)]
    cdst = [torch.empty_like(s0) for _ in range(4)]
    for i in range(4):
        cdst[i].copy_(csrc[i])
    torch.cuda.synchronize()
    ncopy = 64
    e4, e5 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e4.record(stream)
    with torch.cuda.stream(stream):
        for i in range(ncopy):
            cdst[i % 4].copy_(csrc[i % 4])
    e5.record(stream)
    torch.cuda.synchronize()
    copy_us = e4.elapsed_time(e5) * 1e3 / ncopy
    copy_gbs = 2 * s0.numel() * 4 / (copy_us * 1e-6) / 1e9
    del csrc, cdst
    dtr = load_traffic("decode_bf16_B128_H16_d128", DECODE_SOURCES)
    # the roofline takes the rotating measurement: four state sets (512 MiB) exceed the
    # 256 MB MALL, so each step streams its state from and to HBM, as in a many-layer model
    decode = {
        "workload": wd.name, "steps": nsteps, "steps_per_s": round(1e6 / dec4_us, 1),
        "us_per_step": round(dec4_us, 2), "tokens_per_s": round(B * 1e6 / dec4_us, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs4, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs4 / PEAK_HBM_GBS, 4),
                     "traffic": None if dtr is None else dtr["bytes_per_launch"],
                     "algorithmic_bytes_per_launch": dbytes,
                     "measured_on": "4 state sets in rotation (512 MiB)"},
        "one_state_set": {"us_per_step": round(dec_us, 2),
                          "steps_per_s": round(1e6 / dec_us, 1),
                          "achieved_GBs": round(gbs, 1),
                          "frac": round(gbs / PEAK_HBM_GBS, 4)},
        "copy_reference": {"what": "torch copy_ of one state set's bytes (%d MB read, %d MB "
                                   "written), four pairs in rotation" % (
                                       s0.numel() * 4 // 10**6, s0.numel() * 4 // 10**6),
                           "us": round(copy_us, 2), "achieved_GBs": round(copy_gbs, 1),
                           "frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
                           "decode_frac_of_copy": round(gbs4 / copy_gbs, 4)},
    }

    # ------------------------------------------------------------------ layer steps
    # the steps either side of the rule at the prefill workload's shape (bf16, H*d = 2048
    # channels, conv width 4): each is one streaming pass, timed after a cache flush
    layer = None
    if not args.no_layer_steps:
        li = wl.layer_step_inputs([w.T] * nseq, H, d, 4, "bf16", seed=2)
        C = H * d
        lx = wl.to_torch(li["x_q"], dev, "bf16")
        lw = torch.from_numpy(li["w_q"]).to(dev)
        ls_in = torch.from_numpy(li["s_q"]).to(dev)
        ls_out = torch.empty_like(ls_in)
        lo = torch.empty_like(lx)
        la, lb = (torch.from_numpy(li[n]).to(dev) for n in ("a", "b"))
        lA, lba = (torch.from_numpy(li[n]).to(dev) for n in ("A", "b_alpha"))
        lal, lbe = torch.empty_like(la), torch.empty_like(la)
        ly, lz = wl.to_torch(li["y"], dev, "bf16"), wl.to_torch(li["z"], dev, "bf16")
        lnw = torch.from_numpy(li["norm_w"]).to(dev)
        lout = torch.empty_like(ly)
        e2b = T * C * 2
        steps_def = {
            "short_conv_silu_l2norm": (lambda: gdn.gdn_short_conv(
                lx, lw, num_seqs=nseq, head_dim=d, out=lo, state_in=ls_in, state_out=ls_out),
                2 * e2b + C * 4 * 4 + 2 * nseq * C * 3 * 4),
            "gates": (lambda: gdn.gdn_gates(la, lb, lA, lba, alpha=lal, beta=lbe),
                      4 * T * H * 4 + 2 * H * 4),
            "output_gate": (lambda: gdn.gdn_output_gate(ly, lz, lnw, out=lout),
                            3 * e2b + d * 4),
        }
        layer = {"workload": "bf16 T=%d (%d x %d) H=%d d=%d conv width 4" % (T, nseq, w.T, H, d)}
        for name, (fn, nbytes) in steps_def.items():
            for _ in range(3):
                fn()
            times = []
            for _ in range(10):
                cache_flush()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3)
            us = float(np.median(times))
            gb = nbytes / (us * 1e-6) / 1e9
            layer[name] = {"us": round(us, 2), "algorithmic_bytes": nbytes,
                           "achieved_GBs": round(gb, 1), "frac_of_hbm_peak": round(gb / PEAK_HBM_GBS, 4)}
        del lx, lo, ly, lz, lout

    # ------------------------------------------------------------------ backward
    # the chunked backward of the same prefill (dy ~ N(0, 1) bf16, zero final-state
    # adjoint), timed after a cache flush like the forward
    backward = None
    if not args.no_backward:
        adj = wl.backward_inputs(inp, None, seed=2)
        bdy = wl.to_torch(adj["dy"], dev, "bf16")
        bout = (torch.empty((T, H, d), dtype=torch.bfloat16, device=dev),
                torch.empty((T, H, d), dtype=torch.bfloat16, device=dev),
                torch.empty((T, H, d), dtype=torch.bfloat16, device=dev),
                torch.empty((T, H), dtype=torch.float32, device=dev),
                torch.empty((T, H), dtype=torch.float32, device=dev),
                torch.empty((nseq, H, d, d), dtype=torch.float32, device=dev))
        bneed = gdn.gdn_prefill_backward_workspace_bytes(nseq, T, H, d, d)
        bws = torch.empty(bneed, dtype=torch.uint8, device=dev)

        def run_backward():
            gdn.gdn_prefill_backward(q, k, v, alpha, beta, bdy, num_seqs=nseq, workspace=bws,
                                     out=bout)

        for _ in range(3):
            run_backward()
        times = []
        for _ in range(10):
            cache_flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_backward()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        bms = float(np.median(times))
        bflops = backward_flops_per_token_head(d) * T * H
        btf = bflops / (bms * 1e-3) / 1e12
        btr = load_traffic("backward_bf16_B4_H16_T4096_d128", BACKWARD_SOURCES)
        bbytes = backward_bytes(T, H, d, nseq)
        backward = {"workload": w.name, "ms_median": round(bms, 4),
                    "tokens_per_s": round(T / (bms * 1e-3), 1),
                    "flops_per_launch": bflops, "achieved_TFLOPs": round(btf, 2),
                    "frac_of_bf16_peak": round(btf / PEAK_BF16_TFLOPS, 4),
                    "workspace_bytes": bneed,
                    "algorithmic_bytes_per_launch": bbytes,
                    "traffic": None if btr is None else btr["bytes_per_launch"],
                    "kernels": "bwd_prep_kernel<128> + bwd_states_kernel<128,128> + "
                               "bwd_dstates_kernel<128,128> + bwd_chunk_kernel<128,128>"}
        del bws, bout, bdy

    # ------------------------------------------------------------------ channel-wise gates
    # the channel-gated variant (decay per key channel, erase and write gates per value
    # channel), token by token in fp32: at the prefill workload's shape, and as decode steps
    # (one token for each of 128 sequences) over four state sets in rotation
    chan = None
    if not args.no_channel:
        cg = wl.channel_gates(inp, seed=2)
        ca, cb, cw = (torch.from_numpy(cg[n]).to(dev) for n in ("decay", "erase", "write"))
        del cg
        cy = torch.empty_like(y)
        cs = torch.empty_like(sf)

        def run_chan():
            gdn.gdn_channel_gated(q, k, v, ca, cb, cw, num_seqs=nseq, y=cy, final_state=cs)

        for _ in range(2):
            run_chan()
        times = []
        for _ in range(5):
            cache_flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_chan()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        cms = float(np.median(times))
        cflops = 7 * d * d * T * H          # decay, retrieval, write and read-out per token-head
        ctf = cflops / (cms * 1e-3) / 1e12
        del ca, cb, cw, cy, cs
        ns = min(64, nsteps)         # decode steps of the channel-gated variant
        dg = wl.channel_gates({"q": np.empty((ns * B, 1, 1)), "H": Hd, "dk": dh, "dv": dh},
                              seed=3)
        dga, dgb, dgw = (torch.from_numpy(dg[n]).to(dev).view(ns, B, Hd, dh)
                         for n in ("decay", "erase", "write"))
        del dg
        cstates = [s0.clone() for _ in range(4)]
        cyd = torch.empty((B, Hd, dh), dtype=torch.bfloat16, device=dev)

        def run_chan_decode():
            for s in range(ns):
                st = cstates[s % 4]
                gdn.gdn_channel_gated(dq[s], dk_[s], dv_[s], dga[s], dgb[s], dgw[s],
                                      initial_state=st, num_seqs=B, y=cyd, final_state=st)

        run_chan_decode()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_chan_decode()
        e1.record(stream)
        torch.cuda.synchronize()
        cd_us = e0.elapsed_time(e1) * 1e3 / ns
        cdbytes = (2 * dh * dh * 4 + 4 * dh * 2 + 3 * dh * 4) * B * Hd
        cgbs = cdbytes / (cd_us * 1e-6) / 1e9
        ctr_p = load_traffic("channel_prefill_bf16_B4_H16_T4096_d128", CHANNEL_SOURCES)
        ctr_d = load_traffic("channel_decode_bf16_B128_H16_d128", CHANNEL_SOURCES)
        chan = {"kernel": "channel_gated_kernel<128, bf16>",
                "prefill": {"workload": w.name, "ms_median": round(cms, 4),
                            "tokens_per_s": round(T / (cms * 1e-3), 1),
                            "flops_per_launch": cflops,
                            "roofline": {"bound": "alu", "achieved": round(ctf, 2),
                                         "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                                         "frac": round(ctf / PEAK_FP32_VALU_TFLOPS, 4),
                                         "traffic": None if ctr_p is None else ctr_p["bytes_per_launch"]}},
                "decode": {"workload": "B=%d H=%d d=%d, %d steps over 4 state sets" % (B, Hd, dh, ns),
                           "us_per_step": round(cd_us, 2),
                           "algorithmic_bytes_per_launch": cdbytes,
                           "roofline": {"bound": "hbm", "achieved": round(cgbs, 1),
                                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                        "frac": round(cgbs / PEAK_HBM_GBS, 4),
                                        "traffic": None if ctr_d is None else ctr_d["bytes_per_launch"]}}}
        del dga, dgb, dgw, cstates

    # ------------------------------------------------------------------ sparse-attention indexer
    # one sequence of 65,536 tokens, 4 query heads and a key head of 128, budget 512 blocks:
    # normalise/rotate, then block scores and their selection in one streaming kernel; and
    # one sequence of 2^20 tokens (the length the pages time the indexer at)
    qsa_obj = None
    if not args.no_qsa:
        nq = 65536
        qi = wl.qsa_inputs(nq, "bf16", seed=2)
        iq = wl.to_torch(qi["q"], dev, "bf16")
        ik = wl.to_torch(qi["k"], dev, "bf16")
        del qi
        qws = torch.empty(gdn.gdn_qsa_workspace_bytes(nq), dtype=torch.uint8, device=dev)

        def run_qsa():
            return gdn.gdn_qsa_index(iq, ik, block_budget=512, want_blocks=False, workspace=qws)

        for _ in range(2):
            run_qsa()
        times = []
        for _ in range(5):
            cache_flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_qsa()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        qms = float(np.median(times))
        del qws

        def causal_pairs(n_):
            # sum over queries i of min((i + 1) // 4, n_ // 4) visible blocks
            nb_ = n_ // 4
            full = 2 * nb_ * (nb_ - 1) + nb_                # queries 0 .. 4 nb_ - 1
            return full + (n_ - 4 * nb_) * nb_

        pairs = causal_pairs(nq)
        qflops = pairs * 4 * 128 * 2
        # HBM bytes the method cannot avoid: inputs read, token lists written
        qbytes = nq * 5 * 128 * 2 + nq * (4 * 512 + 3) * 4
        # the same at 2^20 tokens: one warm-up and two timed calls
        nl = 1 << 20
        t0 = time.time()
        ql = wl.qsa_inputs(nl, "bf16", seed=3)
        lq, lk = wl.to_torch(ql["q"], dev, "bf16"), wl.to_torch(ql["k"], dev, "bf16")
        del ql
        print("[bench] qsa 2^20 inputs generated in %.1fs" % (time.time() - t0), file=sys.stderr,
              flush=True)
        lws = torch.empty(gdn.gdn_qsa_workspace_bytes(nl), dtype=torch.uint8, device=dev)
        ltok = torch.empty((nl, 4 * 512 + 3), dtype=torch.int32, device=dev)
        gdn.gdn_qsa_index(lq, lk, block_budget=512, want_blocks=False, workspace=lws, tokens=ltok)
        lt = []
        for _ in range(2):
            cache_flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            gdn.gdn_qsa_index(lq, lk, block_budget=512, want_blocks=False, workspace=lws,
                              tokens=ltok)
            e1.record(stream)
            torch.cuda.synchronize()
            lt.append(e0.elapsed_time(e1))
        lms = float(np.median(lt))
        lflops = causal_pairs(nl) * 4 * 128 * 2
        del lq, lk, lws, ltok
        torch.cuda.empty_cache()
        ctr_q = load_traffic("qsa_bf16_n65536_kb512", QSA_SOURCES)
        qsa_obj = {"workload": "one sequence of %d tokens, 4 query heads, d=128, blocks of 4, "
                               "budget 512 blocks" % nq,
                   "ms_median": round(qms, 4), "queries_per_s": round(nq / (qms * 1e-3), 1),
                   "score_flops": qflops,
                   "score_TFLOPs": round(qflops / (qms * 1e-3) / 1e12, 2),
                   "frac_of_bf16_peak": round(qflops / (qms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "algorithmic_bytes": qbytes,
                   "traffic": None if ctr_q is None else ctr_q["bytes_per_launch"],
                   "workspace_bytes": gdn.gdn_qsa_workspace_bytes(nq),
                   "kernels": "qsa_prep_kernel + qsa_select_kernel<16>",
                   "tokens_2p20": {"n": nl, "ms_median": round(lms, 3),
                                   "ms_all": [round(x, 3) for x in lt],
                                   "score_flops": lflops,
                                   "score_TFLOPs": round(lflops / (lms * 1e-3) / 1e12, 2),
                                   "frac_of_bf16_peak": round(lflops / (lms * 1e-3) / 1e12 /
                                                              PEAK_BF16_TFLOPS, 4)}}
        del iq, ik

    # ------------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        nproc = os.cpu_count() or 1
        try:
            avail = len(os.sched_getaffinity(0))
        except AttributeError:
            avail = nproc
        omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
        units = nseq * H
        # one thread per independent (sequence, head) chain, within the cores this process
        # may use (and OMP_NUM_THREADS where the host sets a share)
        use = max(1, min(avail, units, omp if omp > 0 else avail))
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        # whole passes over the workload until at least 10 s of host time (at most 40 passes)
        reps = 0
        c0 = time.perf_counter()
        while True:
            oracle.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None,
                           threads=use, want_y=True, want_state=True)
            reps += 1
            csec = time.perf_counter() - c0
            if csec >= 10.0 or reps >= 40:
                break
        cpu = {"value": round(reps * T / csec, 1), "unit": "tokens/s", "cores": use,
               "kind": "oracle",
               "sample": "%d whole passes over the prefill workload (B=4, H=16, T=4096, d=128), "
                         "fp64 C oracle, %d threads, %.1f s" % (reps, use, csec),
               "nproc": nproc, "cpus_available": avail, "cpu_model": model,
               "independent_units": units}

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": H, "T": w.T, "d_k": d, "d_v": d,
                   "chunk": CHUNK, "dv_tile": tile, "segment_chunks": seg,
                   "parallelism": "single GPU"},
        "prefill": {"ms_median": round(pre_med, 4), "ms_warm_back_to_back": round(warm_ms, 4),
                    "ms_median_after_write_only_flush": round(wo_med, 4),
                    "tokens_per_s_warm": round(T / (warm_ms * 1e-3), 1),
                    "wall_s_timed_loop_incl_flush": round(wall, 4),
                    "output_gated": og_main},
        "roofline": roofline,
        "long_prefill": long_obj,
        "varlen_prefill": varlen_obj,
        "decode": decode,
        "layer_steps": layer,
        "backward": backward,
        "channel_gated": chan,
        "qsa_indexer": qsa_obj,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs for the gated delta rule workloads.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic.  Both the HIP path (through the tests and the benchmark) and the fp64 oracle
take their inputs from here, so the two sides always see bit-identical values.

Recipe (shared by every workload):

* a generator ``numpy.random.default_rng([seed, tensor_id, block])`` per tensor and per
  block of 65,536 packed rows, so large inputs can be drawn block by block, in parallel,
  with a result that does not depend on the order;
* q, k ~ N(0, 1) drawn in fp64, L2-normalised per (row, head) in fp64 (the feature map
  normalises q and k before the recurrence), then rounded once to the storage dtype
  (fp32, or bf16 with round-to-nearest-even);
* v ~ N(0, 1), rounded the same way;
* alpha = sigmoid(N(mu_a, sd_a)) and beta = sigmoid(N(mu_b, sd_b)) in fp64, stored fp32;
* optional initial state S0 ~ N(0, sd_s0) fp32 per (sequence, head);
* variable lengths are integers uniform in [lo, hi], both ends included;
* for the backward: the output adjoint dy ~ N(0, 1) in the storage dtype, and an optional
  final-state adjoint ~ N(0, sd) fp32 per (sequence, head);
* for the channel-wise gated variants: a decay per key channel sigmoid(N(mu_a, sd_a)) and
  erase and write gates per value channel sigmoid(N(mu_b, sd_b)), fp32;
* for the sparse-attention indexer: projected queries [n, 4, 128] and keys [n, 128], N(0, 1)
  in the storage dtype.

bf16 tensors are handled as ``uint16`` bit patterns on the numpy side and viewed as
``torch.bfloat16`` when moved to the GPU.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

BLOCK_ROWS = 65536
T_Q, T_K, T_V, T_ALPHA, T_BETA, T_S0, T_LENS, T_DY, T_DSF, T_CA, T_CB, T_CW, T_IQ, T_IK = range(14)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtypes and value distributions."""
    name: str
    kind: str                      # "prefill" or "decode"
    H: int
    dk: int
    dv: int
    dtype: str                     # "f32" or "bf16" (q, k, v and y)
    alpha: Tuple[float, float]     # (mu, sd) of the pre-sigmoid normal
    beta: Tuple[float, float]
    seed: int
    B: int = 1                     # equal-length sequences (prefill) / batch (decode)
    T: int = 0                     # tokens per sequence (equal-length prefill)
    lengths: Optional[Tuple[int, int, int]] = None   # (count, lo, hi) for packed varlen
    s0_sd: Optional[float] = None  # None = no initial state (zeros)
    steps: int = 0                 # decode steps
    extra: dict = field(default_factory=dict, compare=False, hash=False)


# The five workloads.  Shapes and distributions follow the task's configuration list;
# seeds are the workload number.
TINY = Workload("tiny_fp32_B1_H2_T256_d64", "prefill", H=2, dk=64, dv=64, dtype="f32",
                alpha=(3.0, 1.0), beta=(0.0, 1.0), seed=1, B=1, T=256)
PREFILL = Workload("prefill_bf16_B4_H16_T4096_d128", "prefill", H=16, dk=128, dv=128,
                   dtype="bf16", alpha=(3.0, 1.0), beta=(0.0, 1.0), seed=2, B=4, T=4096)
DECODE = Workload("decode_bf16_B128_H16_d128_1024steps", "decode", H=16, dk=128, dv=128,
                  dtype="bf16", alpha=(3.0, 1.0), beta=(0.0, 1.0), seed=3, B=128,
                  s0_sd=0.02, steps=1024)
LONG = Workload("long_bf16_B1_H16_T1048576_d128", "prefill", H=16, dk=128, dv=128,
                dtype="bf16", alpha=(4.0, 1.0), beta=(0.0, 1.0), seed=4, B=1, T=1 << 20)
VARLEN = Workload("varlen_bf16_32seqs_512to16384_H16_d128", "prefill", H=16, dk=128, dv=128,
                  dtype="bf16", alpha=(1.0, 2.0), beta=(0.0, 1.5), seed=5,
                  lengths=(32, 512, 16384), s0_sd=0.02)

WORKLOADS = {1: TINY, 2: PREFILL, 3: DECODE, 4: LONG, 5: VARLEN}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (round to nearest, ties to even) and return the uint16 bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f64":
        return x
    raise ValueError(dtype)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _rows_blocks(rows: int):
    return [(b, b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS))
            for b in range((rows + BLOCK_ROWS - 1) // BLOCK_ROWS)]


def _fill(out: np.ndarray, seed: int, tid: int, fn):
    """Fill out[r0:r1] block by block with fn(rng, n_rows) in parallel threads."""
    rows = out.shape[0]

    def work(blk):
        b, r0, r1 = blk
        rng = np.random.default_rng([seed, tid, b])
        out[r0:r1] = fn(rng, r1 - r0)

    blocks = _rows_blocks(rows)
    if len(blocks) == 1:
        work(blocks[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, blocks))


def draw_qk(rows: int, H: int, d: int, dtype: str, seed: int, tid: int) -> np.ndarray:
    out = np.empty((rows, H, d), dtype=np.uint16 if dtype == "bf16" else
                   (np.float32 if dtype == "f32" else np.float64))

    def fn(rng, n):
        x = rng.standard_normal((n, H, d))
        x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return _store(x, dtype)

    _fill(out, seed, tid, fn)
    return out


def draw_v(rows: int, H: int, d: int, dtype: str, seed: int, tid: int = T_V) -> np.ndarray:
    out = np.empty((rows, H, d), dtype=np.uint16 if dtype == "bf16" else
                   (np.float32 if dtype == "f32" else np.float64))
    _fill(out, seed, tid, lambda rng, n: _store(rng.standard_normal((n, H, d)), dtype))
    return out


def draw_gate(rows: int, H: int, mu: float, sd: float, seed: int, tid: int) -> np.ndarray:
    out = np.empty((rows, H), dtype=np.float32)
    _fill(out, seed, tid,
          lambda rng, n: _sigmoid(mu + sd * rng.standard_normal((n, H))).astype(np.float32))
    return out


def draw_lengths(count: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, T_LENS, 0])
    return rng.integers(lo, hi, size=count, endpoint=True).astype(np.int64)


def draw_s0(nseq: int, H: int, dk: int, dv: int, sd: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, T_S0, 0])
    return (sd * rng.standard_normal((nseq, H, dk, dv))).astype(np.float32)


def make_inputs(lengths, H: int, dk: int, dv: int, dtype: str, alpha=(3.0, 1.0),
                beta=(0.0, 1.0), s0_sd: Optional[float] = None, seed: int = 0,
                varlen: bool = True) -> dict:
    """Packed prefill inputs for the given per-sequence lengths.

    Returns numpy arrays: q, k [rows, H, dk]; v [rows, H, dv] (uint16 bf16 bits, float32 or
    float64); alpha, beta [rows, H] float32; s0 [N, H, dk, dv] float32 or None;
    cu_seqlens [N+1] int32 (None when ``varlen`` is False: N equal sequences).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    rows = int(cu[-1])
    inp = dict(
        q=draw_qk(rows, H, dk, dtype, seed, T_Q),
        k=draw_qk(rows, H, dk, dtype, seed, T_K),
        v=draw_v(rows, H, dv, dtype, seed),
        alpha=draw_gate(rows, H, alpha[0], alpha[1], seed, T_ALPHA),
        beta=draw_gate(rows, H, beta[0], beta[1], seed, T_BETA),
        s0=None if s0_sd is None else draw_s0(len(lengths), H, dk, dv, s0_sd, seed),
        cu_seqlens=cu.astype(np.int32) if varlen else None,
        lengths=lengths, num_seqs=len(lengths), H=H, dk=dk, dv=dv, dtype=dtype)
    return inp


def backward_inputs(inp: dict, ds_sd: Optional[float] = 0.02, seed: int = 0) -> dict:
    """Adjoints for the backward of the prefill ``inp``: dy [rows, H, dv] in inp's dtype and
    d_final_state [N, H, dk, dv] fp32 (None when ``ds_sd`` is None)."""
    rows = int(inp["q"].shape[0])
    dy = draw_v(rows, inp["H"], inp["dv"], inp["dtype"], seed, T_DY)
    dsf = None
    if ds_sd is not None:
        rng = np.random.default_rng([seed, T_DSF, 0])
        dsf = (ds_sd * rng.standard_normal((inp["num_seqs"], inp["H"], inp["dk"],
                                            inp["dv"]))).astype(np.float32)
    return dict(dy=dy, ds_final=dsf)


def channel_gates(inp: dict, a=(3.0, 1.0), b=(0.0, 1.0), seed: int = 0) -> dict:
    """Channel-wise gates for the prefill ``inp``: decay [rows, H, dk], erase and write
    [rows, H, dv], fp32."""
    rows, H, dk, dv = int(inp["q"].shape[0]), inp["H"], inp["dk"], inp["dv"]

    def draw(tid, d, mu, sd):
        out = np.empty((rows, H, d), dtype=np.float32)
        _fill(out, seed, tid, lambda rng, n: _sigmoid(mu + sd * rng.standard_normal((n, H, d))).astype(np.float32))
        return out

    return dict(decay=draw(T_CA, dk, *a), erase=draw(T_CB, dv, *b), write=draw(T_CW, dv, *b))


def qsa_inputs(n: int, dtype: str = "bf16", seed: int = 0) -> dict:
    """Indexer inputs for one sequence of n tokens: q [n, 4, 128], k [n, 128]."""
    q = np.empty((n, 4, 128), dtype=np.uint16 if dtype == "bf16" else np.float32)
    k = np.empty((n, 128), dtype=q.dtype)
    _fill(q, seed, T_IQ, lambda rng, m: _store(rng.standard_normal((m, 4, 128)), dtype))
    _fill(k, seed, T_IK, lambda rng, m: _store(rng.standard_normal((m, 128)), dtype))
    return dict(q=q, k=k, n=n, dtype=dtype)


def workload_inputs(w: Workload) -> dict:
    """Inputs of a prefill workload (equal-length or packed varlen)."""
    if w.kind != "prefill":
        raise ValueError("use decode_inputs for decode workloads")
    if w.lengths is not None:
        count, lo, hi = w.lengths
        lens = draw_lengths(count, lo, hi, w.seed)
        return make_inputs(lens, w.H, w.dk, w.dv, w.dtype, w.alpha, w.beta, w.s0_sd, w.seed,
                           varlen=True)
    return make_inputs([w.T] * w.B, w.H, w.dk, w.dv, w.dtype, w.alpha, w.beta, w.s0_sd,
                       w.seed, varlen=False)


def decode_inputs(w: Workload, steps: Optional[int] = None, B: Optional[int] = None) -> dict:
    """Inputs of a decode workload: per-step q, k, v [steps, B, H, d], gates [steps, B, H],
    and the initial state [B, H, dk, dv]."""
    steps = w.steps if steps is None else steps
    B = w.B if B is None else B
    rows = steps * B
    H, dk, dv = w.H, w.dk, w.dv
    q = draw_qk(rows, H, dk, w.dtype, w.seed, T_Q).reshape(steps, B, H, dk)
    k = draw_qk(rows, H, dk, w.dtype, w.seed, T_K).reshape(steps, B, H, dk)
    v = draw_v(rows, H, dv, w.dtype, w.seed).reshape(steps, B, H, dv)
    a = draw_gate(rows, H, w.alpha[0], w.alpha[1], w.seed, T_ALPHA).reshape(steps, B, H)
    b = draw_gate(rows, H, w.beta[0], w.beta[1], w.seed, T_BETA).reshape(steps, B, H)
    s0 = draw_s0(B, H, dk, dv, w.s0_sd if w.s0_sd is not None else 0.02, w.seed)
    return dict(q=q, k=k, v=v, alpha=a, beta=b, s0=s0, steps=steps, B=B, H=H, dk=dk, dv=dv,
                dtype=w.dtype)


def to_torch(arr: np.ndarray, device, dtype: str):
    """Move a generated array to torch, viewing uint16 bit patterns as bfloat16."""
    import torch
    if dtype == "bf16" and arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def layer_step_inputs(lengths, H: int, d: int, width: int, dtype: str, seed: int,
                      with_state: bool = True) -> dict:
    """Seeded random inputs of the steps either side of the rule (random draws only):
    projections x_q, x_k, x_v [T, H*d] and the output gate's z and y [T, H, d] in ``dtype``;
    conv weights [H*d, width] ~ N(0, 1/width) and carried conv states [N, H*d, width-1]
    ~ N(0, 1) in fp32; gate pre-activations a, b [T, H] ~ N(0, 2^2), time constants
    A [H] ~ U(-2, 1), biases b_alpha [H] ~ N(0, 1) and the norm offset [d] ~ N(0, 0.1^2)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    C = H * d
    N = len(lengths)
    rng = np.random.default_rng([seed, 9001])
    out = {"lengths": lengths, "T": T, "H": H, "d": d, "C": C, "W": width, "N": N,
           "dtype": dtype,
           "cu_seqlens": np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)}
    for n in ("x_q", "x_k", "x_v"):
        out[n] = _store(rng.standard_normal((T, C)), dtype)
    for n in ("w_q", "w_k", "w_v"):
        out[n] = (rng.standard_normal((C, width)) / np.sqrt(width)).astype(np.float32)
    for n in ("s_q", "s_k", "s_v"):
        out[n] = (rng.standard_normal((N, C, width - 1)).astype(np.float32)
                  if with_state and width > 1 else None)
    out["a"] = (2.0 * rng.standard_normal((T, H))).astype(np.float32)
    out["b"] = (2.0 * rng.standard_normal((T, H))).astype(np.float32)
    out["A"] = rng.uniform(-2.0, 1.0, H).astype(np.float32)
    out["b_alpha"] = rng.standard_normal(H).astype(np.float32)
    out["z"] = _store(rng.standard_normal((T, H, d)), dtype)
    out["y"] = _store(rng.standard_normal((T, H, d)), dtype)
    out["norm_w"] = (0.1 * rng.standard_normal(d)).astype(np.float32)
    return out


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values a stored array holds, as float64."""
    if dtype == "bf16" and arr.dtype == np.uint16:
        return bf16_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)

"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its Python binding) never
imports, links or calls it, and it shares no code with that path.

Two implementations of the same definition live here:

* ``gdn_oracle.c`` (compiled by :func:`build`) -- plain C, fp64, one token at a time,
  OpenMP over independent (sequence, head) pairs.  Used for every size.
* :func:`chain_numpy` -- the same recurrence in numpy, for tiny cases and as an
  independent cross-check of the C code's indexing.

Both follow the jianyuh.github.io reading notes on Qwen3.8-Next, section 2.1 "Gated
DeltaNet" (the four-line gated delta recurrence):

    S~ = alpha_t S,   e_t = v_t - S~^T k_t,   S_t = S~ + beta_t k_t e_t^T,   y_t = S_t^T q_t

with S in R^{d_k x d_v} (rows over the key dimension).  Pins against closed forms, brute
force and invariants live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.gdn_oracle_run.restype = ctypes.c_int
        lib.gdn_oracle_run.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bf16 bit patterns
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError("q/k/v must be float32, float64 or uint16 (bf16 bits), got %s" % a.dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def run(q, k, v, alpha, beta, seq_row0, seq_len, row_step, s0=None,
        heads: Optional[Sequence[int]] = None, want_y=True, want_state=True,
        threads: int = 0):
    """General entry: see gdn_oracle_run in gdn_oracle.c for the row addressing.

    q, k: [rows, H, d_k]; v: [rows, H, d_v] (float32 / float64 / uint16 bf16 bits, all the
    same dtype); alpha, beta: [rows, H]; s0: [nseq, H, d_k, d_v] or None.
    Returns (y [rows, nh, d_v] float64 or None, s_final [nseq, nh, d_k, d_v] float64 or None).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k and v must share one dtype")
    rows, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (rows, H, dk) or v.shape[:2] != (rows, H):
        raise ValueError("shape mismatch between q, k and v")
    alpha = np.ascontiguousarray(alpha, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    if alpha.shape != (rows, H) or beta.shape != (rows, H):
        raise ValueError("alpha/beta must be [rows, H]")
    seq_row0 = np.ascontiguousarray(seq_row0, dtype=np.int64)
    seq_len = np.ascontiguousarray(seq_len, dtype=np.int64)
    nseq = int(seq_row0.shape[0])
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        if s0.shape != (nseq, H, dk, dv):
            raise ValueError("s0 must be [nseq, H, d_k, d_v]")
    h_lo, h_hi = (0, H) if heads is None else (int(heads[0]), int(heads[1]))
    nh = h_hi - h_lo
    y = np.zeros((rows, nh, dv), dtype=np.float64) if want_y else None
    sf = np.zeros((nseq, nh, dk, dv), dtype=np.float64) if want_state else None
    rc = _load().gdn_oracle_run(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(alpha), _ptr(beta), _ptr(s0),
        _ptr(seq_row0), _ptr(seq_len), int(row_step),
        nseq, H, dk, dv, h_lo, h_hi, _ptr(y), _ptr(sf), int(threads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_run failed with code %d" % rc)
    return y, sf


def prefill(q, k, v, alpha, beta, cu_seqlens=None, s0=None, heads=None, threads: int = 0,
            want_y=True, want_state=True):
    """Packed prefill: rows = total tokens; cu_seqlens [N+1] (None = one sequence)."""
    rows = q.shape[0]
    if cu_seqlens is None:
        cu = np.array([0, rows], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    return run(q, k, v, alpha, beta, cu[:-1], np.diff(cu), 1, s0=s0, heads=heads,
               threads=threads, want_y=want_y, want_state=want_state)


def decode(q, k, v, alpha, beta, s0, threads: int = 0, heads=None):
    """A stack of single-token steps.

    q, k: [steps, B, H, d_k]; v: [steps, B, H, d_v]; alpha, beta: [steps, B, H];
    s0: [B, H, d_k, d_v].  Returns (y [steps, B, nh, d_v], state after the last step).
    """
    steps, B, H, dk = q.shape
    dv = v.shape[3]
    y, sf = run(q.reshape(steps * B, H, dk), k.reshape(steps * B, H, dk),
                v.reshape(steps * B, H, dv), np.asarray(alpha).reshape(steps * B, H),
                np.asarray(beta).reshape(steps * B, H),
                np.arange(B, dtype=np.int64), np.full(B, steps, dtype=np.int64), B,
                s0=s0, heads=heads, threads=threads)
    nh = y.shape[1]
    return y.reshape(steps, B, nh, dv), sf


def chain_numpy(q, k, v, alpha, beta, s0=None):
    """One (sequence, head) chain in numpy, fp64, token by token.

    q, k: [T, d_k]; v: [T, d_v]; alpha, beta: [T]; s0: [d_k, d_v] or None.
    Returns (y [T, d_v], S_T [d_k, d_v]).  Same definition as the C oracle (section 2.1
    of the reading notes): decay, residual against the decayed state, rank-one write,
    read-out from the updated state.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    y = np.zeros((T, dv))
    for t in range(T):
        S_dec = float(alpha[t]) * S                     # S~ = alpha_t S
        e = v[t] - S_dec.T @ k[t]                        # e_t = v_t - S~^T k_t
        S = S_dec + float(beta[t]) * np.outer(k[t], e)   # S_t = S~ + beta_t k_t e_t^T
        y[t] = S.T @ q[t]                                # y_t = S_t^T q_t
    return y, S


def chain_c(q, k, v, alpha, beta, s0=None):
    """One chain through the C oracle (same signature as :func:`chain_numpy`)."""
    q = np.asarray(q, dtype=np.float64)[:, None, :]
    k = np.asarray(k, dtype=np.float64)[:, None, :]
    v = np.asarray(v, dtype=np.float64)[:, None, :]
    T = q.shape[0]
    a = np.asarray(alpha, dtype=np.float64).reshape(T, 1)
    b = np.asarray(beta, dtype=np.float64).reshape(T, 1)
    s = None if s0 is None else np.asarray(s0, dtype=np.float64)[None, None]
    y, sf = run(q, k, v, a, b, [0], [T], 1, s0=s, threads=1)
    return y[:, 0, :], sf[0, 0]

"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its Python binding) never
imports, links or calls it, and it shares no code with that path.

Two implementations of the same definition live here:

* ``gdn_oracle.c`` (compiled by :func:`build`) -- plain C, fp64, one token at a time,
  OpenMP over independent (sequence, head) pairs.  Used for every size.
* :func:`chain_numpy` -- the same recurrence in numpy, for tiny cases and as an
  independent cross-check of the C code's indexing.

The channel-wise gated variants (a decay per key channel, erase and write gates per value
channel; the rule is the special case of uniform gates) are :func:`channel_prefill` (C) and
:func:`channel_chain_numpy` (numpy).

The derivative of the same recurrence (for training) is :func:`prefill_backward` (C) and
:func:`chain_backward_numpy` (numpy): reverse mode, token by token, through the four lines
below.

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
_LIB_SAN = os.path.join(_HERE, "libgdn_oracle_san.so")     # AddressSanitizer + UBSan build
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  Returns the library path.  With
    sanitize, a separate copy instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
    (loaded when GDN_ORACLE_LIB names it, in a process that preloads libasan)."""
    lib = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        san = (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer", "-g"] if sanitize else [])
        cmd = (["gcc", "-O1" if sanitize else "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                "-ffp-contract=off"] + san + ["-o", tmp, _SRC, "-lm"])
        subprocess.check_call(cmd)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("GDN_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(path)
        lib.gdn_oracle_run.restype = ctypes.c_int
        lib.gdn_oracle_run.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.gdn_oracle_backward.restype = ctypes.c_int
        lib.gdn_oracle_backward.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.gdn_oracle_channel_run.restype = ctypes.c_int
        lib.gdn_oracle_channel_run.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
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


def prefill_backward(q, k, v, alpha, beta, dy, cu_seqlens=None, s0=None, ds_final=None,
                     heads=None, threads: int = 0):
    """Reverse-mode derivative of :func:`prefill` for L = <dy, y> + <ds_final, S_T>.

    dy: [rows, H, d_v] (any float dtype, widened to float64); ds_final: [nseq, H, d_k, d_v]
    or None (zero).  Returns a dict of float64 arrays holding heads ``heads`` (all by
    default): dq, dk [rows, nh, d_k], dv [rows, nh, d_v], dalpha, dbeta [rows, nh] and
    ds0 [nseq, nh, d_k, d_v].  See gdn_oracle_backward in gdn_oracle.c.
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k and v must share one dtype")
    rows, H, dk = q.shape
    dv = v.shape[2]
    alpha = np.ascontiguousarray(alpha, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    if dy.shape != (rows, H, dv) or alpha.shape != (rows, H) or beta.shape != (rows, H):
        raise ValueError("shape mismatch")
    cu = np.array([0, rows], dtype=np.int64) if cu_seqlens is None else \
        np.asarray(cu_seqlens, dtype=np.int64)
    row0 = np.ascontiguousarray(cu[:-1])
    lens = np.ascontiguousarray(np.diff(cu))
    nseq = int(row0.shape[0])
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        if s0.shape != (nseq, H, dk, dv):
            raise ValueError("s0 must be [nseq, H, d_k, d_v]")
    if ds_final is not None:
        ds_final = np.ascontiguousarray(ds_final, dtype=np.float64)
        if ds_final.shape != (nseq, H, dk, dv):
            raise ValueError("ds_final must be [nseq, H, d_k, d_v]")
    h_lo, h_hi = (0, H) if heads is None else (int(heads[0]), int(heads[1]))
    nh = h_hi - h_lo
    out = dict(dq=np.zeros((rows, nh, dk)), dk=np.zeros((rows, nh, dk)),
               dv=np.zeros((rows, nh, dv)), dalpha=np.zeros((rows, nh)),
               dbeta=np.zeros((rows, nh)), ds0=np.zeros((nseq, nh, dk, dv)))
    rc = _load().gdn_oracle_backward(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(alpha), _ptr(beta), _ptr(s0),
        _ptr(row0), _ptr(lens), 1, nseq, H, dk, dv, h_lo, h_hi, _ptr(dy), _ptr(ds_final),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]),
        _ptr(out["dbeta"]), _ptr(out["ds0"]), int(threads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_backward failed with code %d" % rc)
    return out


def chain_backward_c(q, k, v, alpha, beta, s0, dy, ds_final):
    """One chain through the C backward (same signature as :func:`chain_backward_numpy`)."""
    q = np.asarray(q, dtype=np.float64)[:, None, :]
    k = np.asarray(k, dtype=np.float64)[:, None, :]
    v = np.asarray(v, dtype=np.float64)[:, None, :]
    T = q.shape[0]
    a = np.asarray(alpha, dtype=np.float64).reshape(T, 1)
    b = np.asarray(beta, dtype=np.float64).reshape(T, 1)
    s = None if s0 is None else np.asarray(s0, dtype=np.float64)[None, None]
    d = None if ds_final is None else np.asarray(ds_final, dtype=np.float64)[None, None]
    o = prefill_backward(q, k, v, a, b, np.asarray(dy, np.float64)[:, None, :], s0=s,
                         ds_final=d, threads=1)
    return dict(dq=o["dq"][:, 0], dk=o["dk"][:, 0], dv=o["dv"][:, 0],
                dalpha=o["dalpha"][:, 0], dbeta=o["dbeta"][:, 0], ds0=o["ds0"][0, 0])


def chain_backward_numpy(q, k, v, alpha, beta, s0, dy, ds_final):
    """One (sequence, head) chain of the derivative in numpy, fp64, token by token.

    q, k: [T, d_k]; v, dy: [T, d_v]; alpha, beta: [T]; s0, ds_final: [d_k, d_v] or None.
    Returns dict(dq, dk, dv, dalpha, dbeta, ds0) for L = <dy, y> + <ds_final, S_T>.  The
    forward states are kept whole (tiny cases only); each line of the recurrence is then
    taken backwards as in gdn_oracle_backward.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = [np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)]
    for t in range(T):
        St = float(alpha[t]) * S[-1]
        e = v[t] - St.T @ k[t]
        S.append(St + float(beta[t]) * np.outer(k[t], e))
    D = np.zeros((dk, dv)) if ds_final is None else np.array(ds_final, dtype=np.float64)
    out = dict(dq=np.zeros((T, dk)), dk=np.zeros((T, dk)), dv=np.zeros((T, dv)),
               dalpha=np.zeros(T), dbeta=np.zeros(T))
    for t in range(T - 1, -1, -1):
        a, b = float(alpha[t]), float(beta[t])
        D = D + np.outer(q[t], dy[t])                  # y_t = S_t^T q_t
        out["dq"][t] = S[t + 1] @ dy[t]
        St = a * S[t]                                  # S~ = alpha_t S_{t-1}
        e = v[t] - St.T @ k[t]                         # e = v_t - S~^T k_t
        de = b * (D.T @ k[t])                          # S_t = S~ + beta_t k_t e^T
        out["dbeta"][t] = k[t] @ D @ e
        out["dv"][t] = de
        out["dk"][t] = b * (D @ e) - St @ de
        dSt = D - np.outer(k[t], de)
        out["dalpha"][t] = np.sum(dSt * S[t])
        D = a * dSt
    out["ds0"] = D
    return out


def channel_prefill(q, k, v, a, b, w, cu_seqlens=None, s0=None, heads=None, threads: int = 0,
                    want_y=True, want_state=True, seq_row0=None, seq_len=None, row_step=1):
    """Channel-wise gated variants (see gdn_oracle_channel_run in gdn_oracle.c).

    q, k: [rows, H, d_k]; v: [rows, H, d_v] (one dtype); a: [rows, H, d_k] decay per key
    channel; b, w: [rows, H, d_v] erase and write gates per value channel; s0:
    [nseq, H, d_k, d_v] or None.  Rows follow cu_seqlens (packed) unless seq_row0/seq_len/
    row_step give them explicitly.  Returns (y [rows, nh, d_v], s_final [nseq, nh, d_k, d_v])."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k and v must share one dtype")
    rows, H, dk = q.shape
    dv = v.shape[2]
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    if a.shape != (rows, H, dk) or b.shape != (rows, H, dv) or w.shape != (rows, H, dv):
        raise ValueError("gate shapes")
    if seq_row0 is None:
        cu = np.array([0, rows], dtype=np.int64) if cu_seqlens is None else \
            np.asarray(cu_seqlens, dtype=np.int64)
        seq_row0, seq_len = cu[:-1], np.diff(cu)
    seq_row0 = np.ascontiguousarray(seq_row0, dtype=np.int64)
    seq_len = np.ascontiguousarray(seq_len, dtype=np.int64)
    nseq = int(seq_row0.shape[0])
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        if s0.shape != (nseq, H, dk, dv):
            raise ValueError("s0 must be [nseq, H, d_k, d_v]")
    h_lo, h_hi = (0, H) if heads is None else (int(heads[0]), int(heads[1]))
    nh = h_hi - h_lo
    y = np.zeros((rows, nh, dv)) if want_y else None
    sf = np.zeros((nseq, nh, dk, dv)) if want_state else None
    rc = _load().gdn_oracle_channel_run(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(a), _ptr(b), _ptr(w), _ptr(s0), _ptr(seq_row0),
        _ptr(seq_len), int(row_step), nseq, H, dk, dv, h_lo, h_hi, _ptr(y), _ptr(sf),
        int(threads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_channel_run failed with code %d" % rc)
    return y, sf


def channel_chain_c(q, k, v, a, b, w, s0=None):
    """One chain through the C version (same signature as :func:`channel_chain_numpy`)."""
    T = np.asarray(q).shape[0]
    y, sf = channel_prefill(np.asarray(q, np.float64)[:, None], np.asarray(k, np.float64)[:, None],
                            np.asarray(v, np.float64)[:, None], np.asarray(a)[:, None],
                            np.asarray(b)[:, None], np.asarray(w)[:, None],
                            s0=None if s0 is None else np.asarray(s0, np.float64)[None, None],
                            threads=1)
    return y[:, 0], sf[0, 0]


def channel_chain_numpy(q, k, v, a, b, w, s0=None):
    """One (sequence, head) chain of the channel-wise gated form in numpy, fp64.

    q, k, a: [T, d_k]; v, b, w: [T, d_v]; s0: [d_k, d_v] or None.  Returns (y, S_T):
    decay each key channel, retrieve with the key, write the gated value minus the gated
    retrieval along the key, read with the query."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    y = np.zeros((T, dv))
    for t in range(T):
        St = np.asarray(a[t], np.float64)[:, None] * S          # S~ = Diag(a_t) S
        e = np.asarray(w[t]) * v[t] - np.asarray(b[t]) * (St.T @ k[t])
        S = St + np.outer(k[t], e)                             # S = S~ + k_t e^T
        y[t] = S.T @ q[t]                                      # y_t = S_t^T q_t
    return y, S

"""Python binding of libgdn (the gfx950 gated delta rule library).

Argument marshalling only: every function passes device pointers, sizes and the current HIP
stream to the C ABI of the same name (include/gdn.h) and raises ``GdnError`` on a non-OK
status.  All computation happens in the library's HIP kernels; there is no fallback path, and
a missing library is an error.

Tensors are torch tensors on the GPU (torch is used for device memory and streams only).
q, k, v and y are float32 or bfloat16; gates and states are float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARGUMENT = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_WORKSPACE_TOO_SMALL = 3
GDN_ERR_HIP = 4
GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

_lib = None


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s" % (fn, status_str(status)))
        self.status = status


def load(path: Optional[str] = None):
    """Load libgdn.so (built by ``linear_attention_recurrence_chunked_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("GDN_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build() or "
                           "python -m linear_attention_recurrence_chunked_amd.build" % p)
    lib = ctypes.CDLL(p)
    c = ctypes
    vp, i32, i64, sz = c.c_void_p, c.c_int32, c.c_int64, c.c_size_t
    lib.gdn_status_str.restype = c.c_char_p
    lib.gdn_status_str.argtypes = [i32]
    lib.gdn_version.restype = c.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_prefill_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.gdn_prefill_workspace_bytes_ex.restype = sz
    lib.gdn_prefill_workspace_bytes_ex.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32]
    lib.gdn_prefill_plan.restype = i32
    lib.gdn_prefill_plan.argtypes = [i32, i64, i32, i32, i32, i32,
                                     c.POINTER(i32), c.POINTER(i32)]
    pre = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.gdn_prefill.restype = i32
    lib.gdn_prefill.argtypes = pre
    lib.gdn_prefill_ex.restype = i32
    lib.gdn_prefill_ex.argtypes = pre + [i32, i32]
    lib.gdn_prefill_output_gated.restype = i32
    lib.gdn_prefill_output_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                             i32, vp, vp, c.c_float, vp, vp, vp, sz, vp, i32,
                                             i32]
    lib.gdn_prefill_gated.restype = i32
    lib.gdn_prefill_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                      i32, i32, vp, vp, vp, sz, vp]
    lib.gdn_noalloc_scratch_bytes.restype = sz
    lib.gdn_noalloc_scratch_bytes.argtypes = []
    lib.gdn_prefill_noalloc.restype = i32
    lib.gdn_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                        i32, vp, vp, vp]
    lib.gdn_prefill_backward_workspace_bytes.restype = sz
    lib.gdn_prefill_backward_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.gdn_prefill_backward.restype = i32
    lib.gdn_prefill_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                         i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_channel_gated.restype = i32
    lib.gdn_channel_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                      i32, vp, vp, vp]
    lib.gdn_qsa_workspace_bytes.restype = sz
    lib.gdn_qsa_workspace_bytes.argtypes = [i64]
    lib.gdn_qsa_index.restype = i32
    lib.gdn_qsa_index.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, sz, vp]
    lib.gdn_decode_step.restype = i32
    lib.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.gdn_short_conv.restype = i32
    lib.gdn_short_conv.argtypes = [vp, vp, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.gdn_gates.restype = i32
    lib.gdn_gates.argtypes = [vp, vp, vp, vp, i64, i32, vp, vp, vp]
    lib.gdn_output_gate.restype = i32
    lib.gdn_output_gate.argtypes = [vp, vp, vp, i64, i32, c.c_float, i32, vp, vp]
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().gdn_status_str(int(status)).decode()


gdn_status_str = status_str


def gdn_version() -> str:
    return load().gdn_version().decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    raise TypeError("q/k/v must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn: str, status: int):
    if status != GDN_OK:
        raise GdnError(fn, status)


def gdn_prefill_workspace_bytes(num_seqs: int, total_T: int, H: int, d_k: int, d_v: int,
                                dtype: int, dv_tile: int = 0, segment_chunks: int = 0) -> int:
    return int(load().gdn_prefill_workspace_bytes_ex(num_seqs, total_T, H, d_k, d_v, dtype,
                                                     dv_tile, segment_chunks))


def gdn_prefill_plan(num_seqs: int, total_T: int, H: int, d_k: int, d_v: int,
                     dtype: int) -> Tuple[int, int]:
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check("gdn_prefill_plan", load().gdn_prefill_plan(num_seqs, total_T, H, d_k, d_v, dtype,
                                                       ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def gdn_prefill(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, num_seqs=None,
                y=None, final_state=None, workspace=None, stream=None, dv_tile: int = 0,
                segment_chunks: int = 0, want_final_state: bool = True):
    """Chunked prefill.  q, k: [T, H, d_k]; v: [T, H, d_v]; alpha, beta: [T, H] fp32;
    initial_state: [N, H, d_k, d_v] fp32 or None; cu_seqlens: int32 [N+1] on the device or
    None (N equal sequences, ``num_seqs`` required).  Returns (y, final_state)."""
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if cu_seqlens is not None:
        n = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != n:
            raise ValueError("num_seqs does not match cu_seqlens")
        num_seqs = n
    elif num_seqs is None:
        num_seqs = 1
    if y is None:
        y = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and want_final_state:
        final_state = torch.empty((num_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    need = gdn_prefill_workspace_bytes(num_seqs, T, H, dk, dv, dt, dv_tile, segment_chunks)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gdn_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(initial_state), _ptr(cu_seqlens), num_seqs, T, H, dk, dv,
                               dt, _ptr(y), _ptr(final_state), _ptr(workspace), wbytes,
                               _stream(stream), dv_tile, segment_chunks)
    _check("gdn_prefill", st)
    return y, final_state


def gdn_prefill_output_gated(q, k, v, alpha, beta, z, weight, eps: float = 1e-6,
                             initial_state=None, cu_seqlens=None, num_seqs=None, out=None,
                             final_state=None, workspace=None, stream=None, dv_tile: int = 0,
                             segment_chunks: int = 0, want_final_state: bool = True):
    """Chunked prefill followed by the output gate: out = sigmoid(z) * RMSNorm(y) * (1 +
    weight) per (token, head) row, with z [T, H, d_v] in q's dtype and weight [d_v] fp32.
    Other arguments as gdn_prefill.  Returns (out, final_state)."""
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if cu_seqlens is not None:
        n = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != n:
            raise ValueError("num_seqs does not match cu_seqlens")
        num_seqs = n
    elif num_seqs is None:
        num_seqs = 1
    if out is None:
        out = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and want_final_state:
        final_state = torch.empty((num_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    need = gdn_prefill_workspace_bytes(num_seqs, T, H, dk, dv, dt, dv_tile, segment_chunks)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gdn_prefill_output_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                         _ptr(initial_state), _ptr(cu_seqlens), num_seqs, T, H,
                                         dk, dv, dt, _ptr(z), _ptr(weight), float(eps), _ptr(out),
                                         _ptr(final_state), _ptr(workspace), wbytes,
                                         _stream(stream), dv_tile, segment_chunks)
    _check("gdn_prefill_output_gated", st)
    return out, final_state


def gdn_noalloc_scratch_bytes() -> int:
    return int(load().gdn_noalloc_scratch_bytes())


def gdn_prefill_noalloc(q, k, v, alpha, beta, y, final_state=None, initial_state=None,
                        cu_seqlens=None, num_seqs=None, stream=None):
    """gdn_prefill with the library's fixed per-GPU workspace: nothing is allocated, so y
    [T, H, d_v] and final_state [N, H, d_k, d_v] fp32 (or None) come from the caller.
    Returns (y, final_state)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if cu_seqlens is not None:
        n = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != n:
            raise ValueError("num_seqs does not match cu_seqlens")
        num_seqs = n
    elif num_seqs is None:
        num_seqs = 1
    st = load().gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(initial_state), _ptr(cu_seqlens), num_seqs, T, H, dk,
                                    dv, dt, _ptr(y), _ptr(final_state), _stream(stream))
    _check("gdn_prefill_noalloc", st)
    return y, final_state


def gdn_prefill_gated(q, k, v, a, b, A, b_alpha, initial_state=None, cu_seqlens=None,
                      num_seqs=None, y=None, final_state=None, workspace=None, stream=None,
                      want_final_state: bool = True):
    """Chunked prefill with the gates as pre-activations: a, b [T, H] fp32 and A, b_alpha [H]
    fp32 (alpha = exp(-exp(A) softplus(a + b_alpha)), beta = sigmoid(b)); bf16 q, k, v.
    Returns (y, final_state)."""
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if cu_seqlens is not None:
        n = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != n:
            raise ValueError("num_seqs does not match cu_seqlens")
        num_seqs = n
    elif num_seqs is None:
        num_seqs = 1
    if y is None:
        y = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and want_final_state:
        final_state = torch.empty((num_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    need = gdn_prefill_workspace_bytes(num_seqs, T, H, dk, dv, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().gdn_prefill_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A),
                                  _ptr(b_alpha), _ptr(initial_state), _ptr(cu_seqlens),
                                  num_seqs, T, H, dk, dv, dt, _ptr(y), _ptr(final_state),
                                  _ptr(workspace), wbytes, _stream(stream))
    _check("gdn_prefill_gated", st)
    return y, final_state


def gdn_prefill_backward_workspace_bytes(num_seqs: int, total_T: int, H: int, d_k: int,
                                         d_v: int, dtype: int = GDN_DTYPE_BF16) -> int:
    return int(load().gdn_prefill_backward_workspace_bytes(num_seqs, total_T, H, d_k, d_v,
                                                           dtype))


def gdn_prefill_backward(q, k, v, alpha, beta, dy, initial_state=None, d_final_state=None,
                         cu_seqlens=None, num_seqs=None, workspace=None, stream=None,
                         want_d_initial_state: bool = True, out=None):
    """Backward of :func:`gdn_prefill` for L = <dy, y> + <d_final_state, S_T> (bf16).
    Returns (dq, dk, dv, dalpha, dbeta, d_initial_state); ``out`` may supply that tuple of
    preallocated tensors (d_initial_state may be None)."""
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if cu_seqlens is not None:
        n = cu_seqlens.shape[0] - 1
        if num_seqs is not None and num_seqs != n:
            raise ValueError("num_seqs does not match cu_seqlens")
        num_seqs = n
    elif num_seqs is None:
        num_seqs = 1
    if out is None:
        dev = q.device
        out = (torch.empty((T, H, dk), dtype=q.dtype, device=dev),
               torch.empty((T, H, dk), dtype=q.dtype, device=dev),
               torch.empty((T, H, dv), dtype=q.dtype, device=dev),
               torch.empty((T, H), dtype=torch.float32, device=dev),
               torch.empty((T, H), dtype=torch.float32, device=dev),
               torch.empty((num_seqs, H, dk, dv), dtype=torch.float32, device=dev)
               if want_d_initial_state else None)
    gq, gk, gv, ga, gb, gs = out
    need = gdn_prefill_backward_workspace_bytes(num_seqs, T, H, dk, dv, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = load().gdn_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
        _ptr(cu_seqlens), num_seqs, T, H, dk, dv, dt, _ptr(dy), _ptr(d_final_state),
        _ptr(gq), _ptr(gk), _ptr(gv), _ptr(ga), _ptr(gb), _ptr(gs), _ptr(workspace), wbytes,
        _stream(stream))
    _check("gdn_prefill_backward", st)
    return gq, gk, gv, ga, gb, gs


def gdn_channel_gated(q, k, v, decay, erase, write, initial_state=None, cu_seqlens=None,
                      num_seqs=None, y=None, final_state=None, want_final_state=True,
                      stream=None):
    """Channel-wise gated variants: decay [T, H, d_k], erase and write [T, H, d_v] fp32
    gates; otherwise as :func:`gdn_prefill`.  final_state may be initial_state (in place).
    Returns (y, final_state)."""
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        num_seqs = cu_seqlens.shape[0] - 1
    elif num_seqs is None:
        num_seqs = 1
    if y is None:
        y = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None and want_final_state:
        final_state = torch.empty((num_seqs, H, dk, dv), dtype=torch.float32, device=q.device)
    st = load().gdn_channel_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(erase),
                                  _ptr(write), _ptr(initial_state), _ptr(cu_seqlens), num_seqs,
                                  T, H, dk, dv, _dtype_code(q), _ptr(y), _ptr(final_state),
                                  _stream(stream))
    _check("gdn_channel_gated", st)
    return y, final_state


def gdn_qsa_workspace_bytes(n: int) -> int:
    return int(load().gdn_qsa_workspace_bytes(n))


def gdn_qsa_index(q, k, block_budget: int = 512, want_blocks: bool = True,
                  want_tokens: bool = True, workspace=None, stream=None, blocks=None,
                  tokens=None):
    """Sparse-attention block indexer for one sequence: q [n, 4, 128], k [n, 128]
    (bf16 or fp32).  Returns (blocks [n, budget] int32 or None, tokens [n, 4 budget + 3]
    int32 or None), both ascending and -1 padded; given output tensors are written in
    place."""
    import torch
    n = q.shape[0]
    if blocks is None and want_blocks:
        blocks = torch.empty((n, block_budget), dtype=torch.int32, device=q.device)
    if tokens is None and want_tokens:
        tokens = torch.empty((n, 4 * block_budget + 3), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(gdn_qsa_workspace_bytes(n), 16), dtype=torch.uint8,
                                device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = load().gdn_qsa_index(_ptr(q), _ptr(k), n, _dtype_code(q), block_budget,
                              _ptr(blocks), _ptr(tokens), _ptr(workspace), wbytes,
                              _stream(stream))
    _check("gdn_qsa_index", st)
    return blocks, tokens


def gdn_decode_step(q, k, v, alpha, beta, state, y=None, stream=None):
    """One decode step: q, k [B, H, d_k]; v [B, H, d_v]; alpha, beta [B, H] fp32;
    state [B, H, d_k, d_v] fp32 updated in place.  Returns y [B, H, d_v]."""
    import torch
    B, H, dk = q.shape
    dv = v.shape[2]
    if y is None:
        y = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    st = load().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(state), _ptr(y), B, H, dk, dv, _dtype_code(q),
                                _stream(stream))
    _check("gdn_decode_step", st)
    return y


# ---- the steps either side of the rule ------------------------------------------------------

def gdn_short_conv(x, weight, cu_seqlens=None, num_seqs=None, head_dim: int = 0, out=None,
                   state_in=None, state_out=None, stream=None):
    """Causal depthwise convolution + SiLU (+ per-head L2Norm when head_dim > 0).
    x: [T, C] (or [T, H, d], taken as [T, H*d]) float32/bfloat16; weight: [C, W] fp32;
    state_in/state_out: [N, C, W-1] fp32 or None.  Returns out (same shape as x)."""
    import torch
    T = x.shape[0]
    C = x.numel() // T if T else int(torch.tensor(x.shape[1:]).prod())
    W = weight.shape[1]
    if cu_seqlens is not None:
        num_seqs = cu_seqlens.shape[0] - 1
    elif num_seqs is None:
        num_seqs = 1
    if out is None:
        out = torch.empty_like(x)
    st = load().gdn_short_conv(_ptr(x), _ptr(weight), _ptr(cu_seqlens), num_seqs, T, C, W,
                               head_dim, _dtype_code(x), _ptr(out), _ptr(state_in),
                               _ptr(state_out), _stream(stream))
    _check("gdn_short_conv", st)
    return out


def gdn_gates(a, b, A, b_alpha, alpha=None, beta=None, stream=None):
    """alpha = exp(-exp(A) softplus(a + b_alpha)), beta = sigmoid(b); a, b [T, H] fp32,
    A, b_alpha [H] fp32.  Returns (alpha, beta)."""
    import torch
    T, H = a.shape
    if alpha is None:
        alpha = torch.empty_like(a)
    if beta is None:
        beta = torch.empty_like(a)
    st = load().gdn_gates(_ptr(a), _ptr(b), _ptr(A), _ptr(b_alpha), T, H, _ptr(alpha),
                          _ptr(beta), _stream(stream))
    _check("gdn_gates", st)
    return alpha, beta


def gdn_output_gate(y, z, weight, eps: float = 1e-6, out=None, stream=None):
    """sigmoid(z) * RMSNorm(y) * (1 + weight) over the last axis (d_v in {64, 128});
    y, z [..., d_v] float32/bfloat16, weight [d_v] fp32.  Returns out (may be y)."""
    import torch
    dv = y.shape[-1]
    rows = y.numel() // dv
    if out is None:
        out = torch.empty_like(y)
    st = load().gdn_output_gate(_ptr(y), _ptr(z), _ptr(weight), rows, dv, float(eps),
                                _dtype_code(y), _ptr(out), _stream(stream))
    _check("gdn_output_gate", st)
    return out

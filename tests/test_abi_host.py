"""The C ABI on the host (no GPU needed): the library loads, exports every declared symbol,
and rejects every invalid argument before anything reaches the HIP runtime.

The pointers below are fake but aligned device addresses; every call here fails validation,
so nothing is ever launched or dereferenced.
"""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_chunked_amd import gdn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "gdn.h")
G = 1 << 32   # spacing between fake buffers (no two overlap)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build()")
    return gdn.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "gdn_prefill" in names and "gdn_decode_step" in names
    for n in names:
        assert hasattr(lib, n), "symbol %s missing from libgdn.so" % n


def test_status_strings_and_version(lib):
    assert gdn.status_str(0) == "GDN_OK"
    assert gdn.status_str(3) == "GDN_ERR_WORKSPACE_TOO_SMALL"
    assert gdn.status_str(99) == "GDN_ERR_UNKNOWN"
    assert gdn.gdn_version().startswith("gdn-gfx950")


def test_plans_for_the_workloads(lib):
    # 64 chains (B=4, H=16): split the state columns, never the sequences
    t, s = gdn.gdn_prefill_plan(4, 4 * 4096, 16, 128, 128, gdn.GDN_DTYPE_BF16)
    assert t in (32, 64) and s == -1
    # 16 chains of 1M tokens: the one-launch scan with the whole state per workgroup, one
    # segment of about 1,024 chunks per job (256 jobs)
    t, s = gdn.gdn_prefill_plan(1, 1 << 20, 16, 128, 128, gdn.GDN_DTYPE_BF16)
    assert t == 128 and 1000 <= s <= 1100
    # its workspace: the segment table, a control block, flags and one fp32 end state per
    # (segment, head)
    entries = 1 + -(-(1 << 20) // (s * 64))
    w = gdn.gdn_prefill_workspace_bytes(1, 1 << 20, 16, 128, 128, 1)
    assert entries * 16 * 128 * 128 * 4 < w < entries * 16 * 128 * 128 * 4 + (64 << 10)
    # 512 chains of mixed lengths, 266 chunk steps per CU: the one-launch scan in segments of
    # about 89 chunks (three jobs per CU)
    t, s = gdn.gdn_prefill_plan(32, 270336, 16, 128, 128, gdn.GDN_DTYPE_BF16)
    assert t == 128 and 85 <= s <= 95
    # 64 chains of 256 chunks (64 chunk steps per CU): the two-launch column-split scan
    t, s = gdn.gdn_prefill_plan(4, 4 * 16384, 16, 128, 128, gdn.GDN_DTYPE_BF16)
    assert t in (32, 64) and s == -1
    # bf16 column-split plans: one 8448-byte record (T', g) per chunk slot and head
    slots = 270336 // 64 + 32
    assert gdn.gdn_prefill_workspace_bytes(32, 270336, 16, 128, 128, 1, 32, -1) == slots * 16 * 8448
    # the one-launch scan on request: segments of 16 chunks for 64 chains by default
    assert gdn.gdn_prefill_workspace_bytes(4, 4 * 4096, 16, 128, 128, 1, 128, 0) > 0
    # fp32 without segments needs no workspace
    assert gdn.gdn_prefill_workspace_bytes(1, 256, 2, 64, 64, 0) == 0
    # fp32 tiles stay within the LDS budget
    t, s = gdn.gdn_prefill_plan(1, 256, 2, 64, 64, gdn.GDN_DTYPE_F32)
    assert t in (16, 32, 64)


def test_workspace_query_rejects_bad_shapes(lib):
    assert gdn.gdn_prefill_workspace_bytes(0, 10, 1, 128, 128, 1) == 0
    assert gdn.gdn_prefill_workspace_bytes(1, 10, 1, 96, 128, 1) == 0
    assert gdn.gdn_prefill_workspace_bytes(1, 10, 1, 128, 128, 7) == 0
    # explicit segmentation needs table + per-segment matrices
    w = gdn.gdn_prefill_workspace_bytes(2, 1000, 3, 64, 128, 1, 32, 2)
    assert w >= 3 * 8 * (64 * 128 + 64 * 64) * 4


def prefill(lib, **kw):
    a = dict(q=1 * G, k=2 * G, v=3 * G, alpha=4 * G, beta=5 * G, s0=None, cu=None,
             n=2, T=256, H=2, dk=128, dv=128, dt=1, y=6 * G, sf=7 * G, ws=9 * G, wsb=G,
             stream=None, tile=0, seg=-1)
    a.update(kw)
    return lib.gdn_prefill_ex(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"], a["cu"],
                              a["n"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], a["y"],
                              a["sf"], a["ws"], a["wsb"], a["stream"], a["tile"], a["seg"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(alpha=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(y=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(n=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(H=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(T=255), gdn.GDN_ERR_INVALID_ARGUMENT),          # not a multiple of n without cu
    (dict(dk=96), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dv=256), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dt=5), gdn.GDN_ERR_UNSUPPORTED),
    (dict(tile=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dt=0, tile=128), gdn.GDN_ERR_UNSUPPORTED),      # fp32 tile over the LDS budget
    (dict(dt=0, tile=32), gdn.GDN_ERR_UNSUPPORTED),       # fp32, d_k = 128: 16 columns only
    (dict(seg=-2), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(k=2 * G + 4), gdn.GDN_ERR_INVALID_ARGUMENT),    # misaligned (16 B required)
    (dict(k=2 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),    # bf16: eight elements too
    (dict(dt=0, k=2 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(v=3 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(y=6 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(alpha=4 * G + 2), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(sf=7 * G + 4), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(y=1 * G + 4096), gdn.GDN_ERR_INVALID_ARGUMENT), # y overlaps q
    (dict(sf=5 * G), gdn.GDN_ERR_INVALID_ARGUMENT),       # final state overlaps beta
    (dict(s0=8 * G, y=8 * G), gdn.GDN_ERR_INVALID_ARGUMENT),   # y overlaps initial state
    (dict(s0=8 * G, sf=8 * G + 256), gdn.GDN_ERR_INVALID_ARGUMENT),  # partial overlap
    (dict(s0=8 * G, sf=8 * G, seg=2), gdn.GDN_ERR_INVALID_ARGUMENT),  # in place + split
    (dict(tile=32, ws=None, wsb=0), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),   # bf16 chunk records
    (dict(tile=32, wsb=6 * 2 * 8448 - 1), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),
    (dict(seg=2, ws=None, wsb=0), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),   # segments too
    (dict(seg=2, ws=9 * G, wsb=64), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),
])
def test_prefill_rejects(lib, kw, code):
    assert prefill(lib, **kw) == code


def prefill_noalloc(lib, **kw):
    a = dict(q=1 * G, k=2 * G, v=3 * G, alpha=4 * G, beta=5 * G, s0=None, cu=None,
             n=2, T=256, H=2, dk=128, dv=128, dt=1, y=6 * G, sf=7 * G, stream=None)
    a.update(kw)
    return lib.gdn_prefill_noalloc(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"],
                                   a["cu"], a["n"], a["T"], a["H"], a["dk"], a["dv"], a["dt"],
                                   a["y"], a["sf"], a["stream"])


def prefill_og(lib, **kw):
    a = dict(q=1 * G, k=2 * G, v=3 * G, alpha=4 * G, beta=5 * G, s0=None, cu=None, n=2, T=256,
             H=2, dk=128, dv=128, dt=1, z=8 * G, w=10 * G, eps=1e-6, out=6 * G, sf=7 * G,
             ws=9 * G, wsb=G, stream=None, tile=0, seg=-1)
    a.update(kw)
    return lib.gdn_prefill_output_gated(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"],
                                        a["cu"], a["n"], a["T"], a["H"], a["dk"], a["dv"],
                                        a["dt"], a["z"], a["w"], a["eps"], a["out"], a["sf"],
                                        a["ws"], a["wsb"], a["stream"], a["tile"], a["seg"])


# rejected on the host before anything is enqueued
@pytest.mark.parametrize("kw", [
    dict(z=None), dict(w=None),                          # missing gate inputs
    dict(z=8 * G + 8), dict(w=10 * G + 2),               # misaligned
    dict(eps=-1e-6), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(z=6 * G),                                       # z is the output
    dict(w=6 * G + 256),                                 # weight inside the output
    dict(n=0), dict(H=0),
])
def test_prefill_output_gated_rejects(lib, kw):
    assert prefill_og(lib, **kw) == gdn.GDN_ERR_INVALID_ARGUMENT


def test_prefill_output_gated_unsupported(lib):
    assert prefill_og(lib, dk=96) == gdn.GDN_ERR_UNSUPPORTED
    assert prefill_og(lib, dt=4) == gdn.GDN_ERR_UNSUPPORTED


def test_noalloc_scratch_size(lib):
    assert gdn.gdn_noalloc_scratch_bytes() == 64 << 20


# rejected before any HIP call (the size check is a function of the arguments alone)
@pytest.mark.parametrize("kw,code", [
    (dict(n=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(H=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(dk=96), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dt=5), gdn.GDN_ERR_UNSUPPORTED),
    # a workspace larger than the fixed array: 64 sequences of 65,536 tokens, 16 bf16 heads
    # (chunk records for 2^22 tokens)
    (dict(n=64, T=1 << 22, H=16), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),
])
def test_prefill_noalloc_rejects(lib, kw, code):
    need = gdn.gdn_prefill_workspace_bytes(kw.get("n", 2), kw.get("T", 256), kw.get("H", 2),
                                           kw.get("dk", 128), 128, kw.get("dt", 1))
    if code == gdn.GDN_ERR_WORKSPACE_TOO_SMALL:
        assert need > gdn.gdn_noalloc_scratch_bytes()
    assert prefill_noalloc(lib, **kw) == code


def decode(lib, **kw):
    a = dict(q=1 * G, k=2 * G, v=3 * G, alpha=4 * G, beta=5 * G, state=6 * G, y=7 * G,
             B=4, H=2, dk=128, dv=128, dt=1, stream=None)
    a.update(kw)
    return lib.gdn_decode_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"],
                               a["y"], a["B"], a["H"], a["dk"], a["dv"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(v=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(B=-1), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(H=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(dk=32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dt=2), gdn.GDN_ERR_UNSUPPORTED),
    (dict(q=1 * G + 2), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(q=1 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(state=6 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(y=6 * G + 1024), gdn.GDN_ERR_INVALID_ARGUMENT),   # y inside the state
    (dict(state=1 * G), gdn.GDN_ERR_INVALID_ARGUMENT),      # state over q
    (dict(y=3 * G), gdn.GDN_ERR_INVALID_ARGUMENT),          # y over v
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code


def test_decode_empty_batch_is_a_no_op(lib):
    # B = 0 returns before any HIP call
    assert decode(lib, B=0) == gdn.GDN_OK


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        gdn.load(str(tmp_path / "missing.so"))


# ---- the layer steps --------------------------------------------------------------------

def short_conv(lib, **kw):
    a = dict(x=1 * G, w=2 * G, cu=None, N=2, T=64, C=256, W=4, hd=128, dt=1, out=3 * G,
             sin=4 * G, sout=5 * G, stream=None)
    a.update(kw)
    return lib.gdn_short_conv(a["x"], a["w"], a["cu"], a["N"], a["T"], a["C"], a["W"], a["hd"],
                              a["dt"], a["out"], a["sin"], a["sout"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(C=100), gdn.GDN_ERR_INVALID_ARGUMENT),            # not a multiple of 64
    (dict(W=5), gdn.GDN_ERR_UNSUPPORTED),
    (dict(W=0), gdn.GDN_ERR_UNSUPPORTED),
    (dict(hd=32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(C=192, hd=128), gdn.GDN_ERR_INVALID_ARGUMENT),    # heads do not tile the channels
    (dict(T=63), gdn.GDN_ERR_INVALID_ARGUMENT),             # T not a multiple of N
    (dict(N=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(dt=2), gdn.GDN_ERR_UNSUPPORTED),
    (dict(x=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(w=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(x=1 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(out=1 * G + 256), gdn.GDN_ERR_INVALID_ARGUMENT),  # out overlaps x
    (dict(sout=2 * G), gdn.GDN_ERR_INVALID_ARGUMENT),       # state over the weights
    (dict(sout=4 * G + 4), gdn.GDN_ERR_INVALID_ARGUMENT),   # state partly over state_in
])
def test_short_conv_rejects(lib, kw, code):
    assert short_conv(lib, **kw) == code


def gates(lib, **kw):
    a = dict(a=1 * G, b=2 * G, A=3 * G, ba=4 * G, T=64, H=16, al=5 * G, be=6 * G, stream=None)
    a.update(kw)
    return lib.gdn_gates(a["a"], a["b"], a["A"], a["ba"], a["T"], a["H"], a["al"], a["be"],
                         a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(A=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(al=1 * G + 2), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(al=1 * G), gdn.GDN_ERR_INVALID_ARGUMENT),         # alpha over a
    (dict(be=5 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),     # beta over alpha
])
def test_gates_reject(lib, kw, code):
    assert gates(lib, **kw) == code


def output_gate(lib, **kw):
    a = dict(y=1 * G, z=2 * G, w=3 * G, rows=64, dv=128, eps=1e-6, dt=1, out=4 * G, stream=None)
    a.update(kw)
    return lib.gdn_output_gate(a["y"], a["z"], a["w"], a["rows"], a["dv"], a["eps"], a["dt"],
                               a["out"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dv=96), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dt=3), gdn.GDN_ERR_UNSUPPORTED),
    (dict(rows=-1), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(eps=-1.0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(eps=float("nan")), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(z=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(y=1 * G + 4), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(out=2 * G + 256), gdn.GDN_ERR_INVALID_ARGUMENT),  # out over z
    (dict(out=1 * G + 256), gdn.GDN_ERR_INVALID_ARGUMENT),  # out partly over y
])
def test_output_gate_rejects(lib, kw, code):
    assert output_gate(lib, **kw) == code


def test_layer_steps_empty_is_a_no_op(lib):
    assert gates(lib, T=0) == gdn.GDN_OK
    assert output_gate(lib, rows=0) == gdn.GDN_OK


# ---- backward -------------------------------------------------------------------------------

def backward(lib, **kw):
    a = dict(q=1 * G, k=2 * G, v=3 * G, alpha=4 * G, beta=5 * G, s0=None, cu=None, N=2,
             T=256, H=2, dk=128, dv=128, dt=1, dy=6 * G, dsf=None, dq=7 * G, dkk=8 * G,
             dvv=9 * G, da=10 * G, db=11 * G, ds0=12 * G, ws=13 * G, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return lib.gdn_prefill_backward(
        a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"], a["cu"], a["N"], a["T"],
        a["H"], a["dk"], a["dv"], a["dt"], a["dy"], a["dsf"], a["dq"], a["dkk"], a["dvv"],
        a["da"], a["db"], a["ds0"], a["ws"], a["wsb"], a["stream"])


def test_backward_workspace_query(lib):
    # records (T' and P in bf16, g in fp32: 16,640 bytes) plus the kept states and adjoints
    slots = 4 * 4096 // 64 + 4
    rec = slots * 16 * (2 * 64 * 64 * 2 + 64 * 4)
    st = slots * 16 * 128 * 128 * 4
    assert gdn.gdn_prefill_backward_workspace_bytes(4, 4 * 4096, 16, 128, 128) == rec + 2 * st
    assert gdn.gdn_prefill_backward_workspace_bytes(4, 4 * 4096, 16, 128, 128,
                                                    gdn.GDN_DTYPE_F32) == 0
    assert gdn.gdn_prefill_backward_workspace_bytes(0, 16, 16, 128, 128) == 0
    assert gdn.gdn_prefill_backward_workspace_bytes(1, 16, 16, 96, 128) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dt=0), gdn.GDN_ERR_UNSUPPORTED),                # bf16 only
    (dict(dk=32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(N=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(T=255), gdn.GDN_ERR_INVALID_ARGUMENT),          # N equal lengths must divide T
    (dict(dy=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(da=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(dq=7 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),   # 16-byte alignment
    (dict(dsf=14 * G + 4), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(db=11 * G + 2), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(dq=1 * G), gdn.GDN_ERR_INVALID_ARGUMENT),       # dq over q
    (dict(dvv=6 * G + 256), gdn.GDN_ERR_INVALID_ARGUMENT),  # dv inside dy
    (dict(ds0=7 * G), gdn.GDN_ERR_INVALID_ARGUMENT),      # dS0 over dq
    (dict(s0=14 * G, ds0=14 * G), gdn.GDN_ERR_INVALID_ARGUMENT),  # dS0 over S0
    (dict(ws=12 * G + 1024), gdn.GDN_ERR_INVALID_ARGUMENT),       # workspace over dS0
    (dict(ws=None), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),
    (dict(wsb=1024), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),
])
def test_backward_rejects(lib, kw, code):
    assert backward(lib, **kw) == code


def qsa(lib, **kw):
    a = dict(q=1 * G, k=2 * G, n=4096, dt=gdn.GDN_DTYPE_BF16, kb=512, blocks=3 * G,
             tokens=4 * G, ws=5 * G, wsb=1 << 31, stream=None)
    a.update(kw)
    return lib.gdn_qsa_index(a["q"], a["k"], a["n"], a["dt"], a["kb"], a["blocks"],
                             a["tokens"], a["ws"], a["wsb"], a["stream"])


def test_qsa_workspace_query():
    # bf16 normalised queries [n, 4, 128] and block keys [n/4, 128], each region rounded up to
    # 256 bytes: O(n), no score matrix
    al = lambda x: (x + 255) // 256 * 256
    n = 4096
    assert gdn.gdn_qsa_workspace_bytes(n) == al(n * 4 * 128 * 2) + al(n // 4 * 128 * 2)
    assert gdn.gdn_qsa_workspace_bytes(1030) == al(1030 * 4 * 128 * 2) + al(257 * 128 * 2)
    assert gdn.gdn_qsa_workspace_bytes(3) == al(3 * 4 * 128 * 2) + al(128 * 2)
    assert gdn.gdn_qsa_workspace_bytes(0) == 0
    n = 1 << 20
    assert gdn.gdn_qsa_workspace_bytes(n) == al(n * 4 * 128 * 2) + al(n // 4 * 128 * 2)
    assert gdn.gdn_qsa_workspace_bytes(n + 1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(n=(1 << 20) + 1), gdn.GDN_ERR_UNSUPPORTED),      # beyond 2^20 tokens
    (dict(kb=(1 << 24) + 1), gdn.GDN_ERR_UNSUPPORTED),
    (dict(n=16384, kb=2049), gdn.GDN_ERR_UNSUPPORTED),     # budget > 2,048 below 4,096 blocks
    (dict(n=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(kb=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(ws=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(blocks=None, tokens=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(k=2 * G + 8), gdn.GDN_ERR_INVALID_ARGUMENT),     # 16-byte alignment
    (dict(tokens=4 * G + 2), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(blocks=1 * G + 4096), gdn.GDN_ERR_INVALID_ARGUMENT),   # blocks over q
    (dict(tokens=3 * G + 1024), gdn.GDN_ERR_INVALID_ARGUMENT),   # tokens over blocks
    (dict(ws=4 * G + 4096), gdn.GDN_ERR_INVALID_ARGUMENT),       # workspace over tokens
    (dict(wsb=1 << 20), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),
])
def test_qsa_rejects(lib, kw, code):
    assert qsa(lib, **kw) == code


def prefill_gated(lib, **kw):
    a = dict(q=1 * G, k=2 * G, v=3 * G, ga=4 * G, gb=5 * G, A=10 * G, bal=11 * G, s0=None,
             cu=None, n=2, T=256, H=2, dk=128, dv=128, dt=1, y=6 * G, sf=7 * G, ws=9 * G,
             wsb=G, stream=None)
    a.update(kw)
    return lib.gdn_prefill_gated(a["q"], a["k"], a["v"], a["ga"], a["gb"], a["A"], a["bal"],
                                 a["s0"], a["cu"], a["n"], a["T"], a["H"], a["dk"], a["dv"],
                                 a["dt"], a["y"], a["sf"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dt=0), gdn.GDN_ERR_UNSUPPORTED),                # bf16 only
    (dict(dk=32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(A=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(bal=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(ga=None), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(A=10 * G + 2), gdn.GDN_ERR_INVALID_ARGUMENT),   # 4-byte alignment
    (dict(A=6 * G + 64), gdn.GDN_ERR_INVALID_ARGUMENT),   # A inside y
    (dict(bal=7 * G), gdn.GDN_ERR_INVALID_ARGUMENT),      # b_alpha under the final state
    # sequences long enough to be split into segments need a workspace
    (dict(T=2 * 8192, wsb=16), gdn.GDN_ERR_WORKSPACE_TOO_SMALL),
])
def test_prefill_gated_rejects(lib, kw, code):
    assert prefill_gated(lib, **kw) == code

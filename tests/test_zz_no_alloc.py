"""gdn_prefill_noalloc (the prefill with the library's fixed per-GPU workspace) against
gdn_prefill (caller-provided workspace) and the fp64 oracle, through the C ABI: two calls in
a row on one GPU, the second on a smaller problem, so the second runs on an array that still
holds the first call's data."""
import numpy as np
import pytest

from gpu_util import TOL, cu_of, say, slice_rel_err, state_rel_err, torch_inputs

torch = pytest.importorskip("torch")


def _inputs(lengths, H, seed):
    from linear_attention_recurrence_chunked_amd import workloads as wl
    return wl.make_inputs(lengths, H, 128, 128, "bf16", alpha=(3.0, 1.0), beta=(0.0, 1.0),
                          s0_sd=0.02, seed=seed)


@pytest.mark.gpu
def test_noalloc_matches_prefill_twice(oracle_lib):
    from linear_attention_recurrence_chunked_amd import gdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    cases = [([1500, 7, 0, 2222, 130], 4, 61), ([300, 65], 2, 62)]
    for lengths, H, seed in cases:
        inp = _inputs(lengths, H, seed)
        t = torch_inputs(inp, dev)
        T = inp["q"].shape[0]
        N = len(lengths)
        need = gdn.gdn_prefill_workspace_bytes(N, T, H, 128, 128, gdn.GDN_DTYPE_BF16)
        assert 0 < need <= gdn.gdn_noalloc_scratch_bytes()
        say("[gpu] noalloc lengths=%s H=%d workspace %d bytes" % (lengths, H, need))
        y_na = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device=dev)
        s_na = torch.full((N, H, 128, 128), float("nan"), dtype=torch.float32, device=dev)
        gdn.gdn_prefill_noalloc(t["q"], t["k"], t["v"], t["alpha"], t["beta"], y_na, s_na,
                                initial_state=t["s0"], cu_seqlens=t["cu"])
        y_ref, s_ref = gdn.gdn_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"],
                                       initial_state=t["s0"], cu_seqlens=t["cu"])
        torch.cuda.synchronize()
        gy, gs = y_na.float().cpu().numpy(), s_na.cpu().numpy()
        assert np.all(np.isfinite(gy)) and np.all(np.isfinite(gs))
        ry, rs = oracle_lib.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                    cu_of(inp), s0=inp["s0"])
        ey = slice_rel_err(gy, ry, cu_of(inp))
        es = state_rel_err(gs, rs)
        dy = slice_rel_err(gy, y_ref.float().cpu().numpy().astype(np.float64), cu_of(inp))
        ds = state_rel_err(gs, s_ref.cpu().numpy().astype(np.float64))
        say("    vs oracle: y %.3e state %.3e; vs gdn_prefill: y %.3e state %.3e"
            % (ey, es, dy, ds))
        assert ey <= TOL["bf16"] and es <= TOL["bf16"]
        assert dy <= TOL["bf16"] and ds <= TOL["bf16"]

"""Pins of the fp64 backward oracle (oracle.prefill_backward, oracle.chain_backward_numpy).

The derivative is fixed by the forward recurrence (reading notes, Gated DeltaNet, section
2.1), which the forward pins already hold.  Each pin below checks the backward oracle against
something other than itself:

* central finite differences of the pinned forward oracle, for every input;
* torch autograd (float64, CPU) through a forward written here in torch ops;
* exact adjoint identities that follow from the linearity of (y, S_T) in (V, S0) and of y
  in q for fixed states;
* the closed form of the beta = 0 case, where the state only decays.

Mutants (plausible mistakes in the reverse pass) must each fail at least one pin.
"""
import numpy as np
import pytest

import oracle


def _chain(rng, T, dk, dv, a_lo=0.3):
    q = rng.normal(size=(T, dk))
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.normal(size=(T, dv))
    a = rng.uniform(a_lo, 1.0, size=T)
    b = rng.uniform(0.0, 1.0, size=T)
    if T >= 4:       # the closed ends of the gate domains
        a[1] = 1.0
        b[2] = 0.0
        b[3] = 1.0
    s0 = rng.normal(size=(dk, dv))
    dy = rng.normal(size=(T, dv))
    dsT = rng.normal(size=(dk, dv))
    return q, k, v, a, b, s0, dy, dsT


def _loss(q, k, v, a, b, s0, dy, dsT):
    y, S = oracle.chain_numpy(q, k, v, a, b, s0)
    return float(np.sum(y * dy) + np.sum(S * dsT))


def _close(got, want, rtol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = max(np.abs(want).max(), 1e-300)
    err = np.abs(got - want).max() / scale
    assert err <= rtol, "%s: relative error %.3e > %.1e" % (what, err, rtol)


# ---- pins: each takes a backward implementation with chain_backward_numpy's signature ------

def pin_bwd_finite_differences(bwd):
    rng = np.random.default_rng(101)
    args = list(_chain(rng, 9, 3, 2))
    g = bwd(*args)
    h = 1e-6
    names = ["dq", "dk", "dv", "dalpha", "dbeta", "ds0"]
    for pos, name in zip([0, 1, 2, 3, 4, 5], names):
        x = args[pos]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = list(args)
            am = list(args)
            ap[pos] = xp
            am[pos] = xm
            fd[idx] = (_loss(*ap) - _loss(*am)) / (2 * h)
        _close(g[name], fd, 1e-7, "finite differences, " + name)


def pin_bwd_torch_autograd(bwd):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(202)
    q, k, v, a, b, s0, dy, dsT = _chain(rng, 21, 4, 3)
    tq, tk, tv, ta, tb, ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True)
                              for x in (q, k, v, a, b, s0)]
    S = ts
    ys = []
    for t in range(q.shape[0]):
        St = ta[t] * S
        e = tv[t] - St.T @ tk[t]
        S = St + tb[t] * torch.outer(tk[t], e)
        ys.append(S.T @ tq[t])
    L = (torch.stack(ys) * torch.tensor(dy)).sum() + (S * torch.tensor(dsT)).sum()
    L.backward()
    g = bwd(q, k, v, a, b, s0, dy, dsT)
    for name, t in zip(["dq", "dk", "dv", "dalpha", "dbeta", "ds0"], [tq, tk, tv, ta, tb, ts]):
        _close(g[name], t.grad.numpy(), 1e-12, "autograd, " + name)


def pin_bwd_adjoint_identities(bwd):
    # (y, S_T) is linear in (V, S0) for fixed q, k, alpha, beta, so the adjoint map satisfies
    # <dV, V> + <dS0, S0> = <dy, y> + <dS_T, S_T>; and y_t = S_t^T q_t is linear in q_t with
    # the states fixed, so <dq, q> = <dy, y>.
    rng = np.random.default_rng(303)
    q, k, v, a, b, s0, dy, dsT = _chain(rng, 40, 5, 4)
    y, S = oracle.chain_numpy(q, k, v, a, b, s0)
    g = bwd(q, k, v, a, b, s0, dy, dsT)
    lhs = np.sum(g["dv"] * v) + np.sum(g["ds0"] * s0)
    rhs = np.sum(dy * y) + np.sum(dsT * S)
    assert abs(lhs - rhs) <= 1e-11 * (abs(rhs) + np.abs(dy * y).sum()), (lhs, rhs)
    lq = np.sum(g["dq"] * q)
    rq = np.sum(dy * y)
    assert abs(lq - rq) <= 1e-11 * np.abs(dy * y).sum(), (lq, rq)


def pin_bwd_beta_zero(bwd):
    # beta = 0: S_t = gamma_t S0 with gamma_t = prod_{s<=t} alpha_s, so
    #   y_t = gamma_t S0^T q_t,  dq_t = gamma_t S0 dy_t,  dk = dv = 0,
    #   dS0 = sum_t gamma_t q_t dy_t^T + gamma_T dS_T,
    #   dalpha_s = (1/alpha_s) [sum_{t>=s} gamma_t <S0^T q_t, dy_t> + gamma_T <S0, dS_T>],
    #   dbeta_t = k_t^T D_t e_t with D_t = sum_{r>=t} (gamma_r/gamma_t) q_r dy_r^T
    #             + (gamma_T/gamma_t) dS_T and e_t = v_t - gamma_t S0^T k_t.
    rng = np.random.default_rng(404)
    q, k, v, a, b, s0, dy, dsT = _chain(rng, 12, 4, 3)
    b = np.zeros_like(b)
    T = q.shape[0]
    gam = np.cumprod(a)
    g = bwd(q, k, v, a, b, s0, dy, dsT)
    _close(g["dq"], gam[:, None] * (dy @ s0.T), 1e-13, "beta=0 dq")
    assert np.all(g["dk"] == 0) and np.all(g["dv"] == 0), "beta=0: dk and dv must vanish"
    ds0 = sum(gam[t] * np.outer(q[t], dy[t]) for t in range(T)) + gam[-1] * dsT
    _close(g["ds0"], ds0, 1e-13, "beta=0 dS0")
    r = np.array([np.dot(s0.T @ q[t], dy[t]) for t in range(T)])
    tail = np.cumsum((gam * r)[::-1])[::-1] + gam[-1] * np.sum(s0 * dsT)
    _close(g["dalpha"], tail / a, 1e-13, "beta=0 dalpha")
    db = np.zeros(T)
    for t in range(T):
        D = sum((gam[r_] / gam[t]) * np.outer(q[r_], dy[r_]) for r_ in range(t, T))
        D = D + (gam[-1] / gam[t]) * dsT
        e = v[t] - gam[t] * (s0.T @ k[t])
        db[t] = k[t] @ D @ e
    _close(g["dbeta"], db, 1e-12, "beta=0 dbeta")


PINS = [pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_adjoint_identities,
        pin_bwd_beta_zero]


@pytest.fixture(params=["c", "numpy"])
def bwd(request, oracle_lib):
    return oracle.chain_backward_c if request.param == "c" else oracle.chain_backward_numpy


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(bwd, pin):
    pin(bwd)


def test_c_and_numpy_agree_on_a_long_chain(oracle_lib):
    # several kept-state blocks of the C backward, a ragged last block
    rng = np.random.default_rng(505)
    args = _chain(rng, 200, 6, 5, a_lo=0.8)
    gc = oracle.chain_backward_c(*args)
    gn = oracle.chain_backward_numpy(*args)
    for name in gn:
        _close(gc[name], gn[name], 1e-12, "C vs numpy, " + name)


def test_packed_backward_equals_per_sequence(oracle_lib):
    rng = np.random.default_rng(606)
    lens = [0, 70, 1, 130]
    cu = np.concatenate([[0], np.cumsum(lens)])
    R, H, dk, dv = int(cu[-1]), 2, 4, 3
    q = rng.normal(size=(R, H, dk))
    k = rng.normal(size=(R, H, dk)) / 2
    v = rng.normal(size=(R, H, dv))
    a = rng.uniform(0.5, 1, size=(R, H))
    b = rng.uniform(0, 1, size=(R, H))
    s0 = rng.normal(size=(len(lens), H, dk, dv))
    dsT = rng.normal(size=(len(lens), H, dk, dv))
    dy = rng.normal(size=(R, H, dv))
    o = oracle.prefill_backward(q, k, v, a, b, dy, cu_seqlens=cu, s0=s0, ds_final=dsT)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        for h in range(H):
            g = oracle.chain_backward_numpy(q[s:e, h], k[s:e, h], v[s:e, h], a[s:e, h],
                                            b[s:e, h], s0[n, h], dy[s:e, h], dsT[n, h])
            for name in ["dq", "dk", "dv"]:
                np.testing.assert_allclose(o[name][s:e, h], g[name], rtol=1e-12, atol=1e-12)
            for name in ["dalpha", "dbeta"]:
                np.testing.assert_allclose(o[name][s:e, h], g[name], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(o["ds0"][n, h], g["ds0"], rtol=1e-12, atol=1e-12)
    # an empty sequence passes the final-state adjoint straight through
    np.testing.assert_array_equal(o["ds0"][0], dsT[0])


# ---- mutants: the reverse pass with one planted mistake each -------------------------------

def _mutant_bwd(mut):
    def bwd(q, k, v, alpha, beta, s0, dy, ds_final):
        T, dk = k.shape
        dv = v.shape[1]
        S = [np.array(s0, dtype=np.float64)]
        for t in range(T):
            St = alpha[t] * S[-1]
            e = v[t] - St.T @ k[t]
            S.append(St + beta[t] * np.outer(k[t], e))
        D = np.zeros((dk, dv)) if (ds_final is None or mut == "ignores_final_adjoint") \
            else np.array(ds_final, dtype=np.float64)
        out = dict(dq=np.zeros((T, dk)), dk=np.zeros((T, dk)), dv=np.zeros((T, dv)),
                   dalpha=np.zeros(T), dbeta=np.zeros(T))
        for t in range(T - 1, -1, -1):
            a, b = alpha[t], beta[t]
            if mut != "query_added_after_write":
                D = D + np.outer(q[t], dy[t])
            out["dq"][t] = (S[t] if mut == "dq_from_previous_state" else S[t + 1]) @ dy[t]
            St = a * S[t]
            e = v[t] - St.T @ k[t]
            de = (1.0 if mut == "dv_without_beta" else b) * (D.T @ k[t])
            out["dbeta"][t] = k[t] @ D @ (v[t] if mut == "dbeta_against_v" else e)
            out["dv"][t] = de
            erase = (S[t] if mut == "erase_with_undecayed_state" else St) @ de
            out["dk"][t] = b * (D @ e) - (0.0 if mut == "dk_without_erase" else erase)
            dSt = D - np.outer(k[t], de)
            if mut == "dalpha_against_updated_state":
                out["dalpha"][t] = np.sum(dSt * S[t + 1])
            elif mut == "dalpha_without_erase":
                out["dalpha"][t] = np.sum(D * S[t])
            else:
                out["dalpha"][t] = np.sum(dSt * S[t])
            D = dSt if mut == "adjoint_not_decayed" else a * dSt
            if mut == "query_added_after_write":
                D = D + a * np.outer(q[t], dy[t])
        out["ds0"] = D
        return out
    return bwd


MUTANTS = ["dq_from_previous_state", "dk_without_erase", "erase_with_undecayed_state",
           "dalpha_against_updated_state", "dalpha_without_erase", "dbeta_against_v",
           "adjoint_not_decayed", "dv_without_beta", "query_added_after_write",
           "ignores_final_adjoint"]


def test_unmutated_copy_passes_every_pin():
    for pin in PINS:
        pin(_mutant_bwd(None))


@pytest.mark.parametrize("name", MUTANTS)
def test_every_backward_mutant_fails_a_pin(name):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant_bwd(name))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passes every pin" % name

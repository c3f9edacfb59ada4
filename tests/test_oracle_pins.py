"""The oracle against what the pages and the mathematics fix (CPU only).

Every pin runs against both oracle implementations (the C one used at scale and the numpy
one).  A mutation test then checks that each plausible mistake in the recurrence fails at
least one pin, so the pins can tell a right oracle from a wrong one.
"""
import numpy as np
import pytest

import pins
from checkers import MUTANTS



@pytest.fixture(scope="module", params=["c", "numpy"])
def impl(request, oracle_lib):
    return oracle_lib.chain_c if request.param == "c" else oracle_lib.chain_numpy


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(impl, pin):
    pin(impl)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_fails_a_pin(name):
    mutant = MUTANTS[name]
    caught = []
    for pin in pins.PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passes every pin" % name


def test_undecayed_residual_is_a_different_recurrence(oracle_lib):
    """The one-token snippet on the ta-paperlens walkthrough ("Inside GDN") takes the residual
    against the undecayed state.  The reading notes' recurrence (section 2.1) and its boxed
    transition form do not; the oracle follows the latter, so the two must differ visibly
    once alpha < 1 (a negative control, not a pin)."""
    rng = np.random.default_rng(3)
    T, dk, dv = 64, 16, 8
    q, k, v, a, b, s0 = pins._rand_chain(rng, T, dk, dv, a_lo=0.6, a_hi=0.95)
    y, S = oracle_lib.chain_c(q, k, v, a, b, s0)
    y2, S2 = MUTANTS["undecayed_residual"](q, k, v, a, b, s0)
    assert np.max(np.abs(S - S2)) > 1e-2 * np.max(np.abs(S))


# ---- the C oracle's batch interface -------------------------------------------------------

def _rand_batch(rng, lengths, H, dk, dv, dtype=np.float64):
    rows = int(sum(lengths))
    q = rng.standard_normal((rows, H, dk))
    k = rng.standard_normal((rows, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((rows, H, dv))
    a = rng.uniform(0.5, 1.0, (rows, H))
    b = rng.uniform(0.0, 1.0, (rows, H))
    s0 = rng.standard_normal((len(lengths), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q.astype(dtype), k.astype(dtype), v.astype(dtype), a, b, s0, cu


def test_packed_varlen_equals_per_sequence(oracle_lib):
    """Packed sequences never see each other's tokens: each restarts from its own S0."""
    rng = np.random.default_rng(4)
    lengths = [5, 0, 13, 1, 9]
    H, dk, dv = 3, 6, 4
    q, k, v, a, b, s0, cu = _rand_batch(rng, lengths, H, dk, dv)
    y, sf = oracle_lib.prefill(q, k, v, a, b, cu, s0=s0, threads=3)
    for n in range(len(lengths)):
        r0, r1 = cu[n], cu[n + 1]
        for h in range(H):
            ey, eS = oracle_lib.chain_numpy(q[r0:r1, h], k[r0:r1, h], v[r0:r1, h],
                                            a[r0:r1, h], b[r0:r1, h], s0[n, h])
            np.testing.assert_allclose(y[r0:r1, h], ey, rtol=0, atol=1e-13)
            np.testing.assert_allclose(sf[n, h], eS, rtol=0, atol=1e-13)
    # zero-length sequence: the final state is S0 itself
    assert np.array_equal(sf[1], s0[1])


def test_decode_stack_equals_prefill(oracle_lib):
    """T single-token steps equal one T-token prefill of the same sequence."""
    rng = np.random.default_rng(5)
    steps, B, H, dk, dv = 7, 3, 2, 5, 4
    q, k, v, a, b, s0, _ = _rand_batch(rng, [steps * B], H, dk, dv)
    s0 = rng.standard_normal((B, H, dk, dv))
    yd, sd = oracle_lib.decode(q.reshape(steps, B, H, dk), k.reshape(steps, B, H, dk),
                               v.reshape(steps, B, H, dv), a.reshape(steps, B, H),
                               b.reshape(steps, B, H), s0)
    for bb in range(B):
        sel = slice(bb, None, B)
        yp, sp = oracle_lib.prefill(q[sel], k[sel], v[sel], a[sel], b[sel], None,
                                    s0=s0[bb:bb + 1])
        np.testing.assert_array_equal(yd[:, bb], yp)
        np.testing.assert_array_equal(sd[bb], sp[0])


def test_head_subset_and_threads_are_bitwise_stable(oracle_lib):
    rng = np.random.default_rng(6)
    lengths = [11, 7]
    q, k, v, a, b, s0, cu = _rand_batch(rng, lengths, 4, 5, 3)
    y1, s1 = oracle_lib.prefill(q, k, v, a, b, cu, s0=s0, threads=1)
    y4, s4 = oracle_lib.prefill(q, k, v, a, b, cu, s0=s0, threads=4)
    ys, ss = oracle_lib.prefill(q, k, v, a, b, cu, s0=s0, heads=(1, 3), threads=2)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(s1, s4)
    np.testing.assert_array_equal(ys, y1[:, 1:3])
    np.testing.assert_array_equal(ss, s1[:, 1:3])


def test_bf16_and_f32_inputs_widen_exactly(oracle_lib):
    """bf16 bit patterns and fp32 values reach the recurrence unchanged."""
    from linear_attention_recurrence_chunked_amd.workloads import bf16_bits, bf16_to_f64
    rng = np.random.default_rng(7)
    q, k, v, a, b, s0, cu = _rand_batch(rng, [9, 4], 2, 8, 8)
    for conv, back in ((bf16_bits, bf16_to_f64),
                       (lambda x: x.astype(np.float32), lambda x: x.astype(np.float64))):
        qs, ks, vs = conv(q), conv(k), conv(v)
        y1, s1 = oracle_lib.prefill(qs, ks, vs, a, b, cu, s0=s0)
        y2, s2 = oracle_lib.prefill(back(qs), back(ks), back(vs), a, b, cu, s0=s0)
        np.testing.assert_array_equal(y1, y2)
        np.testing.assert_array_equal(s1, s2)


def test_bf16_rounding_is_round_to_nearest_even():
    from linear_attention_recurrence_chunked_amd.workloads import bf16_bits, bf16_to_f64
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties go to 1 + 2^-6
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0, 1.0 + 2.0 ** -7])
    got = bf16_to_f64(bf16_bits(x))
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2.0 ** -6, -2.5, 0.0, 1.0 + 2.0 ** -7])


def test_placed_step_at_the_rule_is_the_oracle(oracle_lib):
    """The mutants' shared step, at the rule's own placement (residual against the decayed
    state, decay before the write), reproduces the oracle; so the misplaced settings differ
    from it by the placement alone."""
    from checkers import _mutant, _placed_step
    rng = np.random.default_rng(4)
    q, k, v, a, b, s0 = pins._rand_chain(rng, 48, 16, 8, a_lo=0.6, a_hi=0.95)
    y, S = oracle_lib.chain_c(q, k, v, a, b, s0)
    y2, S2 = _mutant(_placed_step("decayed", "before"))(q, k, v, a, b, s0)
    assert np.allclose(y2, y, rtol=1e-12, atol=1e-12 * np.max(np.abs(y)))
    assert np.allclose(S2, S, rtol=1e-12, atol=1e-12 * np.max(np.abs(S)))

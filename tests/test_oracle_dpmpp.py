"""Pins of the oracle's DPM++ 2M sampler (reading S22), CPU only.

What fixes them, beyond the oracle's own formulas:
  - exactness on a straight path: with the exact velocity of a single data
    point, (x - x0) / sigma, every step lands on (1 - sigma) x0 + sigma eps and
    the last on x0 (float64 rounding);
  - the method's order: on Gaussian data, whose probability-flow solution is
    known in closed form, the final error falls ~4x per halving of the step
    (second order) where Euler's falls ~2x, and a single step at a strongly
    non-uniform step ratio has O(h^3) local error; planted mistakes in the
    second-order term (sign, r inverted, dropped) fall to O(h^2);
  - the fp32 update rounds each operation once in the stated order (exact
    rational arithmetic);
  - the library's host coefficients equal the oracle's after rounding to fp32
    on the FlowMatch schedules (host logic, no GPU)."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import dit
from tests.oracle_plant import planted

MU, SD = 0.7, 0.3


def _gauss_vel(x, sg):
    # velocity dx/dsigma of the probability-flow ODE for data N(MU, SD^2)
    a = 1.0 - sg
    q = math.sqrt(a * a * SD * SD + sg * sg)
    return -MU + (-a * SD * SD + sg) / q * ((x - a * MU) / q)


def _gauss_err(sample, K, end=0.05):
    z = np.linspace(-3, 3, 101)
    sig = np.linspace(1.0, end, K + 1)
    a = 1.0 - end
    exact = a * MU + math.sqrt(a * a * SD * SD + end * end) * z
    return float(np.abs(sample(_gauss_vel, z.copy(), sig) - exact).max())


def _euler_sample(vel_fn, x, sigmas):
    for i in range(len(sigmas) - 1):
        x = x + (sigmas[i + 1] - sigmas[i]) * vel_fn(x, sigmas[i])
    return x


def test_straight_path_is_exact():
    rng = np.random.default_rng(0)
    x0, eps = rng.standard_normal(64), rng.standard_normal(64)
    sig, _ = dit.flow_sigmas(20, 4096)
    sig = sig.astype(np.float64)
    x = eps.copy()
    x0_prev, s_prev = None, None
    for i in range(20):
        a, b, c1, c2, order = dit.dpmpp_2m_coeffs(s_prev, sig[i], sig[i + 1])
        pred = x - sig[i] * ((x - x0) / sig[i])
        d = pred if order == 1 else c1 * pred - c2 * x0_prev
        x = a * x - b * d
        x0_prev, s_prev = pred, sig[i]
        target = (1.0 - sig[i + 1]) * x0 + sig[i + 1] * eps
        assert np.allclose(x, target, rtol=0, atol=1e-12), i
    assert np.allclose(x, x0, rtol=0, atol=1e-12)


def test_second_order_convergence():
    e40, e80 = _gauss_err(dit.dpmpp_2m_sample, 40), _gauss_err(dit.dpmpp_2m_sample, 80)
    u40, u80 = _gauss_err(_euler_sample, 40), _gauss_err(_euler_sample, 80)
    assert e40 / e80 > 3.5, (e40, e80)
    assert 1.8 < u40 / u80 < 2.2, (u40, u80)
    assert e80 < u80 / 5


def _local_err(coeffs, h, r=3.0):
    """One second-order step from exact trajectory points at lambda = -r h and
    0 to lambda = h (a strongly non-uniform step ratio r), against the exact
    solution."""
    def sig_of(lam):
        return 1.0 / (1.0 + math.exp(lam))

    def exact_x(z, s):
        a = 1.0 - s
        return a * MU + math.sqrt(a * a * SD * SD + s * s) * z

    z = np.linspace(-3, 3, 41)
    sp, sc, sn = sig_of(-r * h), sig_of(0.0), sig_of(h)
    xp, xc = exact_x(z, sp), exact_x(z, sc)
    x0p, x0c = xp - sp * _gauss_vel(xp, sp), xc - sc * _gauss_vel(xc, sc)
    a, b, c1, c2, order = coeffs(sp, sc, sn)
    assert order == 2
    return float(np.abs(a * xc - b * (c1 * x0c - c2 * x0p) - exact_x(z, sn)).max())


def _local_ratio(coeffs):
    return _local_err(coeffs, 0.1) / _local_err(coeffs, 0.05)


def test_local_error_is_third_order_at_any_step_ratio():
    """A multistep second-order method has O(h^3) local error whatever the
    step ratio: ~8x per halving."""
    assert _local_ratio(dit.dpmpp_2m_coeffs) > 7.0


@pytest.mark.parametrize("old,new", [("c2 = 1.0 / (2.0 * r)", "c2 = -1.0 / (2.0 * r)"),
                                     ("c2 = 1.0 / (2.0 * r)", "c2 = r / 2.0"),
                                     ("c2 = 1.0 / (2.0 * r)", "c2 = 0.0 * r")])
def test_planted_second_order_mistakes_fail(old, new):
    """A wrong sign, an inverted step ratio or a dropped correction each fall
    to O(h^2) local error (~4x)."""
    bad = planted(dit.dpmpp_2m_coeffs, old, new)
    assert _local_ratio(bad) < 5.0


def test_fp32_step_rounds_each_op():
    rng = np.random.default_rng(1)
    x, v, xp = (rng.standard_normal(512).astype(np.float32) for _ in range(3))
    sig, _ = dit.flow_sigmas(30, 1024)
    for i in (0, 1, 5, 29):
        prev = None if i == 0 else sig[i - 1]
        got, x0 = dit.dpmpp_2m_step(x, v, xp, prev, sig[i], sig[i + 1])
        coef = dit.dpmpp_2m_coeffs(prev, sig[i], sig[i + 1])
        a, b, c1, c2 = (np.float32(c) for c in coef[:4])
        order = coef[4]
        r32 = lambda q: np.float32(float(q))  # noqa: E731  (the rational is exact in float64 here)
        F = lambda v_: Fraction(float(v_))     # noqa: E731
        for j in range(0, 512, 7):
            p = r32(F(sig[i]) * F(v[j]))
            pred = r32(F(x[j]) - F(p))
            assert x0[j] == pred
            d = pred if order == 1 else r32(F(r32(F(c1) * F(pred))) - F(r32(F(c2) * F(xp[j]))))
            want = r32(F(r32(F(a) * F(x[j]))) - F(r32(F(b) * F(d))))
            assert got[j] == want, (i, j)


def test_library_host_coefficients_match_oracle():
    import block_causal_attention_qi_amd as qi
    for steps, n in ((40, 4096), (25, 4096), (6, 64), (40, 16384)):
        sig, _ = qi.flow_sigmas(steps, n)
        prev = None
        for i in range(steps):
            got = qi.dpmpp_2m_coeffs(prev, sig[i], sig[i + 1])
            ref = dit.dpmpp_2m_coeffs(prev, sig[i], sig[i + 1])
            assert got[4] == ref[4]
            assert all(np.float32(g) == np.float32(r) for g, r in zip(got[:4], ref[:4])), (steps, n, i, got, ref)
            prev = sig[i]
    with pytest.raises(qi.QiError):
        qi.dpmpp_2m_coeffs(None, 0.5, 0.6)    # sigma must decrease

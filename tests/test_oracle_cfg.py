"""Pins of the oracle's true-CFG combination and its Euler update (CPU only).

What fixes them: the formula the MLX page gives for true CFG ("Optional
modes": noise = neg + g * (pos - neg)) read as fp32 operations in the written
order (reading S20), checked against exact rational arithmetic; special cases
the formula reduces to (g = 0 gives the negative branch, equal branches give
that branch for any g); and the S14 Euler update it feeds."""
from fractions import Fraction

import numpy as np

from oracle import dit
from tests.oracle_plant import planted


def _f(v) -> Fraction:
    return Fraction(float(v))


def _r32(q: Fraction) -> np.float32:
    # round a rational to the nearest fp32 (through float64: the values here
    # are exact in float64 before the single rounding to fp32)
    return np.float32(float(q))


def _inputs(n=2048, seed=0):
    rng = np.random.default_rng(seed)
    pos = rng.standard_normal(n).astype(np.float32)
    neg = (pos + 0.3 * rng.standard_normal(n)).astype(np.float32)
    return pos, neg


def _rational_mismatches(fn, pos, neg, g) -> int:
    got = fn(pos, neg, g)
    g32 = np.float32(g)
    bad = 0
    for i in range(0, len(pos), 5):
        d = _r32(_f(pos[i]) - _f(neg[i]))            # exact in float64, one rounding
        gd = _r32(_f(g32) * _f(d))                   # product of two fp32: exact in float64
        want = _r32(_f(neg[i]) + _f(gd))             # sum of two fp32: exact in float64
        bad += int(got[i] != want)
    return bad


def test_cfg_combine_rounds_each_op_in_order():
    pos, neg = _inputs()
    for g in (2.5, -0.75, 7.0, 1.0):
        assert _rational_mismatches(dit.cfg_combine, pos, neg, g) == 0, g


def test_cfg_special_cases():
    pos, neg = _inputs()
    assert np.array_equal(dit.cfg_combine(pos, neg, 0.0), neg)           # g = 0: the negative branch
    for g in (0.5, 2.5, -3.0):
        assert np.array_equal(dit.cfg_combine(pos, pos, g), pos)         # equal branches
    # g = 1 gives pos up to the two roundings
    one = dit.cfg_combine(pos, neg, 1.0).astype(np.float64)
    bound = 2 * np.finfo(np.float32).eps * (np.abs(pos) + np.abs(neg)).astype(np.float64)
    assert np.all(np.abs(one - pos) <= bound)


def test_cfg_euler_reduces_to_plain_euler():
    pos, neg = _inputs()
    x = np.random.default_rng(3).standard_normal(len(pos)).astype(np.float32)
    sc, sn = np.float32(0.7), np.float32(0.675)
    assert np.array_equal(dit.euler_update_cfg(x, pos, neg, 0.0, sc, sn), dit.euler_update(x, neg, sc, sn))
    assert np.array_equal(dit.euler_update_cfg(x, pos, pos, 4.0, sc, sn), dit.euler_update(x, pos, sc, sn))
    noise = dit.cfg_combine(pos, neg, 2.5)
    assert np.array_equal(dit.euler_update_cfg(x, pos, neg, 2.5, sc, sn), dit.euler_update(x, noise, sc, sn))


def test_cfg_pins_catch_planted_mistakes():
    """Swapped branches, the wrong base term and a combination rounded only
    once (float64 inside) each fail one of the pins above."""
    pos, neg = _inputs()
    swapped = planted(dit.cfg_combine, "d = (pos - neg)", "d = (neg - pos)")
    assert _rational_mismatches(swapped, pos, neg, 2.5) > 0
    wrong_base = planted(dit.cfg_combine, "return (neg + gd)", "return (pos + gd)")
    assert not np.array_equal(wrong_base(pos, neg, 0.0), neg)
    once = planted(dit.cfg_combine, "d = (pos - neg).astype(F32)\n    gd = (F32(g) * d).astype(F32)",
                   "d = pos.astype(np.float64) - neg\n    gd = np.float64(g) * d")
    assert _rational_mismatches(once, pos, neg, 2.5) > 0

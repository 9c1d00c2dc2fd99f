"""Pins of the oracle's FlowMatch Euler schedule and Euler update (CPU only).

What fixes them: the values the pages print (mu at three sizes, sigma_1 at
256^2, the terminal value 0.02, 41 sigmas ending in 0) and exact rational
arithmetic for the fp32 rounding of the Euler step."""
import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import dit

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


def test_mu_printed_values():
    g = GOLD["mu"]
    for n, v in g["values"].items():
        digits = g["digits_printed"][n]
        got = dit.flow_mu(int(n))
        # the pages truncate ("0.5387..."): the printed digits must be a prefix
        assert math.floor(got * 10 ** digits) / 10 ** digits == v, (n, got)


def test_sigma1_at_256_printed():
    g = GOLD["sigma1_256"]
    s, ts = dit.flow_sigmas(GOLD["steps"]["value"], 256)
    assert abs(float(s[1]) - g["value"]) < g["tol"]
    # and it is NOT the unshifted linspace value
    assert abs(float(s[1]) - g["linspace_value"]) > 5e-3


def test_schedule_shape_and_ends():
    steps = GOLD["steps"]["value"]
    for n in (64, 256, 1024, 4096, 16384):
        s, ts = dit.flow_sigmas(steps, n)
        assert s.dtype == np.float32 and ts.dtype == np.float32
        assert s.shape == (steps + 1,) and ts.shape == (steps,)
        assert s[0] == 1.0 and s[-1] == 0.0
        assert abs(float(s[-2]) - GOLD["shift_terminal"]["value"]) < 1e-6
        assert np.all(np.diff(s) < 0)
        assert np.array_equal(ts, s[:-1] * np.float32(1000))


def test_shift_grows_with_resolution():
    s256, _ = dit.flow_sigmas(40, 256)
    s4096, _ = dit.flow_sigmas(40, 4096)
    assert np.all(s4096[1:-2] > s256[1:-2])


def test_timestep_input_is_ts_over_1000_in_fp32():
    _, ts = dit.flow_sigmas(40, 4096)
    for i in (0, 20, 39):
        t = dit.timestep_input(ts, i)
        assert isinstance(t, np.float32)
        assert t == np.float32(ts[i]) / np.float32(1000)


def test_euler_update_rounds_each_op_to_fp32():
    """x + (s_next - s_cur) * vel with every operation rounded to fp32: check
    against exact rational arithmetic and a planted fused multiply-add."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4096).astype(np.float32)
    vel = rng.standard_normal(4096).astype(np.float32)
    sc, sn = np.float32(0.98696375), np.float32(0.9684019)
    got = dit.euler_update(x, vel, sc, sn)
    ds = Fraction(float(sn)) - Fraction(float(sc))
    ds32 = Fraction(float(np.float32(float(ds))))
    n_fma_diff = 0
    for i in range(0, 4096, 7):
        prod = ds32 * Fraction(float(vel[i]))
        # the product of two fp32 values is exact in float64, so rounding the
        # float64 value to fp32 is the correctly rounded fp32 product
        p32 = Fraction(float(np.float32(float(prod))))
        s = Fraction(float(x[i])) + p32
        r = np.float32(float(s))   # x + p32 is exact in float64 here
        assert got[i] == r
        fused = np.float32(float(Fraction(float(x[i])) + prod))
        n_fma_diff += int(fused != r)
    assert n_fma_diff > 0   # the fused form is distinguishable on these inputs

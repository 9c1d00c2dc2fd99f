"""Pins of the oracle's RoPE tables, positions and rotation (CPU only).

What fixes them: the host contract's section 4 (positions, table rows, the
polar formula, axis 1 == axis 2, the h = 16 example) and the mathematics of
rotations (pos 0 is the identity, odd/even symmetry, relative positions)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dit

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


def _ulp_diff(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    # map sign-magnitude to a monotone integer line
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def test_table_shapes_and_rows():
    g = GOLD["rope_table"]
    for d, wdt in zip(g["axis_dims"], g["widths"]):
        c, s = dit.rope_axis_table(d)
        assert c.shape == (g["rows"], wdt) and s.shape == (g["rows"], wdt)
        assert c.dtype == np.float32 and s.dtype == np.float32


def test_position_zero_is_identity():
    for d in (16, 56):
        c, s = dit.rope_axis_table(d)
        r0 = 0 - dit.ROPE_POS_MIN
        assert np.all(c[r0] == 1.0) and np.all(s[r0] == 0.0)


def test_first_frequency_is_one():
    # k = 0 has 1/10000^0 = 1: the angle is the integer position itself.
    c, s = dit.rope_axis_table(56)
    pos = np.arange(dit.ROPE_POS_MIN, dit.ROPE_POS_MAX + 1)
    for p in (-1024, -7, -1, 1, 2, 3, 100, 4095, 8191):
        r = p - dit.ROPE_POS_MIN
        assert c[r, 0] == np.float32(math.cos(p)) and s[r, 0] == np.float32(math.sin(p))
    assert len(pos) == c.shape[0]


def test_closed_form_second_frequency():
    # d = 16, k = 1: 10000^(-2/16) = 10^(-1/2) exactly in real arithmetic.
    c, s = dit.rope_axis_table(16)
    r1 = 1 - dit.ROPE_POS_MIN
    w = 10.0 ** -0.5
    assert abs(float(c[r1, 1]) - math.cos(w)) < 2e-7
    assert abs(float(s[r1, 1]) - math.sin(w)) < 2e-7
    # d = 56, last column: 10000^(-54/56)
    c56, s56 = dit.rope_axis_table(56)
    w = 10000.0 ** (-54 / 56)
    r5 = 5 - dit.ROPE_POS_MIN
    assert abs(float(s56[r5, 27]) - math.sin(5 * w)) < 2e-7


def test_odd_even_symmetry_exact():
    for d in (16, 56):
        c, s = dit.rope_axis_table(d)
        for p in range(1, 1025):
            rp, rn = p - dit.ROPE_POS_MIN, -p - dit.ROPE_POS_MIN
            assert np.array_equal(c[rp], c[rn])
            assert np.array_equal(s[rp], -s[rn])


def test_axis1_axis2_byte_identical():
    a1 = dit.rope_axis_table(56)
    a2 = dit.rope_axis_table(56)
    assert a1[0].tobytes() == a2[0].tobytes() and a1[1].tobytes() == a2[1].tobytes()


def test_matches_torch_polar_within_one_ulp():
    """The host contract defines the tables as torch.polar(1, outer(pos,
    1/10000^(arange(0,d,2)/d))).  torch's CPU cos/sin are not correctly
    rounded, so the pin is <= 1 ulp, with the count of differing values
    reported."""
    pos = torch.arange(dit.ROPE_POS_MIN, dit.ROPE_POS_MAX + 1)
    for d in (16, 56):
        freqs = 1.0 / torch.pow(10000, torch.arange(0, d, 2).to(torch.float32) / d)
        ang = torch.outer(pos.to(torch.float32), freqs)
        z = torch.polar(torch.ones_like(ang), ang)
        tc, ts = z.real.numpy(), z.imag.numpy()
        c, s = dit.rope_axis_table(d)
        assert _ulp_diff(c, tc).max() <= 1
        assert _ulp_diff(s, ts).max() <= 1
        frac = float(((c != tc) | (s != ts)).mean())
        assert frac < 0.05, frac


def test_positions_printed_example():
    g = GOLD["image_rows_h16"]
    txt, img = dit.token_positions(L=22, h=g["h"], w=g["h"])
    assert img[:, 1].min() == g["rows"][0] and img[:, 1].max() == g["rows"][1]
    assert img[:, 2].min() == g["rows"][0] and img[:, 2].max() == g["rows"][1]
    assert np.all(img[:, 0] == 22)                      # frame position = L
    assert np.array_equal(txt, np.stack([np.arange(22)] * 3, axis=1))
    # raster order: token index y*w + x
    y, x = 3, 5
    assert tuple(img[y * 16 + x]) == (22, 3 - 8, 5 - 8)


def test_positions_odd_grid():
    _, img = dit.token_positions(L=9, h=5, w=3)
    # h - h//2 = 3 -> rows -3..1 ; w - w//2 = 2 -> cols -2..0
    assert img[:, 1].min() == -3 and img[:, 1].max() == 1
    assert img[:, 2].min() == -2 and img[:, 2].max() == 0


def test_rope_rows_concatenation():
    L, h, w = 22, 16, 16
    tc, ts, ic, is_ = dit.rope_rows(L, h, w)
    assert tc.shape == (L, 64) and ic.shape == (h * w, 64)
    a0, a1 = dit.rope_axis_table(16), dit.rope_axis_table(56)
    tok = 3 * w + 5
    exp_c = np.concatenate([a0[0][L + 1024], a1[0][-5 + 1024], a1[0][-3 + 1024]])
    exp_s = np.concatenate([a0[1][L + 1024], a1[1][-5 + 1024], a1[1][-3 + 1024]])
    assert np.array_equal(ic[tok], exp_c) and np.array_equal(is_[tok], exp_s)
    i = 7
    assert np.array_equal(tc[i], np.concatenate([a0[0][i + 1024], a1[0][i + 1024], a1[0][i + 1024]]))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rope_apply_equals_complex_multiply():
    T, heads = 12, 3
    x = _rand((T, heads, 128), 1)
    tc, ts, ic, is_ = dit.rope_rows(4, 2, 4)
    cos = np.concatenate([tc, ic])[:T]
    sin = np.concatenate([ts, is_])[:T]
    got = dit.rope_apply(x, cos, sin)
    xc = torch.view_as_complex(torch.from_numpy(x.reshape(T, heads, 64, 2)).contiguous())
    rot = torch.complex(torch.from_numpy(cos.astype(np.float64)), torch.from_numpy(sin.astype(np.float64)))
    ref = torch.view_as_real(xc * rot[:, None, :]).reshape(T, heads, 128).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def test_rope_apply_preserves_pair_norm():
    x = _rand((5, 2, 128), 2)
    tc, ts, _, _ = dit.rope_rows(5, 1, 1)
    y = dit.rope_apply(x, tc, ts)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(nx - ny)) < 1e-5 * np.max(nx)


def test_rope_relative_position():
    """<R(p) q, R(p') k> depends on p - p' only, per axis (fp32 tables)."""
    tabs = [dit.rope_axis_table(d) for d in dit.ROPE_AXES]

    def row(p3):
        c = np.concatenate([tabs[a][0][p3[a] + 1024] for a in range(3)])[None]
        s = np.concatenate([tabs[a][1][p3[a] + 1024] for a in range(3)])[None]
        return c, s

    q = _rand((1, 1, 128), 3)
    k = _rand((1, 1, 128), 4)
    d0 = None
    for base in [(0, 0, 0), (5, -3, 2), (40, 7, -11)]:
        p = base
        pp = (base[0] + 3, base[1] - 2, base[2] + 4)
        rq = dit.rope_apply(q, *row(p))
        rk = dit.rope_apply(k, *row(pp))
        dot = float(np.sum(rq * rk))
        if d0 is None:
            d0 = dot
        assert abs(dot - d0) < 1e-4 * max(1.0, abs(d0))


def test_negative_control_rotate_half_fails_complex_pin(monkeypatch):
    """A plausible mistake (rotate-half pairing instead of adjacent pairs)
    must fail the complex-multiply pin."""
    def rotate_half(x, cos, sin):
        c = cos[:, None, :]
        s = sin[:, None, :]
        a, b = x[..., :64], x[..., 64:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)

    T, heads = 6, 2
    x = _rand((T, heads, 128), 5)
    tc, ts, _, _ = dit.rope_rows(T, 1, 1)
    xc = torch.view_as_complex(torch.from_numpy(x.reshape(T, heads, 64, 2)).contiguous())
    rot = torch.complex(torch.from_numpy(tc.astype(np.float64)), torch.from_numpy(ts.astype(np.float64)))
    ref = torch.view_as_real(xc * rot[:, None, :]).reshape(T, heads, 128).numpy()
    assert np.max(np.abs(rotate_half(x, tc, ts) - ref)) > 1e-2

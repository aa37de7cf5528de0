"""Pins for the oracle's NVFP4 fake quantization (CPU only).

Each check ties ``oracle.nvfp4`` to something other than itself: a library's
E4M3 cast, exact rational arithmetic (``fractions.Fraction``) on exhaustive and
random groups, hand-derived tie cases (tests/golden/nvfp4_ties.json) and closed
forms of the format (grid membership, odd symmetry, the group maximum landing on
6 * scale, idempotence where it holds).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4
from synthetic import f32_from_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_ties.json")

E2M1_EXACT = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
              Fraction(3), Fraction(4), Fraction(6)]


def _e4m3_exact_grid():
    # Independent enumeration from the bit fields via Fraction arithmetic.
    out = []
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            out.append(Fraction(m, 512))
        else:
            out.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return out


E4M3_EXACT = _e4m3_exact_grid()


def _nearest_even(r: Fraction, grid):
    """Nearest grid value to r >= 0, ties to the even index, saturating."""
    if r >= grid[-1]:
        return len(grid) - 1
    best = None
    for i, g in enumerate(grid):
        d = abs(r - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def _fq_group_exact(xs):
    """Reference F1..F5 on one group of floats, with exact rationals."""
    fr = [Fraction(float(x)) for x in xs]
    a = max(abs(v) for v in fr)
    si = _nearest_even(a / 6, E4M3_EXACT)
    s = E4M3_EXACT[si]
    out = []
    for x, v in zip(xs, fr):
        if s == 0:
            y = 0.0
        else:
            y = float(E2M1_EXACT[_nearest_even(abs(v) / s, E2M1_EXACT)] * s)
        out.append(float(np.copysign(y, x)))
    return out, si


def test_e4m3_grid_matches_torch_float8():
    codes = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(nvfp4.E4M3_GRID, codes)
    assert nvfp4.E4M3_GRID[-1] == 448.0
    assert [float(v) for v in E4M3_EXACT] == list(nvfp4.E4M3_GRID)


def test_e2m1_grid():
    assert list(nvfp4.E2M1_GRID) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_round_matches_torch_cast():
    rs = np.random.RandomState(7)
    v = np.concatenate([
        rs.uniform(0, 448, 20000),
        np.exp(rs.uniform(np.log(1e-5), np.log(448), 20000)),
        # exact midpoints of neighbouring grid values
        (nvfp4.E4M3_GRID[:-1] + nvfp4.E4M3_GRID[1:]) / 2,
    ]).astype(np.float32).astype(np.float64)
    ours = nvfp4.e4m3_round(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_saturates():
    assert nvfp4.e4m3_round(np.array([448.0, 460.0, 464.0, 1e9])).tolist() == [448.0] * 4


def test_golden_ties_and_scales():
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["cases"]:
        grp = np.zeros(16)
        grp[0] = 6 * c["s"]
        grp[1] = c["x"]
        y, codes = nvfp4.fake_quant(grp, return_scale_codes=True)
        assert nvfp4.E4M3_GRID[codes[0]] == c["s"], c
        assert y[1] == c["y"] and np.signbit(y[1]) == np.signbit(c["y"]), c
        assert y[0] == 6 * c["s"]
    for c in g["scale_cases"]["cases"]:
        grp = np.zeros(16)
        grp[3] = c["a"]
        _, codes = nvfp4.fake_quant(grp, return_scale_codes=True)
        assert nvfp4.E4M3_GRID[codes[0]] == c["s"], c


def _all_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    return f32_from_bf16_bits(bits).astype(np.float64)


def test_exhaustive_bf16_per_scale_exact():
    """Every non-zero E4M3 scale s, every positive bf16 x in [s/16, 6s]: group [6s, x, 0..]."""
    xs_all = _all_positive_bf16()
    for si in range(1, 127):
        s = float(E4M3_EXACT[si])
        xs = xs_all[(xs_all >= s / 16) & (xs_all <= 6 * s)]
        groups = np.zeros((len(xs), 16))
        groups[:, 0] = 6 * s
        groups[:, 1] = xs
        y, codes = nvfp4.fake_quant(groups, axis=-1, return_scale_codes=True)
        assert np.all(codes[:, 0] == si)
        sF = E4M3_EXACT[si]
        exp = np.array([float(E2M1_EXACT[_nearest_even(Fraction(x) / sF, E2M1_EXACT)] * sF)
                        for x in xs])
        np.testing.assert_array_equal(y[:, 1], exp)


def test_random_groups_exact_reference():
    rs = np.random.RandomState(11)
    groups = []
    for mag in [1e-4, 3e-3, 1e-2, 0.05, 0.3, 1.0, 10.0, 300.0, 3000.0]:
        x = (rs.standard_normal((150, 16)) * mag).astype(np.float32)
        groups.append(f32_from_bf16_bits((x.view(np.uint32) >> 16).astype(np.uint16)))
    groups = np.concatenate(groups).astype(np.float64)
    y, codes = nvfp4.fake_quant(groups, axis=-1, return_scale_codes=True)
    for i in range(len(groups)):
        ref, si = _fq_group_exact(groups[i])
        assert codes[i, 0] == si
        np.testing.assert_array_equal(y[i], ref)
        assert np.array_equal(np.signbit(y[i]), np.signbit(np.array(ref)))


def test_partial_tail_group_and_axis():
    rs = np.random.RandomState(3)
    x = rs.standard_normal((37, 5)).astype(np.float32).astype(np.float64)
    y = nvfp4.fake_quant(x, axis=0)
    for c in range(5):
        for g0 in range(0, 37, 16):
            seg = x[g0:g0 + 16, c]
            ref, _ = _fq_group_exact(seg)
            np.testing.assert_array_equal(y[g0:g0 + 16, c], ref)
    y1 = nvfp4.fake_quant(x.T, axis=-1)
    np.testing.assert_array_equal(y1, y.T)


def test_closed_forms():
    rs = np.random.RandomState(5)
    x = (rs.standard_normal((4000, 16)) * np.exp(rs.uniform(-8, 6, (4000, 1))))
    x = x.astype(np.float32).astype(np.float64)
    y, codes = nvfp4.fake_quant(x, return_scale_codes=True)
    s = nvfp4.E4M3_GRID[codes[:, 0]]
    nz = s > 0
    ratio = np.abs(y[nz]) / s[nz, None]
    assert np.all(np.isin(ratio, nvfp4.E2M1_GRID))
    # odd symmetry, bit for bit including signed zeros
    yn = nvfp4.fake_quant(-x)
    assert np.array_equal(yn, -y) and np.array_equal(np.signbit(yn), ~np.signbit(y))
    # group maximum lands on +-6 s when the scale is normal and unsaturated
    a = np.max(np.abs(x), axis=-1)
    normal = (s >= 2.0 ** -6) & (a / 6 < 448)
    amax_idx = np.argmax(np.abs(x), axis=-1)
    got = np.abs(y[np.arange(len(x)), amax_idx])
    np.testing.assert_array_equal(got[normal], 6 * s[normal])
    # all-zero group
    z, zc = nvfp4.fake_quant(np.zeros((2, 16)), return_scale_codes=True)
    assert np.all(z == 0) and np.all(zc == 0)
    # single non-zero element in the normal range -> +-6 * E4M3(|x|/6)
    v = np.array([0.7, -3.3, 100.0, 1500.0, 0.2])
    g = np.zeros((5, 16))
    g[:, 4] = v
    yy = nvfp4.fake_quant(g)
    np.testing.assert_array_equal(yy[:, 4], np.sign(v) * 6 * nvfp4.e4m3_round(np.abs(v) / 6))


def test_idempotence_where_it_holds():
    rs = np.random.RandomState(9)
    x = (rs.standard_normal((6000, 16)) * np.exp(rs.uniform(-9, 7, (6000, 1))))
    y, codes = nvfp4.fake_quant(x, return_scale_codes=True)
    s = nvfp4.E4M3_GRID[codes[:, 0]]
    a = np.max(np.abs(x), axis=-1)
    domain = (s == 0) | (s >= 2.0 ** -6)      # zero, normal or saturated scale
    yy = nvfp4.fake_quant(y)
    np.testing.assert_array_equal(yy[domain], y[domain])
    # inside the subnormal-scale band 6*2^-10 < a < 0.0879 it can fail; make
    # sure the test domain is the documented one
    band = (a > 6 * 2.0 ** -10) & (a < 0.087890625)
    assert np.all(domain | band)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 33])
def test_lengths(n):
    rs = np.random.RandomState(n)
    x = rs.standard_normal(n)
    y = nvfp4.fake_quant(x)
    ref = []
    for g0 in range(0, n, 16):
        ref += _fq_group_exact(x[g0:g0 + 16])[0]
    np.testing.assert_array_equal(y, ref)


def test_row_flip_tolerant_comparison():
    """The comparison used where the P quantizer's decisions are ill-conditioned
    (scales near the E4M3 subnormal floor): each row is scored against its
    closest candidate, and a row that matches no candidate still counts."""
    from tests.helpers import rel_l2, rel_l2_best_rows
    a = np.random.default_rng(3).standard_normal((4, 8))
    b = a.copy()
    b[2] = 0.0
    got = b.copy()                       # row 2 took the other decision
    assert rel_l2(got, a) > 0.1
    assert rel_l2_best_rows(got, [a, b]) == 0.0
    got[1] += 1.0                        # a wrong row
    assert rel_l2_best_rows(got, [a, b]) == pytest.approx(np.sqrt(8.0) / np.linalg.norm(a))
    z = np.zeros((2, 3))
    assert rel_l2_best_rows(z, [z]) == 0.0
    assert rel_l2_best_rows(np.ones((2, 3)), [z]) == float("inf")

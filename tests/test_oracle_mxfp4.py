"""Pins of the MXFP4 oracle (oracle/mxfp4.py) to facts other than itself:
hand-worked blocks (tests/golden/mxfp4_blocks.json), exact rational
arithmetic on random blocks, closed forms of the format (power-of-two scale
with amax / X in [4, 8), grid values unchanged, exact power-of-two scaling),
and attention cases with known answers (one key, identical keys, LSE as the
log-sum-exp of the quantized scores)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.json")
GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _e2m1_exact(v: Fraction) -> Fraction:
    """Nearest grid magnitude to v >= 0, ties to the even code, saturating at 6."""
    if v >= 6:
        return Fraction(6)
    best = None
    for i, g in enumerate(GRID):
        d = abs(v - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i, g)
    return best[2]


def _block_exact(xs):
    fr = [Fraction(float(x)) for x in xs]
    amax = max(abs(f) for f in fr)
    if amax == 0:
        return [0.0] * len(fr)
    e = 0
    while Fraction(2) ** (e + 1) <= amax:
        e += 1
    while Fraction(2) ** e > amax:
        e -= 1
    X = Fraction(2) ** (e - 2)
    return [float((1 if f >= 0 else -1) * _e2m1_exact(abs(f) / X) * X) for f in fr]


def test_golden_blocks():
    for case in json.load(open(GOLDEN))["cases"]:
        y, se = mxfp4.quant(np.array(case["x"]), return_exponents=True)
        assert int(se[0]) == case["exponent"], case["why"]
        np.testing.assert_array_equal(y, case["y"], err_msg=case["why"])


def test_random_blocks_against_exact_arithmetic():
    rng = np.random.default_rng(3)
    for trial in range(40):
        scale = 2.0 ** rng.integers(-20, 20)
        x = (rng.standard_normal(32) * scale).astype(np.float32).astype(np.float64)
        if trial % 5 == 0:
            x[rng.integers(0, 32, 5)] = 0.0
        np.testing.assert_array_equal(mxfp4.quant(x), _block_exact(x))


def test_scale_closed_form_and_grid_values():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 96)) * np.exp(rng.uniform(-30, 30, (50, 1)))
    y, se = mxfp4.quant(x, return_exponents=True)
    amax = np.abs(x).reshape(50, 3, 32).max(axis=-1)
    r = amax / np.ldexp(1.0, se)
    assert np.all((r >= 4) & (r < 8))
    # values that are grid points times X, with a block maximum of 4 X or 6 X, are unchanged
    codes = rng.integers(0, 8, (20, 32))
    g = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[codes] * np.where(rng.random((20, 32)) < .5, -1, 1)
    g[:, 0] = np.where(np.arange(20) % 2 == 0, 4.0, 6.0)
    e = rng.integers(-30, 30, (20, 1))
    xg = np.ldexp(g, e)
    np.testing.assert_array_equal(mxfp4.quant(xg), xg)
    # exact power-of-two scaling, partial last block padded with zeros
    z = rng.standard_normal((4, 70))
    np.testing.assert_array_equal(mxfp4.quant(z * 2.0 ** 7), mxfp4.quant(z) * 2.0 ** 7)
    np.testing.assert_array_equal(mxfp4.quant(z[:, 64:]), mxfp4.quant(z)[:, 64:])
    np.testing.assert_array_equal(mxfp4.quant(np.zeros(40)), np.zeros(40))


def test_axis_argument():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 40, 8))
    np.testing.assert_array_equal(mxfp4.quant(x, axis=1),
                                  np.swapaxes(mxfp4.quant(np.swapaxes(x, 1, 2), axis=-1), 1, 2))


def test_single_key_and_identical_keys():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 5, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    v = rng.standard_normal((1, 1, 1, 64))
    O, L = mxfp4.forward(q, k, v, 0.3)
    vq = mxfp4.quant(v, axis=-2)
    np.testing.assert_array_equal(O, np.broadcast_to(vq[0, 0, 0], (1, 1, 5, 64)))
    S = 0.3 * mxfp4.quant(q) @ np.swapaxes(mxfp4.quant(k), -1, -2)
    np.testing.assert_allclose(L, S[..., 0], rtol=1e-15)
    # identical keys: every P~ is exactly 1, so O is the mean of the quantized V rows
    k5 = np.repeat(k, 45, axis=2)
    v5 = rng.standard_normal((1, 1, 45, 64))
    O5, L5 = mxfp4.forward(q, k5, v5, 0.3)
    np.testing.assert_allclose(O5, np.broadcast_to(mxfp4.quant(v5, axis=-2).mean(axis=2, keepdims=True),
                                                   O5.shape), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(L5, S[..., 0] + np.log(45), rtol=1e-14)


@pytest.mark.parametrize("Nq,Nk", [(7, 100), (33, 64)])
def test_lse_and_power_of_two_v(Nq, Nk):
    rng = np.random.default_rng(Nq + Nk)
    q, k, v = (rng.standard_normal((1, 2, n, 32)) for n in (Nq, Nk, Nk))
    O, L = mxfp4.forward(q, k, v, 0.5)
    S = 0.5 * mxfp4.quant(q) @ np.swapaxes(mxfp4.quant(k), -1, -2)
    np.testing.assert_allclose(L, logsumexp(S, axis=-1), rtol=1e-13)
    O2, L2 = mxfp4.forward(q, k, v * 2.0 ** -5, 0.5)
    np.testing.assert_allclose(O2, O * 2.0 ** -5, rtol=1e-13, atol=1e-300)
    np.testing.assert_array_equal(L2, L)
    # each row's output is a combination of the quantized V rows with weights summing to at most ~1
    assert np.all(np.abs(O) <= np.abs(mxfp4.quant(v, axis=-2)).max() * 1.2)


def test_p_quantized_per_32_key_block():
    """Hand-built row: key 0 has S = 0 (P~ = 1), keys 1..31 have S = -48, and
    key 32, alone in the second 32-key block, has S = -0.75 (P~ = 0.4724).
    In its own block P~_32 / 2^-4 = 7.56 clips to 6, so it counts as 0.375;
    quantized against the row's maximum it would be 0.5, and unquantized
    0.4724. Every operand is a grid value times a power of two, so MX(Q),
    MX(K), MX(V) are exact; V rows: token 0 -> 2 e0, token 32 -> 4 e1,
    tokens 1..31 -> e2 (their P~ = e^-48 quantizes to 0 in block 0)."""
    D = 32
    q = np.zeros((1, 1, 1, D)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 33, D)); k[..., 1:32, 0] = -48.0; k[..., 32, 0] = -0.75
    v = np.zeros((1, 1, 33, D)); v[..., 0, 0] = 2.0; v[..., 32, 1] = 4.0; v[..., 1:32, 2] = 1.0
    O, L = mxfp4.forward(q, k, v, 1.0)
    l = 1.0 + 31 * np.exp(-48.0) + np.exp(-0.75)
    want = np.zeros(D); want[0] = 2.0 / l; want[1] = 4.0 * 0.375 / l
    np.testing.assert_allclose(O[0, 0, 0], want, rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(L[0, 0, 0], np.log(l), rtol=1e-15)

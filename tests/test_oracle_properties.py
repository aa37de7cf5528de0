"""Property tests of the oracle (CPU only), driven by hypothesis.

They check laws that the NVFP4 format and the attention definition imply,
on inputs hypothesis generates and shrinks, so that a mistake that the fixed
pins happen to miss (an off-by-one in the grouping, a sign lost in one
branch, a wrong axis) still fails somewhere:

* fake quantization is odd (FQ(-x) = -FQ(x)), scales exactly with powers of
  two while every group scale stays a normal E4M3 value, puts every value on
  the grid {E2M1} x s of its group with the group maximum at 6 s when s is
  normal, acts on each 16-element group independently of the others, and is
  idempotent on groups whose scale is normal;
* attention with every quantizer on is unchanged when whole 16-key groups of
  K and V are permuted together (each group of P and of V moves as a unit),
  and with every quantizer off under any permutation of the keys; LSE is the
  log-sum-exp of the scores in both cases.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import attention as oatt
from oracle import nvfp4

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _groups(draw, n_groups, lo_exp=-4, hi_exp=4):
    """float64 array of n_groups x 16 values with per-group magnitudes
    2^e, e in [lo_exp, hi_exp] (E4M3 scales of amax / 6 stay normal)."""
    seed = draw(st.integers(0, 2**31 - 1))
    rs = np.random.RandomState(seed)
    mags = 2.0 ** rs.randint(lo_exp, hi_exp + 1, size=(n_groups, 1))
    x = rs.standard_normal((n_groups, 16)) * mags
    # sprinkle exact zeros and ties of the format
    x[rs.rand(n_groups, 16) < 0.05] = 0.0
    return x


@st.composite
def group_arrays(draw, max_groups=6):
    return _groups(draw, draw(st.integers(1, max_groups)))


@SETTINGS
@given(group_arrays())
def test_fake_quant_is_odd(x):
    np.testing.assert_array_equal(nvfp4.fake_quant(-x), -nvfp4.fake_quant(x))


@SETTINGS
@given(group_arrays(), st.integers(-3, 3))
def test_fake_quant_scales_with_powers_of_two(x, k):
    # groups whose amax / 6 is a normal E4M3 magnitude (below 224, away from
    # saturation) before and after the scaling: multiplying the input by 2^k
    # then multiplies each scale, hence each output, by exactly 2^k
    amax = np.abs(x).max(axis=1)

    def normal(a):
        return (a / 6 >= 2.0 ** -6) & (a / 6 <= 224)

    ok = (amax == 0) | (normal(amax) & normal(amax * 2.0 ** k))
    x = x[ok]
    if x.size == 0:
        return
    np.testing.assert_array_equal(nvfp4.fake_quant(x * 2.0 ** k), nvfp4.fake_quant(x) * 2.0 ** k)


@SETTINGS
@given(group_arrays())
def test_fake_quant_values_on_group_grid(x):
    y, codes = nvfp4.fake_quant(x, return_scale_codes=True)
    s = nvfp4.e4m3fn_grid()[codes.astype(np.int64)][:, 0]
    for g in range(x.shape[0]):
        if s[g] == 0:
            assert np.all(y[g] == 0)
            continue
        q = np.abs(y[g]) / s[g]
        assert np.all(np.isin(q, E2M1)), (x[g], s[g])
        # a normal E4M3 scale is amax / 6 within a relative 2^-4, so amax / s
        # lies in [6 / (1 + 2^-4), 6 / (1 - 2^-4)] = [5.65, 6.4], which
        # rounds (or saturates) to 6: the group maximum lands on 6 s
        if s[g] >= 2.0 ** -6:
            assert q.max() == 6.0, (x[g], s[g])


@SETTINGS
@given(group_arrays(max_groups=8))
def test_fake_quant_groups_are_independent(x):
    y = nvfp4.fake_quant(x.reshape(-1)).reshape(x.shape)
    for g in range(x.shape[0]):
        np.testing.assert_array_equal(y[g], nvfp4.fake_quant(x[g]))


@SETTINGS
@given(group_arrays())
def test_fake_quant_idempotent_for_normal_unrounded_scales(x):
    # FQ(FQ(x)) = FQ(x) holds when the scale of FQ(x) is the scale of x: the
    # group maximum of FQ(x) is 6 s, so E4M3(6 s / 6) = s whenever s itself is
    # a normal E4M3 value and the maximum's ratio rounded to 6
    y, codes = nvfp4.fake_quant(x, return_scale_codes=True)
    grid = nvfp4.e4m3fn_grid()
    s = grid[codes.astype(np.int64)][:, 0]
    keep = (s >= 2.0 ** -6) & (np.abs(y).max(axis=1) == 6 * s)
    np.testing.assert_array_equal(nvfp4.fake_quant(y[keep]), y[keep])


def _attn_inputs(seed, n_groups, D=16, Nq=5):
    rs = np.random.RandomState(seed)
    Nk = 16 * n_groups
    q = rs.standard_normal((1, 1, Nq, D))
    k = rs.standard_normal((1, 1, Nk, D))
    v = rs.standard_normal((1, 1, Nk, D))
    return q, k, v


@SETTINGS
@given(st.integers(0, 2**31 - 1), st.integers(2, 4), st.data())
def test_attention_invariant_under_group_permutations(seed, n_groups, data):
    q, k, v = _attn_inputs(seed, n_groups)
    perm = data.draw(st.permutations(range(n_groups)))
    idx = np.concatenate([np.arange(16 * g, 16 * g + 16) for g in perm])
    O, L = oatt.forward(q, k, v, 0.5, oatt.MASK_ALL)
    O2, L2 = oatt.forward(q, k[:, :, idx], v[:, :, idx], 0.5, oatt.MASK_ALL)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L2, L, rtol=1e-12, atol=1e-12)


@SETTINGS
@given(st.integers(0, 2**31 - 1), st.integers(1, 3), st.data())
def test_plain_attention_invariant_under_key_permutations(seed, n_groups, data):
    q, k, v = _attn_inputs(seed, n_groups)
    perm = np.array(data.draw(st.permutations(range(16 * n_groups))))
    O, L = oatt.forward(q, k, v, 0.5, 0)
    O2, L2 = oatt.forward(q, k[:, :, perm], v[:, :, perm], 0.5, 0)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-12)
    S = 0.5 * q[0, 0] @ k[0, 0].T
    m = S.max(axis=1)
    np.testing.assert_allclose(L[0, 0], m + np.log(np.exp(S - m[:, None]).sum(axis=1)), rtol=1e-13)


def test_group_permutation_changes_output_when_groups_split():
    # guard against the permutation test passing vacuously: moving a single
    # key across a group boundary does change the quantized output
    q, k, v = _attn_inputs(5, 2)
    idx = np.arange(32)
    idx[[15, 16]] = idx[[16, 15]]
    O, _ = oatt.forward(q, k, v, 0.5, oatt.MASK_ALL)
    O2, _ = oatt.forward(q, k[:, :, idx], v[:, :, idx], 0.5, oatt.MASK_ALL)
    assert np.abs(O2 - O).max() > 1e-6

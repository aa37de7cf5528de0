"""Pins for the oracle's attention forward/backward and block-sparse path (CPU).

* quantization off: textbook attention through torch's fp64 SDPA and autograd;
* uniform attention (identical keys): hand-derived closed forms for the
  quantized P, no renormalisation (tests/golden/uniform_attention.json);
* quantization axes: operands checked group by group against an exact-rational
  quantizer; a V built so that the token axis and the head axis disagree;
* quantization on: central finite differences of the straight-through
  surrogate loss;
* invariants: LSE of identical keys, sum_j dK_j = 0 with P quantization off;
* block selection: brute force with exact rationals, including a tie.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import block_sparse as bsp
from oracle import nvfp4
from synthetic import f32_from_bf16_bits, random_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "uniform_attention.json")


def _bf16(seed, shape, scale=1.0):
    return f32_from_bf16_bits(random_bf16(seed, shape, scale)).astype(np.float64)


def _sdpa_fp64(q, k, v, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    lse = torch.logsumexp(scale * (qt @ kt.transpose(-1, -2)), dim=-1)
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("Nq,Nk,D", [(64, 64, 32), (40, 72, 16), (33, 17, 64)])
def test_forward_quant_off_matches_sdpa(Nq, Nk, D):
    q = _bf16(1, (2, 3, Nq, D))
    k = _bf16(2, (2, 3, Nk, D))
    v = _bf16(3, (2, 3, Nk, D))
    scale = 1 / math.sqrt(D)
    O, L = att.forward(q, k, v, scale, mask=0, row_block=16)
    Or, Lr = _sdpa_fp64(q, k, v, scale)
    np.testing.assert_allclose(O, Or, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lr, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Nq,Nk,D", [(48, 48, 32), (24, 40, 16)])
def test_backward_quant_off_matches_autograd(Nq, Nk, D):
    q = _bf16(4, (1, 2, Nq, D))
    k = _bf16(5, (1, 2, Nk, D))
    v = _bf16(6, (1, 2, Nk, D))
    do = _bf16(7, (1, 2, Nq, D))
    scale = 0.37
    dq, dk, dv = att.backward(q, k, v, do, scale, mask=0, row_block=16)
    qt, kt, vt = (torch.from_numpy(a).requires_grad_() for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    o.backward(torch.from_numpy(do))
    for ours, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_identical_keys_lse_closed_form():
    q = _bf16(8, (1, 1, 5, 16))
    krow = _bf16(9, (1, 1, 1, 16))
    for Nk in (3, 16, 100):
        k = np.repeat(krow, Nk, axis=2)
        v = _bf16(10, (1, 1, Nk, 16))
        _, L = att.forward(q, k, v, 0.25, mask=0)
        S = 0.25 * (q[0, 0] @ krow[0, 0, 0])
        np.testing.assert_allclose(L[0, 0], S + math.log(Nk), rtol=0, atol=1e-13)


def test_uniform_attention_p_quant_closed_forms():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        Nk = c["Nk"]
        q = _bf16(11, (1, 1, 4, 16))
        k = np.repeat(_bf16(12, (1, 1, 1, 16)), Nk, axis=2)
        v = _bf16(13, (1, 1, Nk, 16))
        O, _ = att.forward(q, k, v, 0.25, mask=att.MASK_P)
        expect = c["c"] * np.mean(v[0, 0], axis=0)
        np.testing.assert_allclose(O[0, 0], np.broadcast_to(expect, O[0, 0].shape),
                                   rtol=1e-12, atol=1e-15)


ROWMAX_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rowmax_p_quant.json")


def test_rowmax_uniform_attention_closed_form():
    """Row-max-relative P quantization on identical keys: O = 1.03125 mean(Vq)
    for every Nk, including lengths where the normalised P flushes to zero."""
    with open(ROWMAX_GOLDEN) as f:
        cases = json.load(f)["uniform"]["cases"]
    for c in cases:
        Nk = c["Nk"]
        q = _bf16(31, (1, 1, 4, 16))
        k = np.repeat(_bf16(32, (1, 1, 1, 16)), Nk, axis=2)
        v = _bf16(33, (1, 1, Nk, 16))
        O, _ = att.forward(q, k, v, 0.25, mask=att.MASK_P, p_mode=att.P_ROWMAX)
        expect = c["c"] * np.mean(v[0, 0], axis=0)
        np.testing.assert_allclose(O[0, 0], np.broadcast_to(expect, O[0, 0].shape),
                                   rtol=1e-12, atol=1e-15)


def test_rowmax_worked_row():
    """exp(S - m) = 2^-j over keys 0..15 and 1 over keys 16..31: the
    hand-derived codes at s = 0.171875, divided by l; the normalised reading
    gives a different result on the same row."""
    with open(ROWMAX_GOLDEN) as f:
        g = json.load(f)["worked_row"]
    sm = 0.5
    q = np.zeros((1, 1, 1, 32))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, 32, 32))
    k[0, 0, :16, 0] = -np.arange(16) * math.log(2.0) / sm   # S_j = -j ln 2, then S_j = 0
    v = np.eye(32)[None, None]                               # O row = Pq row
    O, L = att.forward(q, k, v, sm, mask=att.MASK_P, p_mode=att.P_ROWMAX)
    expect = np.array(g["codes"]) * g["s"] / g["l"]
    np.testing.assert_allclose(O[0, 0, 0], expect, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(L[0, 0, 0], math.log(g["l"]), rtol=0, atol=1e-14)
    On, _ = att.forward(q, k, v, sm, mask=att.MASK_P)
    assert np.abs(On[0, 0, 0] - expect).max() > 1e-3


def test_rowmax_equals_normalised_without_p_quant():
    q, k, v = _bf16(34, (1, 2, 24, 16)), _bf16(35, (1, 2, 40, 16)), _bf16(36, (1, 2, 40, 16))
    for mask in (0, att.MASK_Q | att.MASK_K | att.MASK_V):
        O0, L0 = att.forward(q, k, v, 0.3, mask=mask)
        O1, L1 = att.forward(q, k, v, 0.3, mask=mask, p_mode=att.P_ROWMAX)
        np.testing.assert_allclose(O1, O0, rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(L1, L0)


def _fq_exact_vec(xs):
    fr = [Fraction(float(x)) for x in xs]
    grid4 = [Fraction(float(g)) for g in nvfp4.E4M3_GRID]
    grid2 = [Fraction(float(g)) for g in nvfp4.E2M1_GRID]

    def near(r, grid):
        if r >= grid[-1]:
            return grid[-1]
        best = min(range(len(grid)), key=lambda i: (abs(r - grid[i]), i % 2))
        return grid[best]
    s = near(max(abs(v) for v in fr) / 6, grid4)
    return [0.0 if s == 0 else math.copysign(float(near(abs(v) / s, grid2) * s), float(x))
            for x, v in zip(xs, fr)]


def test_operand_quantization_axes():
    q = _bf16(14, (1, 1, 20, 32))
    k = _bf16(15, (1, 1, 20, 32))
    v = _bf16(16, (1, 1, 20, 32))
    qq, kq, vq = att.quantize_operands(q, k, v, att.MASK_ALL)
    for r in range(20):
        for g in range(2):
            sl = slice(16 * g, 16 * g + 16)
            assert list(qq[0, 0, r, sl]) == _fq_exact_vec(q[0, 0, r, sl])
            assert list(kq[0, 0, r, sl]) == _fq_exact_vec(k[0, 0, r, sl])
    for c in range(32):
        for t0 in (0, 16):
            sl = slice(t0, min(20, t0 + 16))
            assert list(vq[0, 0, sl, c]) == _fq_exact_vec(v[0, 0, sl, c])
    # cleared bits leave the operand untouched
    q2, k2, v2 = att.quantize_operands(q, k, v, att.MASK_P)
    assert np.array_equal(q2, q) and np.array_equal(k2, k) and np.array_equal(v2, v)


def test_v_quantized_along_tokens():
    """Hand-built V: per column, tokens carry [6, 2.5, 1.75, 5] * sigma_c."""
    D = 16
    sig = np.array([2.0 ** (c % 4 - 2) for c in range(D)])
    v = np.zeros((1, 1, 16, D))
    for t, mult in enumerate([6.0, 2.5, 1.75, 5.0]):
        v[0, 0, t] = mult * sig
    # along tokens the scale is sigma_c and the column becomes [6, 2, 2, 4] * sigma_c
    k = np.zeros((1, 1, 16, D))       # all scores equal -> P = 1/16
    q = _bf16(17, (1, 1, 3, D))
    O, _ = att.forward(q, k, v, 0.5, mask=att.MASK_V)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(14.0 / 16.0 * sig, (3, D)),
                               rtol=1e-14)


def _surrogate_loss(Q, K, V, W, rQ, rK, rV, lse0, R, scale):
    S = scale * (Q + rQ) @ (K + rK).T
    m = S.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))
    P = np.exp(S - lse)
    Pt = P + np.exp(lse0[:, None] - lse) * R
    return float(np.sum(W * (Pt @ (V + rV))))


@pytest.mark.parametrize("N,D,seed,p_mode", [(32, 16, 0, 0), (40, 32, 1, 0), (32, 16, 2, 1),
                                           (40, 32, 3, 1)])
def test_backward_quant_on_finite_differences(N, D, seed, p_mode):
    """Central differences of the straight-through surrogate loss.

    Residuals r = FQ(x0) - x0 are frozen at the base point and the quantized P
    enters as P + exp(LSE0 - LSE) * (Pq0 - P0). At the base point the
    surrogate's output is the quantized forward, and its gradient is the
    straight-through backward with D = rowsum(dO * O).
    """
    # Scores spread wide enough that many P groups keep a non-zero scale.
    Q = _bf16(100 + seed, (N, D), 1.5)
    K = _bf16(200 + seed, (N, D), 1.5)
    V = _bf16(300 + seed, (N, D))
    W = _bf16(400 + seed, (N, D))
    scale = 1 / math.sqrt(D)
    Qq = nvfp4.fake_quant(Q, -1)
    Kq = nvfp4.fake_quant(K, -1)
    Vq = nvfp4.fake_quant(V, -2)
    rQ, rK, rV = Qq - Q, Kq - K, Vq - V
    S0 = scale * Qq @ Kq.T
    lse0 = np.log(np.exp(S0).sum(axis=1))
    P0 = np.exp(S0 - lse0[:, None])
    if p_mode == att.P_ROWMAX:
        # exp(S - m) quantized, divided by l = exp(LSE - m)
        m0 = S0.max(axis=1, keepdims=True)
        Pq0 = nvfp4.fake_quant(np.exp(S0 - m0), -1) / np.exp(lse0[:, None] - m0)
    else:
        Pq0 = nvfp4.fake_quant(P0, -1)
    R = Pq0 - P0
    assert np.count_nonzero(Pq0) > N  # P quantization is active

    O, L = att.forward(Q[None, None], K[None, None], V[None, None], scale, att.MASK_ALL,
                       p_mode=p_mode)
    np.testing.assert_allclose(O[0, 0], (P0 + R) @ Vq, rtol=1e-12, atol=1e-14)
    dq, dk, dv = att.backward(Q[None, None], K[None, None], V[None, None], W[None, None],
                              scale, att.MASK_ALL, p_mode=p_mode)
    h = 1e-6
    for X, G in ((Q, dq[0, 0]), (K, dk[0, 0]), (V, dv[0, 0])):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _surrogate_loss(Q, K, V, W, rQ, rK, rV, lse0, R, scale)
            X[idx] = old - h
            fm = _surrogate_loss(Q, K, V, W, rQ, rK, rV, lse0, R, scale)
            X[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - G) / np.linalg.norm(G)
        assert err < 1e-7, err


def _surrogate_loss_ste(Q, K, V, W, rQ, rK, rV, R, scale):
    S = scale * (Q + rQ) @ (K + rK).T
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    P = P / P.sum(axis=1, keepdims=True)
    return float(np.sum(W * ((P + R) @ (V + rV))))


@pytest.mark.parametrize("N,D,seed", [(32, 16, 5), (40, 32, 6)])
def test_backward_additive_ste_delta_finite_differences(N, D, seed):
    """With the quantized P entering as P + (Pq0 - P0) (difference frozen, no
    LSE factor), central differences give the backward whose delta is
    D' = rowsum(dO * O_ste), O_ste = P Vq: the oracle's backward fed O_ste."""
    Q = _bf16(500 + seed, (N, D), 1.5)
    K = _bf16(600 + seed, (N, D), 1.5)
    V = _bf16(700 + seed, (N, D))
    W = _bf16(800 + seed, (N, D))
    scale = 1 / math.sqrt(D)
    Qq, Kq, Vq = nvfp4.fake_quant(Q, -1), nvfp4.fake_quant(K, -1), nvfp4.fake_quant(V, -2)
    rQ, rK, rV = Qq - Q, Kq - K, Vq - V
    S0 = scale * Qq @ Kq.T
    P0 = np.exp(S0 - np.log(np.exp(S0).sum(axis=1))[:, None])
    R = nvfp4.fake_quant(P0, -1) - P0
    O, L, Os = att.forward(Q[None, None], K[None, None], V[None, None], scale, att.MASK_ALL,
                           with_ste=True)
    np.testing.assert_allclose(Os[0, 0], P0 @ Vq, rtol=1e-12, atol=1e-14)
    dq, dk, dv = att.backward(Q[None, None], K[None, None], V[None, None], W[None, None],
                              scale, att.MASK_ALL, O=Os, lse=L)
    h = 1e-6
    for X, G in ((Q, dq[0, 0]), (K, dk[0, 0]), (V, dv[0, 0])):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _surrogate_loss_ste(Q, K, V, W, rQ, rK, rV, R, scale)
            X[idx] = old - h
            fm = _surrogate_loss_ste(Q, K, V, W, rQ, rK, rV, R, scale)
            X[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - G) / np.linalg.norm(G)
        assert err < 1e-7, err
    # and it differs from the delta of the quantized output
    dq2, _, _ = att.backward(Q[None, None], K[None, None], V[None, None], W[None, None],
                             scale, att.MASK_ALL, O=O, lse=L)
    assert np.linalg.norm(dq2 - dq) > 1e-3 * np.linalg.norm(dq)


def test_ste_output_equals_output_without_p_quant():
    q, k, v = _bf16(37, (1, 1, 20, 16)), _bf16(38, (1, 1, 30, 16)), _bf16(39, (1, 1, 30, 16))
    for mask in (0, att.MASK_Q | att.MASK_K | att.MASK_V):
        O, L, Os = att.forward(q, k, v, 0.3, mask=mask, with_ste=True)
        np.testing.assert_array_equal(Os, O)


def test_dk_sums_to_zero_without_p_quant():
    q = _bf16(20, (1, 1, 48, 32))
    k = _bf16(21, (1, 1, 48, 32))
    v = _bf16(22, (1, 1, 48, 32))
    do = _bf16(23, (1, 1, 48, 32))
    dq, dk, dv = att.backward(q, k, v, do, 0.2, mask=att.MASK_Q | att.MASK_K | att.MASK_V)
    assert np.abs(dk.sum(axis=2)).max() < 1e-10 * np.abs(dk).max()
    # with P quantization on the sum is in general not zero
    dq, dk, dv = att.backward(q * 3, k * 3, v, do, 0.2, mask=att.MASK_ALL)
    assert np.abs(dk.sum(axis=2)).max() > 1e-6


def test_sampled_rows_and_keys_match_full():
    q = _bf16(30, (1, 1, 80, 32), 2.0)
    k = _bf16(31, (1, 1, 72, 32), 2.0)
    v = _bf16(32, (1, 1, 72, 32))
    do = _bf16(33, (1, 1, 80, 32))
    sc = 0.25
    O, L = att.forward(q, k, v, sc)
    dq, dk, dv = att.backward(q, k, v, do, sc)
    qq, kq, vq = att.quantize_operands(q[0, 0], k[0, 0], v[0, 0], att.MASK_ALL)
    rows = np.array([0, 5, 79, 33])
    Or, Lr = att.head_forward(qq, kq, vq, sc, att.MASK_ALL, rows=rows)
    np.testing.assert_allclose(Or, O[0, 0, rows], rtol=1e-13, atol=1e-15)
    dqr = att.head_backward_rows(qq, kq, vq, do[0, 0, rows], Or, Lr, rows, sc, att.MASK_ALL)
    np.testing.assert_allclose(dqr, dq[0, 0, rows], rtol=1e-11, atol=1e-14)
    keys = np.array([3, 17, 71, 64, 65])
    dkk, dvk = att.head_backward_keys(qq, kq, vq, do[0, 0], O[0, 0], L[0, 0], sc,
                                      att.MASK_ALL, keys, row_block=32)
    np.testing.assert_allclose(dkk, dk[0, 0, keys], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dvk, dv[0, 0, keys], rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------------------
# block selection and block-sparse attention


def test_effective_topk_formula():
    assert bsp.effective_topk(256, 0.9) == 26
    assert bsp.effective_topk(5, 0.9) == 1
    assert bsp.effective_topk(10, 0.0) == 10


def _bf16_exact(r: Fraction) -> Fraction:
    if r == 0:
        return Fraction(0)
    sgn = 1 if r > 0 else -1
    a = abs(r)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    return sgn * round(a / ulp) * ulp        # round() on Fraction: half to even


def test_bf16_round_matches_exact():
    rs = np.random.RandomState(40)
    x = rs.standard_normal(3000) * np.exp(rs.uniform(-20, 20, 3000))
    ours = bsp.bf16_round(x)
    ref = [float(_bf16_exact(Fraction(v))) for v in x]
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("N,bt,topk", [(8 * 16, 16, 3), (7 * 16 + 5, 16, 2)])
def test_block_selection_brute_force(N, bt, topk):
    q = _bf16(41, (1, 2, N, 8))
    k = _bf16(42, (1, 2, N, 8))
    k[0, 0, 2 * bt:3 * bt] = k[0, 0, 5 * bt:6 * bt]       # blocks 2 and 5 tie exactly
    idx = bsp.select_blocks(q, k, bt, topk)
    nb = -(-N // bt)
    for h in range(2):
        means_q, means_k = [], []
        for j in range(nb):
            t0, t1 = j * bt, min(N, (j + 1) * bt)
            means_q.append([_bf16_exact(sum(Fraction(float(x)) for x in q[0, h, t0:t1, c]) / (t1 - t0))
                            for c in range(8)])
            means_k.append([_bf16_exact(sum(Fraction(float(x)) for x in k[0, h, t0:t1, c]) / (t1 - t0))
                            for c in range(8)])
        for i in range(nb):
            sc = [_bf16_exact(sum(a * b for a, b in zip(means_q[i], means_k[j]))) for j in range(nb)]
            best = sorted(range(nb), key=lambda j: (-sc[j], j))[:topk]
            assert list(idx[0, h, i]) == sorted(best)
    # the tie: whenever block 5 is chosen, block 2 is chosen too
    for i in range(nb):
        sel = set(idx[0, 0, i].tolist())
        if 5 in sel:
            assert 2 in sel


def _masked_dense(q, k, v, do, scale, idx, bt, mask):
    """Dense attention in which the unselected keys get probability exactly 0."""
    N = q.shape[0]
    allow = np.zeros((N, k.shape[0]), dtype=bool)
    for i in range(idx.shape[0]):
        for j in idx[i]:
            allow[i * bt:(i + 1) * bt, j * bt:(j + 1) * bt] = True
    qq, kq, vq = att.quantize_operands(q, k, v, mask)
    S = np.where(allow, scale * qq @ kq.T, -np.inf)
    m = S.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
    P = np.exp(S - lse[:, None])
    Pq = nvfp4.fake_quant(P, -1) if mask & att.MASK_P else P
    O = Pq @ vq
    Dd = (do * O).sum(axis=1)
    dS = P * (do @ vq.T - Dd[:, None])
    return O, lse, scale * dS @ kq, scale * dS.T @ qq, Pq.T @ do


@pytest.mark.parametrize("mask", [0, 15])
def test_block_sparse_equals_masked_dense(mask):
    bt, nb, topk = 32, 6, 2
    N = bt * nb
    q = _bf16(50, (1, 1, N, 16), 2.0)
    k = _bf16(51, (1, 1, N, 16), 2.0)
    v = _bf16(52, (1, 1, N, 16))
    do = _bf16(53, (1, 1, N, 16))
    idx = bsp.select_blocks(q, k, bt, topk)
    O, L = bsp.forward(q, k, v, 0.25, idx, bt, mask)
    dq, dk, dv = bsp.backward(q, k, v, do, 0.25, idx, bt, mask)
    Or, Lr, dqr, dkr, dvr = _masked_dense(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.25,
                                          idx[0, 0], bt, mask)
    for a, b in ((O[0, 0], Or), (L[0, 0], Lr), (dq[0, 0], dqr), (dk[0, 0], dkr), (dv[0, 0], dvr)):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)
    if mask == 0:
        # quant off, every block selected -> textbook attention
        idx_all = np.tile(np.arange(nb, dtype=np.int32), (1, 1, nb, 1))
        O2, _ = bsp.forward(q, k, v, 0.25, idx_all, bt, 0)
        Or2, _ = _sdpa_fp64(q, k, v, 0.25)
        np.testing.assert_allclose(O2, Or2, rtol=1e-12, atol=1e-13)


def test_block_sparse_rowmax_equals_masked_dense():
    """Row-max variant, sparse: the row maximum is taken over the selected
    keys only, as in dense attention with the unselected keys masked out."""
    N, bt, D, topk = 384, 128, 16, 2
    q, k, v, do = (_bf16(60 + i, (1, 1, N, D)) for i in range(4))
    idx = bsp.select_blocks(q, k, bt, topk)
    O, L = bsp.forward(q, k, v, 0.3, idx, bt, att.MASK_ALL, p_mode=att.P_ROWMAX)
    qq, kq, vq = att.quantize_operands(q, k, v, att.MASK_ALL)
    for i in range(N // bt):
        keys = np.concatenate([np.arange(j * bt, (j + 1) * bt) for j in idx[0, 0, i]])
        S = 0.3 * qq[0, 0, i * bt:(i + 1) * bt] @ kq[0, 0, keys].T
        m = S.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
        Pq = nvfp4.fake_quant(np.exp(S - m), -1) / np.exp(lse[:, None] - m)
        np.testing.assert_allclose(O[0, 0, i * bt:(i + 1) * bt], Pq @ vq[0, 0, keys], rtol=1e-12,
                                   atol=1e-14)
        np.testing.assert_allclose(L[0, 0, i * bt:(i + 1) * bt], lse, rtol=0, atol=1e-12)


def test_block_helpers_match_full_sparse_oracle():
    bt, nb, topk = 32, 5, 2
    N = bt * nb - 7                       # ragged last block
    q = _bf16(60, (1, 1, N, 16), 2.0)
    k = _bf16(61, (1, 1, N, 16), 2.0)
    v = _bf16(62, (1, 1, N, 16))
    do = _bf16(63, (1, 1, N, 16))
    idx = bsp.select_blocks(q, k, bt, topk)
    O, L = bsp.forward(q, k, v, 0.3, idx, bt, 15)
    dq, dk, dv = bsp.backward(q, k, v, do, 0.3, idx, bt, 15, O, L)
    qq, kq, vq = att.quantize_operands(q[0, 0], k[0, 0], v[0, 0], 15)
    for i in range(nb):
        r0, r1 = i * bt, min(N, (i + 1) * bt)
        _, Oi, Li, _, _ = bsp.query_block_forward(qq, kq, vq, idx[0, 0, i], r0, r1, bt, 0.3, 15)
        np.testing.assert_allclose(Oi, O[0, 0, r0:r1], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(Li, L[0, 0, r0:r1], rtol=1e-13)
        dqi = bsp.query_block_backward(qq, kq, vq, do[0, 0], Oi, idx[0, 0, i], r0, r1, bt, 0.3, 15)
        np.testing.assert_allclose(dqi, dq[0, 0, r0:r1], rtol=1e-11, atol=1e-14)
    for j in range(nb):
        dkj, dvj = bsp.key_block_backward(qq, kq, vq, do[0, 0], idx[0, 0], j, bt, 0.3, 15)
        k0, k1 = j * bt, min(N, (j + 1) * bt)
        np.testing.assert_allclose(dkj, dk[0, 0, k0:k1], rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(dvj, dv[0, 0, k0:k1], rtol=1e-11, atol=1e-14)


def test_parallel_full_head_forward_matches():
    q = _bf16(70, (1, 1, 300, 32), 2.0)
    k = _bf16(71, (1, 1, 250, 32), 2.0)
    v = _bf16(72, (1, 1, 250, 32))
    qq, kq, vq = att.quantize_operands(q[0, 0], k[0, 0], v[0, 0], 15)
    O1, L1 = att.head_forward(qq, kq, vq, 0.2, 15)
    O2, L2 = att.head_forward_all(qq, kq, vq, 0.2, 15, workers=2, chunk=64)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_block_sparse_ste_output():
    """Sparse O_ste: with every key block selected it is the dense O_ste; with
    P unquantized it is the sparse O."""
    N, bt, D = 96, 32, 16
    q, k, v = (_bf16(70 + i, (1, 1, N, D)) for i in range(3))
    idx_all = np.arange(3, dtype=np.int32)[None, None, None].repeat(3, axis=2)
    _, _, Os = bsp.forward(q, k, v, 0.3, idx_all, bt, att.MASK_ALL, with_ste=True)
    _, _, Osd = att.forward(q, k, v, 0.3, att.MASK_ALL, with_ste=True)
    np.testing.assert_allclose(Os, Osd, rtol=1e-12, atol=1e-14)
    idx = bsp.select_blocks(q, k, bt, 1)
    O, _, Os = bsp.forward(q, k, v, 0.3, idx, bt, att.MASK_Q | att.MASK_K | att.MASK_V,
                           with_ste=True)
    np.testing.assert_array_equal(Os, O)

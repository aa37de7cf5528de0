"""Pins of the VSA coarse-branch oracle (oracle/vsa.py) to facts other than
itself: the dense softmax-attention oracle (pinned to torch SDPA) applied to
the block means, central finite differences of the coarse branch and of the
whole gated combination with quantization off, and invariants of the block
pooling."""
import numpy as np
import pytest

from oracle import attention as att
from oracle import block_sparse as bsp
from oracle import vsa


def _rand(seed, shape, scale=1.0):
    return bsp.bf16_round(np.random.default_rng(seed).standard_normal(shape) * scale)


def test_coarse_equals_dense_attention_on_block_means():
    """Coarse attention is softmax attention of the query-block means over the
    key-block means: the dense oracle with quantization off gives the same."""
    q, k, v = _rand(1, (1, 2, 300, 16)), _rand(2, (1, 2, 200, 16)), _rand(3, (1, 2, 200, 16))
    oc, L, (qb, kb, vb, _) = vsa.coarse_forward(q, k, v, 0.7, 64)
    assert qb.shape == (1, 2, 5, 16) and kb.shape == (1, 2, 4, 16)
    O, Ld = att.forward(qb, kb, vb, 0.7, mask=0)
    np.testing.assert_allclose(oc, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L, Ld, rtol=1e-12, atol=1e-14)


def test_constant_blocks():
    """When every token of a block is the same vector, the block means are
    those vectors, and each token gets its block's coarse output."""
    rng = np.random.default_rng(5)
    qv = bsp.bf16_round(rng.standard_normal((3, 8)))
    kv = bsp.bf16_round(rng.standard_normal((2, 8)))
    vv = bsp.bf16_round(rng.standard_normal((2, 8)))
    q = np.repeat(qv, 4, axis=0)[None, None]
    k = np.repeat(kv, 4, axis=0)[None, None]
    v = np.repeat(vv, 4, axis=0)[None, None]
    oc, _, (qb, kb, vb, P) = vsa.coarse_forward(q, k, v, 0.5, 4)
    np.testing.assert_array_equal(qb[0, 0], qv)
    s = 0.5 * qv @ kv.T
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(oc[0, 0], w @ vv, rtol=1e-13)
    g = _rand(6, q.shape)
    o = vsa.combine(np.zeros_like(q), g, oc, 4)
    np.testing.assert_allclose(o[0, 0, 5], g[0, 0, 5] * oc[0, 0, 1], rtol=1e-15)


def test_zero_gate_gives_the_fine_branch():
    N, bt = 96, 32
    q, k, v, do = (_rand(10 + i, (1, 1, N, 16)) for i in range(4))
    idx = bsp.select_blocks(q, k, bt, 2)
    g = np.zeros_like(q)
    O, Of, L = vsa.forward(q, k, v, g, 0.3, idx, bt)
    np.testing.assert_array_equal(O, Of)
    dq, dk, dv, dG = vsa.backward(q, k, v, g, do, 0.3, idx, bt)
    fq, fk, fv = bsp.backward(q, k, v, do, 0.3, idx, bt, 15)
    np.testing.assert_array_equal(dq, fq)
    np.testing.assert_array_equal(dk, fk)
    np.testing.assert_array_equal(dv, fv)
    # the gate gradient does not depend on the gate
    oc, _, _ = vsa.coarse_forward(q, k, v, 0.3, bt)
    np.testing.assert_allclose(dG, do * vsa.broadcast(oc, N, bt), rtol=1e-15)


def _fd_check(fun, args, grads, names, rng, h=1e-6, n=6, rtol=2e-6):
    for name, x, gx in zip(names, args, grads):
        for _ in range(n):
            i = tuple(rng.integers(0, s) for s in x.shape)
            x0 = x[i]
            x[i] = x0 + h
            fp = fun()
            x[i] = x0 - h
            fm = fun()
            x[i] = x0
            fd = (fp - fm) / (2 * h)
            assert abs(fd - gx[i]) <= rtol * (abs(fd) + 1e-3), (name, i, fd, gx[i])


@pytest.mark.parametrize("Nq,Nk,bt", [(40, 24, 16), (32, 32, 8)])
def test_coarse_backward_finite_differences(Nq, Nk, bt):
    """Gradients of sum(W * G * O_c[block(t)]) with exact (unrounded) block
    means, partial last blocks and Nq != Nk included."""
    rng = np.random.default_rng(Nq + Nk)
    q = rng.standard_normal((1, 1, Nq, 8))
    k = rng.standard_normal((1, 1, Nk, 8))
    v = rng.standard_normal((1, 1, Nk, 8))
    g = rng.standard_normal((1, 1, Nq, 8))
    w = rng.standard_normal((1, 1, Nq, 8))

    def loss():
        oc, _, _ = vsa.coarse_forward(q, k, v, 0.6, bt, round_bf16=False)
        return float(np.sum(w * vsa.combine(np.zeros_like(g), g, oc, bt)))

    dq, dk, dv, dG = vsa.coarse_backward(q, k, v, g, w, 0.6, bt, round_bf16=False)
    _fd_check(loss, [q, k, v, g], [dq, dk, dv, dG], ["q", "k", "v", "g"], rng)


def test_whole_vsa_backward_finite_differences():
    """Quantization off: the gradient of sum(W * O) for O = O_fine + G * O_c
    (fixed block selection, exact block means) is the fine backward taken with
    the fine output plus the coarse contributions."""
    rng = np.random.default_rng(21)
    N, bt, D = 48, 16, 8
    q, k, v, g, w = (rng.standard_normal((1, 1, N, D)) for _ in range(5))
    idx = np.array([[[[0, 2], [1, 2], [0, 1]]]], np.int32)

    def loss():
        of, _ = bsp.forward(q, k, v, 0.5, idx, bt, mask=0)
        oc, _, _ = vsa.coarse_forward(q, k, v, 0.5, bt, round_bf16=False)
        return float(np.sum(w * vsa.combine(of, g, oc, bt)))

    of, L = bsp.forward(q, k, v, 0.5, idx, bt, mask=0)
    fq, fk, fv = bsp.backward(q, k, v, w, 0.5, idx, bt, 0, of, L)
    cq, ck, cv, dG = vsa.coarse_backward(q, k, v, g, w, 0.5, bt, round_bf16=False)
    _fd_check(loss, [q, k, v, g], [fq + cq, fk + ck, fv + cv, dG], ["q", "k", "v", "g"], rng)


def test_pooling_gradient_invariants():
    """Every token of a block receives the same coarse gradient, and the
    block's tokens together receive exactly the gradient of its mean."""
    q, k, v, g, do = (_rand(30 + i, (1, 1, 70, 8)) for i in range(5))
    dq, dk, dv, _ = vsa.coarse_backward(q, k, v, g, do, 0.4, 32)
    for x in (dq, dk, dv):
        for j, (t0, t1) in enumerate([(0, 32), (32, 64), (64, 70)]):
            np.testing.assert_array_equal(x[0, 0, t0:t1], np.broadcast_to(x[0, 0, t0], (t1 - t0, 8)))

"""LDS-poisoning debug build against the release library (GPU).

``libattnqat_ldspoison.so`` is the same sources compiled with AQ_LDS_POISON:
every kernel fills the LDS arrays that stage operands, exchange products and
hold partial results with NaN (as bf16, fp16, fp32 and fp64) before first
use. If a kernel read LDS it had not written (tile padding, an exchange slot
of a skipped step, rows past a ragged tail), the NaN would reach its
outputs. Each case runs both builds on the same inputs and requires every
output to match bit for bit: dense and block-sparse forward and backward with
ragged tails, the split last round of pass 2 and dQ, the straight-through and
row-max variants, quantization off, the MXFP4 forward, block selection and the
VSA coarse branch.
"""
import contextlib

import numpy as np
import pytest
import torch

import quantization_aware_attention_amd as qaa
from quantization_aware_attention_amd.build import POISON_PATH
from synthetic import random_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def poison_lib(gpu_lib):
    return qaa.open_library(POISON_PATH)


@contextlib.contextmanager
def _using(lib):
    old = qaa._lib
    qaa._lib = lib
    try:
        yield
    finally:
        qaa._lib = old


def _both(poison_lib, run):
    """run() with the release library, then with the poisoning one; each
    returns a dict of tensors."""
    ref = run()
    torch.cuda.synchronize()
    with _using(poison_lib):
        got = run()
        torch.cuda.synchronize()
    return ref, got


def _same(ref, got, label):
    for k in ref:
        a, b = ref[k], got[k]
        if a is None:
            continue
        assert a.dtype == b.dtype and a.shape == b.shape, (label, k)
        av = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
        bv = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
        ndiff = int((av != bv).sum())
        assert ndiff == 0, f"{label}: {k} differs in {ndiff} elements"
        if a.is_floating_point():
            assert bool(torch.isfinite(b.float()).all()), f"{label}: {k} not finite"


def _inputs(seed, shape, scale=1.0):
    return {k: torch.from_numpy(random_bf16(seed + i, shape, scale).view(np.int16))
            .view(torch.bfloat16).cuda() for i, k in enumerate(("q", "k", "v", "do"))}


@pytest.mark.parametrize("shape,quant", [((1, 2, 300, 128), "qkvp"), ((1, 3, 200, 64), "qkvp"),
                                         ((2, 2, 2100, 128), "qkvp"), ((1, 2, 300, 128), "p"),
                                         ((1, 2, 300, 128), "qkv")])
def test_dense_forward_backward(poison_lib, shape, quant):
    """Ragged tails (300, 200 tokens), the shared-out last round of pass 2
    and dQ (2 x 2 heads x 2100 tokens), P-only and no-P quantization (the
    single-pass forward)."""
    t = _inputs(700, shape)
    sc = 1.0 / np.sqrt(shape[-1])

    def run():
        o, lse = qaa.fwd(t["q"], t["k"], t["v"], sc, quant)
        dq, dk, dv = qaa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, quant)
        return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)

    _same(*_both(poison_lib, run), f"dense {shape} {quant}")


@pytest.mark.parametrize("N", [600, 1050])
def test_sparse_forward_backward(poison_lib, N):
    """Block-sparse with the partial last key block selected (600 = 4 x 128
    + 88, 1050 = 8 x 128 + 26 tokens)."""
    t = _inputs(720, (1, 2, N, 128))
    nb = (N + 127) // 128
    rows = np.array([[i % (nb - 1), nb - 1] for i in range(nb)], np.int32)
    idx = torch.from_numpy(np.broadcast_to(rows, (1, 2, nb, 2)).copy()).cuda()
    sc = 0.0884

    def run():
        o, lse = qaa.fwd(t["q"], t["k"], t["v"], sc, "qkvp", idx)
        dq, dk, dv = qaa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, "qkvp", idx)
        return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)

    _same(*_both(poison_lib, run), f"sparse N={N}")


@pytest.mark.parametrize("N,sparse", [(700, False), (2100, False), (600, True)])
def test_variants(poison_lib, N, sparse):
    """The straight-through output (dense pass 2 with its own split at 2,100
    tokens; sparse) and the row-max-relative P quantization."""
    t = _inputs(740, (1, 2, N, 128))
    idx = None
    if sparse:
        nb = (N + 127) // 128
        rows = np.array([[0, nb - 1]] * nb, np.int32)
        idx = torch.from_numpy(np.broadcast_to(rows, (1, 2, nb, 2)).copy()).cuda()
    sc = 0.0884

    def run():
        ost = torch.empty_like(t["q"])
        o, lse = qaa.fwd(t["q"], t["k"], t["v"], sc, "qkvp", idx, o_ste=ost)
        g = qaa.bwd(t["q"], t["k"], t["v"], ost, lse, t["do"], sc, "qkvp", idx)
        o2, lse2, m = qaa.fwd(t["q"], t["k"], t["v"], sc, "qkvp", idx, p_mode=qaa.P_ROWMAX)
        g2 = qaa.bwd(t["q"], t["k"], t["v"], o2, lse2, t["do"], sc, "qkvp", idx,
                     p_mode=qaa.P_ROWMAX, row_max=m)
        return dict(o=o, ost=ost, lse=lse, dq=g[0], dk=g[1], dv=g[2], o2=o2, lse2=lse2, m=m,
                    dq2=g2[0], dk2=g2[1], dv2=g2[2])

    _same(*_both(poison_lib, run), f"variants N={N} sparse={sparse}")


@pytest.mark.parametrize("N,D", [(1000, 128), (300, 64)])
def test_mxfp4_forward(poison_lib, N, D):
    t = _inputs(760, (1, 2, N, D))

    def run():
        o, lse = qaa.mxfp4_fwd(t["q"], t["k"], t["v"], 1.0 / np.sqrt(D))
        return dict(o=o, lse=lse)

    _same(*_both(poison_lib, run), f"mxfp4 N={N} D={D}")


def test_selection_and_vsa(poison_lib):
    """Block selection, the fine branch on its index, and the VSA coarse
    branch forward and backward (1,000 tokens: a partial last block)."""
    N, D = 1000, 128
    t = _inputs(780, (1, 2, N, D), 1.5)
    g = torch.from_numpy(random_bf16(785, (1, 2, N, D)).view(np.int16)).view(torch.bfloat16).cuda()
    sc = 1.0 / np.sqrt(D)

    def run():
        idx = qaa.block_select(t["q"], t["k"], 2)
        of, lse = qaa.fwd(t["q"], t["k"], t["v"], sc, "qkvp", idx)
        o = qaa.vsa_fwd(t["q"], t["k"], t["v"], g, of, sc)
        dq, dk, dv = qaa.bwd(t["q"], t["k"], t["v"], of, lse, t["do"], sc, "qkvp", idx)
        dq, dk, dv, dg = qaa.vsa_bwd(t["q"], t["k"], t["v"], g, t["do"], dq, dk, dv, sc)
        return dict(idx=idx, o=o, lse=lse, dq=dq, dk=dk, dv=dv, dg=dg)

    _same(*_both(poison_lib, run), "selection + VSA")

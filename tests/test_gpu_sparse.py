"""GPU parity of VSA-style block selection and block-sparse fine attention
against the full oracle, at sizes the oracle finishes in seconds."""
import numpy as np
import pytest
import torch

from oracle import block_sparse as bsp
from oracle.block_sparse import bf16_round
from synthetic import random_bf16
from tests.helpers import TOL_LSE, dev_f64, rel_l2, to_dev, to_f64, tol_for

pytestmark = pytest.mark.gpu


def _inputs(seed, shape, scale=1.0):
    return {k: random_bf16(seed + i, shape, scale) for i, k in enumerate(("q", "k", "v", "do"))}


@pytest.mark.parametrize("N,D,topk", [(1024, 64, 3), (1000, 128, 2), (640, 128, 5), (300, 64, 1)])
def test_selection_exact(gpu_lib, N, D, topk):
    bits = _inputs(N + D, (2, 2, N, D))
    idx_g = gpu_lib.block_select(to_dev(bits["q"]), to_dev(bits["k"]), topk, 128)
    idx_r = bsp.select_blocks(to_f64(bits["q"]), to_f64(bits["k"]), 128, topk)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_r)


def test_selection_ties_go_to_lower_index(gpu_lib):
    bits = _inputs(5, (1, 1, 1024, 64))
    k = bits["k"].copy()
    k[0, 0, 3 * 128:4 * 128] = k[0, 0, 6 * 128:7 * 128]   # blocks 3 and 6 score equally
    k[0, 0, 5 * 128:6 * 128] = k[0, 0, 6 * 128:7 * 128]   # and block 5 too
    idx_g = gpu_lib.block_select(to_dev(bits["q"]), to_dev(k), 2, 128)
    idx_r = bsp.select_blocks(to_f64(bits["q"]), to_f64(k), 128, 2)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_r)


@pytest.mark.parametrize("N,D,topk,mask", [(1024, 64, 3, 15), (1000, 128, 2, 15),
                                           (768, 128, 6, 0), (1000, 64, 8, 15)])
def test_sparse_attention(gpu_lib, N, D, topk, mask):
    bits = _inputs(100 + N, (1, 2, N, D), 1.5)
    f = {k: to_f64(v) for k, v in bits.items()}
    idx = bsp.select_blocks(f["q"], f["k"], 128, topk)
    sc = 1.0 / np.sqrt(D)
    O, L = bsp.forward(f["q"], f["k"], f["v"], sc, idx, 128, mask)
    dq, dk, dv = bsp.backward(f["q"], f["k"], f["v"], f["do"], sc, idx, 128, mask,
                              bf16_round(O), L)
    t = {k: to_dev(v) for k, v in bits.items()}
    it = torch.from_numpy(idx).to("cuda")
    o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, it)
    gdq, gdk, gdv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, mask, it)
    torch.cuda.synchronize()
    errs = {"o": rel_l2(dev_f64(o), O), "dq": rel_l2(dev_f64(gdq), dq, exact_zero=False),
            "dk": rel_l2(dev_f64(gdk), dk, exact_zero=False), "dv": rel_l2(dev_f64(gdv), dv)}
    lse_err = float(np.abs(lse.cpu().numpy() - L).max())
    msg = f"sparse N={N} D={D} topk={topk} mask={mask} {errs} lse {lse_err:.2e}"
    print(msg, flush=True)
    assert lse_err <= TOL_LSE, msg
    for e in errs.values():
        assert e <= tol_for(mask), msg


def test_sparse_all_blocks_equals_dense(gpu_lib):
    bits = _inputs(7, (1, 2, 512, 64), 1.5)
    t = {k: to_dev(v) for k, v in bits.items()}
    idx = torch.arange(4, dtype=torch.int32, device="cuda").repeat(1, 2, 4, 1).contiguous()
    o1, l1 = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15, idx)
    o2, l2 = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15)
    d1 = gpu_lib.bwd(t["q"], t["k"], t["v"], o1, l1, t["do"], 0.125, 15, idx)
    d2 = gpu_lib.bwd(t["q"], t["k"], t["v"], o2, l2, t["do"], 0.125, 15)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(d1, d2):
        assert torch.equal(a, b)

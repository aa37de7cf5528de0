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


def _all_blocks_vs_dense(gpu_lib, seed, shape):
    N = shape[2]
    nb = (N + 127) // 128
    bits = _inputs(seed, shape, 1.5)
    t = {k: to_dev(v) for k, v in bits.items()}
    idx = torch.arange(nb, dtype=torch.int32, device="cuda").repeat(1, shape[1], nb, 1).contiguous()
    o1, l1 = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15, idx)
    o2, l2 = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15)
    d1 = gpu_lib.bwd(t["q"], t["k"], t["v"], o1, l1, t["do"], 0.125, 15, idx)
    d2 = gpu_lib.bwd(t["q"], t["k"], t["v"], o2, l2, t["do"], 0.125, 15)
    torch.cuda.synchronize()
    return (o1, l1) + tuple(d1), (o2, l2) + tuple(d2)


def test_sparse_all_blocks_equals_dense(gpu_lib):
    """Selecting every key block reproduces the dense path. LSE accumulates
    in the same order and matches bit for bit. Dense forward pass 2, dK/dV
    and dQ launches whose workgroups do not fill whole rounds of compute
    units split the last round's blocks into parts (along the keys for O and
    dQ, the queries for dK/dV) summed in fp32 afterwards (a different
    summation order), so here O, dQ, dK and dV may differ by bf16 rounding
    flips only."""
    sp, de = _all_blocks_vs_dense(gpu_lib, 7, (1, 2, 512, 64))
    assert torch.equal(sp[1], de[1]), "lse"
    for name, a, b in zip(("o", "dq", "dk", "dv"), sp[:1] + sp[2:], de[:1] + de[2:]):
        a, b = a.float(), b.float()
        tol = 2.0 ** -7 * a.abs().maximum(b.abs()) + 1e-3 * float(b.abs().max())
        assert bool(((a - b).abs() <= tol).all()), name


def test_sparse_all_blocks_equals_dense_unsplit(gpu_lib):
    """With twice as many 128-key blocks and as many 256-query blocks as
    compute units the dense pass 2, dK/dV and dQ launches run whole blocks
    only, and every output matches the sparse path bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert cus <= 256
    sp, de = _all_blocks_vs_dense(gpu_lib, 8, (1, 2, 128 * cus, 64))
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), sp, de):
        assert torch.equal(a, b), name


def _index_with_last_block(seed, B, H, nbq, nbk, topk):
    """Ascending rows of `topk` key blocks, each holding the sequence's last
    (partial) block, so that every query block visits the masked tail."""
    rs = np.random.RandomState(seed)
    idx = np.empty((B, H, nbq, topk), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nbq):
                rest = rs.choice(nbk - 1, topk - 1, replace=False)
                idx[b, h, i] = np.sort(np.concatenate([rest, [nbk - 1]]))
    return idx


@pytest.mark.parametrize("N,D,topk,mask", [(1050, 128, 3, 15), (1025, 64, 2, 15),
                                           (1100, 128, 4, 15), (1050, 64, 3, 0),
                                           (129, 128, 1, 15)])
def test_sparse_partial_last_block(gpu_lib, N, D, topk, mask):
    """The last key block holds N % 128 keys (26, 1, 76, 26, 1): both of its
    64-key tiles run masked whether the first or only the second is partial,
    so keys past N add nothing to LSE, P or the gradients."""
    bits = _inputs(300 + N + D, (1, 2, N, D), 1.5)
    f = {k: to_f64(v) for k, v in bits.items()}
    nb = -(-N // 128)
    idx = _index_with_last_block(N + topk, 1, 2, nb, nb, topk)
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
    msg = f"sparse tail N={N} D={D} topk={topk} mask={mask} {errs} lse {lse_err:.2e}"
    print(msg, flush=True)
    assert lse_err <= TOL_LSE, msg
    for e in errs.values():
        assert e <= tol_for(mask), msg


@pytest.mark.parametrize("fault", ["out_of_range", "negative", "descending", "duplicate"])
def test_bad_block_index_is_caught_on_the_device(gpu_lib, fault):
    """An index entry outside [0, nbk) or a row that is not strictly ascending
    is found by the library's device-side check: no sparse kernel follows it,
    the outputs are NaN, and the binding raises."""
    N, D, topk = 512, 64, 2
    bits = _inputs(11, (1, 2, N, D))
    t = {k: to_dev(v) for k, v in bits.items()}
    idx = np.tile(np.array([0, 2], np.int32), (1, 2, 4, 1))
    bad = {"out_of_range": (1, 3, 1, 4), "negative": (0, 1, 0, -1),
           "descending": (0, 0, 0, 3), "duplicate": (1, 1, 0, 2)}[fault]
    idx[0, bad[0], bad[1], bad[2]] = bad[3]
    it = torch.from_numpy(idx).to("cuda")
    with pytest.raises(gpu_lib.AttnQatError, match="kv_block_idx"):
        gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15, it)
    o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15, it, validate_index=False)
    good = torch.from_numpy(np.tile(np.array([0, 2], np.int32), (1, 2, 4, 1))).to("cuda")
    og, lg = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15, good)
    with pytest.raises(gpu_lib.AttnQatError, match="kv_block_idx"):
        gpu_lib.bwd(t["q"], t["k"], t["v"], og, lg, t["do"], 0.125, 15, it)
    grads = gpu_lib.bwd(t["q"], t["k"], t["v"], og, lg, t["do"], 0.125, 15, it,
                        validate_index=False)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
    for g in grads:
        assert torch.isnan(g.float()).all()
    # a valid index afterwards runs normally on the same workspace size
    assert torch.isfinite(og.float()).all() and torch.isfinite(lg).all()


def test_block_index_layout_checks(gpu_lib):
    """int64 indices (what torch.topk returns), a wrong shape, or a
    non-contiguous view are rejected by the binding before any call."""
    bits = _inputs(12, (1, 1, 256, 64))
    t = {k: to_dev(v) for k, v in bits.items()}
    good = torch.zeros((1, 1, 2, 1), dtype=torch.int32, device="cuda")
    strided = torch.zeros((1, 1, 2, 2), dtype=torch.int32, device="cuda")[..., :1]
    assert not strided.is_contiguous()
    for bad in (good.long(), good[:, :, :1], strided, good.cpu()):
        with pytest.raises(gpu_lib.AttnQatError, match="kv_block_idx"):
            gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15, bad)
    o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15, good)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()

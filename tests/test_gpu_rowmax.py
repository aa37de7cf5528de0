"""GPU parity of the row-max-relative P quantization variant (p_mode
P_ROWMAX) against the fp64 oracle: every quant mask on the tiny workload,
ragged and cross-attention shapes, a length where the normalised P flushes
to zero, and the block-sparse path. The forward's row maxima are checked
against the oracle's; the oracle's backward takes D from its own forward
output rounded to bf16 (never from the GPU's output)."""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import block_sparse as bsp
from oracle.block_sparse import bf16_round
from synthetic import WORKLOADS, make_inputs, random_bf16
from tests.helpers import TOL_LSE, dev_f64, rel_l2, to_dev, to_f64, tol_for

pytestmark = pytest.mark.gpu
ROWMAX = oatt.P_ROWMAX


def _gpu(gpu_lib, bits, mask, sc, idx=None):
    t = {k: to_dev(v) for k, v in bits.items()}
    it = None if idx is None else torch.from_numpy(idx).to("cuda")
    o, lse, m = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, it, p_mode=ROWMAX)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, mask, it,
                             p_mode=ROWMAX, row_max=m)
    torch.cuda.synchronize()
    return {k: dev_f64(v) for k, v in dict(o=o, lse=lse, m=m, dq=dq, dk=dk, dv=dv).items()}


def _oracle(bits, mask, sc):
    f = {k: to_f64(v) for k, v in bits.items()}
    O, L, M = oatt.forward(f["q"], f["k"], f["v"], sc, mask, p_mode=ROWMAX, with_max=True)
    dq, dk, dv = oatt.backward(f["q"], f["k"], f["v"], f["do"], sc, mask, bf16_round(O), L,
                               p_mode=ROWMAX)
    return dict(o=O, lse=L, m=M, dq=dq, dk=dk, dv=dv)


def _compare(got, ref, mask, label):
    tol = tol_for(mask)
    errs = {k: rel_l2(got[k], ref[k], exact_zero=k in ("o", "dv"))
            for k in ("o", "dq", "dk", "dv")}
    lse_err = float(np.abs(got["lse"] - ref["lse"]).max())
    m_err = float(np.abs(got["m"] - ref["m"]).max())
    msg = f"rowmax {label} mask={mask} rel-L2 {errs} lse {lse_err:.2e} row max {m_err:.2e}"
    print(msg, flush=True)
    assert lse_err <= TOL_LSE and m_err <= TOL_LSE, msg
    for e in errs.values():
        assert e <= tol, msg


@pytest.mark.parametrize("mask", [15, 8, 12, 0])
def test_rowmax_tiny(gpu_lib, mask):
    w = WORKLOADS[1]
    bits = make_inputs(1)
    _compare(_gpu(gpu_lib, bits, mask, w.sm_scale), _oracle(bits, mask, w.sm_scale), mask, "tiny")


@pytest.mark.parametrize("Nq,Nk,D", [(100, 333, 128), (333, 77, 64), (1, 17, 128), (640, 640, 128)])
def test_rowmax_ragged_and_cross(gpu_lib, Nq, Nk, D):
    bits = {"q": random_bf16(41, (1, 2, Nq, D)), "k": random_bf16(42, (1, 2, Nk, D)),
            "v": random_bf16(43, (1, 2, Nk, D)), "do": random_bf16(44, (1, 2, Nq, D))}
    sc = 1.0 / np.sqrt(D)
    _compare(_gpu(gpu_lib, bits, 15, sc), _oracle(bits, 15, sc), 15, f"Nq={Nq} Nk={Nk} D={D}")


def test_rowmax_long_rows_keep_p_groups(gpu_lib):
    """At 4096 keys of i.i.d. scores the normalised P flushes most group scales
    to zero (its output keeps about a quarter of the norm); the row-max-relative
    P keeps them, and matches the oracle."""
    N, D = 4096, 64
    bits = {"q": random_bf16(51, (1, 1, N, D)), "k": random_bf16(52, (1, 1, N, D)),
            "v": random_bf16(53, (1, 1, N, D)), "do": random_bf16(54, (1, 1, N, D))}
    sc = 1.0 / np.sqrt(D)
    got = _gpu(gpu_lib, bits, 15, sc)
    ref = _oracle(bits, 15, sc)
    assert np.abs(ref["o"]).max() > 0.01
    _compare(got, ref, 15, f"N={N}")
    t = {k: to_dev(v) for k, v in bits.items()}
    o_n, _ = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, 15)
    assert np.linalg.norm(dev_f64(o_n)) < 0.5 * np.linalg.norm(got["o"])


def test_rowmax_sparse(gpu_lib):
    N, D, topk, mask = 1000, 128, 2, 15
    bits = {k: random_bf16(70 + i, (1, 2, N, D), 1.5) for i, k in enumerate(("q", "k", "v", "do"))}
    f = {k: to_f64(v) for k, v in bits.items()}
    idx = bsp.select_blocks(f["q"], f["k"], 128, topk)
    sc = 1.0 / np.sqrt(D)
    O, L = bsp.forward(f["q"], f["k"], f["v"], sc, idx, 128, mask, p_mode=ROWMAX)
    dq, dk, dv = bsp.backward(f["q"], f["k"], f["v"], f["do"], sc, idx, 128, mask, bf16_round(O),
                              L, p_mode=ROWMAX)
    got = _gpu(gpu_lib, bits, mask, sc, idx)
    ref = dict(o=O, dq=dq, dk=dk, dv=dv)
    errs = {k: rel_l2(got[k], ref[k], exact_zero=False) for k in ref}
    lse_err = float(np.abs(got["lse"] - L).max())
    msg = f"rowmax sparse {errs} lse {lse_err:.2e}"
    print(msg, flush=True)
    assert lse_err <= TOL_LSE, msg
    for e in errs.values():
        assert e <= tol_for(mask), msg

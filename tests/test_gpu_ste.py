"""GPU parity of the additive straight-through output O_ste = P Vq (the
forward's optional second output) and of the backward that takes its delta
from it (O_ste passed as the backward's o), against the fp64 oracle. The
oracle's backward gets its own O_ste rounded to bf16 (never the GPU's)."""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import block_sparse as bsp
from oracle.block_sparse import bf16_round
from synthetic import WORKLOADS, make_inputs, random_bf16
from tests.helpers import TOL_LSE, dev_f64, rel_l2, to_dev, to_f64, tol_for

pytestmark = pytest.mark.gpu


def _gpu(gpu_lib, bits, mask, sc, p_mode=0, idx=None):
    t = {k: to_dev(v) for k, v in bits.items()}
    it = None if idx is None else torch.from_numpy(idx).to("cuda")
    os_ = torch.empty_like(t["q"])
    res = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, it, p_mode=p_mode, o_ste=os_)
    o, lse = res[0], res[1]
    rm = res[2] if p_mode == oatt.P_ROWMAX else None
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], os_, lse, t["do"], sc, mask, it,
                             p_mode=p_mode, row_max=rm)
    torch.cuda.synchronize()
    return {k: dev_f64(v) for k, v in dict(o=o, os=os_, lse=lse, dq=dq, dk=dk, dv=dv).items()}


def _check(got, ref, mask, label):
    tol = tol_for(mask)
    errs = {k: rel_l2(got[k], ref[k], exact_zero=k in ("o", "dv")) for k in ref if k != "lse"}
    lse_err = float(np.abs(got["lse"] - ref["lse"]).max())
    msg = f"ste {label} mask={mask} rel-L2 {errs} lse {lse_err:.2e}"
    print(msg, flush=True)
    assert lse_err <= TOL_LSE, msg
    for e in errs.values():
        assert e <= tol, msg


def _oracle(bits, mask, sc, p_mode=0):
    f = {k: to_f64(v) for k, v in bits.items()}
    O, L, Os = oatt.forward(f["q"], f["k"], f["v"], sc, mask, p_mode=p_mode, with_ste=True)
    dq, dk, dv = oatt.backward(f["q"], f["k"], f["v"], f["do"], sc, mask, bf16_round(Os), L,
                               p_mode=p_mode)
    return dict(o=O, os=Os, lse=L, dq=dq, dk=dk, dv=dv)


@pytest.mark.parametrize("mask", [15, 8, 0])
def test_ste_tiny(gpu_lib, mask):
    w = WORKLOADS[1]
    bits = make_inputs(1)
    _check(_gpu(gpu_lib, bits, mask, w.sm_scale), _oracle(bits, mask, w.sm_scale), mask, "tiny")


@pytest.mark.parametrize("Nq,Nk,D", [(100, 333, 128), (333, 77, 64), (640, 640, 128)])
def test_ste_ragged_and_cross(gpu_lib, Nq, Nk, D):
    bits = {"q": random_bf16(81, (1, 2, Nq, D)), "k": random_bf16(82, (1, 2, Nk, D)),
            "v": random_bf16(83, (1, 2, Nk, D)), "do": random_bf16(84, (1, 2, Nq, D))}
    sc = 1.0 / np.sqrt(D)
    _check(_gpu(gpu_lib, bits, 15, sc), _oracle(bits, 15, sc), 15, f"Nq={Nq} Nk={Nk} D={D}")


def test_ste_with_rowmax(gpu_lib):
    w = WORKLOADS[1]
    bits = make_inputs(1)
    _check(_gpu(gpu_lib, bits, 15, w.sm_scale, p_mode=oatt.P_ROWMAX),
           _oracle(bits, 15, w.sm_scale, p_mode=oatt.P_ROWMAX), 15, "tiny rowmax")


def test_ste_sparse(gpu_lib):
    N, D, topk, mask = 1000, 128, 2, 15
    bits = {k: random_bf16(90 + i, (1, 2, N, D), 1.5) for i, k in enumerate(("q", "k", "v", "do"))}
    f = {k: to_f64(v) for k, v in bits.items()}
    idx = bsp.select_blocks(f["q"], f["k"], 128, topk)
    sc = 1.0 / np.sqrt(D)
    O, L, Os = bsp.forward(f["q"], f["k"], f["v"], sc, idx, 128, mask, with_ste=True)
    dq, dk, dv = bsp.backward(f["q"], f["k"], f["v"], f["do"], sc, idx, 128, mask, bf16_round(Os), L)
    got = _gpu(gpu_lib, bits, mask, sc, idx=idx)
    errs = {k: rel_l2(got[k], r, exact_zero=False)
            for k, r in dict(o=O, os=Os, dq=dq, dk=dk, dv=dv).items()}
    msg = f"ste sparse {errs} lse {float(np.abs(got['lse'] - L).max()):.2e}"
    print(msg, flush=True)
    for e in errs.values():
        assert e <= tol_for(mask), msg

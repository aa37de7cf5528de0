"""Parity of the P-quantizer variants and the VSA coarse branch at the sizes
the benchmark times them, in the launch configuration it uses.

* Row-max-relative P (p_mode P_ROWMAX) and the additive straight-through
  output (o_ste) at the kernel-timing workload (6 heads x 31,200 tokens, 1% of
  key rows x8): sampled query rows of three heads (O, O_ste, LSE, row maxima,
  dQ) and whole 16-key groups of one head (dK, dV, which need that head's full
  forward).
* The VSA step at its own workload (12 heads x 32,768 tokens, top-26 of 256
  blocks): coarse output and combination, the gate's gradient, and the summed
  fine + coarse gradients of sampled query and key blocks.

The GPU computes every output; the oracle recomputes the samples from the same
inputs (never from a GPU output).
"""
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import block_sparse as bsp
from oracle import vsa
from oracle.block_sparse import bf16_round
from synthetic import WORKLOADS, make_inputs, random_bf16
from tests.helpers import TOL_LSE, TOL_PLAIN, TOL_QUANT, dev_f64, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)
ROWMAX = oatt.P_ROWMAX


def _check(label, errs, stat_errs, tol):
    msg = f"{label} rel-L2 {errs} max-abs {stat_errs}"
    print(msg, flush=True)
    for e in stat_errs.values():
        assert e <= TOL_LSE, msg
    for e in errs.values():
        assert e <= tol, msg


def _rows(N, seed):
    rs = np.random.RandomState(seed)
    return np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N),
                                     rs.choice(N, 8, replace=False)]))


def _key_groups(N):
    ng = (N + 15) // 16
    return np.concatenate([np.arange(g * 16, min(N, g * 16 + 16)) for g in (0, ng // 2, ng - 1)])


def test_rowmax_full_size(gpu_lib):
    w = WORKLOADS[3]
    B, H, N, D = w.shape
    print(f"workload {w.name} {w.shape} p_mode=rowmax", flush=True)
    bits = make_inputs(3)
    t = {k: to_dev(v) for k, v in bits.items()}
    sc, mask = w.sm_scale, 15
    o, lse, m = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, p_mode=ROWMAX)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, mask, p_mode=ROWMAX,
                             row_max=m)
    torch.cuda.synchronize()
    rows = _rows(N, 31)
    for b, h in ((0, 0), (0, H // 2), (0, H - 1)):
        f = {k: to_f64(bits[k][b, h]) for k in bits}
        qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
        Or, Lr, Mr = oatt.head_forward(qq, kq, vq, sc, mask, rows=rows, p_mode=ROWMAX,
                                       with_max=True)
        dqr = oatt.head_backward_rows(qq, kq, vq, f["do"][rows], bf16_round(Or), Lr, rows, sc,
                                      mask)
        errs = {"o": rel_l2(dev_f64(o[b, h, rows]), Or),
                "dq": rel_l2(dev_f64(dq[b, h, rows]), dqr, exact_zero=False)}
        stats = {"lse": float(np.abs(lse[b, h, rows].cpu().numpy() - Lr).max()),
                 "row_max": float(np.abs(m[b, h, rows].cpu().numpy() - Mr).max())}
        _check(f"rowmax b={b} h={h} rows", errs, stats, TOL_QUANT)
    b, h = 0, 0
    f = {k: to_f64(bits[k][b, h]) for k in bits}
    qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
    Of, Lf, Mf = oatt.head_forward_all(qq, kq, vq, sc, mask, workers=WORKERS, p_mode=ROWMAX,
                                       with_max=True)
    keys = _key_groups(N)
    dkr, dvr = oatt.head_backward_keys(qq, kq, vq, f["do"], bf16_round(Of), Lf, sc, mask, keys,
                                       p_mode=ROWMAX, row_max=Mf)
    errs = {"o_head": rel_l2(dev_f64(o[b, h]), Of),
            "dk_keys": rel_l2(dev_f64(dk[b, h, keys]), dkr, exact_zero=False),
            "dv_keys": rel_l2(dev_f64(dv[b, h, keys]), dvr)}
    stats = {"lse": float(np.abs(lse[b, h].cpu().numpy() - Lf).max()),
             "row_max": float(np.abs(m[b, h].cpu().numpy() - Mf).max())}
    _check(f"rowmax b={b} h={h} full head", errs, stats, TOL_QUANT)


def test_ste_delta_full_size(gpu_lib):
    w = WORKLOADS[3]
    B, H, N, D = w.shape
    print(f"workload {w.name} {w.shape} o_ste", flush=True)
    bits = make_inputs(3)
    t = {k: to_dev(v) for k, v in bits.items()}
    sc, mask = w.sm_scale, 15
    os_ = torch.empty_like(t["q"])
    o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, o_ste=os_)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], os_, lse, t["do"], sc, mask)
    torch.cuda.synchronize()
    rows = _rows(N, 37)
    for b, h in ((0, 0), (0, H // 2), (0, H - 1)):
        f = {k: to_f64(bits[k][b, h]) for k in bits}
        qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
        Or, Lr, Osr = oatt.head_forward(qq, kq, vq, sc, mask, rows=rows, with_ste=True)
        dqr = oatt.head_backward_rows(qq, kq, vq, f["do"][rows], bf16_round(Osr), Lr, rows, sc,
                                      mask)
        errs = {"o": rel_l2(dev_f64(o[b, h, rows]), Or),
                "o_ste": rel_l2(dev_f64(os_[b, h, rows]), Osr),
                "dq": rel_l2(dev_f64(dq[b, h, rows]), dqr, exact_zero=False)}
        stats = {"lse": float(np.abs(lse[b, h, rows].cpu().numpy() - Lr).max())}
        _check(f"ste b={b} h={h} rows", errs, stats, TOL_QUANT)
    b, h = 0, 0
    f = {k: to_f64(bits[k][b, h]) for k in bits}
    qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
    Of, Lf, Osf = oatt.head_forward_all(qq, kq, vq, sc, mask, workers=WORKERS, with_ste=True)
    keys = _key_groups(N)
    dkr, dvr = oatt.head_backward_keys(qq, kq, vq, f["do"], bf16_round(Osf), Lf, sc, mask, keys)
    errs = {"o_head": rel_l2(dev_f64(o[b, h]), Of),
            "o_ste_head": rel_l2(dev_f64(os_[b, h]), Osf),
            "dk_keys": rel_l2(dev_f64(dk[b, h, keys]), dkr, exact_zero=False),
            "dv_keys": rel_l2(dev_f64(dv[b, h, keys]), dvr)}
    stats = {"lse": float(np.abs(lse[b, h].cpu().numpy() - Lf).max())}
    _check(f"ste b={b} h={h} full head", errs, stats, TOL_QUANT)


def test_vsa_full_size(gpu_lib):
    w = WORKLOADS[5]
    B, H, N, D = w.shape
    sc, bt, mask = w.sm_scale, w.block_tokens, 15
    print(f"workload {w.name} {w.shape} vsa topk={w.topk}", flush=True)
    bits = make_inputs(5)
    gbits = random_bf16(5006, w.shape)
    t = {k: to_dev(v) for k, v in bits.items()}
    g = to_dev(gbits)
    idx = bsp.select_blocks(to_f64(bits["q"]), to_f64(bits["k"]), bt, w.topk)
    it = torch.from_numpy(idx).to("cuda")
    of, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, it)
    o = gpu_lib.vsa_fwd(t["q"], t["k"], t["v"], g, of, sc)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], of, lse, t["do"], sc, mask, it)
    _, _, _, dg = gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], g, t["do"], dq, dk, dv, sc)
    torch.cuda.synchronize()
    nb = N // bt
    for h in (0, H - 1):
        f = {k: to_f64(bits[k][0, h]) for k in bits}
        gh = to_f64(gbits[0, h])
        oc, _, _ = vsa.coarse_forward(f["q"], f["k"], f["v"], sc, bt)
        cq, ck, cv, cg = vsa.coarse_backward(f["q"], f["k"], f["v"], gh, f["do"], sc, bt)
        qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
        # the combination adds gate * O_c of the token's block to the fine output
        # (compared as the GPU's o - o_fine against the oracle's gate * O_c)
        comb = dev_f64(o[0, h]) - dev_f64(of[0, h])
        errs = {"coarse_term": rel_l2(comb, gh * vsa.broadcast(oc, N, bt), exact_zero=False),
                "dgate": rel_l2(dev_f64(dg[0, h]), cg, exact_zero=False)}
        _check(f"vsa h={h} coarse", errs, {}, TOL_PLAIN)
        for i in (0, nb // 2, nb - 1):
            r0, r1 = i * bt, (i + 1) * bt
            _, Oi, Li, _, _ = bsp.query_block_forward(qq, kq, vq, idx[0, h, i], r0, r1, bt, sc,
                                                      mask)
            dqi = bsp.query_block_backward(qq, kq, vq, f["do"], bf16_round(Oi), idx[0, h, i],
                                           r0, r1, bt, sc, mask)
            errs = {"dq": rel_l2(dev_f64(dq[0, h, r0:r1]), dqi + cq[r0:r1], exact_zero=False)}
            stats = {"lse": float(np.abs(lse[0, h, r0:r1].cpu().numpy() - Li).max())}
            _check(f"vsa h={h} qblock={i}", errs, stats, TOL_QUANT)
        for j in (2, nb - 3):
            k0, k1 = j * bt, (j + 1) * bt
            dkj, dvj = bsp.key_block_backward(qq, kq, vq, f["do"], idx[0, h], j, bt, sc, mask,
                                              o_round=bf16_round)
            errs = {"dk": rel_l2(dev_f64(dk[0, h, k0:k1]), dkj + ck[k0:k1], exact_zero=False),
                    "dv": rel_l2(dev_f64(dv[0, h, k0:k1]), dvj + cv[k0:k1], exact_zero=False)}
            _check(f"vsa h={h} kblock={j}", errs, {}, TOL_QUANT)

"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

The GPU computes every output; the oracle checks samples it can afford:
query rows of three heads (O, LSE, dQ), every row of one head (O, LSE), and
whole 16-key groups of that head (dK, dV, which need that head's full forward).
With every quantizer off, sum_j dK_j is checked against the value shift
invariance gives it over every head.
"""
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle.block_sparse import bf16_round
from oracle.nvfp4 import fake_quant
from synthetic import WORKLOADS, make_inputs
from tests.helpers import (LSE_FLIP, TOL_LSE, best_candidate, dev_f64, rel_l2, rel_l2_best_rows,
                           to_dev, to_f64, tol_for)

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _check(label, errs, lse_err, tol):
    msg = f"{label} rel-L2 {errs} lse {lse_err:.2e}"
    print(msg, flush=True)
    assert lse_err <= TOL_LSE, msg
    for k, e in errs.items():
        assert e <= tol, msg


@pytest.mark.parametrize("cid,mask", [(2, 15), (3, 15), (4, 15), (4, 0)])
def test_full_size(gpu_lib, cid, mask):
    w = WORKLOADS[cid]
    print(f"workload {w.name} {w.shape} mask={mask}", flush=True)
    bits = make_inputs(cid)
    t = {k: to_dev(v) for k, v in bits.items()}
    sc = w.sm_scale
    o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, mask)
    torch.cuda.synchronize()
    B, H, N, D = w.shape
    tol = tol_for(mask)
    rs = np.random.RandomState(cid * 10 + mask)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N),
                                     rs.choice(N, 8, replace=False)]))
    heads = [(0, 0), (B - 1, H // 2), (B - 1, H - 1)]
    for b, h in heads:
        f = {k: to_f64(bits[k][b, h]) for k in bits}
        qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
        Or, Lr = oatt.head_forward(qq, kq, vq, sc, mask, rows=rows)
        dqr = oatt.head_backward_rows(qq, kq, vq, f["do"][rows], bf16_round(Or), Lr, rows, sc,
                                      mask)
        errs = {"o": rel_l2(dev_f64(o[b, h, rows]), Or),
                "dq": rel_l2(dev_f64(dq[b, h, rows]), dqr, exact_zero=False)}
        lse_err = float(np.abs(lse[b, h, rows].cpu().numpy() - Lr).max())
        _check(f"{w.name} b={b} h={h} rows", errs, lse_err, tol)

    # one head in full: O and LSE of every row, dK/dV of whole key groups
    b, h = 0, 0
    f = {k: to_f64(bits[k][b, h]) for k in bits}
    qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
    Of, Lf = oatt.head_forward_all(qq, kq, vq, sc, mask, workers=WORKERS)
    errs = {"o_head": rel_l2(dev_f64(o[b, h]), Of)}
    lse_err = float(np.abs(lse[b, h].cpu().numpy() - Lf).max())
    ng = (N + 15) // 16
    groups = [0, ng // 2, ng - 1]
    keys = np.concatenate([np.arange(g * 16, min(N, g * 16 + 16)) for g in groups])
    dkr, dvr = oatt.head_backward_keys(qq, kq, vq, f["do"], bf16_round(Of), Lf, sc, mask, keys)
    errs["dk_keys"] = rel_l2(dev_f64(dk[b, h, keys]), dkr, exact_zero=False)
    errs["dv_keys"] = rel_l2(dev_f64(dv[b, h, keys]), dvr)
    _check(f"{w.name} b={b} h={h} full head", errs, lse_err, tol)
    if np.linalg.norm(Of) == 0:
        # every quantized probability of this head flushed to zero
        assert torch.count_nonzero(o[b, h]) == 0 and torch.count_nonzero(dv[b, h]) == 0
    if mask == 0:
        # Shift invariance. With P = softmax(S) exactly, sum_j dS_ij =
        # dO_i . O_i - D_i, which is zero for D formed from the exact O; the
        # backward forms D from the stored bf16 O, so
        #   sum_j dK_j = c sum_i (dO_i . (O_i - Ostored_i)) Q_i
        # up to rounding. Rounding model (u = 2^-8 / sqrt 3 bounds the standard
        # deviation of one bf16 rounding, relative): each stored dK_j; dS,
        # rounded to bf16 before its products (half the relative size, and
        # the terms of dK_j have random signs, so its share is a quarter of
        # the stored dK's); and, where the exact O is not known, the D term
        # above as rounding noise of the stored O.
        u2 = (2.0 ** -8) ** 2 / 3
        g = dk.double()
        s = g.sum(dim=2)
        store = g.pow(2).sum(dim=2) * u2
        dsr = store / 4
        dD2 = (t["do"].double().pow(2) * o.double().pow(2)).sum(dim=3) * u2
        dterm = sc ** 2 * (dD2[..., None] * t["q"].double().pow(2)).sum(dim=2)
        ratio = (s.abs() / (store + dsr + dterm).sqrt().clamp_min(1e-30)).max().item()
        print(f"every head: max |sum_j dK_j| / sigma = {ratio:.2f}", flush=True)
        assert ratio <= 5.0
        # head (0, 0): the D term from the oracle's exact O, leaving rounding
        pred = sc * ((f["do"] * (Of - dev_f64(o[b, h]))).sum(axis=1) @ qq)
        res = np.abs(s[b, h].cpu().numpy() - pred)
        sig = np.sqrt((store[b, h] + dsr[b, h]).cpu().numpy())
        r0 = float((res / np.maximum(sig, 1e-30)).max())
        print(f"head (0, 0): max |sum_j dK_j - D term| / sigma = {r0:.2f} "
              f"(D term {np.abs(pred).max() / sig.max():.2f} sigma)", flush=True)
        assert r0 <= 5.0


def test_sparse_full_size(gpu_lib):
    from oracle import block_sparse as bsp
    w = WORKLOADS[5]
    bits = make_inputs(5)
    t = {k: to_dev(v) for k, v in bits.items()}
    B, H, N, D = w.shape
    sc, bt = w.sm_scale, w.block_tokens
    print(f"workload {w.name} {w.shape} topk={w.topk}", flush=True)
    idx_g = gpu_lib.block_select(t["q"], t["k"], w.topk, bt)
    idx_r = bsp.select_blocks(to_f64(bits["q"]), to_f64(bits["k"]), bt, w.topk)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_r)
    idx_t = torch.from_numpy(idx_r).to("cuda")
    o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, 15, idx_t)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, 15, idx_t)
    torch.cuda.synchronize()
    nb = N // bt
    for h in (0, H - 1):
        f = {k: to_f64(bits[k][0, h]) for k in bits}
        qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], 15)
        for i in (0, nb // 3, nb - 1):
            r0, r1 = i * bt, (i + 1) * bt
            keys, Oi, Li, Pi, _ = bsp.query_block_forward(qq, kq, vq, idx_r[0, h, i], r0, r1, bt,
                                                          sc, 15)
            dqi = bsp.query_block_backward(qq, kq, vq, f["do"], bf16_round(Oi), idx_r[0, h, i],
                                           r0, r1, bt, sc, 15)
            # these rows' largest probabilities are 0.003-0.014, so the P
            # quantizer's scales are near the E4M3 subnormal floor: accept the
            # decisions the oracle takes at LSE -/+ LSE_FLIP as well
            cands = [Oi] + [fake_quant(Pi * np.exp(-s), axis=-1) @ vq[keys]
                            for s in (-LSE_FLIP, LSE_FLIP)]
            og = dev_f64(o[0, h, r0:r1])
            errs = {"o": rel_l2_best_rows(og, cands),
                    "dq": rel_l2(dev_f64(dq[0, h, r0:r1]), dqi, exact_zero=False)}
            dl = np.abs(lse[0, h, r0:r1].cpu().numpy() - Li)
            lse_err = float(dl.max())
            # a row may match a shifted candidate only if the kernel's LSE is
            # within that shift of the oracle's
            flipped = best_candidate(og, cands) > 0
            flip_err = float(dl[flipped].max()) if flipped.any() else 0.0
            print(f"sparse h={h} qblock={i}: {int(flipped.sum())} rows matched at LSE -/+ "
                  f"{LSE_FLIP:g}, their max |dLSE| {flip_err:.2e}", flush=True)
            assert flip_err <= LSE_FLIP
            _check(f"sparse h={h} qblock={i}", errs, lse_err, 1e-2)
        for j in (1, nb - 2):
            dkj, dvj = bsp.key_block_backward(qq, kq, vq, f["do"], idx_r[0, h], j, bt, sc, 15,
                                              o_round=bf16_round)
            errs = {"dk": rel_l2(dev_f64(dk[0, h, j * bt:(j + 1) * bt]), dkj, exact_zero=False),
                    "dv": rel_l2(dev_f64(dv[0, h, j * bt:(j + 1) * bt]), dvj)}
            _check(f"sparse h={h} kblock={j}", errs, 0.0, 1e-2)

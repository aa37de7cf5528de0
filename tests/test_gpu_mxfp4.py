"""GPU parity of the real-FP4 (MXFP4) inference forward (attnqat_mxfp4_fwd)
against the fp64 oracle (oracle/mxfp4.py): ragged and cross-attention
shapes, d = 64 and 128, a single key, the tiny workload, strided inputs,
determinism, and sampled query rows at the timing workload's full size.
Tolerances are those of the quantized path (O rel-L2 1e-2, LSE 1e-3): the
products of FP4 operands are exact, and the two sides differ by fp32
rounding of the sums and of exp, which can move a P~ across an E2M1 rounding
boundary."""
import numpy as np
import pytest
import torch

from oracle import mxfp4
from synthetic import WORKLOADS, make_inputs, random_bf16
from tests.helpers import TOL_LSE, TOL_QUANT, dev_f64, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _check(label, o, lse, ref_o, ref_l):
    e = rel_l2(dev_f64(o), ref_o)
    le = float(np.abs(lse.cpu().numpy() - ref_l).max())
    msg = f"mxfp4 {label} rel-L2 o={e:.3e} lse={le:.2e}"
    print(msg, flush=True)
    assert le <= TOL_LSE, msg
    assert e <= TOL_QUANT, msg


@pytest.mark.parametrize("B,H,Nq,Nk,D", [(1, 2, 300, 300, 128), (1, 2, 100, 333, 64),
                                         (2, 1, 77, 1000, 128), (1, 1, 5, 1, 64),
                                         (1, 3, 640, 256, 128)])
def test_mxfp4_against_oracle(gpu_lib, B, H, Nq, Nk, D):
    s = 11 + Nq + Nk + D
    bits = {"q": random_bf16(s, (B, H, Nq, D), 1.5), "k": random_bf16(s + 1, (B, H, Nk, D), 1.5),
            "v": random_bf16(s + 2, (B, H, Nk, D))}
    t = {n: to_dev(x) for n, x in bits.items()}
    sc = 1.0 / np.sqrt(D)
    o, lse = gpu_lib.mxfp4_fwd(t["q"], t["k"], t["v"], sc)
    torch.cuda.synchronize()
    O, L = mxfp4.forward(to_f64(bits["q"]), to_f64(bits["k"]), to_f64(bits["v"]), sc)
    _check(f"B={B} H={H} Nq={Nq} Nk={Nk} D={D}", o, lse, O, L)


def test_mxfp4_tiny_workload_strided_and_deterministic(gpu_lib):
    w = WORKLOADS[1]
    bits = make_inputs(1)
    B, H, N, D = w.shape
    O, L = mxfp4.forward(to_f64(bits["q"]), to_f64(bits["k"]), to_f64(bits["v"]), w.sm_scale)
    t = {n: to_dev(bits[n]) for n in ("q", "k", "v")}
    o1, l1 = gpu_lib.mxfp4_fwd(t["q"], t["k"], t["v"], w.sm_scale)
    o2, l2 = gpu_lib.mxfp4_fwd(t["q"], t["k"], t["v"], w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _check("tiny", o1, l1, O, L)
    # [B, N, H, D] storage viewed as [B, H, N, D], output into a strided view
    ts = {n: to_dev(bits[n]).transpose(1, 2).contiguous().transpose(1, 2) for n in ("q", "k", "v")}
    out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o3, l3 = gpu_lib.mxfp4_fwd(ts["q"], ts["k"], ts["v"], w.sm_scale, out=out)
    torch.cuda.synchronize()
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_mxfp4_full_size_sampled_rows(gpu_lib):
    """The timing workload (6 heads x 31,200 tokens, d = 128) in the launch
    configuration the benchmark times: sampled query rows of two heads."""
    w = WORKLOADS[3]
    bits = make_inputs(3)
    t = {n: to_dev(bits[n]) for n in ("q", "k", "v")}
    o, lse = gpu_lib.mxfp4_fwd(t["q"], t["k"], t["v"], w.sm_scale)
    torch.cuda.synchronize()
    B, H, N, D = w.shape
    rows = np.unique(np.concatenate([np.arange(4), np.arange(N - 4, N),
                                     np.random.RandomState(7).choice(N, 8, replace=False)]))
    for b, h in ((0, 0), (B - 1, H - 1)):
        f = {n: to_f64(bits[n][b, h]) for n in ("q", "k", "v")}
        O, L = mxfp4.forward(f["q"][rows], f["k"], f["v"], w.sm_scale)
        _check(f"full size b={b} h={h}", o[b, h, rows], lse[b, h, rows], O, L)

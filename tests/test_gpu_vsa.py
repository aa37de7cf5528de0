"""GPU parity of the VSA coarse branch and gated combination (attnqat_vsa_fwd,
attnqat_vsa_bwd) against the fp64 oracle (oracle/vsa.py): the coarse
contribution alone (zero fine output and zero incoming gradients), the
in-place accumulation onto given gradients, the whole VSA pipeline (selection,
fine branch, coarse branch) with every quantizer on, ragged and
cross-attention lengths, d = 64, a single block, and a zero gate."""
import numpy as np
import pytest
import torch

from oracle import block_sparse as bsp
from oracle import vsa
from oracle.block_sparse import bf16_round
from synthetic import random_bf16
from tests.helpers import TOL_PLAIN, TOL_QUANT, dev_f64, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _bits(seed, B, H, Nq, Nk, D):
    return {"q": random_bf16(seed, (B, H, Nq, D)), "k": random_bf16(seed + 1, (B, H, Nk, D)),
            "v": random_bf16(seed + 2, (B, H, Nk, D)), "g": random_bf16(seed + 3, (B, H, Nq, D)),
            "do": random_bf16(seed + 4, (B, H, Nq, D))}


def _report(label, errs):
    msg = f"vsa {label} rel-L2 " + " ".join(f"{k}={v:.2e}" for k, v in errs.items())
    print(msg, flush=True)
    return msg


@pytest.mark.parametrize("Nq,Nk,D", [(1000, 1000, 128), (300, 700, 64), (100, 90, 128),
                                     (640, 384, 128)])
def test_vsa_coarse_parts(gpu_lib, Nq, Nk, D):
    """Coarse output with a zero fine output, and coarse gradients added to
    zero gradients, against the oracle's coarse branch."""
    bits = _bits(7 + Nq + D, 1, 2, Nq, Nk, D)
    t = {k: to_dev(v) for k, v in bits.items()}
    f = {k: to_f64(v) for k, v in bits.items()}
    sc = 1.0 / np.sqrt(D)
    zero = torch.zeros_like(t["q"])
    o = gpu_lib.vsa_fwd(t["q"], t["k"], t["v"], t["g"], zero, sc)
    dq, dk, dv = torch.zeros_like(t["q"]), torch.zeros_like(t["k"]), torch.zeros_like(t["v"])
    _, _, _, dg = gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], t["g"], t["do"], dq, dk, dv, sc)
    torch.cuda.synchronize()
    oc, _, _ = vsa.coarse_forward(f["q"], f["k"], f["v"], sc, 128)
    ref_o = vsa.combine(np.zeros_like(f["q"]), f["g"], oc, 128)
    cq, ck, cv, cg = vsa.coarse_backward(f["q"], f["k"], f["v"], f["g"], f["do"], sc, 128)
    errs = {"o": rel_l2(dev_f64(o), ref_o, exact_zero=False),
            "dq": rel_l2(dev_f64(dq), cq, exact_zero=False),
            "dk": rel_l2(dev_f64(dk), ck, exact_zero=False),
            "dv": rel_l2(dev_f64(dv), cv, exact_zero=False),
            "dg": rel_l2(dev_f64(dg), cg, exact_zero=False)}
    msg = _report(f"coarse Nq={Nq} Nk={Nk} D={D}", errs)
    for e in errs.values():
        assert e <= TOL_PLAIN, msg


def test_vsa_accumulates_and_zero_gate(gpu_lib):
    """vsa_bwd adds to the gradients it is given; a zero gate leaves the fine
    output unchanged bit for bit and adds no coarse gradient."""
    bits = _bits(51, 1, 1, 512, 512, 128)
    t = {k: to_dev(v) for k, v in bits.items()}
    f = {k: to_f64(v) for k, v in bits.items()}
    sc = 0.0884
    base = {n: random_bf16(60 + i, (1, 1, 512, 128)) for i, n in enumerate(("dq", "dk", "dv", "of"))}
    g = {n: to_dev(v) for n, v in base.items()}
    dq, dk, dv = g["dq"].clone(), g["dk"].clone(), g["dv"].clone()
    gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], t["g"], t["do"], dq, dk, dv, sc, want_dgate=False)
    zg = torch.zeros_like(t["g"])
    o0 = gpu_lib.vsa_fwd(t["q"], t["k"], t["v"], zg, g["of"], sc)
    zq, zk, zv = g["dq"].clone(), g["dk"].clone(), g["dv"].clone()
    _, _, _, dg0 = gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], zg, t["do"], zq, zk, zv, sc)
    torch.cuda.synchronize()
    cq, ck, cv, _ = vsa.coarse_backward(f["q"], f["k"], f["v"], f["g"], f["do"], sc, 128)
    errs = {n: rel_l2(dev_f64(x), to_f64(base[n]) + c, exact_zero=False)
            for n, x, c in (("dq", dq, cq), ("dk", dk, ck), ("dv", dv, cv))}
    msg = _report("accumulate", errs)
    for e in errs.values():
        assert e <= TOL_PLAIN, msg
    assert torch.equal(o0, g["of"])
    # dk, dv get exactly zero added (rounding the unchanged bf16 value); dq too
    assert torch.equal(zq, g["dq"]) and torch.equal(zk, g["dk"]) and torch.equal(zv, g["dv"])
    oc, _, _ = vsa.coarse_forward(f["q"], f["k"], f["v"], sc, 128)
    assert rel_l2(dev_f64(dg0), f["do"] * vsa.broadcast(oc, 512, 128), exact_zero=False) <= TOL_PLAIN


@pytest.mark.parametrize("N,topk", [(1000, 2), (1536, 3)])
def test_vsa_pipeline(gpu_lib, N, topk):
    """Selection (the oracle's index, as for the sparse tests), fine branch
    with every quantizer on, coarse branch and combination; backward as the
    training step runs it: fine backward with o = o_fine, then vsa_bwd."""
    D, mask = 128, 15
    bits = _bits(90 + N, 1, 2, N, N, D)
    for key in ("q", "k"):
        bits[key] = random_bf16(95 + N + len(key), (1, 2, N, D), 1.5)
    t = {k: to_dev(v) for k, v in bits.items()}
    f = {k: to_f64(v) for k, v in bits.items()}
    sc = 1.0 / np.sqrt(D)
    idx = bsp.select_blocks(f["q"], f["k"], 128, topk)
    it = torch.from_numpy(idx).to("cuda")
    of, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, it)
    o = gpu_lib.vsa_fwd(t["q"], t["k"], t["v"], t["g"], of, sc)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], of, lse, t["do"], sc, mask, it)
    _, _, _, dg = gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], t["g"], t["do"], dq, dk, dv, sc)
    torch.cuda.synchronize()
    O, Of, L = vsa.forward(f["q"], f["k"], f["v"], f["g"], sc, idx, 128, mask)
    rq, rk, rv, rg = vsa.backward(f["q"], f["k"], f["v"], f["g"], f["do"], sc, idx, 128, mask,
                                  bf16_round(Of), L)
    errs = {"o": rel_l2(dev_f64(o), O, exact_zero=False),
            "dq": rel_l2(dev_f64(dq), rq, exact_zero=False),
            "dk": rel_l2(dev_f64(dk), rk, exact_zero=False),
            "dv": rel_l2(dev_f64(dv), rv, exact_zero=False),
            "dg": rel_l2(dev_f64(dg), rg, exact_zero=False)}
    msg = _report(f"pipeline N={N} topk={topk}", errs)
    for e in errs.values():
        assert e <= TOL_QUANT, msg


def test_vsa_strided(gpu_lib):
    """Non-contiguous [B,H,N,D] views (heads interleaved) for every tensor."""
    B, H, N, D = 1, 2, 384, 64
    raw = {k: random_bf16(120 + i, (B, N, H, D)) for i, k in enumerate(("q", "k", "v", "g", "do", "of"))}
    t = {k: to_dev(v).permute(0, 2, 1, 3) for k, v in raw.items()}
    f = {k: to_f64(v).transpose(0, 2, 1, 3) for k, v in raw.items()}
    sc = 0.125
    out = torch.empty_like(to_dev(raw["of"])).permute(0, 2, 1, 3)
    o = gpu_lib.vsa_fwd(t["q"], t["k"], t["v"], t["g"], t["of"], sc, out=out)
    dq = torch.zeros_like(to_dev(raw["q"])).permute(0, 2, 1, 3)
    dk = torch.zeros_like(to_dev(raw["k"])).permute(0, 2, 1, 3)
    dv = torch.zeros_like(to_dev(raw["v"])).permute(0, 2, 1, 3)
    dg = torch.empty_like(to_dev(raw["g"])).permute(0, 2, 1, 3)
    gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], t["g"], t["do"], dq, dk, dv, sc, dgate=dg)
    torch.cuda.synchronize()
    oc, _, _ = vsa.coarse_forward(f["q"], f["k"], f["v"], sc, 128)
    cq, ck, cv, cg = vsa.coarse_backward(f["q"], f["k"], f["v"], f["g"], f["do"], sc, 128)
    errs = {"o": rel_l2(dev_f64(o), vsa.combine(f["of"], f["g"], oc, 128), exact_zero=False),
            "dq": rel_l2(dev_f64(dq), cq, exact_zero=False),
            "dk": rel_l2(dev_f64(dk), ck, exact_zero=False),
            "dv": rel_l2(dev_f64(dv), cv, exact_zero=False),
            "dg": rel_l2(dev_f64(dg), cg, exact_zero=False)}
    msg = _report("strided", errs)
    for e in errs.values():
        assert e <= TOL_PLAIN, msg


def test_vsa_autograd_matches_entry_points(gpu_lib):
    """The autograd wrapper runs exactly the entry-point sequence (bitwise)."""
    bits = _bits(140, 1, 2, 700, 700, 128)
    t = {k: to_dev(v) for k, v in bits.items()}
    sc = 1.0 / np.sqrt(128)
    idx = gpu_lib.block_select(t["q"], t["k"], 2)
    leaves = {n: t[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g")}
    o = gpu_lib.vsa_attention(leaves["q"], leaves["k"], leaves["v"], leaves["g"], sm_scale=sc,
                              kv_block_idx=idx)
    o.backward(t["do"])
    of, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, "qkvp", idx)
    o2 = gpu_lib.vsa_fwd(t["q"], t["k"], t["v"], t["g"], of, sc)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], of, lse, t["do"], sc, "qkvp", idx)
    _, _, _, dg = gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], t["g"], t["do"], dq, dk, dv, sc)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for n, ref in (("q", dq), ("k", dk), ("v", dv), ("g", dg)):
        assert torch.equal(leaves[n].grad, ref), n
    assert gpu_lib.effective_topk(6, 0.9) == 1 and gpu_lib.effective_topk(256, 0.9) == 26


def test_vsa_pipeline_partial_last_block(gpu_lib):
    """1,050 tokens (a last block of 26) with that block selected by every
    query block: the fine branch's masked tail and the coarse branch's
    partial-block means together, forward and backward."""
    N, D, topk, mask = 1050, 128, 3, 15
    bits = _bits(333, 1, 2, N, N, D)
    t = {k: to_dev(v) for k, v in bits.items()}
    f = {k: to_f64(v) for k, v in bits.items()}
    sc = 1.0 / np.sqrt(D)
    nb = -(-N // 128)
    rs = np.random.RandomState(5)
    idx = np.empty((1, 2, nb, topk), np.int32)
    for h in range(2):
        for i in range(nb):
            idx[0, h, i] = np.sort(np.concatenate([rs.choice(nb - 1, topk - 1, replace=False),
                                                   [nb - 1]]))
    it = torch.from_numpy(idx).to("cuda")
    of, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask, it)
    o = gpu_lib.vsa_fwd(t["q"], t["k"], t["v"], t["g"], of, sc)
    dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], of, lse, t["do"], sc, mask, it)
    _, _, _, dg = gpu_lib.vsa_bwd(t["q"], t["k"], t["v"], t["g"], t["do"], dq, dk, dv, sc)
    torch.cuda.synchronize()
    O, Of, L = vsa.forward(f["q"], f["k"], f["v"], f["g"], sc, idx, 128, mask)
    rq, rk, rv, rg = vsa.backward(f["q"], f["k"], f["v"], f["g"], f["do"], sc, idx, 128, mask,
                                  bf16_round(Of), L)
    errs = {"o": rel_l2(dev_f64(o), O, exact_zero=False),
            "dq": rel_l2(dev_f64(dq), rq, exact_zero=False),
            "dk": rel_l2(dev_f64(dk), rk, exact_zero=False),
            "dv": rel_l2(dev_f64(dv), rv, exact_zero=False),
            "dg": rel_l2(dev_f64(dg), rg, exact_zero=False)}
    msg = _report(f"pipeline N={N} partial last block", errs)
    assert float(np.abs(lse.cpu().numpy() - L).max()) <= 1e-3, msg
    for e in errs.values():
        assert e <= TOL_QUANT, msg

"""GPU parity of the Attn-QAT forward and backward against the fp64 oracle.

Small sizes the oracle finishes in seconds, spanning several 128-token tiles
and ragged tails; every quantization mask on the tiny workload; cross-attention
with Nq != Nk; determinism, stream order, strided layouts and input
immutability.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle.block_sparse import bf16_round
from synthetic import WORKLOADS, bf16_bits_from_f32, make_inputs, random_bf16
from tests.helpers import TOL_LSE, dev_bits, dev_f64, rel_l2, to_dev, to_f64, tol_for

pytestmark = pytest.mark.gpu


def _run_pair(gpu_lib, bits, mask, sc, do_bwd=True):
    t = {k: to_dev(v) for k, v in bits.items()}
    o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], sc, mask)
    out = {"o": o, "lse": lse}
    if do_bwd:
        dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], sc, mask)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k: dev_f64(v) for k, v in out.items()}


def _oracle(bits, mask, sc, do_bwd=True):
    """Oracle forward; its backward takes D from the forward output as returned,
    i.e. rounded to the bf16 output dtype (never from the GPU's output)."""
    f = {k: to_f64(v) for k, v in bits.items()}
    O, L = oatt.forward(f["q"], f["k"], f["v"], sc, mask)
    res = {"o": O, "lse": L}
    if do_bwd:
        res["dq"], res["dk"], res["dv"] = oatt.backward(f["q"], f["k"], f["v"], f["do"], sc, mask,
                                                        bf16_round(O), L)
    return res


def _compare(got, ref, mask, label):
    tol = tol_for(mask)
    errs = {k: rel_l2(got[k], ref[k], exact_zero=k in ("o", "dv")) for k in got if k != "lse"}
    lse_err = float(np.abs(got["lse"] - ref["lse"]).max())
    msg = f"{label} mask={mask} rel-L2 {errs} lse {lse_err:.2e}"
    print(msg, flush=True)
    assert lse_err <= TOL_LSE, msg
    for k, e in errs.items():
        assert e <= tol, msg


@pytest.mark.parametrize("mask", list(range(16)))
def test_tiny_all_masks(gpu_lib, mask):
    w = WORKLOADS[1]
    bits = make_inputs(1)
    got = _run_pair(gpu_lib, bits, mask, w.sm_scale)
    ref = _oracle(bits, mask, w.sm_scale)
    _compare(got, ref, mask, "tiny")


@pytest.mark.parametrize("Nq,Nk,D", [(200, 200, 64), (100, 333, 128), (333, 77, 64),
                                     (1, 17, 128), (130, 1, 64), (384, 256, 128)])
@pytest.mark.parametrize("mask", [15, 0])
def test_ragged_and_cross(gpu_lib, Nq, Nk, D, mask):
    bits = {"q": random_bf16(11, (2, 2, Nq, D)), "k": random_bf16(12, (2, 2, Nk, D)),
            "v": random_bf16(13, (2, 2, Nk, D)), "do": random_bf16(14, (2, 2, Nq, D))}
    sc = 1.0 / np.sqrt(D)
    got = _run_pair(gpu_lib, bits, mask, sc)
    ref = _oracle(bits, mask, sc)
    _compare(got, ref, mask, f"Nq={Nq} Nk={Nk} D={D}")


@pytest.mark.parametrize("Nq,Nk,D", [(2100, 2100, 128), (1500, 1500, 64), (1100, 2400, 64)])
def test_last_round_shared_out(gpu_lib, Nq, Nk, D):
    """Dense pass 2 and dQ run one workgroup per 256 queries; a round that
    does not fill the compute units is shared out along the key tiles (2 x 2
    heads x 2100 tokens: 36 query blocks of 33 tiles in chunks of 9 tiles, so
    chunks cross block boundaries; 1500 tokens: 24 blocks of 24 tiles in
    chunks of 8; 1100 queries against 2400 keys: 20 blocks of 38 tiles in
    chunks of 8, crossing) and a fixup adds the partial sums; ragged last
    query block and key tile."""
    bits = {"q": random_bf16(61, (2, 2, Nq, D)), "k": random_bf16(62, (2, 2, Nk, D)),
            "v": random_bf16(63, (2, 2, Nk, D)), "do": random_bf16(64, (2, 2, Nq, D))}
    sc = 1.0 / np.sqrt(D)
    got = _run_pair(gpu_lib, bits, 15, sc)
    ref = _oracle(bits, 15, sc)
    _compare(got, ref, 15, f"shared-out Nq={Nq} Nk={Nk} D={D}")


def test_sm_scale_is_honoured(gpu_lib):
    bits = make_inputs(1)
    for sc in (0.05, 0.3):
        got = _run_pair(gpu_lib, bits, 15, sc)
        ref = _oracle(bits, 15, sc)
        _compare(got, ref, 15, f"sm_scale={sc}")


def test_wide_scores_keep_p_groups(gpu_lib):
    """Larger logits so that many P groups keep a non-zero scale at N = 640."""
    bits = {"q": random_bf16(21, (1, 2, 640, 128), 2.0), "k": random_bf16(22, (1, 2, 640, 128), 2.0),
            "v": random_bf16(23, (1, 2, 640, 128)), "do": random_bf16(24, (1, 2, 640, 128))}
    got = _run_pair(gpu_lib, bits, 15, 1 / np.sqrt(128))
    ref = _oracle(bits, 15, 1 / np.sqrt(128))
    assert np.linalg.norm(ref["o"]) > 0
    _compare(got, ref, 15, "wide")


@pytest.mark.parametrize("mask", [15, 8])
def test_growing_scores_move_the_reference_maximum(gpu_lib, mask):
    """Scores that grow along the keys, so that forward pass 1 keeps moving
    its reference maximum: head 0 gains about 32 nats per 32-key block and
    jumps by 120 nats at key 200 (the block sum against the old maximum
    overflows to inf); head 1 gains 8 nats per block, so several blocks sum
    against a stale maximum before it moves."""
    N, D = 384, 64
    f = {n: to_f64(random_bf16(70 + i, (1, 2, N, D), 0.25)) for i, n in enumerate(("q", "k"))}
    f["q"][..., 0] = 1.0
    j = np.arange(N, dtype=np.float64)
    f["k"][0, 0, :, 0] = j + np.where(j >= 200, 120.0, 0.0)
    f["k"][0, 1, :, 0] = j / 4
    bits = {n: bf16_bits_from_f32(f[n].astype(np.float32)) for n in ("q", "k")}
    bits["v"] = random_bf16(72, (1, 2, N, D))
    bits["do"] = random_bf16(73, (1, 2, N, D))
    got = _run_pair(gpu_lib, bits, mask, 1.0)
    ref = _oracle(bits, mask, 1.0)
    assert ref["lse"][0, 0].max() > 300 and ref["lse"][0, 1].max() > 80
    # Every key carries a large component k_j0 (up to ~500) that differs by
    # about 1 between the keys holding the probability mass, so dQ = sum_j dS_j
    # k_j (with sum_j dS_j = 0) cancels to a few hundredths of its terms, and
    # dK = sum_i dS_i q_i partly too: the bf16 rounding of dS (an operand of
    # the BF16 products, exact in the fp64 oracle) is amplified there, and the
    # oracle's own dQ moves by 1.6-3.3% when O is not rounded to bf16. A
    # rounding of dS by a relative 2^-9 moves each dQ entry by at most 2^-9
    # sum_j |dS_j| |k_j|, so dQ and dK are compared against the size of their
    # terms: |error| over those sums of absolute values, at the same 1e-2.
    # Head 0 with Q and K unquantized (mask 8) is left out of that check: its
    # scores reach ~500, where the fp32 products carry absolute errors of
    # ~1e-4, enough to flip P-quantization decisions (O moves by ~0.6%), and
    # the resulting change of D = rowsum(dO O) enters dQ through the same
    # cancellation. (With K quantized its rows reduce to the one large
    # component and the scores are exact.)
    heads = [0, 1] if mask & oatt.MASK_K else [1]
    aq, ak = _abs_terms(bits, mask, 1.0)
    for k, a in (("dq", aq), ("dk", ak)):
        g, r = got.pop(k)[:, heads], ref.pop(k)[:, heads]
        e = float(np.linalg.norm(g - r) / np.linalg.norm(a[:, heads]))
        print(f"growing scores mask={mask} heads {heads} {k}: |error| / |sum of |terms|| = "
              f"{e:.2e}", flush=True)
        assert e <= tol_for(mask)
    _compare(got, ref, mask, "growing scores")


def _abs_terms(bits, mask, sc):
    """sc |dS| |Kq| and sc |dS|^T |Qq|: the sums of absolute values of the
    terms that make up dQ and dK (dS from the oracle's forward, D taken from
    its output rounded to bf16 as in _oracle)."""
    f = {k: to_f64(v) for k, v in bits.items()}
    O, L = oatt.forward(f["q"], f["k"], f["v"], sc, mask)
    qq, kq, vq = oatt.quantize_operands(f["q"], f["k"], f["v"], mask)
    Ob = bf16_round(O)
    aq, ak = np.zeros_like(qq), np.zeros_like(kq)
    for b in range(qq.shape[0]):
        for h in range(qq.shape[1]):
            P = np.exp(sc * (qq[b, h] @ kq[b, h].T) - L[b, h][:, None])
            Dl = np.sum(f["do"][b, h] * Ob[b, h], axis=-1)
            dS = np.abs(P * (f["do"][b, h] @ vq[b, h].T - Dl[:, None]))
            aq[b, h] = sc * (dS @ np.abs(kq[b, h]))
            ak[b, h] = sc * (dS.T @ np.abs(qq[b, h]))
    return aq, ak


def test_deterministic_and_inputs_unchanged(gpu_lib):
    bits = {"q": random_bf16(31, (1, 3, 300, 128)), "k": random_bf16(32, (1, 3, 300, 128)),
            "v": random_bf16(33, (1, 3, 300, 128)), "do": random_bf16(34, (1, 3, 300, 128))}
    t = {k: to_dev(v) for k, v in bits.items()}
    outs = []
    for _ in range(2):
        o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.1, 15)
        dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], 0.1, 15)
        torch.cuda.synchronize()
        outs.append([dev_bits(x) if x.dtype == torch.bfloat16 else x.cpu().numpy()
                     for x in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    for k, v in bits.items():
        np.testing.assert_array_equal(dev_bits(t[k]), v)


def test_non_default_stream_and_strides(gpu_lib):
    B, H, N, D = 1, 2, 260, 64
    bits = {k: random_bf16(40 + i, (B, N, H, D)) for i, k in enumerate(("q", "k", "v", "do"))}
    t = {k: to_dev(v).permute(0, 2, 1, 3) for k, v in bits.items()}   # BSHD memory, BHSD view
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.125, 15)
        dq, dk, dv = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], 0.125, 15)
    s.synchronize()
    ref = _oracle({k: np.ascontiguousarray(v.transpose(0, 2, 1, 3)) for k, v in bits.items()},
                  15, 0.125)
    got = {"o": dev_f64(o), "lse": lse.cpu().numpy(), "dq": dev_f64(dq), "dk": dev_f64(dk),
           "dv": dev_f64(dv)}
    _compare(got, ref, 15, "strided+stream")


def test_autograd_function(gpu_lib):
    bits = make_inputs(1)
    t = {k: to_dev(v).requires_grad_(k != "do") for k, v in bits.items()}
    o = gpu_lib.attention(t["q"], t["k"], t["v"])
    o.backward(t["do"])
    ref = _oracle(bits, 15, WORKLOADS[1].sm_scale)
    assert rel_l2(dev_f64(o), ref["o"]) <= 1e-2
    for n in ("q", "k", "v"):
        assert rel_l2(dev_f64(t[n].grad), ref["d" + n]) <= 1e-2

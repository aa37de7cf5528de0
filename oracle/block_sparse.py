"""VSA-style block selection and block-sparse fine attention (fp64 numpy).

TEST INFRASTRUCTURE: part of the CPU oracle; only tests, the smoke check and the
benchmark's CPU-baseline leg may import it.

Source: FastVideo VSA checkpoint metadata, ``attention`` object:
``cube_shape`` [4, 4, 8] (128-token blocks), ``precision.coarse`` "BF16" with
``quantize_coarse`` false, ``precision.fine`` "NVFP4 fake-quant with BF16
matmul", and ``selection.effective_topk`` = max(1, min(ceil((1 - sparsity) *
num_blocks), num_blocks)) with sparsity 0.9.

Readings where the page is silent:

* Coarse scores: mean-pool Q and K over each block of ``block_tokens`` tokens
  (a partial last block is averaged over its own tokens); the pooled means and
  the block-pair scores are rounded to bfloat16 (the coarse precision) from
  their exact values. Pooled sums of bf16 inputs and dot products of bf16
  means are exact in float64 for the value ranges used, so the rounding
  decisions do not depend on summation order. No softmax scale is applied:
  a positive scale does not change the ordering.
* Selection: the ``topk`` highest scores per query block, ties to the lower
  key-block index; the chosen block indices are returned in ascending order.
  The page names the mode "top-p" next to a count formula; the count formula is
  the one that fixes a number, so it is the one used.
* Fine attention: each query row attends only to the keys of the blocks its
  query block selected, visited in ascending order. LSE and P are over those
  keys only, and the 16-key P groups align within each block.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import MASK_ALL, MASK_P, P_NORMALISED, probabilities, quantize_operands, _lse
from .nvfp4 import fake_quant


def effective_topk(num_blocks: int, sparsity: float) -> int:
    return max(1, min(int(math.ceil((1.0 - sparsity) * num_blocks)), num_blocks))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of float64 values, as float64.

    Written on the value: split off the binary exponent and round the
    significand to 8 bits with numpy's round-half-even.
    """
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                     # x = m * 2^e, 0.5 <= |m| < 1
    r = np.round(m * 256.0) / 256.0        # 8 significant bits, ties to even
    return np.ldexp(r, e)


def pooled_means(x: np.ndarray, block_tokens: int) -> np.ndarray:
    """bf16-rounded per-block means over the token axis: [..., N, D] -> [..., nb, D]."""
    N = x.shape[-2]
    nb = -(-N // block_tokens)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]))
    for j in range(nb):
        t0, t1 = j * block_tokens, min(N, (j + 1) * block_tokens)
        out[..., j, :] = bf16_round(np.sum(x[..., t0:t1, :], axis=-2) / (t1 - t0))
    return out


def coarse_scores(q: np.ndarray, k: np.ndarray, block_tokens: int) -> np.ndarray:
    """bf16-rounded block scores C[..., i, j] = qbar_i . kbar_j."""
    qb = pooled_means(np.asarray(q, np.float64), block_tokens)
    kb = pooled_means(np.asarray(k, np.float64), block_tokens)
    return bf16_round(np.einsum("...id,...jd->...ij", qb, kb))


def select_blocks(q, k, block_tokens: int, topk: int) -> np.ndarray:
    """int32 [B, H, nbq, topk] ascending key-block indices per query block."""
    C = coarse_scores(q, k, block_tokens)
    B, H, nbq, nbk = C.shape
    if topk > nbk:
        raise ValueError("topk exceeds the number of key blocks")
    idx = np.empty((B, H, nbq, topk), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nbq):
                # sort by descending score, then ascending block index
                order = sorted(range(nbk), key=lambda j: (-C[b, h, i, j], j))
                idx[b, h, i] = np.sort(np.array(order[:topk], dtype=np.int32))
    return idx


def _keys_of(blocks, block_tokens: int, Nk: int) -> np.ndarray:
    return np.concatenate([np.arange(j * block_tokens, min(Nk, (j + 1) * block_tokens))
                           for j in blocks])


def forward(q, k, v, sm_scale: float, idx: np.ndarray, block_tokens: int,
            mask: int = MASK_ALL, p_mode: int = P_NORMALISED, with_ste: bool = False):
    """Block-sparse O [B,H,Nq,D] and LSE [B,H,Nq] for the selection ``idx``
    (``p_mode`` as in ``oracle.attention``: the row maximum is taken over the
    selected keys), then O_ste = P Vq over the selected keys with
    ``with_ste``."""
    q = np.asarray(q, np.float64)
    B, H, Nq, D = q.shape
    Nk = np.asarray(k).shape[2]
    qq, kq, vq = quantize_operands(q, k, v, mask)
    O = np.zeros((B, H, Nq, vq.shape[-1]))
    Os = np.zeros((B, H, Nq, vq.shape[-1]))
    L = np.zeros((B, H, Nq))
    nbq = idx.shape[2]
    for b in range(B):
        for h in range(H):
            for i in range(nbq):
                r0, r1 = i * block_tokens, min(Nq, (i + 1) * block_tokens)
                keys = _keys_of(idx[b, h, i], block_tokens, Nk)
                S = sm_scale * (qq[b, h, r0:r1] @ kq[b, h, keys].T)
                lse = _lse(S)
                P, Pq = probabilities(S, lse, mask, p_mode)
                O[b, h, r0:r1] = Pq @ vq[b, h, keys]
                Os[b, h, r0:r1] = P @ vq[b, h, keys]
                L[b, h, r0:r1] = lse
    return (O, L) + ((Os,) if with_ste else ())


def backward(q, k, v, do, sm_scale: float, idx: np.ndarray, block_tokens: int,
             mask: int = MASK_ALL, O=None, lse=None, p_mode: int = P_NORMALISED):
    """Block-sparse STE backward: dQ, dK, dV (same formulas as the dense path)."""
    q = np.asarray(q, np.float64)
    do = np.asarray(do, np.float64)
    B, H, Nq, D = q.shape
    Nk = np.asarray(k).shape[2]
    if O is None or lse is None:
        O, lse = forward(q, k, v, sm_scale, idx, block_tokens, mask, p_mode)
    qq, kq, vq = quantize_operands(q, k, v, mask)
    dq = np.zeros_like(qq)
    dk = np.zeros_like(kq)
    dv = np.zeros_like(vq)
    nbq = idx.shape[2]
    for b in range(B):
        for h in range(H):
            Dd = np.sum(do[b, h] * O[b, h], axis=-1)
            for i in range(nbq):
                r0, r1 = i * block_tokens, min(Nq, (i + 1) * block_tokens)
                keys = _keys_of(idx[b, h, i], block_tokens, Nk)
                S = sm_scale * (qq[b, h, r0:r1] @ kq[b, h, keys].T)
                P, Pq = probabilities(S, lse[b, h, r0:r1], mask, p_mode)
                dv[b, h, keys] += Pq.T @ do[b, h, r0:r1]
                dP = do[b, h, r0:r1] @ vq[b, h, keys].T
                dS = P * (dP - Dd[r0:r1, None])
                dq[b, h, r0:r1] = sm_scale * (dS @ kq[b, h, keys])
                dk[b, h, keys] += sm_scale * (dS.T @ qq[b, h, r0:r1])
    return dq, dk, dv


def query_block_forward(qq, kq, vq, blocks, r0: int, r1: int, block_tokens: int,
                        sm_scale: float, mask: int):
    """One head, query rows [r0, r1) of one query block attending to ``blocks``.

    Operands are already quantized ([N, D] arrays). Returns (keys, O, LSE, P, Pq)
    where ``keys`` are the attended key indices in visiting order.
    """
    keys = _keys_of(blocks, block_tokens, kq.shape[0])
    S = sm_scale * (qq[r0:r1] @ kq[keys].T)
    lse = _lse(S)
    P = np.exp(S - lse[:, None])
    Pq = fake_quant(P, axis=-1) if mask & MASK_P else P
    return keys, Pq @ vq[keys], lse, P, Pq


def query_block_backward(qq, kq, vq, do, O, blocks, r0: int, r1: int, block_tokens: int,
                         sm_scale: float, mask: int):
    """dQ of query rows [r0, r1) of one head (one query block) attending to
    ``blocks``; ``O`` is the forward output of those rows (D = rowsum(dO O))."""
    keys, _, lse, P, Pq = query_block_forward(qq, kq, vq, blocks, r0, r1, block_tokens,
                                              sm_scale, mask)
    Dd = np.sum(do[r0:r1] * O, axis=-1)
    dS = P * (do[r0:r1] @ vq[keys].T - Dd[:, None])
    return sm_scale * (dS @ kq[keys])


def key_block_backward(qq, kq, vq, do, idx_h, j: int, block_tokens: int, sm_scale: float,
                       mask: int, o_round=None):
    """dK, dV of key block ``j`` of one head: the sum over every query block
    whose selection ``idx_h`` [nbq, topk] contains j. The forward output of
    those query blocks is recomputed here; ``o_round`` (optional) maps it to
    the stored output dtype before it enters D = rowsum(dO O)."""
    Nq, Nk = qq.shape[0], kq.shape[0]
    k0, k1 = j * block_tokens, min(Nk, (j + 1) * block_tokens)
    dk = np.zeros((k1 - k0, kq.shape[1]))
    dv = np.zeros((k1 - k0, vq.shape[1]))
    for i in range(idx_h.shape[0]):
        if j not in set(int(x) for x in idx_h[i]):
            continue
        r0, r1 = i * block_tokens, min(Nq, (i + 1) * block_tokens)
        keys, O, lse, P, Pq = query_block_forward(qq, kq, vq, idx_h[i], r0, r1, block_tokens,
                                                  sm_scale, mask)
        if o_round is not None:
            O = o_round(O)
        sel = np.nonzero((keys >= k0) & (keys < k1))[0]
        Dd = np.sum(do[r0:r1] * O, axis=-1)
        dP = do[r0:r1] @ vq[keys[sel]].T
        dS = P[:, sel] * (dP - Dd[:, None])
        dv += Pq[:, sel].T @ do[r0:r1]
        dk += sm_scale * (dS.T @ qq[r0:r1])
    return dk, dv

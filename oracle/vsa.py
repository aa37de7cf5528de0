"""VSA coarse branch and its gated combination with the fine branch (fp64 numpy).

TEST INFRASTRUCTURE: part of the CPU oracle; only tests, the smoke check and the
benchmark's CPU-baseline leg may import it.

Source: FastVideo VSA checkpoint metadata, ``attention`` object (``kind`` vsa,
backend VSA_QAT_TRAIN_C128, ``cube_shape`` [4, 4, 8], ``precision.coarse``
"BF16" with ``quantize_coarse`` false, ``compression_gates`` "trained"), and
the fastvideo-kernel commit message (frozen VSA gates in the distillation
recipe; the VSA inference layout step scatters Q, K, V and the gate into one
tile buffer, so the gate is a per-token tensor shaped like them).

Readings where the pages are silent:

* Coarse branch: each 128-token block is represented by the mean of its
  tokens' Q, K and V (the raw inputs: the coarse branch is not quantized),
  rounded to bfloat16 exactly as for the block selection. Coarse attention is
  plain softmax attention of the query-block means over all key-block means
  with the caller's softmax scale: O_c = softmax(sm_scale Qbar Kbar^T) Vbar,
  one row per query block. The products are taken in full precision here;
  the GPU accumulates them in fp32 from the bf16 means.
* Combination: O = O_fine + G * O_c[block(t)], elementwise, where O_fine is
  the block-sparse fine attention output and G the gate tensor ([B,H,Nq,D],
  applied to the compressed branch only, as its name says). A gate of zero
  gives the fine branch alone.
* Backward: the fine branch's gradients are those of ``block_sparse.backward``
  with O_fine (its softmax delta uses O_fine, not O). The coarse branch adds
  the gradient of its output through the pooling: dO_c[i] = sum over the
  tokens t of block i of G_t * dO_t; the softmax backward gives dQbar, dKbar,
  dVbar; each token of a block receives its block mean's gradient divided by
  the block's token count (the bf16 rounding of the means is passed straight
  through). The gate's gradient is dG = dO * O_c[block(t)].
"""
from __future__ import annotations

import numpy as np

from . import block_sparse as bsp
from .block_sparse import bf16_round


def _means(x: np.ndarray, block_tokens: int, round_bf16: bool) -> np.ndarray:
    """Per-block means over the token axis: [..., N, D] -> [..., nb, D]."""
    if round_bf16:
        return bsp.pooled_means(x, block_tokens)
    N = x.shape[-2]
    nb = -(-N // block_tokens)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]))
    for j in range(nb):
        t0, t1 = j * block_tokens, min(N, (j + 1) * block_tokens)
        out[..., j, :] = np.mean(np.asarray(x, np.float64)[..., t0:t1, :], axis=-2)
    return out


def block_sizes(N: int, block_tokens: int) -> np.ndarray:
    """Token count of each block (the last one may be partial)."""
    nb = -(-N // block_tokens)
    return np.array([min(N, (j + 1) * block_tokens) - j * block_tokens for j in range(nb)], np.float64)


def broadcast(xb: np.ndarray, N: int, block_tokens: int) -> np.ndarray:
    """Block rows to token rows: [..., nb, D] -> [..., N, D], token t gets row t // block_tokens."""
    return np.repeat(xb, block_tokens, axis=-2)[..., :N, :]


def block_sums(x: np.ndarray, block_tokens: int) -> np.ndarray:
    """Per-block sums over the token axis: [..., N, D] -> [..., nb, D]."""
    N = x.shape[-2]
    nb = -(-N // block_tokens)
    return np.stack([x[..., j * block_tokens:min(N, (j + 1) * block_tokens), :].sum(axis=-2)
                     for j in range(nb)], axis=-2)


def coarse_forward(q, k, v, sm_scale: float, block_tokens: int = 128, round_bf16: bool = True):
    """O_c [B,H,nbq,D] and the coarse LSE [B,H,nbq] of the query-block means
    against all key-block means; also returns (Qbar, Kbar, Vbar, P)."""
    qb = _means(q, block_tokens, round_bf16)
    kb = _means(k, block_tokens, round_bf16)
    vb = _means(v, block_tokens, round_bf16)
    S = sm_scale * (qb @ np.swapaxes(kb, -1, -2))
    m = S.max(axis=-1, keepdims=True)
    L = m[..., 0] + np.log(np.exp(S - m).sum(axis=-1))
    P = np.exp(S - L[..., None])
    return P @ vb, L, (qb, kb, vb, P)


def combine(o_fine, gate, oc, block_tokens: int = 128) -> np.ndarray:
    """O = O_fine + G * O_c[block(t)]."""
    o_fine = np.asarray(o_fine, np.float64)
    return o_fine + np.asarray(gate, np.float64) * broadcast(oc, o_fine.shape[-2], block_tokens)


def coarse_backward(q, k, v, gate, do, sm_scale: float, block_tokens: int = 128,
                    round_bf16: bool = True):
    """Coarse-branch contributions to dQ, dK, dV and the gate gradient dG."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    do = np.asarray(do, np.float64)
    Nq, Nk = q.shape[-2], k.shape[-2]
    oc, _, (qb, kb, vb, P) = coarse_forward(q, k, v, sm_scale, block_tokens, round_bf16)
    dG = do * broadcast(oc, Nq, block_tokens)
    doc = block_sums(np.asarray(gate, np.float64) * do, block_tokens)
    dvb = np.swapaxes(P, -1, -2) @ doc
    dP = doc @ np.swapaxes(vb, -1, -2)
    Dc = np.sum(doc * oc, axis=-1, keepdims=True)
    dS = P * (dP - Dc)
    dqb = sm_scale * (dS @ kb)
    dkb = sm_scale * (np.swapaxes(dS, -1, -2) @ qb)
    nq = block_sizes(Nq, block_tokens)[:, None]
    nk = block_sizes(Nk, block_tokens)[:, None]
    dq = broadcast(dqb / nq, Nq, block_tokens)
    dk = broadcast(dkb / nk, Nk, block_tokens)
    dv = broadcast(dvb / nk, Nk, block_tokens)
    return dq, dk, dv, dG


def forward(q, k, v, gate, sm_scale: float, idx: np.ndarray, block_tokens: int = 128,
            mask: int = 15, p_mode: int = 0):
    """Whole VSA attention: returns (O, O_fine, LSE_fine)."""
    o_f, L = bsp.forward(q, k, v, sm_scale, idx, block_tokens, mask, p_mode)
    oc, _, _ = coarse_forward(q, k, v, sm_scale, block_tokens)
    return combine(o_f, gate, oc, block_tokens), o_f, L


def backward(q, k, v, gate, do, sm_scale: float, idx: np.ndarray, block_tokens: int = 128,
             mask: int = 15, O_fine=None, lse=None, p_mode: int = 0):
    """Whole VSA attention backward: dQ, dK, dV (fine + coarse) and dG.

    ``O_fine`` / ``lse`` are the fine branch's forward output and statistics
    (the oracle's own by default)."""
    dq, dk, dv = bsp.backward(q, k, v, do, sm_scale, idx, block_tokens, mask, O_fine, lse,
                              p_mode=p_mode)
    cq, ck, cv, dG = coarse_backward(q, k, v, gate, do, sm_scale, block_tokens)
    return dq + cq, dk + ck, dv + cv, dG


__all__ = ["coarse_forward", "combine", "coarse_backward", "forward", "backward", "broadcast",
           "block_sums", "block_sizes", "bf16_round"]

"""Attn-QAT attention, forward and straight-through backward (fp64 numpy).

TEST INFRASTRUCTURE: this module is part of the CPU oracle. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.

What is computed (plain reading of the pages, steps in order):

* FastVideo VSA checkpoint metadata, ``precision``: "fine: NVFP4 fake-quant with
  BF16 matmul", ``quant_p`` / ``quant_v`` / ``quantize_fine`` true, no global
  scale factors. So Q, K, V and the probability matrix P are fake-quantized
  (``oracle.nvfp4.fake_quant``) and the two products use the quantized values.
* FastVideo Attn-QAT training guide, environment-variable table
  (``FWD_EXACT_M`` row) and the fastvideo-kernel commit message (SM100 route
  paragraph): the forward saves per-row softmax statistics and the backward
  recomputes P from them, so the quantized P is that of the *normalised*
  probabilities P = exp(S - LSE).

Forward, with quant mask bits Q=1, K=2, V=4, P=8 (a cleared bit means identity)::

    Qq = FQ_d(Q)            groups of 16 along the head dimension
    Kq = FQ_d(K)
    Vq = FQ_tokens(V)       groups of 16 along the key axis
    S  = sm_scale * Qq Kq^T
    LSE_i = ln sum_j exp(S_ij)
    P  = exp(S - LSE)
    Pq = FQ_keys(P)         groups of 16 keys per query row, aligned at key 0
    O  = Pq Vq              (no renormalisation of Pq)

Backward (straight-through estimator: every quantizer passes the gradient as
the identity; the softmax Jacobian uses the unquantized P)::

    dV = Pq^T dO
    dP = dO Vq^T
    D_i = sum_c dO_ic O_ic
    dS = P * (dP - D)
    dQ = sm_scale * dS Kq
    dK = sm_scale * dS^T Qq

Row-max-relative variant (``p_mode=P_ROWMAX``; the first of the pages'
alternative readings of which P is quantized). The quantized quantity is the
probability relative to the row maximum rather than the normalised one::

    m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)      (LSE = m + ln l)
    Pq  = FQ_keys(exp(S - m)) / l                      (values in (0, 1] before FQ)

Everything else is unchanged: O = Pq Vq, and the backward uses this Pq in dV
and the unquantized P = exp(S - LSE) in the softmax Jacobian. With the p bit
clear both modes give Pq = P. Because exp(S - m) has maximum 1, the group
scales do not flush to zero on long rows as those of the normalised P do.

Additive straight-through output (the second alternative reading of the
softmax-backward delta): the forward also forms the STE product of the
unquantized P with Vq, O_ste = P Vq, and the backward takes its delta from
it, D'_i = sum_c dO_ic O_ste_ic (``backward(..., O=O_ste)``). This is the
gradient of the surrogate whose quantized P enters as P + (Pq0 - P0) with
the difference frozen, i.e. Pq with a pure straight-through estimator.

Everything is float64; S and P are materialised in row blocks.
"""
from __future__ import annotations

import numpy as np

from .nvfp4 import fake_quant

MASK_Q, MASK_K, MASK_V, MASK_P = 1, 2, 4, 8
MASK_ALL = 15
P_NORMALISED, P_ROWMAX = 0, 1


def quantize_operands(q, k, v, mask: int):
    """Qq, Kq, Vq for one or many heads (axes [..., N, D])."""
    qq = fake_quant(q, axis=-1) if mask & MASK_Q else np.asarray(q, np.float64)
    kq = fake_quant(k, axis=-1) if mask & MASK_K else np.asarray(k, np.float64)
    vq = fake_quant(v, axis=-2) if mask & MASK_V else np.asarray(v, np.float64)
    return qq, kq, vq


def _lse(S: np.ndarray) -> np.ndarray:
    m = np.max(S, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(S - m), axis=-1, keepdims=True)))[..., 0]


def probabilities(S: np.ndarray, lse: np.ndarray, mask: int, p_mode: int = P_NORMALISED,
                  row_max=None):
    """(P, Pq) for whole score rows S [n, Nk] with their LSE [n].

    P = exp(S - LSE). Pq = FQ_keys(P) (normalised mode) or
    FQ_keys(exp(S - m)) / l with m the row maximum (``row_max`` if given, for
    rows whose S holds only some of the keys) and l = exp(LSE - m).
    """
    P = np.exp(S - lse[:, None])
    if not mask & MASK_P:
        return P, P
    if p_mode == P_ROWMAX:
        m = (np.max(S, axis=-1) if row_max is None else np.asarray(row_max, np.float64))[:, None]
        return P, fake_quant(np.exp(S - m), axis=-1) / np.exp(lse[:, None] - m)
    return P, fake_quant(P, axis=-1)


def head_forward(qq, kq, vq, sm_scale: float, mask: int, rows=None, row_block: int = 512,
                 p_mode: int = P_NORMALISED, with_max: bool = False, with_ste: bool = False):
    """Forward for one head on already-quantized operands.

    ``rows`` (optional index array) restricts the query rows computed; the
    result then has len(rows) rows. Returns (O [n, D], LSE [n]), then the row
    maxima of S [n] with ``with_max`` and O_ste = P Vq [n, D] with ``with_ste``.
    """
    qsel = qq if rows is None else qq[rows]
    n = qsel.shape[0]
    O = np.empty((n, vq.shape[1]))
    Os = np.empty((n, vq.shape[1]))
    L = np.empty(n)
    M = np.empty(n)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        S = sm_scale * (qsel[r0:r1] @ kq.T)
        lse = _lse(S)
        P, Pq = probabilities(S, lse, mask, p_mode)
        O[r0:r1] = Pq @ vq
        if with_ste:
            Os[r0:r1] = P @ vq
        L[r0:r1] = lse
        M[r0:r1] = np.max(S, axis=-1)
    return (O, L) + ((M,) if with_max else ()) + ((Os,) if with_ste else ())


def _forward_rows_task(args):
    qq, kq, vq, sm_scale, mask, r0, r1, kw = args
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            return head_forward(qq[r0:r1], kq, vq, sm_scale, mask, **kw)
    except ImportError:  # pragma: no cover
        return head_forward(qq[r0:r1], kq, vq, sm_scale, mask, **kw)


def head_forward_all(qq, kq, vq, sm_scale: float, mask: int, workers: int = 0,
                     chunk: int = 1024, p_mode: int = P_NORMALISED, with_max: bool = False,
                     with_ste: bool = False):
    """``head_forward`` over every query row, split into row chunks across
    ``workers`` processes (0 or 1: in this process). Rows are independent in
    the forward, so the result is identical to a single call, extra outputs
    (``with_max``, ``with_ste``) included."""
    n = qq.shape[0]
    spans = [(r0, min(n, r0 + chunk)) for r0 in range(0, n, chunk)]
    kw = dict(p_mode=p_mode, with_max=with_max, with_ste=with_ste)
    if workers <= 1:
        parts = [head_forward(qq[a:b], kq, vq, sm_scale, mask, **kw) for a, b in spans]
    else:
        import multiprocessing as mp
        with mp.get_context("fork").Pool(workers) as pool:
            parts = pool.map(_forward_rows_task,
                             [(qq, kq, vq, sm_scale, mask, a, b, kw) for a, b in spans])
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))


def forward(q, k, v, sm_scale: float, mask: int = MASK_ALL, row_block: int = 512,
            p_mode: int = P_NORMALISED, with_max: bool = False, with_ste: bool = False):
    """O [B,H,Nq,D] and LSE [B,H,Nq] for real-valued inputs q, k, v, then the
    row maxima of S [B,H,Nq] with ``with_max`` and the straight-through output
    O_ste = P Vq [B,H,Nq,D] with ``with_ste``."""
    q = np.asarray(q, np.float64)
    B, H, Nq, D = q.shape
    qq, kq, vq = quantize_operands(q, k, v, mask)
    O = np.empty((B, H, Nq, vq.shape[-1]))
    Os = np.empty((B, H, Nq, vq.shape[-1]))
    L = np.empty((B, H, Nq))
    M = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h], M[b, h], Os[b, h] = head_forward(
                qq[b, h], kq[b, h], vq[b, h], sm_scale, mask, row_block=row_block,
                p_mode=p_mode, with_max=True, with_ste=True)
    return (O, L) + ((M,) if with_max else ()) + ((Os,) if with_ste else ())


def head_backward(qq, kq, vq, do, O, lse, sm_scale: float, mask: int,
                  row_block: int = 512, p_mode: int = P_NORMALISED):
    """dQ, dK, dV for one head on quantized operands (STE through quantizers).

    ``O`` and ``lse`` are this head's forward output and statistics (all rows).
    """
    Nq = qq.shape[0]
    dq = np.zeros_like(qq)
    dk = np.zeros_like(kq)
    dv = np.zeros_like(vq)
    Dd = np.sum(do * O, axis=-1)
    for r0 in range(0, Nq, row_block):
        r1 = min(Nq, r0 + row_block)
        S = sm_scale * (qq[r0:r1] @ kq.T)
        P, Pq = probabilities(S, lse[r0:r1], mask, p_mode)
        dv += Pq.T @ do[r0:r1]
        dP = do[r0:r1] @ vq.T
        dS = P * (dP - Dd[r0:r1, None])
        dq[r0:r1] = sm_scale * (dS @ kq)
        dk += sm_scale * (dS.T @ qq[r0:r1])
    return dq, dk, dv


def backward(q, k, v, do, sm_scale: float, mask: int = MASK_ALL, O=None, lse=None,
             row_block: int = 512, p_mode: int = P_NORMALISED):
    """dQ, dK, dV [B,H,N,D]. O / LSE default to this oracle's own forward."""
    q = np.asarray(q, np.float64)
    do = np.asarray(do, np.float64)
    B, H, Nq, D = q.shape
    qq, kq, vq = quantize_operands(q, k, v, mask)
    if O is None or lse is None:
        O, lse = forward(q, k, v, sm_scale, mask, row_block, p_mode=p_mode)
    dq = np.empty_like(qq)
    dk = np.empty_like(kq)
    dv = np.empty_like(vq)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward(
                qq[b, h], kq[b, h], vq[b, h], do[b, h], O[b, h], lse[b, h],
                sm_scale, mask, row_block, p_mode)
    return dq, dk, dv


def head_backward_keys(qq, kq, vq, do, O, lse, sm_scale: float, mask: int, keys,
                       row_block: int = 2048, p_mode: int = P_NORMALISED, row_max=None):
    """dK and dV of one head restricted to the key rows ``keys``.

    Needs this head's O and LSE for all query rows (and, for the row-max
    variant, the row maxima of S over all keys, ``row_max``). P is quantized
    per 16-key group, so every group that contains a requested key is
    evaluated whole. Returns (dK[keys], dV[keys]).
    """
    keys = np.asarray(keys)
    Nk = kq.shape[0]
    groups = np.unique(keys // 16)
    cols = np.concatenate([np.arange(g * 16, min(Nk, g * 16 + 16)) for g in groups])
    pos = {c: i for i, c in enumerate(cols)}
    sel = np.array([pos[c] for c in keys])
    Dd = np.sum(do * O, axis=-1)
    dk = np.zeros((len(cols), kq.shape[1]))
    dv = np.zeros((len(cols), vq.shape[1]))
    Nq = qq.shape[0]
    # Every group in ``cols`` is whole and listed in key order, so quantizing
    # along the gathered axis reproduces the per-group quantization of P.
    starts = np.array([np.searchsorted(cols, g * 16) for g in groups])
    for r0 in range(0, Nq, row_block):
        r1 = min(Nq, r0 + row_block)
        S = sm_scale * (qq[r0:r1] @ kq[cols].T)
        P = np.exp(S - lse[r0:r1, None])
        if mask & MASK_P:
            if p_mode == P_ROWMAX:
                m = np.asarray(row_max, np.float64)[r0:r1, None]
                X, post = np.exp(S - m), 1.0 / np.exp(lse[r0:r1, None] - m)
            else:
                X, post = P, 1.0
            Pq = np.empty_like(P)
            for gi, st in enumerate(starts):
                en = starts[gi + 1] if gi + 1 < len(starts) else len(cols)
                Pq[:, st:en] = fake_quant(X[:, st:en], axis=-1) * post
        else:
            Pq = P
        dv += Pq.T @ do[r0:r1]
        dP = do[r0:r1] @ vq[cols].T
        dS = P * (dP - Dd[r0:r1, None])
        dk += sm_scale * (dS.T @ qq[r0:r1])
    return dk[sel], dv[sel]


def head_backward_rows(qq, kq, vq, do_rows, O_rows, lse_rows, q_rows_idx, sm_scale: float,
                       mask: int):
    """dQ of one head restricted to query rows ``q_rows_idx`` (row-local)."""
    S = sm_scale * (qq[q_rows_idx] @ kq.T)
    P = np.exp(S - lse_rows[:, None])
    Dd = np.sum(do_rows * O_rows, axis=-1)
    dP = do_rows @ vq.T
    dS = P * (dP - Dd[:, None])
    return sm_scale * (dS @ kq)

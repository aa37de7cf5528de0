"""MXFP4 quantization and the real-FP4 inference attention forward (fp64 numpy).

TEST INFRASTRUCTURE: part of the CPU oracle; only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it.

What it computes: the counterpart, on a chip whose FP4 matrix instructions
take microscaled operands, of the pages' real-FP4 inference attention (the
inference-backend pull request's FP4 attention call with its single-level P
quantization option; the Attn-QAT guide's inference route). Readings where
the pages are silent:

* Format (a format change, not NVFP4): blocks of 32 consecutive values share
  one power-of-two scale, the OCP Microscaling (MX) v1.0 rule for FP4 E2M1
  elements: X = 2^(floor(log2 amax) - 2), 2 being the largest E2M1 exponent,
  clamped to the E8M0 range [2^-127, 2^127]; each element is E2M1(x / X),
  round to nearest with ties to even, saturating at 6 (amax / X lies in
  [4, 8), so the largest elements of a block can clip to 6 X). A block of
  zeros quantizes to zeros. NVFP4's E4M3 scale per 16 values carries mantissa
  bits no power-of-two scale has, so this path computes a different format
  than the fake-quantized training path.
* Blocks: Q and K along the head dimension, V along the tokens (per column),
  P along the keys; every block starts at index 0 and a partial last block is
  padded with zeros.
* P is quantized relative to the row maximum: P~ = exp(S - m), m_i = max_j
  S_ij, so the block holding the maximum has amax = 1 exactly. O = MX(P~) V~ / l
  with l_i = sum_j P~_ij (unquantized), and LSE = m + ln l. S = sm_scale
  MX(Q) MX(K)^T, V~ = MX(V).
"""
from __future__ import annotations

import numpy as np

from .nvfp4 import e2m1_round

BLOCK = 32
E8M0_MIN, E8M0_MAX = -127, 127


def block_exponents(amax: np.ndarray) -> np.ndarray:
    """Shared scale exponents floor(log2 amax) - 2 (E8M0-clamped; 0 blocks -> -127)."""
    amax = np.asarray(amax, np.float64)
    pos = amax > 0
    _, e = np.frexp(np.where(pos, amax, 1.0))  # amax = f 2^e, f in [0.5, 1)
    se = np.where(pos, (e - 1) - 2, E8M0_MIN)
    return np.clip(se, E8M0_MIN, E8M0_MAX).astype(np.int64)


def quant(x: np.ndarray, axis: int = -1, return_exponents: bool = False):
    """MX FP4 quantization of ``x`` in blocks of 32 along ``axis`` (dequantized values)."""
    x = np.moveaxis(np.asarray(x, np.float64), axis, -1)
    n = x.shape[-1]
    nb = -(-n // BLOCK)
    xp = np.zeros(x.shape[:-1] + (nb * BLOCK,))
    xp[..., :n] = x
    xb = xp.reshape(x.shape[:-1] + (nb, BLOCK))
    se = block_exponents(np.abs(xb).max(axis=-1))
    X = np.ldexp(1.0, se)[..., None]
    y = np.copysign(e2m1_round(np.abs(xb) / X) * X, xb)
    y = np.moveaxis(y.reshape(xp.shape)[..., :n], -1, axis)
    return (y, se) if return_exponents else y


def forward(q, k, v, sm_scale: float):
    """Real-FP4 inference attention: returns (O, LSE) for [..., N, D] inputs."""
    qq = quant(q, axis=-1)
    kq = quant(k, axis=-1)
    vq = quant(v, axis=-2)
    S = sm_scale * (qq @ np.swapaxes(kq, -1, -2))
    m = S.max(axis=-1, keepdims=True)
    Pt = np.exp(S - m)
    l = Pt.sum(axis=-1, keepdims=True)
    O = (quant(Pt, axis=-1) @ vq) / l
    return O, m[..., 0] + np.log(l[..., 0])


__all__ = ["BLOCK", "block_exponents", "quant", "forward"]

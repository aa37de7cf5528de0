"""Shared helpers for the GPU parity tests (bf16 transfer, error metrics)."""
import numpy as np
import torch

from synthetic import f32_from_bf16_bits

TOL_QUANT = 1e-2       # relative L2, O / dQ / dK / dV with any quantizer on
TOL_PLAIN = 5e-3       # relative L2 with every quantizer off
TOL_LSE = 1e-3         # max absolute error of LSE


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 patterns -> bf16 tensor on the device (bit-identical)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_f64(bits: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(bits).astype(np.float64)


def dev_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


ZERO_GRAD_ABS = 1e-5   # max |dQ|, |dK| when the exact gradient vanishes by cancellation


def rel_l2(got: np.ndarray, ref: np.ndarray, exact_zero: bool = True) -> float:
    """Relative L2 error.

    When the reference is exactly zero: with ``exact_zero`` (O and dV, which
    vanish because every quantized probability is flushed to zero) the result
    must be exactly zero too; otherwise (dQ and dK, which vanish by algebraic
    cancellation of dP - D, e.g. a single key) the largest magnitude must stay
    below ZERO_GRAD_ABS (the error is then reported as 0, else as inf).
    """
    n = np.linalg.norm(ref)
    if n == 0:
        if exact_zero:
            return 0.0 if np.all(got == 0) else float("inf")
        return 0.0 if float(np.abs(got).max()) <= ZERO_GRAD_ABS else float("inf")
    return float(np.linalg.norm(got - ref) / n)


# Where every probability of a row is small, the P quantizer's E4M3 scales sit
# near their subnormal floor, and one rounding decision can switch a whole
# 16-key group, or a whole row, between zero and non-zero. An LSE that differs
# from the oracle's by a few fp32 ulps (the kernels' own rounding) can then
# take the other, equally valid, decision. LSE_FLIP is the LSE shift (about
# 4 ulps for |LSE| < 16) over which such decisions are re-taken by the oracle.
LSE_FLIP = 4e-6


def rel_l2_best_rows(got: np.ndarray, cands) -> float:
    """Relative L2 error of ``got`` against the first of ``cands``, where each
    row is compared with whichever candidate is closest to it (candidates:
    the oracle's output for the same rows with its own decisions and with the
    decisions taken at LSE -/+ LSE_FLIP)."""
    ref = cands[0]
    n = np.linalg.norm(ref)
    err2 = np.min(np.stack([np.sum((got - c) ** 2, axis=-1) for c in cands]), axis=0)
    if n == 0:
        return 0.0 if float(err2.max()) == 0.0 else float("inf")
    return float(np.sqrt(err2.sum()) / n)


def best_candidate(got: np.ndarray, cands) -> np.ndarray:
    """Per row of ``got``, the index of the closest of ``cands`` (the first
    one on ties), as ``rel_l2_best_rows`` chooses it."""
    err2 = np.stack([np.sum((got - c) ** 2, axis=-1) for c in cands])
    return np.argmin(err2, axis=0)


def tol_for(mask: int) -> float:
    return TOL_QUANT if mask else TOL_PLAIN

"""NVFP4 fake quantization, written out from the format definition (fp64 numpy).

TEST INFRASTRUCTURE: this module is part of the CPU oracle. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
HIP library never does.

Source: FastVideo VSA checkpoint metadata, ``linear_quantization.format``
("E2M1 values, 16-element blocks, FP8 E4M3 block scales") together with
``precision.use_global_sf_qkv`` / ``use_global_sf_p`` = false (no global scale
for attention operands). The pages give no formula; the steps below are the
plain reading of that format:

F1  a = max |x_i| over a group of 16 consecutive elements (groups start at
    index 0; a partial last group is padded with zeros, which never raise a).
F2  s = E4M3(a / 6): round to nearest, ties to even, onto the finite OCP
    E4M3FN grid, saturating at 448 (6 is the largest E2M1 magnitude, so the
    group maximum lands on the top of the E2M1 range).
F3  s == 0  ->  y_i = copysign(0, x_i).
F4  q_i = E2M1(|x_i| / s): round to nearest, ties to even, onto
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}, saturating at 6.
F5  y_i = copysign(q_i * s, x_i).

Both roundings are evaluated on exact reals: a/6 and |x|/s are formed in
float64, which is exact enough that no input representable in float32 can be
pushed onto (or off) a rounding midpoint (the nearest non-midpoint value is at
least 2^-29 away in relative terms, far above float64's 2^-53).
"""
from __future__ import annotations

import numpy as np

GROUP = 16


def e4m3fn_grid() -> np.ndarray:
    """All non-negative finite OCP E4M3FN values, indexed by their code 0..126.

    Code c has exponent field c >> 3 and mantissa c & 7 (bias 7). Exponent 0
    is subnormal: m * 2^-9. Code 0x7F is NaN and is excluded, so the largest
    value is 1.75 * 2^8 = 448.
    """
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


def e2m1_grid() -> np.ndarray:
    """Non-negative E2M1 values indexed by code 0..7 (bias 1, exponent 0 subnormal)."""
    vals = []
    for c in range(8):
        e, m = c >> 1, c & 1
        vals.append(m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(vals, dtype=np.float64)


E4M3_GRID = e4m3fn_grid()
E2M1_GRID = e2m1_grid()


def round_to_grid(v: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Round non-negative ``v`` to the sorted ``grid``: nearest, ties to even code.

    Values at or above the last grid point saturate to it. Returns the grid
    index (the format's code for non-negative values). The midpoint between two
    neighbours has few significant bits, so (lo + hi) / 2 and the comparison with
    it are exact in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    lo = np.searchsorted(grid, v, side="right") - 1
    lo = np.clip(lo, 0, len(grid) - 1)
    hi = np.minimum(lo + 1, len(grid) - 1)
    mid = (grid[lo] + grid[hi]) * 0.5
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0) & (hi != lo))
    idx = np.where(pick_hi, hi, lo)
    return idx


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """E4M3FN value nearest to non-negative ``v`` (ties to even, saturating at 448)."""
    return E4M3_GRID[round_to_grid(v, E4M3_GRID)]


def e4m3_code(v: np.ndarray) -> np.ndarray:
    return round_to_grid(v, E4M3_GRID).astype(np.uint8)


def e2m1_round(v: np.ndarray) -> np.ndarray:
    """E2M1 value nearest to non-negative ``v`` (ties to even, saturating at 6)."""
    return E2M1_GRID[round_to_grid(v, E2M1_GRID)]


def fake_quant(x: np.ndarray, axis: int = -1, return_scale_codes: bool = False):
    """NVFP4 fake quantization of ``x`` in groups of 16 along ``axis`` (F1..F5).

    ``x`` holds real values (float32/float64). The result is float64 and every
    element is exactly q * s with q on the E2M1 grid and s on the E4M3 grid.
    With ``return_scale_codes`` the E4M3FN byte of each group is returned too,
    shaped like ``x`` with ``axis`` replaced by the group count.
    """
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    ng = -(-n // GROUP)
    pad = ng * GROUP - n
    if pad:
        xm = np.concatenate([xm, np.zeros(xm.shape[:-1] + (pad,))], axis=-1)
    g = xm.reshape(xm.shape[:-1] + (ng, GROUP))
    a = np.max(np.abs(g), axis=-1)                       # F1
    sidx = round_to_grid(a / 6.0, E4M3_GRID)             # F2
    s = E4M3_GRID[sidx]
    s_b = s[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s_b > 0, np.abs(g) / np.where(s_b > 0, s_b, 1.0), 0.0)
    q = e2m1_round(r)                                    # F4
    y = np.copysign(q * s_b, g)                          # F3, F5 (q * 0 = 0)
    y = y.reshape(xm.shape[:-1] + (ng * GROUP,))[..., :n]
    y = np.moveaxis(y, -1, axis)
    if return_scale_codes:
        return y, np.moveaxis(sidx.astype(np.uint8), -1, axis)
    return y

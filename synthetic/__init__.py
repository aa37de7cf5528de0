"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module only draws random numbers and stores them as bfloat16 bit patterns.
It contains none of the attention or fake-quantization arithmetic, so both the
CPU oracle (``oracle/``) and the HIP library can consume its output without
sharing any method code.

Recipe (identical bytes go to both sides):

* ``numpy.random.RandomState(seed)`` (legacy generator: its stream is stable
  across numpy releases), ``standard_normal`` in float64, cast to float32, then
  rounded to bfloat16 with round-to-nearest-even.
* Each tensor is drawn whole, in C order ``[B, H, N, D]``, from its own
  generator seeded with ``1000 * config + tensor_id`` (Q=1, K=2, V=3, dO=4;
  the outlier-row selection of the timing workload uses id 5).

The workloads mirror the shapes on the source pages: the Wan2.1-T2V-1.3B
transformer (12 heads of dimension 128, 16 latent frames of 448x896 video, i.e.
25,088 tokens; FastVideo VSA checkpoint metadata, ``model.architecture`` and
``training.data``), the kernel-timing shape of 6 heads by 31,200 tokens
(fastvideo-kernel commit message, paragraph on the SM100 Attn-QAT route), a
16,384 + 27 token tail case, and a 256-block VSA-style sparse layout
(``attention.cube_shape`` [4, 4, 8] = 128 tokens per block, sparsity 0.9).
These synthetic tensors stand in for the MixKit activations the pages train on.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4, "outlier_rows": 5}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN is not expected in generated
    data; it would be kept as a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_f32(seed: int, shape) -> np.ndarray:
    rs = np.random.RandomState(seed)
    return rs.standard_normal(size=shape).astype(np.float32)


def normal_bf16(seed: int, shape) -> np.ndarray:
    """i.i.d. N(0, 1) drawn in float64, cast to float32, rounded to bf16 bits."""
    return bf16_bits_from_f32(_normal_f32(seed, shape))


def rms_normalised_bf16(seed: int, shape, eps: float = 1e-6) -> np.ndarray:
    """N(0,1) rows scaled to unit RMS over the last axis (float32), then bf16.

    Each row x becomes x / sqrt(mean(x**2) + eps) with no gain, computed in
    float32: the per-head RMS-normalised queries and keys of a video DiT.
    """
    x = _normal_f32(seed, shape)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
    x = x / np.sqrt(ms + np.float32(eps), dtype=np.float32)
    return bf16_bits_from_f32(x.astype(np.float32))


def outlier_keys_bf16(seed: int, shape, rows_seed: int, frac: float = 0.01,
                      factor: float = 8.0) -> np.ndarray:
    """N(0,1) keys where ``frac`` of each head's rows are multiplied by ``factor``.

    For every (b, h) in C order, ``int(frac * N)`` distinct rows are drawn by
    successive ``choice(N, m, replace=False)`` calls on one
    ``RandomState(rows_seed)``, so the outlier rows differ per head. The scaling
    happens before bf16 rounding; a factor that is a power of two keeps it exact.
    """
    B, H, N, D = shape
    x = _normal_f32(seed, shape)
    rs = np.random.RandomState(rows_seed)
    m = int(frac * N)
    for b in range(B):
        for h in range(H):
            rows = rs.choice(N, m, replace=False)
            x[b, h, rows, :] *= np.float32(factor)
    return bf16_bits_from_f32(x)


@dataclass(frozen=True)
class Workload:
    """One named synthetic workload: shape, value recipe and the softmax scale."""

    cid: int
    name: str
    B: int
    H: int
    N: int
    D: int
    qk_kind: str = "normal"          # "normal", "rms", "outlier_k"
    topk: int = 0                    # >0: block-sparse selection of this many blocks
    block_tokens: int = 128
    note: str = ""
    quant_masks: tuple = field(default=(15,))

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.D)

    def credited_flops(self) -> tuple[float, float]:
        """Forward 4*Nq*Nk*D*B*H and backward 2.5x that; sparse scaled by density."""
        f = 4.0 * self.N * self.N * self.D * self.B * self.H
        if self.topk:
            nb = -(-self.N // self.block_tokens)
            f *= self.topk / nb
        return f, 2.5 * f


WORKLOADS = {
    1: Workload(1, "tiny", 1, 2, 256, 64,
                note="tiny i.i.d. case, every quant mask", quant_masks=tuple(range(16))),
    2: Workload(2, "video_dit_12h_25088", 1, 12, 25088, 128, qk_kind="rms",
                note="Wan2.1 1.3B single attention layer, RMS-normalised Q/K"),
    3: Workload(3, "timing_6h_31200", 1, 6, 31200, 128, qk_kind="outlier_k",
                note="the pages' kernel-timing shape; 1% of K rows x8"),
    4: Workload(4, "tail_2x12h_16411", 2, 12, 16411, 128,
                note="16384 + 27 tokens: partial 128-tile and partial 16-group",
                quant_masks=(15, 0)),
    5: Workload(5, "vsa_sparse_12h_32768", 1, 12, 32768, 128, topk=26,
                note="256 blocks of 128 tokens, top-26 blocks per query block"),
}


def seed_for(cid: int, tensor: str) -> int:
    return 1000 * cid + TENSOR_IDS[tensor]


def make_inputs(cid: int, tensors=("q", "k", "v", "do"), shape=None) -> dict:
    """Return the bf16 bit patterns (uint16, C order [B,H,N,D]) of a workload.

    ``shape`` overrides the workload's shape (used for reduced test sizes); the
    value recipe and seeds stay those of workload ``cid``.
    """
    w = WORKLOADS[cid]
    shp = tuple(shape) if shape is not None else w.shape
    out = {}
    for t in tensors:
        s = seed_for(cid, t)
        if t in ("q", "k") and w.qk_kind == "rms":
            out[t] = rms_normalised_bf16(s, shp)
        elif t == "k" and w.qk_kind == "outlier_k":
            out[t] = outlier_keys_bf16(s, shp, seed_for(cid, "outlier_rows"))
        else:
            out[t] = normal_bf16(s, shp)
    return out


def random_bf16(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Generic helper for tests: N(0, scale^2) as bf16 bits."""
    x = _normal_f32(seed, shape) * np.float32(scale)
    return bf16_bits_from_f32(x)


def sha256_hex(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()

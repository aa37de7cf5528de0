"""GPU parity of the standalone NVFP4 fake-quant kernel: bit-exact vs the oracle."""
import numpy as np
import pytest
import torch

from oracle import nvfp4
from synthetic import bf16_bits_from_f32, random_bf16
from tests.helpers import dev_bits, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _oracle_bits(x_bits, axis):
    y, codes = nvfp4.fake_quant(to_f64(x_bits), axis=axis, return_scale_codes=True)
    return bf16_bits_from_f32(y.astype(np.float32)), codes


def _positive_bf16():
    return np.arange(1, 0x7F80, dtype=np.uint16)   # every positive finite bf16


def test_every_group_maximum(gpu_lib):
    """Scale step: every finite bf16 value (both signs) as the maximum of a group."""
    a = _positive_bf16()
    a = np.concatenate([a, a | 0x8000])
    x = np.zeros((len(a), 16), np.uint16)
    x[:, 3] = a
    x[:, 7] = a ^ 0x8000        # the negated value in the same group
    xb = x.reshape(1, 1, len(a), 16)
    y, codes = gpu_lib.fakequant(to_dev(xb), "d", return_scale_codes=True)
    ry, rc = _oracle_bits(xb, -1)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(dev_bits(y), ry)


def test_every_element_per_scale(gpu_lib):
    """Element step: for each of the 126 non-zero E4M3 scales s, every bf16 x in
    [s/64, 6s] of both signs inside the group [6s, x, 0, ...]."""
    allx = to_f64(_positive_bf16())
    rows = []
    for si in range(1, 127):
        s = nvfp4.E4M3_GRID[si]
        xs = _positive_bf16()[(allx >= s / 64) & (allx <= 6 * s)]
        g = np.zeros((2 * len(xs), 16), np.uint16)
        g[:, 0] = bf16_bits_from_f32(np.array([6 * s], np.float32))[0]
        g[: len(xs), 1] = xs
        g[len(xs):, 1] = xs | 0x8000
        rows.append(g)
    x = np.concatenate(rows).reshape(1, 1, -1, 16)
    y = gpu_lib.fakequant(to_dev(x), "d")
    ry, _ = _oracle_bits(x, -1)
    np.testing.assert_array_equal(dev_bits(y), ry)


@pytest.mark.parametrize("shape", [(2, 3, 257, 64), (1, 2, 33, 128), (1, 1, 5, 16), (2, 1, 300, 48)])
def test_random_axis_d(gpu_lib, shape):
    rs = np.random.RandomState(sum(shape))
    mag = np.exp(rs.uniform(-12, 10, shape[:-1] + (1,))).astype(np.float32)
    x = bf16_bits_from_f32(rs.standard_normal(shape).astype(np.float32) * mag)
    y, codes = gpu_lib.fakequant(to_dev(x), "d", return_scale_codes=True)
    ry, rc = _oracle_bits(x, -1)
    np.testing.assert_array_equal(dev_bits(y), ry)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("shape", [(2, 3, 257, 64), (1, 2, 16, 128), (1, 1, 5, 8), (1, 2, 1000, 24)])
def test_random_axis_n(gpu_lib, shape):
    rs = np.random.RandomState(7 + sum(shape))
    mag = np.exp(rs.uniform(-12, 10, shape[:2] + (1, shape[3]))).astype(np.float32)
    x = bf16_bits_from_f32(rs.standard_normal(shape).astype(np.float32) * mag)
    y, codes = gpu_lib.fakequant(to_dev(x), "n", return_scale_codes=True)
    ry, rc = _oracle_bits(x, -2)
    np.testing.assert_array_equal(dev_bits(y), ry)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def test_strided_input_and_output(gpu_lib):
    x = random_bf16(5, (2, 40, 3, 64))                       # [B, N, H, D] memory order
    xt = to_dev(x).permute(0, 2, 1, 3)                      # view as [B, H, N, D]
    ybig = torch.zeros((2, 3, 40, 80), dtype=torch.bfloat16, device="cuda")
    y = ybig[..., :64]                                      # row stride 80
    L = gpu_lib.load()
    rc = L.attnqat_fakequant_nvfp4(xt.data_ptr(), gpu_lib.strides_of(xt), y.data_ptr(),
                                   gpu_lib.strides_of(y), None, 2, 3, 40, 64, gpu_lib.AXIS_D,
                                   gpu_lib._stream())
    gpu_lib.check(rc)
    ref, _ = _oracle_bits(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), -1)
    np.testing.assert_array_equal(dev_bits(y), ref)
    assert torch.count_nonzero(ybig[..., 64:]) == 0          # untouched padding columns
    # the input is not modified
    np.testing.assert_array_equal(dev_bits(xt.permute(0, 2, 1, 3)), x)


def test_deterministic(gpu_lib):
    x = to_dev(random_bf16(9, (1, 4, 999, 128)))
    a = dev_bits(gpu_lib.fakequant(x, "n"))
    b = dev_bits(gpu_lib.fakequant(x, "n"))
    np.testing.assert_array_equal(a, b)

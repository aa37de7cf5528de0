"""attnqat_fwd_noalloc (fixed device scratch, no workspace) against
attnqat_fwd, called through the C ABI: bitwise equal outputs on two calls in
a row, the second on a smaller problem, then a block-sparse call; problems
larger than the scratch are rejected before any work."""
import ctypes

import numpy as np
import pytest
import torch

from synthetic import random_bf16
from tests.helpers import dev_bits, to_dev

pytestmark = pytest.mark.gpu


def _problem(gpu_lib, t, sc, mask, o, idx=None):
    return gpu_lib.make_problem(t["q"], t["k"], sc, mask, v=t["v"], o=o, kv_block_idx=idx)


def _noalloc(gpu_lib, t, sc, mask, idx=None):
    """Outputs of the no-allocation entry point, called through the C ABI."""
    L = gpu_lib.lib()
    B, H, Nq, D = t["q"].shape
    o = torch.full((B, H, Nq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    p = _problem(gpu_lib, t, sc, mask, o, idx)
    st = torch.cuda.current_stream().cuda_stream
    rc = L.attnqat_fwd_noalloc(ctypes.byref(p), t["q"].data_ptr(), t["k"].data_ptr(),
                               t["v"].data_ptr(), o.data_ptr(), lse.data_ptr(), st)
    assert rc == 0, L.attnqat_last_error()
    return o, lse


def _with_workspace(gpu_lib, t, sc, mask, idx=None):
    """Outputs of attnqat_fwd with its own workspace, through the C ABI."""
    L = gpu_lib.lib()
    B, H, Nq, D = t["q"].shape
    o = torch.empty((B, H, Nq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    p = _problem(gpu_lib, t, sc, mask, o, idx)
    ws = torch.empty(L.attnqat_fwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8,
                     device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = L.attnqat_fwd(ctypes.byref(p), t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                       o.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(), st)
    assert rc == 0, L.attnqat_last_error()
    return o, lse


def _inputs(seed, shape):
    return {k: to_dev(random_bf16(seed + i, shape)) for i, k in enumerate(("q", "k", "v"))}


def _same(a, b):
    (oa, la), (ob, lb) = a, b
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev_bits(oa), dev_bits(ob))
    np.testing.assert_array_equal(la.cpu().numpy().view(np.uint32), lb.cpu().numpy().view(np.uint32))


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    # first call: 4 heads x 1,000 tokens, d = 128, every quantizer on
    big = _inputs(500, (1, 4, 1000, 128))
    _same(_noalloc(gpu_lib, big, 0.0884, 15), _with_workspace(gpu_lib, big, 0.0884, 15))
    # second call on the same GPU: a smaller problem (2 heads x 300 tokens,
    # d = 64) over the scratch the first call left behind
    small = _inputs(510, (1, 2, 300, 64))
    _same(_noalloc(gpu_lib, small, 0.125, 15), _with_workspace(gpu_lib, small, 0.125, 15))
    # a smaller problem whose pass 2 also shares its last round out (2 heads x
    # 700 tokens: 6 query blocks of 11 key tiles in chunks of 9), over the
    # partial sums the first call (16 blocks of 16 tiles, chunks of 8) left
    mid = _inputs(520, (1, 2, 700, 128))
    _same(_noalloc(gpu_lib, mid, 0.0884, 15), _with_workspace(gpu_lib, mid, 0.0884, 15))
    # quantization off (single-pass forward) and a block-sparse call
    _same(_noalloc(gpu_lib, small, 0.125, 0), _with_workspace(gpu_lib, small, 0.125, 0))
    idx = torch.tensor([[0, 2], [1, 2], [0, 1]], dtype=torch.int32,
                       device="cuda").repeat(1, 2, 1, 1).contiguous()
    _same(_noalloc(gpu_lib, small, 0.125, 15, idx), _with_workspace(gpu_lib, small, 0.125, 15, idx))


def test_noalloc_rejects_problems_beyond_its_scratch(gpu_lib):
    L = gpu_lib.lib()
    t = {k: torch.empty((1, 1, 8, 128), dtype=torch.bfloat16, device="cuda") for k in "qkv"}
    o = torch.empty_like(t["q"])
    lse = torch.empty((1, 1, 8), dtype=torch.float32, device="cuda")
    p = _problem(gpu_lib, t, 0.1, 15, o)
    p.H, p.Nq, p.Nk = 64, 4096, 4096      # 3 x 64 x 4096 x 128 x 2 B = 192 MiB of operands
    assert L.attnqat_fwd_workspace_bytes(ctypes.byref(p)) > gpu_lib.NOALLOC_SCRATCH_BYTES
    rc = L.attnqat_fwd_noalloc(ctypes.byref(p), t["q"].data_ptr(), t["k"].data_ptr(),
                               t["v"].data_ptr(), o.data_ptr(), lse.data_ptr(), None)
    assert rc == 2 and b"scratch" in L.attnqat_last_error()

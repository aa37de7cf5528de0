"""Guard tests of the forward and backward calls (GPU).

* Canary regions: every output (O, LSE, dQ, dK, dV) and the workspace are
  views into larger buffers whose margins hold a NaN bit pattern; after the
  calls the margins must be bit-for-bit unchanged (no write outside the
  buffers the ABI hands over) and the outputs equal those of a call on plain
  tensors.
* Workspace poisoning: the same calls with the workspace filled with 0xFF
  bytes (NaN in every float view) and with zeros give bitwise equal results,
  so no kernel reads workspace bytes that the call did not write first.

Dense (ragged 300 tokens) and block-sparse (600 tokens, top-2 of 5 blocks with
the partial last block selected) cases, every quantizer on.
"""
import ctypes

import numpy as np
import pytest
import torch

from helpers import dev_bits, to_dev
from synthetic import random_bf16

pytestmark = pytest.mark.gpu

PAD = 4096  # elements (bytes for the workspace) on each side of a guarded view
NAN16 = 0x7FC1
NAN32 = 0x7FC00001


def _guarded(shape, dtype):
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * PAD, dtype=dtype, device="cuda")
    if dtype == torch.bfloat16:
        buf.view(torch.int16).fill_(NAN16)
    elif dtype == torch.float32:
        buf.view(torch.int32).fill_(NAN32)
    else:
        buf.fill_(0xA5)
    return buf, buf[PAD:PAD + n].view(shape)


def _margins_intact(buf, n):
    if buf.dtype == torch.bfloat16:
        bits, pat = buf.view(torch.int16), NAN16
    elif buf.dtype == torch.float32:
        bits, pat = buf.view(torch.int32), NAN32
    else:
        bits, pat = buf, 0xA5
    return bool((bits[:PAD] == pat).all()) and bool((bits[PAD + n:] == pat).all())


def _case(gpu_lib, sparse):
    if sparse:
        N, shape = 600, (1, 2, 600, 128)
    else:
        N, shape = 300, (1, 2, 300, 128)
    t = {k: to_dev(random_bf16(900 + i, shape)) for i, k in enumerate(("q", "k", "v", "do"))}
    idx = None
    if sparse:
        nb = (N + 127) // 128
        rows = np.array([[0, nb - 1], [1, nb - 1], [2, 3], [1, nb - 1], [0, 2]], np.int32)[:nb]
        idx = torch.from_numpy(np.broadcast_to(rows, (1, 2, nb, 2)).copy()).to("cuda")
    return t, idx


def _ws_bytes(gpu_lib, t, idx, o, fwd):
    L = gpu_lib.lib()
    if fwd:
        p = gpu_lib.make_problem(t["q"], t["k"], 0.0884, 15, v=t["v"], o=o, kv_block_idx=idx)
        return L.attnqat_fwd_workspace_bytes(ctypes.byref(p))
    p = gpu_lib.make_problem(t["q"], t["k"], 0.0884, 15, v=t["v"], o=o, do=t["do"],
                             dq=torch.empty_like(t["q"]), dk=torch.empty_like(t["k"]),
                             dv=torch.empty_like(t["v"]), kv_block_idx=idx)
    return L.attnqat_bwd_workspace_bytes(ctypes.byref(p))


@pytest.mark.parametrize("sparse", [False, True])
def test_outputs_and_workspace_stay_inside_their_buffers(gpu_lib, sparse):
    t, idx = _case(gpu_lib, sparse)
    B, H, N, D = t["q"].shape
    # reference on plain tensors
    o_ref, l_ref = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.0884, 15, idx)
    g_ref = gpu_lib.bwd(t["q"], t["k"], t["v"], o_ref, l_ref, t["do"], 0.0884, 15, idx)
    # guarded outputs and workspaces
    ob, o = _guarded((B, H, N, D), torch.bfloat16)
    lb, lse = _guarded((B, H, N), torch.float32)
    nf = _ws_bytes(gpu_lib, t, idx, o, True)
    wfb, wf = _guarded((nf,), torch.uint8)
    gpu_lib.fwd(t["q"], t["k"], t["v"], 0.0884, 15, idx, out=o, lse=lse, workspace=wf)
    gbufs, gviews = zip(*[_guarded((B, H, N, D), torch.bfloat16) for _ in range(3)])
    nb = _ws_bytes(gpu_lib, t, idx, o, False)
    wbb, wb = _guarded((nb,), torch.uint8)
    gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], 0.0884, 15, idx, dq=gviews[0],
                dk=gviews[1], dv=gviews[2], workspace=wb)
    torch.cuda.synchronize()
    n4 = B * H * N * D
    assert _margins_intact(ob, n4) and _margins_intact(lb, B * H * N)
    assert _margins_intact(wfb, nf) and _margins_intact(wbb, nb)
    for gb in gbufs:
        assert _margins_intact(gb, n4)
    np.testing.assert_array_equal(dev_bits(o), dev_bits(o_ref))
    np.testing.assert_array_equal(lse.cpu().numpy().view(np.uint32), l_ref.cpu().numpy().view(np.uint32))
    for got, ref in zip(gviews, g_ref):
        np.testing.assert_array_equal(dev_bits(got), dev_bits(ref))


@pytest.mark.parametrize("sparse", [False, True])
def test_results_do_not_depend_on_workspace_contents(gpu_lib, sparse):
    t, idx = _case(gpu_lib, sparse)
    outs = []
    for fill in (0x00, 0xFF):
        o0 = torch.empty_like(t["q"])
        nf = _ws_bytes(gpu_lib, t, idx, o0, True)
        nb = _ws_bytes(gpu_lib, t, idx, o0, False)
        wf = torch.full((nf,), fill, dtype=torch.uint8, device="cuda")
        wb = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        o, lse = gpu_lib.fwd(t["q"], t["k"], t["v"], 0.0884, 15, idx, workspace=wf)
        g = gpu_lib.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], 0.0884, 15, idx, workspace=wb)
        torch.cuda.synchronize()
        outs.append([dev_bits(o), lse.cpu().numpy().view(np.uint32)] + [dev_bits(x) for x in g])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    assert np.isfinite(outs[0][1].view(np.float32)).all()

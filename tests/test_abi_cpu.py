"""C-ABI contract checks that need no GPU.

The library loads, exports every function declared in include/attnqat.h, and
rejects every malformed call with the documented status before any HIP call
(so these calls use fake device addresses that are never dereferenced).
"""
import ctypes
import math
import os
import re

import pytest

import quantization_aware_attention_amd as qaa
from quantization_aware_attention_amd import build as qbuild

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "attnqat.h")
OK, E_INVALID, E_UNSUPPORTED, E_MISALIGNED, E_WORKSPACE, E_HIP = 0, 1, 2, 3, 4, 5
A = 1 << 20          # fake, 16-byte (and 256-byte) aligned device addresses, never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qbuild.LIB_PATH):
        qbuild.build()
    return qaa.load()


def _prob(**kw):
    p = qaa.Problem()
    p.B, p.H, p.Nq, p.Nk, p.D = 1, 2, 100, 120, 64
    p.sm_scale = 0.125
    p.quant_mask = 15
    p.block_tokens = 128
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _fwd(L, p, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, ws=6 * A, wsb=1 << 40):
    return L.attnqat_fwd(ctypes.byref(p), q, k, v, o, lse, ws, wsb, None)


def _bwd(L, p, ws=20 * A, wsb=1 << 40, **ptrs):
    d = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, do=6 * A, dq=7 * A, dk=8 * A, dv=9 * A)
    d.update(ptrs)
    return L.attnqat_bwd(ctypes.byref(p), d["q"], d["k"], d["v"], d["o"], d["lse"], d["do"],
                         d["dq"], d["dk"], d["dv"], ws, wsb, None)


def test_exports_every_declared_function(L):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attnqat_\w+)\s*\(", text, re.M))
    assert declared == set(qaa.EXPORTS), declared ^ set(qaa.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.attnqat_abi_version() == 5


def test_status_strings(L):
    for code in range(6):
        assert L.attnqat_status_string(code)
    assert L.attnqat_status_string(99) == b"unknown status"


@pytest.mark.parametrize("field,value,code", [
    ("D", 96, E_UNSUPPORTED), ("D", 256, E_UNSUPPORTED), ("B", 0, E_INVALID),
    ("Nq", 0, E_INVALID), ("Nk", 0, E_INVALID), ("H", -1, E_INVALID),
    ("sm_scale", 0.0, E_INVALID), ("sm_scale", -1.0, E_INVALID),
    ("sm_scale", float("nan"), E_INVALID), ("sm_scale", float("inf"), E_INVALID),
    ("quant_mask", 16, E_INVALID), ("quant_mask", 0x80000000, E_INVALID),
])
def test_forward_rejects_bad_problem(L, field, value, code):
    p = _prob(**{field: value})
    assert _fwd(L, p) == code
    assert L.attnqat_last_error()
    assert L.attnqat_fwd_workspace_bytes(ctypes.byref(p)) == 0


def test_forward_pointer_checks(L):
    p = _prob()
    assert _fwd(L, p, q=0) == E_INVALID
    assert _fwd(L, p, lse=0) == E_INVALID
    assert _fwd(L, p, k=2 * A + 8) == E_MISALIGNED
    assert _fwd(L, p, ws=6 * A + 16) == E_MISALIGNED
    assert _fwd(L, p, lse=5 * A + 2) == E_MISALIGNED
    assert _fwd(L, p, ws=0) == E_WORKSPACE
    need = L.attnqat_fwd_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert _fwd(L, p, wsb=need - 1) == E_WORKSPACE
    assert _fwd(L, p, o=A) == E_INVALID                 # output aliases q
    assert _fwd(L, p, ws=A) == E_INVALID                # workspace overlaps q
    assert b"overlap" in L.attnqat_last_error()


def test_forward_stride_checks(L):
    p = _prob()
    p.q = qaa.Strides(2 * 100 * 64, 100 * 64, 60)       # row stride < D and not a multiple of 8
    assert _fwd(L, p) == E_MISALIGNED
    p.q = qaa.Strides(2 * 100 * 64, 100 * 64, 32)       # rows overlap
    assert _fwd(L, p) == E_INVALID
    p.q = qaa.Strides(-8, 100 * 64, 64)
    assert _fwd(L, p) == E_INVALID


def test_backward_checks(L):
    p = _prob()
    need = L.attnqat_bwd_workspace_bytes(ctypes.byref(p))
    assert need > L.attnqat_fwd_workspace_bytes(ctypes.byref(p))
    assert _bwd(L, p, dq=0) == E_INVALID
    assert _bwd(L, p, wsb=need - 1) == E_WORKSPACE
    assert _bwd(L, p, dk=7 * A) == E_INVALID            # dk overlaps dq
    assert _bwd(L, p, dv=A) == E_INVALID                # dv overlaps q
    assert _bwd(L, p, do=6 * A + 4) == E_MISALIGNED


def test_sparse_problem_checks(L):
    p = _prob(Nq=1024, Nk=1024, block_tokens=64)
    p.kv_block_idx = 30 * A
    p.topk = 2
    assert _fwd(L, p) == E_UNSUPPORTED                  # block_tokens must be 128
    p.block_tokens = 128
    p.topk = 9
    assert _fwd(L, p) == E_INVALID                      # 8 key blocks
    p.topk = 0
    assert _fwd(L, p) == E_INVALID
    p.topk = 3
    dense = _prob(Nq=1024, Nk=1024)
    # the sparse backward adds the reverse index (int32 [BH][nbk][nbq] lists,
    # [BH][nbk] counts and the [BH][nbk] dispatch order, 256-byte aligned)
    # and stages no permuted K^T
    # (bf16 [BH][Nk_pad][D])
    # and the dense one the fp32 partial sums of the key blocks its dK/dV
    # launch may split (at most 4 parts of [dK, dV][128 keys][D] per block,
    # for at most 255 blocks)
    nb = 1024 // 128
    kt = 2 * 1024 * 64 * 2
    rev = -(-2 * nb * nb * 4 // 256) * 256 + 2 * (-(-2 * nb * 4 // 256) * 256)
    part = min(2 * nb, 255) * 4 * 2 * 128 * 64 * 4
    assert (L.attnqat_bwd_workspace_bytes(ctypes.byref(p)) ==
            L.attnqat_bwd_workspace_bytes(ctypes.byref(dense)) - kt - part + rev)


def test_block_select_checks(L):
    p = _prob(Nq=1024, Nk=1024)
    p.topk = 3
    need = L.attnqat_block_select_workspace_bytes(ctypes.byref(p))
    assert need > 0
    sel = L.attnqat_block_select
    assert sel(ctypes.byref(p), A, 2 * A, 0, 6 * A, need, None) == E_INVALID
    assert sel(ctypes.byref(p), A, 2 * A, 3 * A, 6 * A, need - 1, None) == E_WORKSPACE
    assert sel(ctypes.byref(p), A, 2 * A, 3 * A + 2, 6 * A, need, None) == E_MISALIGNED
    p.topk = 9
    assert sel(ctypes.byref(p), A, 2 * A, 3 * A, 6 * A, need, None) == E_INVALID
    p.topk = 3
    p.D = 80
    assert sel(ctypes.byref(p), A, 2 * A, 3 * A, 6 * A, need, None) == E_UNSUPPORTED


def test_fakequant_checks(L):
    s0 = qaa.Strides(0, 0, 0)
    fq = L.attnqat_fakequant_nvfp4
    assert fq(A, s0, 2 * A, s0, None, 1, 1, 16, 64, 2, None) == E_INVALID       # axis
    assert fq(A, s0, 2 * A, s0, None, 1, 1, 16, 40, 0, None) == E_UNSUPPORTED   # D % 16
    assert fq(A, s0, 2 * A, s0, None, 1, 1, 16, 12, 1, None) == E_UNSUPPORTED   # D % 8
    assert fq(0, s0, 2 * A, s0, None, 1, 1, 16, 64, 0, None) == E_INVALID
    assert fq(A, s0, A + 64, s0, None, 1, 1, 16, 64, 0, None) == E_INVALID      # overlap
    assert fq(A + 8, s0, 2 * A, s0, None, 1, 1, 16, 64, 0, None) == E_MISALIGNED
    assert fq(A, s0, 2 * A, s0, None, 0, 1, 16, 64, 0, None) == E_INVALID
    assert fq(A, s0, 2 * A, s0, A + 16, 1, 1, 16, 64, 0, None) == E_INVALID     # codes overlap


def test_profile_read_empty(L):
    assert L.attnqat_profile_enable(1) == OK
    assert L.attnqat_profile_read(None, None, None, 8) == 0
    assert L.attnqat_profile_enable(0) == OK


def test_workspace_sizes_scale_with_problem(L):
    a = L.attnqat_fwd_workspace_bytes(ctypes.byref(_prob(Nq=256, Nk=256)))
    b = L.attnqat_fwd_workspace_bytes(ctypes.byref(_prob(Nq=512, Nk=512)))
    assert b > a > 0 and a % 256 == 0 and b % 256 == 0


def test_mask_parsing():
    assert qaa.parse_mask("qkvp") == 15 and qaa.parse_mask("p") == 8 and qaa.parse_mask(5) == 5
    assert math.isclose(1 / math.sqrt(128), 0.08838834764831845)


def test_row_max_mode_validation(L):
    """p_mode: unknown values, a missing or misaligned row_max, and a row_max
    that overlaps an output or input are rejected before any HIP call."""
    assert _fwd(L, _prob(p_mode=2)) == E_INVALID
    assert _fwd(L, _prob(p_mode=1)) == E_INVALID                       # row_max missing
    assert _fwd(L, _prob(p_mode=1, row_max=30 * A + 2)) == E_MISALIGNED
    assert _fwd(L, _prob(p_mode=1, row_max=5 * A)) == E_INVALID       # overlaps lse
    assert _fwd(L, _prob(p_mode=1, row_max=A)) == E_INVALID           # overlaps q
    assert _bwd(L, _prob(p_mode=1, row_max=7 * A)) == E_INVALID       # overlaps dq
    assert _bwd(L, _prob(p_mode=1)) == E_INVALID
    # the row-max backward needs room for its scaled dO copy and statistics
    need0 = L.attnqat_bwd_workspace_bytes(ctypes.byref(_prob()))
    need1 = L.attnqat_bwd_workspace_bytes(ctypes.byref(_prob(p_mode=1, row_max=30 * A)))
    assert need1 > need0
    # without P quantization the variant is the normalised one: no extra room
    need2 = L.attnqat_bwd_workspace_bytes(ctypes.byref(_prob(p_mode=1, row_max=30 * A,
                                                             quant_mask=7)))
    assert need2 == need0


def test_ste_output_validation(L):
    """o_ste takes o's strides; it must be 16-byte aligned and overlap neither
    an input nor another output."""
    assert _fwd(L, _prob(o_ste=40 * A + 8)) == E_MISALIGNED
    assert _fwd(L, _prob(o_ste=A)) == E_INVALID        # overlaps q
    assert _fwd(L, _prob(o_ste=4 * A)) == E_INVALID    # overlaps o



def _vsa_fwd(L, p, q=A, k=2 * A, v=3 * A, gate=4 * A, of=5 * A, o=6 * A, ws=7 * A, wsb=1 << 40):
    return L.attnqat_vsa_fwd(ctypes.byref(p), q, k, v, gate, of, o, ws, wsb, None)


def _vsa_bwd(L, p, ws=20 * A, wsb=1 << 40, **ptrs):
    d = dict(q=A, k=2 * A, v=3 * A, gate=4 * A, do=5 * A, dq=6 * A, dk=7 * A, dv=8 * A, dg=9 * A)
    d.update(ptrs)
    return L.attnqat_vsa_bwd(ctypes.byref(p), d["q"], d["k"], d["v"], d["gate"], d["do"], d["dq"],
                             d["dk"], d["dv"], d["dg"], ws, wsb, None)


def test_vsa_validation(L):
    """The VSA coarse entry points: 128-token blocks only, workspace size and
    alignment, o / gradient aliasing and pointer alignment are all rejected
    before any HIP call."""
    p = _prob()
    need = L.attnqat_vsa_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert L.attnqat_vsa_workspace_bytes(ctypes.byref(_prob(block_tokens=64))) == 0
    assert _vsa_fwd(L, _prob(block_tokens=64)) == E_UNSUPPORTED
    assert _vsa_fwd(L, p, wsb=need - 1) == E_WORKSPACE
    assert _vsa_fwd(L, p, ws=7 * A + 16) == E_MISALIGNED
    assert _vsa_fwd(L, p, gate=4 * A + 8) == E_MISALIGNED
    assert _vsa_fwd(L, p, o=A) == E_INVALID          # o overlaps q
    assert _vsa_fwd(L, p, o=5 * A) == E_INVALID      # o overlaps o_fine
    assert _vsa_fwd(L, p, ws=4 * A) == E_INVALID     # workspace overlaps the gate
    assert _vsa_fwd(L, _prob(D=96)) == E_UNSUPPORTED
    assert _vsa_bwd(L, _prob(block_tokens=256)) == E_UNSUPPORTED
    assert _vsa_bwd(L, p, dq=7 * A) == E_INVALID      # dq overlaps dk
    assert _vsa_bwd(L, p, dg=6 * A) == E_INVALID      # dgate overlaps dq
    assert _vsa_bwd(L, p, dv=5 * A) == E_INVALID      # dv overlaps dout
    assert _vsa_bwd(L, p, wsb=16) == E_WORKSPACE
    assert _vsa_bwd(L, p, dk=7 * A + 4) == E_MISALIGNED
    assert _vsa_bwd(L, p, q=0) == E_INVALID


def test_batch_heads_limit(L):
    """(batch, head) pairs index the second grid dimension: more than 65535
    is rejected, as unsupported, before any HIP call."""
    assert _fwd(L, _prob(B=2, H=40000)) == E_UNSUPPORTED
    assert L.attnqat_fwd_workspace_bytes(ctypes.byref(_prob(B=2, H=40000))) == 0



def _mx(L, p, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, ws=6 * A, wsb=1 << 40):
    return L.attnqat_mxfp4_fwd(ctypes.byref(p), q, k, v, o, lse, ws, wsb, None)


def test_mxfp4_validation(L):
    """The MXFP4 forward: dense, every quantizer, no straight-through output;
    the exact workspace size (codes and scales of Q, K and V^T, token counts
    padded to 256); workspace, alignment and aliasing errors before any HIP
    call."""
    p = _prob()
    need = L.attnqat_mxfp4_fwd_workspace_bytes(ctypes.byref(p))
    # B H = 2, D = 64, Nq_pad = Nk_pad = 256: 2 * 256 * 32 code bytes and
    # 2 * 256 * 2 scale bytes for each of Q, K and V^T
    assert need == 3 * (2 * 256 * 32) + 3 * (2 * 256 * 2)
    assert L.attnqat_mxfp4_fwd_workspace_bytes(ctypes.byref(_prob(quant_mask=7))) == 0
    assert _mx(L, _prob(quant_mask=7)) == E_UNSUPPORTED
    assert _mx(L, _prob(kv_block_idx=9 * A, topk=1)) == E_UNSUPPORTED
    assert _mx(L, _prob(o_ste=9 * A)) == E_UNSUPPORTED
    assert _mx(L, _prob(D=96)) == E_UNSUPPORTED
    assert _mx(L, p, wsb=need - 1) == E_WORKSPACE
    assert _mx(L, p, ws=6 * A + 16) == E_MISALIGNED
    assert _mx(L, p, lse=5 * A + 2) == E_MISALIGNED
    assert _mx(L, p, o=A) == E_INVALID          # output overlaps q
    assert _mx(L, p, ws=4 * A) == E_INVALID     # workspace overlaps o
    assert _mx(L, p, q=0) == E_INVALID


def test_sequence_length_cap(L):
    """Sequences beyond ATTNQAT_MAX_TOKENS are rejected as unsupported before
    any HIP call (the tile copies form 32-bit byte offsets of up to 128 rows of
    a transposed operand); the cap itself is accepted."""
    cap = qaa.MAX_TOKENS
    text = open(HEADER).read()
    assert f"#define ATTNQAT_MAX_TOKENS {cap}" in text
    assert 128 * cap * 2 < 2 ** 31
    for kw in (dict(Nq=cap + 1), dict(Nk=cap + 1), dict(Nq=1 << 30, Nk=1 << 30)):
        p = _prob(**kw)
        assert _fwd(L, p) == E_UNSUPPORTED
        assert b"sequence length" in L.attnqat_last_error()
        assert _bwd(L, p) == E_UNSUPPORTED
        assert _mx(L, p) == E_UNSUPPORTED
        assert L.attnqat_fwd_workspace_bytes(ctypes.byref(p)) == 0
        assert L.attnqat_bwd_workspace_bytes(ctypes.byref(p)) == 0
    ok = _prob(Nq=cap, Nk=cap)
    assert L.attnqat_fwd_workspace_bytes(ctypes.byref(ok)) > 0
    assert L.attnqat_bwd_workspace_bytes(ctypes.byref(ok)) > 0


def test_effective_topk_matches_the_oracle_formula(L):
    """The library's selection count is the pages' formula, as the oracle
    states it, over a grid of block counts and sparsities."""
    from oracle import block_sparse as bsp
    for n in (1, 2, 5, 6, 10, 100, 244, 256, 1000, 1024):
        for sp in (0.0, 0.1, 0.5, 0.75, 0.9, 0.95, 0.99, 1.0):
            assert L.attnqat_effective_topk(n, sp) == bsp.effective_topk(n, sp), (n, sp)
    assert L.attnqat_effective_topk(256, 0.9) == 26
    assert L.attnqat_effective_topk(0, 0.9) == -E_INVALID
    assert L.attnqat_effective_topk(10, 1.5) == -E_INVALID
    assert L.attnqat_effective_topk(10, float("nan")) == -E_INVALID
    assert qaa.effective_topk(256, 0.9) == 26


def test_block_idx_status_argument_checks(L):
    flag = ctypes.c_int(0)
    assert L.attnqat_block_idx_status(None, ctypes.byref(flag), None) == E_INVALID
    assert L.attnqat_block_idx_status(A, None, None) == E_INVALID
    assert L.attnqat_block_idx_status(A + 16, ctypes.byref(flag), None) == E_MISALIGNED


def test_workspace_starts_with_the_index_flag(L):
    """Both layouts keep the block-index check flag at offset 0 (one 256-byte
    region), which attnqat_block_idx_status reads: the sparse forward's
    workspace is the dense one's operands."""
    dense = _prob(Nq=1024, Nk=1024)
    sparse = _prob(Nq=1024, Nk=1024, kv_block_idx=30 * A, topk=3)
    # operands: Qq, Kq and Vq^T (the forward reads V only transposed) of
    # 2 heads x 1024 tokens x 64 bf16, plus the flag
    ops = 256 + 3 * 2 * 1024 * 64 * 2
    assert L.attnqat_fwd_workspace_bytes(ctypes.byref(sparse)) == ops
    # the dense pass 2 runs 8 workgroups of 256 queries, a partial round on a
    # chip of 256 compute units, so their 8 x 16 key tiles are shared out to
    # 16 workgroups of 8 tiles, each with two partial slots of 256 x 64 fp32
    assert L.attnqat_fwd_workspace_bytes(ctypes.byref(dense)) == ops + 2 * 16 * 256 * 64 * 4


def test_forward_split_region(L):
    """The pass-2 partial region exists only where the dense producer/consumer
    pass 2 runs (P quantized) and its last round is partly filled."""
    def fwd_ws(**kw):
        return L.attnqat_fwd_workspace_bytes(ctypes.byref(_prob(**kw)))
    ops = 256 + 3 * 2 * 1024 * 64 * 2
    assert fwd_ws(Nq=1024, Nk=1024, quant_mask=7) == ops        # no P quantizer: one pass
    # pass 2 with O_ste: 16 blocks of 128 queries x 16 key tiles shared out
    # to 32 workgroups of 8 tiles, two slots of [O, O_ste][128][64] each
    assert fwd_ws(Nq=1024, Nk=1024, o_ste=30 * A) == ops + 2 * 32 * 256 * 64 * 4
    # 256 heads x 256 queries: one whole round of 256 workgroups
    full = 256 + 3 * 256 * 256 * 64 * 2
    assert fwd_ws(H=256, Nq=256, Nk=256) == full
    # 264 heads of 256 tokens: 8 workgroups in the second round with 4 key
    # tiles each, too few to share out in chunks of at least 8 tiles
    assert fwd_ws(H=264, Nq=256, Nk=256) == 256 + 3 * 264 * 256 * 64 * 2
    # 264 heads of 1024 tokens: 32 last-round workgroups x 16 key tiles shared
    # out to 64 workgroups of 8 tiles
    assert (fwd_ws(H=264, Nq=1024, Nk=1024) ==
            256 + 3 * 264 * 1024 * 64 * 2 + 2 * 64 * 256 * 64 * 4)
    # a single key tile cannot be split (Kq and Vq^T padded to 256 tokens)
    assert fwd_ws(Nq=1024, Nk=64) == 256 + 2 * 1024 * 64 * 2 + 2 * (2 * 256 * 64 * 2)


def test_noalloc_host_checks(L):
    """attnqat_fwd_noalloc validates like attnqat_fwd and rejects, before any
    HIP call, a problem whose workspace would not fit its fixed scratch."""
    assert _fwd_noalloc(L, _prob(D=96)) == E_UNSUPPORTED
    assert _fwd_noalloc(L, _prob(B=0)) == E_INVALID
    big = _prob(H=64, Nq=4096, Nk=4096, D=128)
    assert L.attnqat_fwd_workspace_bytes(ctypes.byref(big)) > qaa.NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(L, big) == E_UNSUPPORTED
    assert b"scratch" in L.attnqat_last_error()


def _fwd_noalloc(L, p, q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A):
    return L.attnqat_fwd_noalloc(ctypes.byref(p), q, k, v, o, lse, None)


def test_lds_poison_build_carries_the_poison():
    """The debug twin that the GPU poisoning test compares with the release
    library stores the poison word (0x7FF87FF8, as an instruction literal) in
    its kernels; the release library does not."""
    from quantization_aware_attention_amd.build import LIB_PATH, POISON_PATH
    word = (0x7FF87FF8).to_bytes(4, "little")
    with open(POISON_PATH, "rb") as f:
        assert f.read().count(word) > 0
    with open(LIB_PATH, "rb") as f:
        assert f.read().count(word) == 0

"""Python binding of the Attn-QAT HIP library (``libattnqat.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attnqat.h``. PyTorch provides
device memory and the current stream. There is no CPU path: if the library is
not built or no gfx950 GPU is present, calls raise.

    o, lse = fwd(q, k, v)                     # bf16 [B,H,N,D] tensors on the GPU
    dq, dk, dv = bwd(q, k, v, o, lse, do)
    y = fakequant(x, axis="d")               # NVFP4 fake quantization
    idx = block_select(q, k, topk=26)        # VSA-style block selection
    o = attention(q, k, v)                   # autograd-aware wrapper
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # noqa: F401  (load torch's HIP runtime before the library)

from .build import LIB_PATH

QUANT_Q, QUANT_K, QUANT_V, QUANT_P = 1, 2, 4, 8
QUANT_ALL = 15
AXIS_D, AXIS_N = 0, 1
P_NORMALISED, P_ROWMAX = 0, 1

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "misaligned",
          4: "workspace too small", 5: "HIP error"}


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("Nq", ctypes.c_int64),
        ("Nk", ctypes.c_int64), ("D", ctypes.c_int64), ("sm_scale", ctypes.c_float),
        ("quant_mask", ctypes.c_uint32),
        ("q", Strides), ("k", Strides), ("v", Strides), ("o", Strides),
        ("dout", Strides), ("dq", Strides), ("dk", Strides), ("dv", Strides),
        ("kv_block_idx", ctypes.c_void_p), ("topk", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("p_mode", ctypes.c_uint32), ("row_max", ctypes.c_void_p), ("o_ste", ctypes.c_void_p),
    ]


EXPORTS = [
    "attnqat_abi_version", "attnqat_status_string", "attnqat_last_error",
    "attnqat_fakequant_nvfp4", "attnqat_fwd_workspace_bytes", "attnqat_fwd",
    "attnqat_bwd_workspace_bytes", "attnqat_bwd", "attnqat_block_select_workspace_bytes",
    "attnqat_block_select", "attnqat_vsa_workspace_bytes", "attnqat_vsa_fwd", "attnqat_vsa_bwd",
    "attnqat_mxfp4_fwd_workspace_bytes", "attnqat_mxfp4_fwd",
    "attnqat_profile_enable", "attnqat_profile_read", "attnqat_block_idx_status",
    "attnqat_effective_topk", "attnqat_fwd_noalloc",
]
NOALLOC_SCRATCH_BYTES = 64 << 20
MAX_TOKENS = 4194304

_lib = None


class AttnQatError(RuntimeError):
    pass


def _hip_runtimes_mapped() -> set:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                p = line.split()[-1] if line.strip() else ""
                if "libamdhip64.so" in p:
                    paths.add(os.path.realpath(p))
    except OSError:
        pass
    return paths


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path or LIB_PATH)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Open a build of the library at `path` and declare its C signatures,
    without making it the one the functions below call (load does that)."""
    if not os.path.exists(path):
        raise AttnQatError(f"{path} is missing: build it with quantization_aware_attention_amd."
                           "build.build() (there is no fallback path)")
    lib = ctypes.CDLL(path)
    P, V, I64, SZ = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    pp = ctypes.POINTER(Problem)
    lib.attnqat_abi_version.restype = ctypes.c_int
    lib.attnqat_status_string.restype = ctypes.c_char_p
    lib.attnqat_status_string.argtypes = [ctypes.c_int]
    lib.attnqat_last_error.restype = ctypes.c_char_p
    lib.attnqat_fakequant_nvfp4.restype = ctypes.c_int
    lib.attnqat_fakequant_nvfp4.argtypes = [P, Strides, P, Strides, P, I64, I64, I64, I64,
                                            ctypes.c_int, V]
    lib.attnqat_fwd_workspace_bytes.restype = SZ
    lib.attnqat_fwd_workspace_bytes.argtypes = [pp]
    lib.attnqat_fwd.restype = ctypes.c_int
    lib.attnqat_fwd.argtypes = [pp, P, P, P, P, P, P, SZ, V]
    lib.attnqat_fwd_noalloc.restype = ctypes.c_int
    lib.attnqat_fwd_noalloc.argtypes = [pp, P, P, P, P, P, V]
    lib.attnqat_bwd_workspace_bytes.restype = SZ
    lib.attnqat_bwd_workspace_bytes.argtypes = [pp]
    lib.attnqat_bwd.restype = ctypes.c_int
    lib.attnqat_bwd.argtypes = [pp, P, P, P, P, P, P, P, P, P, P, SZ, V]
    lib.attnqat_block_select_workspace_bytes.restype = SZ
    lib.attnqat_block_select_workspace_bytes.argtypes = [pp]
    lib.attnqat_block_select.restype = ctypes.c_int
    lib.attnqat_block_select.argtypes = [pp, P, P, P, P, SZ, V]
    lib.attnqat_vsa_workspace_bytes.restype = SZ
    lib.attnqat_vsa_workspace_bytes.argtypes = [pp]
    lib.attnqat_vsa_fwd.restype = ctypes.c_int
    lib.attnqat_vsa_fwd.argtypes = [pp, P, P, P, P, P, P, P, SZ, V]
    lib.attnqat_vsa_bwd.restype = ctypes.c_int
    lib.attnqat_vsa_bwd.argtypes = [pp, P, P, P, P, P, P, P, P, P, P, SZ, V]
    lib.attnqat_mxfp4_fwd_workspace_bytes.restype = SZ
    lib.attnqat_mxfp4_fwd_workspace_bytes.argtypes = [pp]
    lib.attnqat_mxfp4_fwd.restype = ctypes.c_int
    lib.attnqat_mxfp4_fwd.argtypes = [pp, P, P, P, P, P, P, SZ, V]
    lib.attnqat_block_idx_status.restype = ctypes.c_int
    lib.attnqat_block_idx_status.argtypes = [P, ctypes.POINTER(ctypes.c_int), V]
    lib.attnqat_effective_topk.restype = ctypes.c_int
    lib.attnqat_effective_topk.argtypes = [I64, ctypes.c_double]
    lib.attnqat_profile_enable.restype = ctypes.c_int
    lib.attnqat_profile_enable.argtypes = [ctypes.c_int]
    lib.attnqat_profile_read.restype = ctypes.c_int
    lib.attnqat_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int), ctypes.c_int]
    rts = _hip_runtimes_mapped()
    if len(rts) > 1:
        raise AttnQatError(f"two HIP runtimes are mapped ({sorted(rts)}); streams would not "
                           "be shared with torch")
    return lib


def lib() -> ctypes.CDLL:
    return load()


def check(rc: int) -> None:
    if rc != 0:
        msg = _lib.attnqat_last_error().decode() if _lib else ""
        raise AttnQatError(f"attnqat status {rc} ({STATUS.get(rc, '?')}): {msg}")


def parse_mask(quant) -> int:
    if isinstance(quant, int):
        return quant
    m = 0
    for ch in str(quant).lower():
        m |= {"q": QUANT_Q, "k": QUANT_K, "v": QUANT_V, "p": QUANT_P}[ch]
    return m


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check4(name, t):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
        raise AttnQatError(f"{name} must be a bf16 CUDA tensor")
    if t.dim() != 4 or t.stride(-1) != 1:
        raise AttnQatError(f"{name} must be [B,H,N,D] with a contiguous last dimension")


def strides_of(t: torch.Tensor) -> Strides:
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _check_block_idx(idx, B, H, Nq, block_tokens, device):
    """Layout checks of a block index (the ranges and the ascending order of
    its entries are checked on the device by the library)."""
    if not isinstance(idx, torch.Tensor) or idx.dtype != torch.int32:
        raise AttnQatError("kv_block_idx must be an int32 tensor (torch.topk returns int64)")
    if not idx.is_cuda or idx.device != device:
        raise AttnQatError("kv_block_idx must be on the device of q")
    nbq = -(-Nq // block_tokens)
    if idx.dim() != 4 or tuple(idx.shape[:3]) != (B, H, nbq) or idx.shape[3] < 1:
        raise AttnQatError(f"kv_block_idx must be [B, H, ceil(Nq/{block_tokens}), topk] = "
                           f"[{B}, {H}, {nbq}, topk], got {tuple(idx.shape)}")
    if not idx.is_contiguous():
        raise AttnQatError("kv_block_idx must be contiguous")


def block_idx_status(workspace, stream=None) -> bool:
    """True if the device-side check of the block index failed in the last
    block-sparse fwd/bwd that used ``workspace`` (its outputs are then NaN).
    Waits for that call."""
    flag = ctypes.c_int(0)
    check(load().attnqat_block_idx_status(workspace.data_ptr(), ctypes.byref(flag),
                                          _stream(stream)))
    return bool(flag.value)


def _raise_if_bad_index(workspace, stream):
    if block_idx_status(workspace, stream):
        raise AttnQatError("kv_block_idx has an entry outside [0, ceil(Nk/128)) or a row that "
                           "is not strictly ascending; the outputs were filled with NaN")


def make_problem(q, k, sm_scale, quant_mask, *, v=None, o=None, do=None, dq=None, dk=None,
                 dv=None, kv_block_idx=None, block_tokens=128, p_mode=P_NORMALISED,
                 row_max=None, o_ste=None) -> Problem:
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    p = Problem()
    p.B, p.H, p.Nq, p.Nk, p.D = B, H, Nq, Nk, D
    p.sm_scale = float(sm_scale)
    p.quant_mask = parse_mask(quant_mask)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", do), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        if t is not None:
            setattr(p, name, strides_of(t))
    if kv_block_idx is not None:
        _check_block_idx(kv_block_idx, B, H, Nq, block_tokens, q.device)
        p.kv_block_idx = kv_block_idx.data_ptr()
        p.topk = kv_block_idx.shape[-1]
    p.block_tokens = block_tokens
    p.p_mode = int(p_mode)
    if row_max is not None:
        p.row_max = row_max.data_ptr()
    if o_ste is not None:
        p.o_ste = o_ste.data_ptr()
    return p


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte (at least) aligned blocks
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def fakequant(x: torch.Tensor, axis: str = "d", return_scale_codes: bool = False, stream=None,
              out=None):
    """NVFP4 fake quantization of a bf16 [B,H,N,D] tensor along 'd' or 'n'."""
    L = load()
    _check4("x", x)
    B, H, N, D = x.shape
    ax = AXIS_D if axis == "d" else AXIS_N
    y = out if out is not None else torch.empty((B, H, N, D), dtype=torch.bfloat16,
                                                device=x.device)
    _check4("out", y)
    if tuple(y.shape) != (B, H, N, D):
        raise ValueError("out must have the shape of x")
    codes = None
    if return_scale_codes:
        shp = (B, H, N, D // 16) if ax == AXIS_D else (B, H, (N + 15) // 16, D)
        codes = torch.empty(shp, dtype=torch.uint8, device=x.device)
    check(L.attnqat_fakequant_nvfp4(x.data_ptr(), strides_of(x), y.data_ptr(), strides_of(y),
                                    codes.data_ptr() if codes is not None else None,
                                    B, H, N, D, ax, _stream(stream)))
    return (y, codes) if return_scale_codes else y


def fwd(q, k, v, sm_scale=None, quant="qkvp", kv_block_idx=None, block_tokens=128,
        out=None, lse=None, workspace=None, stream=None, p_mode=P_NORMALISED, row_max=None,
        o_ste=None, validate_index=True):
    """O (bf16) and LSE (fp32, natural log) of Attn-QAT attention; with
    p_mode=P_ROWMAX also the row maxima of S (fp32 [B,H,Nq]), which the
    backward of that mode needs: returns (O, LSE, row_max). ``o_ste`` (a bf16
    tensor shaped and strided like the output) also receives the
    straight-through output P Vq; pass it as the backward's ``o`` for the
    additive straight-through delta. With a block index and
    ``validate_index``, the result of the library's device-side index check
    is read back (a wait on the stream) and a failed check raises."""
    L = load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check4(n, t)
    B, H, Nq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty((B, H, Nq, D), dtype=torch.bfloat16,
                                                device=q.device)
    lse = lse if lse is not None else torch.empty((B, H, Nq), dtype=torch.float32,
                                                  device=q.device)
    if p_mode == P_ROWMAX and row_max is None:
        row_max = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if o_ste is not None:
        _check4("o_ste", o_ste)
        if tuple(o_ste.shape) != tuple(o.shape) or o_ste.stride() != o.stride():
            raise ValueError("o_ste must have the shape and strides of the output")
    p = make_problem(q, k, sm_scale, quant, v=v, o=o, kv_block_idx=kv_block_idx,
                     block_tokens=block_tokens, p_mode=p_mode, row_max=row_max, o_ste=o_ste)
    need = L.attnqat_fwd_workspace_bytes(ctypes.byref(p))
    if need == 0:  # invalid problem: the call reports why
        check(L.attnqat_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            o.data_ptr(), lse.data_ptr(), None, 0, _stream(stream)))
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        _workspace(need, q.device)
    check(L.attnqat_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        lse.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    if kv_block_idx is not None and validate_index:
        _raise_if_bad_index(ws, stream)
    return (o, lse, row_max) if p_mode == P_ROWMAX else (o, lse)


def fwd_noalloc(q, k, v, o, lse, sm_scale=None, quant="qkvp", kv_block_idx=None,
                block_tokens=128, stream=None, p_mode=P_NORMALISED, row_max=None, o_ste=None):
    """attnqat_fwd_noalloc: the forward into the caller's o (bf16) and lse
    (fp32 [B,H,Nq]) with the library's fixed device scratch instead of a
    workspace (for code that must not allocate, e.g. under graph capture);
    o, lse (and row_max, o_ste) must be preallocated."""
    L = load()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check4(n, t)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    p = make_problem(q, k, sm_scale, quant, v=v, o=o, kv_block_idx=kv_block_idx,
                     block_tokens=block_tokens, p_mode=p_mode, row_max=row_max, o_ste=o_ste)
    check(L.attnqat_fwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                o.data_ptr(), lse.data_ptr(), _stream(stream)))
    return o, lse


def bwd(q, k, v, o, lse, do, sm_scale=None, quant="qkvp", kv_block_idx=None, block_tokens=128,
        dq=None, dk=None, dv=None, workspace=None, stream=None, p_mode=P_NORMALISED,
        row_max=None, validate_index=True):
    """dQ, dK, dV (bf16) of Attn-QAT attention with straight-through quantizers
    (p_mode=P_ROWMAX needs the forward's row_max). ``validate_index`` as for
    ``fwd``."""
    L = load()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check4(n, t)
    B, H, Nq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dq = dq if dq is not None else torch.empty_like(q, memory_format=torch.contiguous_format)
    dk = dk if dk is not None else torch.empty_like(k, memory_format=torch.contiguous_format)
    dv = dv if dv is not None else torch.empty_like(v, memory_format=torch.contiguous_format)
    p = make_problem(q, k, sm_scale, quant, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv,
                     kv_block_idx=kv_block_idx, block_tokens=block_tokens, p_mode=p_mode,
                     row_max=row_max)
    need = L.attnqat_bwd_workspace_bytes(ctypes.byref(p))
    if need == 0:  # invalid problem: the call reports why
        check(L.attnqat_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                            dk.data_ptr(), dv.data_ptr(), None, 0, _stream(stream)))
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        _workspace(need, q.device)
    check(L.attnqat_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                        dv.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    if kv_block_idx is not None and validate_index:
        _raise_if_bad_index(ws, stream)
    return dq, dk, dv


def block_select(q, k, topk: int, block_tokens: int = 128, stream=None) -> torch.Tensor:
    """int32 [B,H,ceil(Nq/bt),topk] ascending key-block indices (VSA coarse selection)."""
    L = load()
    _check4("q", q)
    _check4("k", k)
    B, H, Nq, D = q.shape
    nbq = -(-Nq // block_tokens)
    idx = torch.empty((B, H, nbq, topk), dtype=torch.int32, device=q.device)
    p = make_problem(q, k, 1.0, 0, block_tokens=block_tokens)
    p.topk = topk
    need = L.attnqat_block_select_workspace_bytes(ctypes.byref(p))
    ws = _workspace(need, q.device)
    check(L.attnqat_block_select(ctypes.byref(p), q.data_ptr(), k.data_ptr(), idx.data_ptr(),
                                 ws.data_ptr(), ws.numel(), _stream(stream)))
    return idx


def mxfp4_fwd(q, k, v, sm_scale=None, out=None, lse=None, workspace=None, stream=None):
    """Real-FP4 inference forward on MXFP4 operands (attnqat_mxfp4_fwd):
    returns (o bf16 [B,H,Nq,D], lse fp32 [B,H,Nq])."""
    L = load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check4(n, t)
    B, H, Nq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty_like(q)
    _check4("out", o)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be a contiguous float32 [B,H,Nq] tensor")
    p = make_problem(q, k, sm_scale, QUANT_ALL, v=v, o=o)
    need = L.attnqat_mxfp4_fwd_workspace_bytes(ctypes.byref(p))
    if need == 0:
        check(L.attnqat_mxfp4_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  o.data_ptr(), lse.data_ptr(), None, 0, _stream(stream)))
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        _workspace(need, q.device)
    check(L.attnqat_mxfp4_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              o.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream(stream)))
    return o, lse


def vsa_fwd(q, k, v, gate, o_fine, sm_scale=None, out=None, workspace=None, stream=None):
    """VSA coarse branch and gated combination: o_fine + gate * O_c[block(t)]
    (bf16 [B,H,Nq,D]; gate, o_fine and the output share one stride layout)."""
    L = load()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("o_fine", o_fine)):
        _check4(n, t)
    B, H, Nq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty_like(o_fine)
    _check4("out", o)
    for n, t in (("gate", gate), ("out", o)):
        if tuple(t.shape) != tuple(o_fine.shape) or t.stride() != o_fine.stride():
            raise ValueError(f"{n} must have the shape and strides of o_fine")
    p = make_problem(q, k, sm_scale, 0, v=v, o=o_fine)
    need = L.attnqat_vsa_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        _workspace(need, q.device)
    check(L.attnqat_vsa_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            gate.data_ptr(), o_fine.data_ptr(), o.data_ptr(), ws.data_ptr(),
                            ws.numel(), _stream(stream)))
    return o


def vsa_bwd(q, k, v, gate, do, dq, dk, dv, sm_scale=None, dgate=None, want_dgate=True,
            workspace=None, stream=None):
    """Adds the coarse branch's gradients to dq, dk, dv in place (they hold
    the fine branch's) and returns (dq, dk, dv, dgate); dgate is shaped and
    strided like gate (None with want_dgate=False)."""
    L = load()
    for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("do", do), ("dq", dq),
                 ("dk", dk), ("dv", dv)):
        _check4(n, t)
    B, H, Nq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if want_dgate and dgate is None:
        dgate = torch.empty_like(gate)
    if dgate is not None:
        _check4("dgate", dgate)
        if tuple(dgate.shape) != tuple(gate.shape) or dgate.stride() != gate.stride():
            raise ValueError("dgate must have the shape and strides of gate")
    p = make_problem(q, k, sm_scale, 0, v=v, o=gate, do=do, dq=dq, dk=dk, dv=dv)
    need = L.attnqat_vsa_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        _workspace(need, q.device)
    check(L.attnqat_vsa_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            gate.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), dgate.data_ptr() if dgate is not None else None,
                            ws.data_ptr(), ws.numel(), _stream(stream)))
    return dq, dk, dv, dgate


def profile_enable(on: bool = True) -> None:
    """Time every kernel this thread enqueues with HIP events on its stream."""
    check(load().attnqat_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kernel kind: (total ms, launches)} since the last read; synchronises."""
    L = load()
    n = 32
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    k = L.attnqat_profile_read(names, ms, cnt, n)
    if k < 0:
        check(-k)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(k)}


class AttnQatFunction(torch.autograd.Function):
    """Autograd wrapper: forward saves (O, LSE[, row maxima]); backward is
    straight-through."""

    @staticmethod
    def forward(ctx, q, k, v, sm_scale, quant, kv_block_idx, p_mode=P_NORMALISED):
        res = fwd(q, k, v, sm_scale, quant, kv_block_idx, p_mode=p_mode)
        o, lse = res[0], res[1]
        row_max = res[2] if p_mode == P_ROWMAX else None
        ctx.save_for_backward(q, k, v, o, lse, kv_block_idx, row_max)
        ctx.sm_scale, ctx.quant, ctx.p_mode = sm_scale, quant, p_mode
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, idx, row_max = ctx.saved_tensors
        do = do.contiguous()
        dq, dk, dv = bwd(q, k, v, o, lse, do, ctx.sm_scale, ctx.quant, idx, p_mode=ctx.p_mode,
                         row_max=row_max, validate_index=False)  # the forward checked it
        return dq, dk, dv, None, None, None, None


def attention(q, k, v, sm_scale=None, quant="qkvp", kv_block_idx=None, p_mode=P_NORMALISED):
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    return AttnQatFunction.apply(q, k, v, sm_scale, quant, kv_block_idx, p_mode)


def effective_topk(num_blocks: int, sparsity: float = 0.9) -> int:
    """Key blocks kept per query block (the library's attnqat_effective_topk)."""
    k = load().attnqat_effective_topk(int(num_blocks), float(sparsity))
    if k < 0:
        check(-k)
    return k


class VsaAttentionFunction(torch.autograd.Function):
    """VSA attention: block-sparse Attn-QAT fine branch over the selected key
    blocks plus the gated coarse branch. Backward: the fine branch's
    straight-through backward (with its own output as o), then the coarse
    branch's gradients added in place, and the gate's gradient."""

    @staticmethod
    def forward(ctx, q, k, v, gate, sm_scale, quant, kv_block_idx):
        o_fine, lse = fwd(q, k, v, sm_scale, quant, kv_block_idx)  # checks the index
        o = vsa_fwd(q, k, v, gate, o_fine, sm_scale)
        ctx.save_for_backward(q, k, v, gate, o_fine, lse, kv_block_idx)
        ctx.sm_scale, ctx.quant = sm_scale, quant
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, gate, o_fine, lse, idx = ctx.saved_tensors
        do = do.contiguous()
        dq, dk, dv = bwd(q, k, v, o_fine, lse, do, ctx.sm_scale, ctx.quant, idx,
                         validate_index=False)  # the forward checked this index
        dq, dk, dv, dgate = vsa_bwd(q, k, v, gate, do, dq, dk, dv, ctx.sm_scale,
                                    want_dgate=ctx.needs_input_grad[3])
        return dq, dk, dv, dgate, None, None, None


def vsa_attention(q, k, v, gate, topk=None, sparsity=0.9, sm_scale=None, quant="qkvp",
                  kv_block_idx=None):
    """VSA attention with 128-token blocks. The key blocks come from the coarse
    selection (top ``topk`` per query block, default effective_topk(blocks,
    sparsity)) unless ``kv_block_idx`` is given."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    if kv_block_idx is None:
        nbk = -(-k.shape[2] // 128)
        kv_block_idx = block_select(q, k, topk if topk is not None else effective_topk(nbk, sparsity))
    return VsaAttentionFunction.apply(q, k, v, gate, sm_scale, quant, kv_block_idx)

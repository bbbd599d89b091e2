"""ctypes binding of ``libnsa_sel.so`` (declared in ``include/nsa_sel.h``).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch supplies device memory and the current stream.  If the
library has not been built, importing this module fails loudly; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnsa_sel.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python nsa_selected_block_amd/build.py` "
        "(or __graft_entry__.build()); there is no non-HIP fallback")

# torch (ROCm build) carries its own HIP runtime, whose SONAME is the same
# libamdhip64.so.7 this library needs.  Loading torch first makes the dynamic
# loader bind this library to that one runtime; loading the library first
# would bring in a second HIP/HSA runtime that cannot see the device.
import torch  # noqa: E402,F401  (must precede the CDLL below)

lib = ctypes.CDLL(LIB_PATH)

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_HIP = -4
ERR_BAD_INPUT = -5

DTYPE_BF16 = 1
DTYPE_F32 = 2
DTYPE_F16 = 3

FLAG_DENSE_SPLIT = 1


class Desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("stage_events", ctypes.c_void_p),  # NULL or hipEvent_t[STAGE_EVENTS] of the caller
    ]


STAGE_EVENTS = 5


_P = ctypes.c_void_p
_D = ctypes.POINTER(Desc)
lib.nsa_sel_version.argtypes = []
lib.nsa_sel_version.restype = ctypes.c_int
lib.nsa_sel_status_string.argtypes = [ctypes.c_int]
lib.nsa_sel_status_string.restype = ctypes.c_char_p
lib.nsa_sel_last_error.argtypes = []
lib.nsa_sel_last_error.restype = ctypes.c_char_p
lib.nsa_sel_validate.argtypes = [_D]
lib.nsa_sel_validate.restype = ctypes.c_int
lib.nsa_sel_index_sizes.argtypes = [_D, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
lib.nsa_sel_index_sizes.restype = ctypes.c_int
lib.nsa_sel_index_workspace_size.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t)]
lib.nsa_sel_index_workspace_size.restype = ctypes.c_int
lib.nsa_sel_fwd_workspace_size.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t)]
lib.nsa_sel_fwd_workspace_size.restype = ctypes.c_int
lib.nsa_sel_build_index.argtypes = [_D, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.nsa_sel_build_index.restype = ctypes.c_int
lib.nsa_sel_attn_fwd.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.nsa_sel_attn_fwd.restype = ctypes.c_int
lib.nsa_sel_attn_fwd_indexed.argtypes = [_D] + [_P] * 10 + [ctypes.c_size_t, _P]
lib.nsa_sel_attn_fwd_indexed.restype = ctypes.c_int
lib.nsa_sel_workspace_size.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t)]
lib.nsa_sel_workspace_size.restype = ctypes.c_int
lib.nsa_sel_bwd_workspace_size.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t)]
lib.nsa_sel_bwd_workspace_size.restype = ctypes.c_int
lib.nsa_sel_attn_bwd.argtypes = [_D] + [_P] * 12 + [ctypes.c_size_t, _P]
lib.nsa_sel_attn_bwd.restype = ctypes.c_int
lib.nsa_sel_window_workspace_size.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t)]
lib.nsa_sel_window_workspace_size.restype = ctypes.c_int
lib.nsa_sel_window_fwd.argtypes = [_D, ctypes.c_int] + [_P] * 7 + [ctypes.c_size_t, _P]
lib.nsa_sel_window_fwd.restype = ctypes.c_int
lib.nsa_sel_window_fwd_noalloc.argtypes = [_D, ctypes.c_int] + [_P] * 7
lib.nsa_sel_window_fwd_noalloc.restype = ctypes.c_int
lib.nsa_sel_select_workspace_size.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t)]
lib.nsa_sel_select_workspace_size.restype = ctypes.c_int
lib.nsa_sel_select_blocks.argtypes = [_D] + [ctypes.c_int] * 4 + [_P] * 5 + [ctypes.c_size_t, _P]
lib.nsa_sel_select_blocks.restype = ctypes.c_int
lib.nsa_sel_check.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_int)]
lib.nsa_sel_check.restype = ctypes.c_int


class NsaSelError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = lib.nsa_sel_status_string(status).decode()
        if status == ERR_HIP:
            msg += ": " + lib.nsa_sel_last_error().decode()
        super().__init__(f"{what}: {msg} ({status})" if what else f"{msg} ({status})")


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise NsaSelError(rc, what)


def version() -> int:
    return lib.nsa_sel_version()


def status_string(status: int) -> str:
    return lib.nsa_sel_status_string(status).decode()


def make_desc(total_tokens: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
              head_dim: int, block_size: int, topk: int, scale: Optional[float] = None,
              dtype: int = DTYPE_BF16, flags: int = 0, stage_events=None) -> Desc:
    """A descriptor; stage_events is None or a ctypes array of STAGE_EVENTS
    hipEvent_t handles (see StageTimer)."""
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    ev = ctypes.cast(stage_events, ctypes.c_void_p) if stage_events is not None else None
    return Desc(ctypes.sizeof(Desc), dtype, num_seqs, num_q_heads, total_tokens, num_kv_heads,
                head_dim, block_size, topk, scale, flags, ev)


def validate(desc: Desc) -> int:
    return lib.nsa_sel_validate(ctypes.byref(desc))


def index_sizes(desc: Desc) -> Tuple[int, int]:
    nb, ne = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.nsa_sel_index_sizes(ctypes.byref(desc), ctypes.byref(nb), ctypes.byref(ne)),
           "nsa_sel_index_sizes")
    return nb.value, ne.value


def index_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.nsa_sel_index_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "nsa_sel_index_workspace_size")
    return n.value


def fwd_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.nsa_sel_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "nsa_sel_fwd_workspace_size")
    return n.value


def bwd_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.nsa_sel_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "nsa_sel_bwd_workspace_size")
    return n.value


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _check_out(out, lse, q, name="out"):
    """The caller's output buffers must be exactly what the kernels write:
    out shaped and typed like q, lse float32 [T, Hq], both on q's device."""
    torch = _torch()
    T, Hq = q.shape[0], q.shape[1]
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape) or out.device != q.device \
            or out.dim() != 3 or not out.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {q.dtype} tensor of q's shape {tuple(q.shape)} "
                         f"on {q.device}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq) or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(T, Hq)} on {q.device}")


def _desc_from(q, k, cu_seqlens, block_idx, block_size, scale, flags=0, stage_events=None):
    torch = _torch()
    dtype = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16, torch.float32: DTYPE_F32}.get(q.dtype)
    if dtype is None:
        raise TypeError("q must be bfloat16, float16 or float32")
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    return make_desc(T, cu_seqlens.shape[0] - 1, Hq, Hkv, D, block_size, block_idx.shape[2],
                     scale, dtype, flags, stage_events)


class Workspace:
    """A reusable device workspace (grown on demand)."""

    def __init__(self, device=None):
        self.buf = None
        self.device = device

    def get(self, nbytes: int, device):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = None
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


def build_index(cu_seqlens, block_idx, num_kv_heads: int, block_size: int,
                total_tokens: Optional[int] = None, workspace: Optional[Workspace] = None):
    """Inverted index (offsets int32 [nb+1], entries int32 [max_entries]) on the device."""
    torch = _torch()
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _require(block_idx, "block_idx", torch.int32, 3)
    T = block_idx.shape[0] if total_tokens is None else total_tokens
    desc = make_desc(T, cu_seqlens.shape[0] - 1, num_kv_heads, num_kv_heads, 64, block_size,
                     block_idx.shape[2])
    nb, ne = index_sizes(desc)
    dev = block_idx.device
    offsets = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    entries = torch.empty(max(ne, 1), dtype=torch.int32, device=dev)
    nbytes = index_workspace_size(desc)
    ws = (workspace or Workspace()).get(nbytes, dev)
    rc = lib.nsa_sel_build_index(ctypes.byref(desc), cu_seqlens.data_ptr(), block_idx.data_ptr(),
                                 offsets.data_ptr(), entries.data_ptr(), ws.data_ptr(), ws.numel(),
                                 _stream_ptr(dev))
    _check(rc, "nsa_sel_build_index")
    return offsets, entries


def attn_fwd(q, k, v, cu_seqlens, block_idx, block_size: int, scale: Optional[float] = None,
             out=None, lse=None, workspace: Optional[Workspace] = None, dense_split: bool = False,
             stage_events=None):
    """Selected-block attention forward: returns (out [T,Hq,d], lse float32 [T,Hq]).

    dense_split=True computes the blocks every token of a token block keeps
    with the dense kernel (NSA_SEL_FLAG_DENSE_SPLIT, bf16); the result is the
    same up to rounding.
    """
    torch = _torch()
    _require(q, "q", q.dtype, 3)
    _require(k, "k", q.dtype, 3)
    _require(v, "v", q.dtype, 3)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _require(block_idx, "block_idx", torch.int32, 3)
    T, Hq, D = q.shape
    if k.shape[0] != T or v.shape != k.shape or k.shape[2] != D or block_idx.shape[0] != T \
            or block_idx.shape[1] != k.shape[1]:
        raise ValueError("shape mismatch between q, k, v and block_idx")
    desc = _desc_from(q, k, cu_seqlens, block_idx, block_size, scale,
                      FLAG_DENSE_SPLIT if dense_split else 0, stage_events)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    _require(out, "out", q.dtype, 3)
    _require(lse, "lse", torch.float32, 2)
    _check_out(out, lse, q)
    nbytes = fwd_workspace_size(desc)
    ws = (workspace or Workspace()).get(nbytes, dev)
    rc = lib.nsa_sel_attn_fwd(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              cu_seqlens.data_ptr(), block_idx.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    _check(rc, "nsa_sel_attn_fwd")
    return out, lse


def attn_fwd_indexed(q, k, v, cu_seqlens, block_idx, offsets, entries, block_size: int,
                     scale: Optional[float] = None, out=None, lse=None, workspace: Optional[Workspace] = None,
                     stage_events=None):
    """The forward on a prebuilt index (offsets, entries from build_index for
    the same cu_seqlens and block_idx): returns (out, lse), bitwise those of
    attn_fwd."""
    torch = _torch()
    for t, name in ((k, "k"), (v, "v")):
        _require(t, name, q.dtype, 3)
    _require(q, "q", q.dtype, 3)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _require(block_idx, "block_idx", torch.int32, 3)
    _require(offsets, "offsets", torch.int32, 1)
    _require(entries, "entries", torch.int32, 1)
    T, Hq, D = q.shape
    if k.shape[0] != T or v.shape != k.shape or k.shape[2] != D or block_idx.shape[0] != T \
            or block_idx.shape[1] != k.shape[1]:
        raise ValueError("shape mismatch between q, k, v and block_idx")
    desc = _desc_from(q, k, cu_seqlens, block_idx, block_size, scale, 0, stage_events)
    nb, ne = index_sizes(desc)
    if offsets.numel() < nb + 1 or entries.numel() < max(ne, 1):
        raise ValueError("offsets / entries smaller than nsa_sel_index_sizes gives")
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    _require(out, "out", q.dtype, 3)
    _require(lse, "lse", torch.float32, 2)
    _check_out(out, lse, q)
    nbytes = fwd_workspace_size(desc)
    ws = (workspace or Workspace()).get(nbytes, dev)
    rc = lib.nsa_sel_attn_fwd_indexed(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      cu_seqlens.data_ptr(), block_idx.data_ptr(), offsets.data_ptr(),
                                      entries.data_ptr(), out.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                                      ws.numel(), _stream_ptr(dev))
    _check(rc, "nsa_sel_attn_fwd_indexed")
    return out, lse


def attn_bwd(q, k, v, out, lse, dout, cu_seqlens, block_idx, block_size: int,
             scale: Optional[float] = None, dq=None, dk=None, dv=None,
             workspace: Optional[Workspace] = None, stage_events=None):
    """Selected-block attention backward (bf16 or fp16): returns (dq, dk, dv).

    out and lse are the forward's results for the same inputs; dout is the
    gradient of the loss with respect to out.
    """
    torch = _torch()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("the backward takes bfloat16 or float16 tensors")
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _require(t, name, q.dtype, 3)
    _require(lse, "lse", torch.float32, 2)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _require(block_idx, "block_idx", torch.int32, 3)
    T, Hq, D = q.shape
    if k.shape[0] != T or v.shape != k.shape or k.shape[2] != D or block_idx.shape[0] != T \
            or block_idx.shape[1] != k.shape[1] or out.shape != q.shape or dout.shape != q.shape \
            or tuple(lse.shape) != (T, Hq):
        raise ValueError("shape mismatch between q, k, v, out, lse, dout and block_idx")
    desc = _desc_from(q, k, cu_seqlens, block_idx, block_size, scale, 0, stage_events)
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", q.dtype, 3)
    _require(dk, "dk", q.dtype, 3)
    _require(dv, "dv", q.dtype, 3)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape or \
            any(t.device != q.device for t in (k, v, out, lse, dout, dq, dk, dv)):
        raise ValueError("gradient buffers must have the shapes of q, k and v, all on q's device")
    nbytes = bwd_workspace_size(desc)
    ws = (workspace or Workspace()).get(nbytes, dev)
    rc = lib.nsa_sel_attn_bwd(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                              cu_seqlens.data_ptr(), block_idx.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream_ptr(dev))
    _check(rc, "nsa_sel_attn_bwd")
    return dq, dk, dv


def window_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.nsa_sel_window_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "nsa_sel_window_workspace_size")
    return n.value


def window_fwd(q, k, v, cu_seqlens, window: int, scale: Optional[float] = None, tile: int = 64,
               out=None, lse=None, workspace: Optional[Workspace] = None, stage_events=None):
    """Sliding-window attention forward (bf16 or fp16): token i attends to the
    keys i - window < p <= i of its sequence.  Returns (out, lse float32)."""
    torch = _torch()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("the window branch takes bfloat16 or float16 tensors")
    _require(q, "q", q.dtype, 3)
    _require(k, "k", q.dtype, 3)
    _require(v, "v", q.dtype, 3)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, Hq, D = q.shape
    if k.shape[0] != T or v.shape != k.shape or k.shape[2] != D:
        raise ValueError("shape mismatch between q, k and v")
    dtype = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    desc = make_desc(T, cu_seqlens.shape[0] - 1, Hq, k.shape[1], D, tile, 1, scale, dtype, 0, stage_events)
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    _require(out, "out", q.dtype, 3)
    _require(lse, "lse", torch.float32, 2)
    _check_out(out, lse, q)
    ws = (workspace or Workspace()).get(window_workspace_size(desc), dev)
    rc = lib.nsa_sel_window_fwd(ctypes.byref(desc), int(window), q.data_ptr(), k.data_ptr(),
                                v.data_ptr(), cu_seqlens.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    _check(rc, "nsa_sel_window_fwd")
    return out, lse


def window_fwd_noalloc(q, k, v, cu_seqlens, window: int, out, lse, scale: Optional[float] = None,
                       tile: int = 64):
    """The sliding-window forward through nsa_sel_window_fwd_noalloc: no
    workspace and no allocation, in the library or here (out and lse are the
    caller's).  Calls that overlap on one GPU share the library's scratch."""
    torch = _torch()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("the window branch takes bfloat16 or float16 tensors")
    _require(q, "q", q.dtype, 3)
    _require(k, "k", q.dtype, 3)
    _require(v, "v", q.dtype, 3)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _require(out, "out", q.dtype, 3)
    _require(lse, "lse", torch.float32, 2)
    T, Hq, D = q.shape
    if k.shape[0] != T or v.shape != k.shape or k.shape[2] != D:
        raise ValueError("shape mismatch between q, k and v")
    _check_out(out, lse, q)
    dtype = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    desc = make_desc(T, cu_seqlens.shape[0] - 1, Hq, k.shape[1], D, tile, 1, scale, dtype)
    rc = lib.nsa_sel_window_fwd_noalloc(ctypes.byref(desc), int(window), q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), cu_seqlens.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                        _stream_ptr(q.device))
    _check(rc, "nsa_sel_window_fwd_noalloc")
    return out, lse


def select_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib.nsa_sel_select_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "nsa_sel_select_workspace_size")
    return n.value


def select_blocks(q, k, cu_seqlens, block_size: int = 64, topk: int = 16, scale: Optional[float] = None,
                  kernel_size: int = 32, kernel_stride: int = 16, init_blocks: int = 1,
                  local_blocks: int = 2, out=None, workspace: Optional[Workspace] = None, stage_events=None):
    """Index producer (bf16 or fp16): block lists [T, Hkv, topk] int32 from
    compressed attention -- init and local blocks first, then the blocks
    with the largest compressed-attention mass over the kv head's query
    heads.  The result feeds attn_fwd / attn_bwd as block_idx."""
    torch = _torch()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("the index producer takes bfloat16 or float16 tensors")
    _require(q, "q", q.dtype, 3)
    _require(k, "k", q.dtype, 3)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, Hq, D = q.shape
    if k.shape[0] != T or k.shape[2] != D:
        raise ValueError("shape mismatch between q and k")
    dtype = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    desc = make_desc(T, cu_seqlens.shape[0] - 1, Hq, k.shape[1], D, block_size, topk, scale, dtype, 0,
                     stage_events)
    dev = q.device
    out = torch.empty((T, k.shape[1], topk), dtype=torch.int32, device=dev) if out is None else out
    _require(out, "out", torch.int32, 3)
    if tuple(out.shape) != (T, k.shape[1], topk) or out.device != q.device:
        raise ValueError("out must be [T, Hkv, topk] on q's device")
    ws = (workspace or Workspace()).get(select_workspace_size(desc), dev)
    rc = lib.nsa_sel_select_blocks(ctypes.byref(desc), int(kernel_size), int(kernel_stride), int(init_blocks),
                                   int(local_blocks), q.data_ptr(), k.data_ptr(), cu_seqlens.data_ptr(),
                                   out.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    _check(rc, "nsa_sel_select_blocks")
    return out


def check(workspace: Workspace, device=None) -> int:
    """Synchronise and return the device's malformed-input bits of the last call."""
    st = ctypes.c_int()
    dev = workspace.buf.device
    rc = lib.nsa_sel_check(workspace.buf.data_ptr(), _stream_ptr(dev), ctypes.byref(st))
    if rc not in (OK, ERR_BAD_INPUT):
        _check(rc, "nsa_sel_check")
    return st.value


FWD_STAGES = ("index", "main", "dense", "merge")
BWD_STAGES = ("index", "delta", "main", "finish_dq_merge")
WIN_STAGES = ("prep", "window", "orphans", "none")
SEL_STAGES = ("prep", "compress", "select", "orphans")


class StageTimer:
    """Caller-owned HIP events for the stage boundaries of up to `calls`
    calls: pass ``timer.next()`` as a wrapper's ``stage_events`` (the library
    records them on its stream through the descriptor and keeps nothing), then
    ``timer.stage_ms(names)`` sums each stage's duration over the calls made.
    The events are torch's; torch creates one at its first record, so each is
    recorded once here before its handle is taken."""

    def __init__(self, calls: int, device=None):
        torch = _torch()
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        stream = torch.cuda.current_stream(dev)
        self.events = [[torch.cuda.Event(enable_timing=True) for _ in range(STAGE_EVENTS)]
                       for _ in range(calls)]
        for evs in self.events:
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize(dev)
        self.arrays = [(ctypes.c_void_p * STAGE_EVENTS)(*[e.cuda_event for e in evs]) for evs in self.events]
        self.used = 0

    def next(self):
        if self.used >= len(self.arrays):
            raise RuntimeError("StageTimer: more calls than events were made for")
        self.used += 1
        return self.arrays[self.used - 1]

    def stage_ms(self, names):
        """{stage name: summed ms over the calls made}; waits for the events."""
        tot = [0.0] * (STAGE_EVENTS - 1)
        for evs in self.events[:self.used]:
            evs[-1].synchronize()
            for i in range(STAGE_EVENTS - 1):
                tot[i] += evs[i].elapsed_time(evs[i + 1])
        return {n: tot[i] for i, n in enumerate(names)}

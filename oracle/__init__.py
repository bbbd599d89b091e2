"""Reference oracle for NSA selected-block attention -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over ``nsa_oracle.c``: plain double-precision CPU loops
written from the definition of selected-block attention (see the header of
``nsa_oracle.c`` for what is computed and which readings of the pages it
takes).  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package; the product path never does, and
this package imports nothing from the product package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB = os.path.join(_HERE, "libnsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into ``libnsa_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64, I32, F64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.nsa_oracle_fwd.argtypes = [I64, I32, P, I32, I32, I32, I32, I32, F64,
                                       P, P, P, P, I64, P, P, P]
        lib.nsa_oracle_fwd.restype = I32
        lib.nsa_oracle_invert.argtypes = [I64, I32, P, I32, I32, I32, P, I64, P, P]
        lib.nsa_oracle_invert.restype = I64
        lib.nsa_oracle_bwd.argtypes = [I64, I32, P, I32, I32, I32, I32, I32, F64,
                                       P, P, P, P, P, P, P, P]
        lib.nsa_oracle_bwd.restype = I32
        lib.nsa_oracle_bwd_dq_rows.argtypes = [I64, I32, P, I32, I32, I32, I32, I32, F64,
                                               P, P, P, P, P, I64, P, P]
        lib.nsa_oracle_bwd_dq_rows.restype = I32
        lib.nsa_oracle_bwd_dkv_blocks.argtypes = [I64, I32, P, I32, I32, I32, I32, I32, F64,
                                                  P, P, P, P, P, I64, P, P, P]
        lib.nsa_oracle_bwd_dkv_blocks.restype = I32
        lib.nsa_oracle_bwd_dkv_all.argtypes = [I64, I32, P, I32, I32, I32, I32, I32, F64,
                                               P, P, P, P, P, P, P, P, P]
        lib.nsa_oracle_bwd_dkv_all.restype = I32
        lib.nsa_oracle_window_fwd.argtypes = [I64, I32, P, I32, I32, I32, I32, F64,
                                              P, P, P, I64, P, P, P]
        lib.nsa_oracle_window_fwd.restype = I32
        lib.nsa_oracle_select.argtypes = [I64, I32, P, I32, I32, I32, I32, I32, I32, I32, I32, I32,
                                          F64, I32, P, P, I64, P, I32, P, P]
        lib.nsa_oracle_select.restype = I32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def nb_cap(total_tokens: int, block_size: int, num_seqs: int) -> int:
    """Upper bound on the number of blocks over all sequences: T // bs + B."""
    return total_tokens // block_size + num_seqs


def fwd(q, k, v, cu_seqlens, block_idx, block_size: int, scale: float,
        rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Selected-block attention forward in double precision.

    q [T, Hq, d], k/v [T, Hkv, d] (float32 values), cu_seqlens int32 [B+1],
    block_idx int32 [T, Hkv, topk].  Without ``rows`` returns out [T, Hq, d]
    and lse [T, Hq]; with ``rows`` (int64 ids t*Hkv + h) returns
    out [n, G, d] and lse [n, G] for just those rows.
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    cu, bi = _i32(cu_seqlens), _i32(block_idx)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    topk = bi.shape[2]
    G = Hq // Hkv
    if rows is None:
        out = np.empty((T, Hq, d), dtype=np.float64)
        lse = np.empty((T, Hq), dtype=np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.shape[0], G, d), dtype=np.float64)
        lse = np.empty((rows.shape[0], G), dtype=np.float64)
        rp, nr = _ptr(rows), rows.shape[0]
    rc = _load().nsa_oracle_fwd(T, cu.shape[0] - 1, _ptr(cu), Hq, Hkv, d, block_size,
                                topk, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(bi),
                                nr, rp, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle fwd: bad arguments")
    return out, lse


def invert(cu_seqlens, block_idx, num_kv_heads: int, block_size: int,
           total_tokens: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Per-block token lists as CSR: (offsets int64 [Hkv*nb_cap + 1], entries int32 [nnz])."""
    cu, bi = _i32(cu_seqlens), _i32(block_idx)
    T = bi.shape[0] if total_tokens is None else total_tokens
    topk = bi.shape[2]
    B = cu.shape[0] - 1
    cap = nb_cap(T, block_size, B)
    offsets = np.zeros(num_kv_heads * cap + 1, dtype=np.int64)
    entries = np.zeros(max(1, T * num_kv_heads * topk), dtype=np.int32)
    nnz = _load().nsa_oracle_invert(T, B, _ptr(cu), num_kv_heads, block_size, topk,
                                    _ptr(bi), cap, _ptr(offsets), _ptr(entries))
    if nnz < 0:
        raise ValueError("oracle invert: bad arguments")
    return offsets, entries[:nnz].copy()


def bwd(q, k, v, cu_seqlens, block_idx, dout, block_size: int, scale: float):
    """Gradients (dq [T,Hq,d], dk [T,Hkv,d], dv [T,Hkv,d]) in double precision."""
    q, k, v, do = _f32(q), _f32(k), _f32(v), _f32(dout)
    cu, bi = _i32(cu_seqlens), _i32(block_idx)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    dq = np.empty((T, Hq, d), dtype=np.float64)
    dk = np.empty((T, Hkv, d), dtype=np.float64)
    dv = np.empty((T, Hkv, d), dtype=np.float64)
    rc = _load().nsa_oracle_bwd(T, cu.shape[0] - 1, _ptr(cu), Hq, Hkv, d, block_size,
                                bi.shape[2], float(scale), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(bi), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle bwd: bad arguments")
    return dq, dk, dv


def bwd_dq_rows(q, k, v, cu_seqlens, block_idx, dout, block_size: int, scale: float, rows):
    """dq for rows t*Hkv + h (all G heads of each): [n, G, d], double precision."""
    q, k, v, do = _f32(q), _f32(k), _f32(v), _f32(dout)
    cu, bi = _i32(cu_seqlens), _i32(block_idx)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], Hq // Hkv, d), dtype=np.float64)
    rc = _load().nsa_oracle_bwd_dq_rows(T, cu.shape[0] - 1, _ptr(cu), Hq, Hkv, d, block_size,
                                        bi.shape[2], float(scale), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(bi), _ptr(do), rows.shape[0], _ptr(rows), _ptr(out))
    if rc != 0:
        raise ValueError("oracle bwd_dq_rows: bad arguments")
    return out


def bwd_dkv_blocks(q, k, v, cu_seqlens, block_idx, dout, block_size: int, scale: float, blocks):
    """dk, dv of the keys of blocks (h, s, j): each [n, block_size, d], double precision."""
    q, k, v, do = _f32(q), _f32(k), _f32(v), _f32(dout)
    cu, bi = _i32(cu_seqlens), _i32(block_idx)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    hsj = np.ascontiguousarray(blocks, dtype=np.int32).reshape(-1, 3)
    n = hsj.shape[0]
    dk = np.empty((n, block_size, d), dtype=np.float64)
    dv = np.empty((n, block_size, d), dtype=np.float64)
    rc = _load().nsa_oracle_bwd_dkv_blocks(T, cu.shape[0] - 1, _ptr(cu), Hq, Hkv, d, block_size,
                                           bi.shape[2], float(scale), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(bi), _ptr(do), n, _ptr(hsj), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle bwd_dkv_blocks: bad arguments")
    return dk, dv


def bwd_dkv_all(q, k, v, cu_seqlens, block_idx, dout, block_size: int, scale: float, lse, D):
    """dk, dv [T, Hkv, d] of every key, double precision, from each row's
    log-sum-exp and D = dout . out ([T, Hq], as ``fwd`` and its output give
    them); one thread per (kv head, sequence, key block)."""
    q, k, v, do = _f32(q), _f32(k), _f32(v), _f32(dout)
    cu, bi = _i32(cu_seqlens), _i32(block_idx)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    lse = np.ascontiguousarray(lse, dtype=np.float64).reshape(T, Hq)
    D = np.ascontiguousarray(D, dtype=np.float64).reshape(T, Hq)
    dk = np.empty((T, Hkv, d), dtype=np.float64)
    dv = np.empty((T, Hkv, d), dtype=np.float64)
    rc = _load().nsa_oracle_bwd_dkv_all(T, cu.shape[0] - 1, _ptr(cu), Hq, Hkv, d, block_size,
                                        bi.shape[2], float(scale), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(bi), _ptr(do), _ptr(lse), _ptr(D), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle bwd_dkv_all: bad arguments")
    return dk, dv


def window_fwd(q, k, v, cu_seqlens, window: int, scale: float,
               rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Sliding-window attention forward in double precision: token i attends to
    keys i - window < p <= i of its sequence.  Shapes as for ``fwd``."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    cu = _i32(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if rows is None:
        out = np.empty((T, Hq, d), dtype=np.float64)
        lse = np.empty((T, Hq), dtype=np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.shape[0], G, d), dtype=np.float64)
        lse = np.empty((rows.shape[0], G), dtype=np.float64)
        rp, nr = _ptr(rows), rows.shape[0]
    rc = _load().nsa_oracle_window_fwd(T, cu.shape[0] - 1, _ptr(cu), Hq, Hkv, d, int(window),
                                       float(scale), _ptr(q), _ptr(k), _ptr(v), nr, rp,
                                       _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle window_fwd: bad arguments")
    return out, lse


DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2}


def select(q, k, cu_seqlens, scale: float, dtype: str = "bf16", kernel_size: int = 32,
           kernel_stride: int = 16, block_size: int = 64, topk: int = 16, init_blocks: int = 1,
           local_blocks: int = 2, rows: Optional[np.ndarray] = None,
           with_importance: bool = False):
    """Block lists from compressed attention (see nsa_oracle_select in the C
    source for every step and reading).  q [T, Hq, d], k [T, Hkv, d] (values
    already in the input format, given as float32), dtype names that format
    (the compressed keys are rounded to it).  Returns block_idx [rows, topk]
    (or [T, Hkv, topk] when rows is None) and, if asked, the block importance
    [rows, nbmax] (-1 past the row's own block)."""
    q, k = _f32(q), _f32(k)
    cu = _i32(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    B = cu.shape[0] - 1
    nbmax = max([int((cu[s + 1] - cu[s] + block_size - 1) // block_size) for s in range(B)] + [1])
    if rows is None:
        n, rp = T * Hkv, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n, rp = rows.shape[0], _ptr(rows)
    bi = np.empty((max(n, 1), topk), dtype=np.int32)
    imp = np.empty((max(n, 1), nbmax), dtype=np.float64) if with_importance else None
    rc = _load().nsa_oracle_select(T, B, _ptr(cu), Hq, Hkv, d, kernel_size, kernel_stride,
                                   block_size, topk, init_blocks, local_blocks, float(scale),
                                   DTYPE_CODE[dtype], _ptr(q), _ptr(k), n if rows is not None else 0,
                                   rp, nbmax, _ptr(bi), _ptr(imp) if imp is not None else None)
    if rc != 0:
        raise ValueError("oracle select: bad arguments")
    bi = bi[:n]
    if rows is None:
        bi = bi.reshape(T, Hkv, topk)
    if with_importance:
        return bi, imp[:n]
    return bi

"""Seeded synthetic inputs for selected-block attention.

This module only draws inputs: Q/K/V values, ``cu_seqlens`` and the per-row
block-index lists.  It holds none of the attention arithmetic, none of the
index inversion and nothing of the GPU path, so the CPU oracle and the HIP
path can both be fed from it without sharing any of the method's code.

The workload shapes follow the Flash-Sparse-Attention project page
(agentlenshq, "Relaxed-System-Lab/Flash-Sparse-Attention", "Quick start":
``block_size=64``, ``topk=16``, one init block, two local blocks, ``head_dim``
128, a varlen batch of lengths 65536 and 32768 packed by ``cu_seqlens``).

Index rule for a token at local position ``i`` in block ``b = i // bs``:
the row is ``[0, b-1, b]`` followed by the seeded extra draws, negative ids
and later duplicates are dropped, the survivors are shifted left and the
row is padded with -1 to ``topk``.  Extra draws are distinct blocks from the
inclusive range ``[1, b-2]``; when that range holds fewer blocks than
requested, all of them are taken.

* ``uniform``: a uniformly random subset, drawn with Floyd's algorithm
  (one vectorised draw per step over all rows of a token block).
* ``zipf``: successive sampling without replacement from the truncated
  Zipf law P(r) ~ r**-a over ranks r = 1..b-2, rank r meaning block
  ``b-1-r`` (rank 1 is the most recent eligible block).  Drawn exactly with
  Gumbel-top-k on the log-weights (Kool, van Hoof and Welling, 2019).

Values are N(0, 1) (times ``value_scale``), drawn in the order q, k, v, then
the indices, then dO; bf16 configs round them to bfloat16 with
round-to-nearest-even and hand both sides the same rounded values.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
import os
from typing import Dict, List, Optional

import numpy as np

GEN_VERSION = 1


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seqlens: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    topk: int
    dtype: str            # "f32" or "bf16"
    seed: int
    value_scale: float = 1.0
    extra: str = "uniform"  # extra-draw law: "uniform" or "zipf"
    zipf_a: float = 1.1
    with_grad: bool = False  # draw dO as well (seed ``grad_seed``)
    grad_seed: int = 4
    description: str = ""

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def n_extra(self) -> int:
        return self.topk - 3


CONFIGS: Dict[str, Config] = {
    "c0": Config("c0", (1024,), 2, 1, 64, 64, 4, "f32", seed=0,
                 description="tiny fp32, T=1024, GQA group 2, d=64, block 64, topk 4"),
    "c1": Config("c1", (32768,), 4, 4, 128, 64, 16, "bf16", seed=1,
                 description="T=32768, 4 q / 4 kv heads, d=128, block 64, topk 16"),
    "c2": Config("c2", (65536, 32768), 32, 8, 128, 64, 16, "bf16", seed=2,
                 value_scale=0.5,
                 description="varlen [65536, 32768], 32 q / 8 kv heads (GQA-4), "
                             "d=128, block 64, topk 16"),
    "c3": Config("c3", (32768,), 64, 8, 128, 128, 8, "bf16", seed=3,
                 extra="zipf",
                 description="T=32768, 64 q / 8 kv heads (GQA-8), d=128, block 128, "
                             "topk 8, Zipf(1.1) recent-skewed extra blocks"),
    "c4": Config("c4", (65536, 32768), 32, 8, 128, 64, 16, "bf16", seed=2,
                 value_scale=0.5, with_grad=True, grad_seed=4,
                 description="c2 plus dO ~ N(0,1) for the backward pass"),
}


# ---------------------------------------------------------------------------
# bf16 helpers (storage format only: round-to-nearest-even of float32)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (RNE) and return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# index rows
# ---------------------------------------------------------------------------

def _floyd_uniform(rng: np.random.Generator, rows: int, n: int, k: int) -> np.ndarray:
    """k distinct values from 1..n per row (Floyd's subset algorithm)."""
    out = np.empty((rows, k), dtype=np.int64)
    for step, jj in enumerate(range(n - k + 1, n + 1)):
        r = rng.integers(1, jj + 1, size=rows)
        if step:
            seen = (out[:, :step] == r[:, None]).any(axis=1)
            r = np.where(seen, jj, r)
        out[:, step] = r
    return out


def _zipf_ranks(rng: np.random.Generator, rows: int, n: int, k: int, a: float) -> np.ndarray:
    """k distinct ranks from 1..n per row, successive sampling with P(r) ~ r**-a."""
    ranks = np.arange(1, n + 1, dtype=np.float64)
    logw = -a * np.log(ranks)
    u = rng.random((rows, n))
    # Gumbel(0,1) = -log(-log U); U == 0 has probability ~2**-53, clamp it.
    u = np.maximum(u, np.finfo(np.float64).tiny)
    keys = logw[None, :] - np.log(-np.log(u))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return order + 1


def _tidy_rows(rows: np.ndarray, topk: int) -> np.ndarray:
    """Drop negative ids and later duplicates, shift left, pad with -1."""
    out = np.full((rows.shape[0], topk), -1, dtype=np.int32)
    width = rows.shape[1]
    keep = rows >= 0
    for c in range(1, width):
        dup = (rows[:, :c] == rows[:, c:c + 1]).any(axis=1)
        keep[:, c] &= ~dup
    pos = np.cumsum(keep, axis=1) - 1
    r_idx, c_idx = np.nonzero(keep)
    out[r_idx, pos[r_idx, c_idx]] = rows[r_idx, c_idx]
    return out


def make_block_idx(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Block-index tensor int32 [T, H_kv, topk] for ``cfg`` (see module doc)."""
    T, H, bs, topk = cfg.total_tokens, cfg.num_kv_heads, cfg.block_size, cfg.topk
    k_extra = cfg.n_extra
    out = np.full((T, H, topk), -1, dtype=np.int32)
    start = 0
    for L in cfg.seqlens:
        nb = (L + bs - 1) // bs
        for b in range(nb):
            t0 = start + b * bs
            t1 = start + min((b + 1) * bs, L)
            rows = (t1 - t0) * H
            n = b - 2
            if n <= 0:
                extra = np.zeros((rows, 0), dtype=np.int64)
            elif n <= k_extra:
                extra = np.broadcast_to(np.arange(1, n + 1, dtype=np.int64), (rows, n))
                if cfg.extra == "zipf":  # rank order: most recent first
                    extra = np.broadcast_to(np.arange(n, 0, -1, dtype=np.int64), (rows, n))
            elif cfg.extra == "uniform":
                extra = _floyd_uniform(rng, rows, n, k_extra)
            elif cfg.extra == "zipf":
                extra = b - 1 - _zipf_ranks(rng, rows, n, k_extra, cfg.zipf_a)
            else:
                raise ValueError(cfg.extra)
            fixed = np.broadcast_to(np.array([0, b - 1, b], dtype=np.int64), (rows, 3))
            row = np.concatenate([fixed, extra], axis=1)
            out[t0:t1] = _tidy_rows(row, topk).reshape(t1 - t0, H, topk)
        start += L
    return out


# ---------------------------------------------------------------------------
# full input sets
# ---------------------------------------------------------------------------

def cu_seqlens_of(seqlens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(seqlens, dtype=np.int64))]).astype(np.int32)


def _normal(rng, shape, scale, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def _cache_dir() -> str:
    return os.environ.get(
        "NSA_INPUT_CACHE",
        os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_cache"))


def make_inputs(cfg, use_cache: bool = True) -> Dict[str, np.ndarray]:
    """Seeded inputs for a config (name or Config).

    Returns a dict with ``q``, ``k``, ``v`` (uint16 bf16 bit patterns for bf16
    configs, float32 otherwise), ``cu_seqlens`` int32 [B+1], ``block_idx``
    int32 [T, H_kv, topk] and, for gradient configs, ``do``.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    names = ["q", "k", "v", "block_idx"]
    key = repr((GEN_VERSION, cfg.seqlens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                cfg.block_size, cfg.topk, cfg.dtype, cfg.seed, cfg.value_scale, cfg.extra,
                cfg.zipf_a))
    cdir = os.path.join(_cache_dir(), hashlib.sha1(key.encode()).hexdigest()[:16])
    if use_cache and all(os.path.exists(os.path.join(cdir, n + ".npy")) for n in names):
        d = {n: np.load(os.path.join(cdir, n + ".npy")) for n in names}
    else:
        rng = np.random.default_rng(cfg.seed)
        T, Hq, Hk, D = cfg.total_tokens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
        d = {
            "q": _normal(rng, (T, Hq, D), cfg.value_scale, cfg.dtype),
            "k": _normal(rng, (T, Hk, D), cfg.value_scale, cfg.dtype),
            "v": _normal(rng, (T, Hk, D), cfg.value_scale, cfg.dtype),
        }
        d["block_idx"] = make_block_idx(cfg, rng)
        if use_cache and T >= 8192:
            os.makedirs(cdir, exist_ok=True)
            for n in names:
                np.save(os.path.join(cdir, n + ".npy"), d[n])
    d["cu_seqlens"] = cu_seqlens_of(cfg.seqlens)
    if cfg.with_grad:
        grng = np.random.default_rng(cfg.grad_seed)
        d["do"] = _normal(grng, (cfg.total_tokens, cfg.num_q_heads, cfg.head_dim), 1.0, cfg.dtype)
    return d


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 view of a value tensor as generated (exact for bf16)."""
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def rows_per_block_nnz(cfg: Config) -> int:
    """Closed-form count of kept (token, kv head, block) triples under the rule:
    a row in block b keeps min(b + 1, topk) blocks."""
    total = 0
    for L in cfg.seqlens:
        nb = (L + cfg.block_size - 1) // cfg.block_size
        for b in range(nb):
            ntok = min((b + 1) * cfg.block_size, L) - b * cfg.block_size
            total += ntok * min(b + 1, cfg.topk)
    return total * cfg.num_kv_heads


def effective_flops(cfg: Config, block_idx: Optional[np.ndarray] = None) -> int:
    """4*d FLOP per (query head, causally visible selected key).

    Without ``block_idx`` this uses the config rule (every kept block but the
    diagonal one is fully visible; the diagonal block shows i mod bs + 1 keys).
    """
    bs, topk, D, G = cfg.block_size, cfg.topk, cfg.head_dim, cfg.group
    keys = 0
    for L in cfg.seqlens:
        i = np.arange(L, dtype=np.int64)
        b = i // bs
        k_row = np.minimum(b + 1, topk)
        keys += int(((k_row - 1) * bs + (i % bs) + 1).sum())
    return 4 * D * G * keys * cfg.num_kv_heads

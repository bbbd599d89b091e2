"""Parity of the HIP sliding-window branch (through the C ABI) with the CPU
oracle: whole outputs on small ragged random shapes (bf16 and fp16, every
tile size and head dim, windows from 1 to longer than the sequence), sampled
rows of the 64K+32K GQA-4 workload at the quick-start window of 512, tokens
outside every sequence, and run-to-run determinism."""
import zlib

import numpy as np
import pytest

import nsa_selected_block_amd as nsa
import oracle
import workloads as W
from helpers import compare, f32_of, from_dev, random_case, to_dev

pytestmark = pytest.mark.gpu


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


# (seqlens, Hkv, G, D, tile, window, dtype)
SMALL = [
    ([300, 1, 0, 130], 2, 4, 128, 64, 100, "bf16"),
    ([700], 1, 2, 64, 32, 1, "bf16"),
    ([1000, 64], 2, 1, 128, 128, 512, "bf16"),
    ([257, 513], 1, 8, 64, 64, 17, "f16"),
    ([900], 2, 4, 128, 64, 5000, "f16"),
    ([2000, 3], 1, 16, 64, 128, 300, "bf16"),
    ([600, 70], 1, 4, 256, 64, 200, "bf16"),
    ([300], 2, 2, 256, 32, 1000, "f16"),
    ([900, 200], 1, 2, 256, 128, 300, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[6]}-G{c[2]}-d{c[3]}-t{c[4]}-w{c[5]}" for c in SMALL])
def test_window_small_random(case):
    import torch
    seqlens, Hkv, G, D, tile, window, dtype = case
    print(f"window small {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    d = random_case(rng, seqlens, Hkv, G, D, tile, 1, dtype)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    scale = 1.0 / np.sqrt(D)
    out, lse = nsa.window_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], window, scale, tile=tile)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.window_fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                                     window, scale)
    compare(from_dev(out), from_dev(lse), ref_o, ref_l, dtype, str(case))


@pytest.mark.parametrize("scale", [-0.11, 0.0])
def test_window_negative_and_zero_scale(scale):
    """A negative softmax scale (its sign goes into the query registers) and
    a zero one (uniform weights over the window)."""
    import torch
    rng = np.random.default_rng(21 if scale else 22)
    d = random_case(rng, [700, 130], 2, 4, 128, 64, 1, "bf16")
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    out, lse = nsa.window_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], 300, scale, tile=64)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.window_fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"], 300,
                                     scale)
    compare(from_dev(out), from_dev(lse), ref_o, ref_l, "bf16", f"scale {scale}")


def test_window_full_size_sampled():
    """seqlens [65536, 32768], 32 / 8 heads, d 128, bf16, window 512."""
    import torch
    cfg = W.CONFIGS["c2"]
    d = W.make_inputs(cfg)
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "v", "cu_seqlens")}
    out, lse = nsa.window_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], 512, cfg.scale, tile=64)
    out2, lse2 = nsa.window_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], 512, cfg.scale, tile=64)
    torch.cuda.synchronize()
    o, l = from_dev(out), from_dev(lse)
    assert np.array_equal(o, from_dev(out2)) and np.array_equal(l, from_dev(lse2))
    assert np.isfinite(o).all() and np.isfinite(l).all()
    rng = np.random.default_rng(300)
    toks = []
    for s, L in enumerate(cfg.seqlens):
        c0 = int(d["cu_seqlens"][s])
        toks += list(range(c0, c0 + 80)) + list(range(c0 + 500, c0 + 530)) + list(range(c0 + L - 40, c0 + L))
    toks += list(rng.choice(cfg.total_tokens, 400, replace=False))
    toks = np.unique(np.array(toks, dtype=np.int64))
    Hkv, G = cfg.num_kv_heads, cfg.group
    rows = (toks[:, None] * Hkv + np.arange(Hkv)[None, :]).reshape(-1)
    ref_o, ref_l = oracle.window_fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                                     512, cfg.scale, rows=rows)
    got_o = o.reshape(cfg.total_tokens, Hkv, G, cfg.head_dim)[rows // Hkv, rows % Hkv]
    got_l = l.reshape(cfg.total_tokens, Hkv, G)[rows // Hkv, rows % Hkv]
    compare(got_o, got_l, ref_o, ref_l, "bf16", f"window 512 sampled {rows.size} rows")


def test_window_full_size_whole():
    """Every element of out and lse of the window branch (window 512) on the
    64K+32K GQA-4 tensors, in the benchmark's launch configuration."""
    import torch
    cfg = W.CONFIGS["c2"]
    d = W.make_inputs(cfg)
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "v", "cu_seqlens")}
    out, lse = nsa.window_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], 512, cfg.scale, tile=64)
    torch.cuda.synchronize()
    o, l = from_dev(out), from_dev(lse)
    del out, lse, dd
    print("oracle: window forward of every row", flush=True)
    ref_o, ref_l = oracle.window_fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                                     512, cfg.scale)
    compare(o, l, ref_o, ref_l, "bf16", "window 512 every element")


def test_window_tokens_outside_sequences():
    import torch
    rng = np.random.default_rng(5)
    d = random_case(rng, [300], 2, 2, 64, 64, 1, "bf16")
    cu = d["cu_seqlens"].copy()
    cu[-1] = 200
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    ws = nsa.Workspace()
    out, lse = nsa.window_fwd(dd["q"], dd["k"], dd["v"], to_dev(cu, dev()), 64, 0.125, workspace=ws)
    assert nsa.check(ws) == 1
    o, l = from_dev(out), from_dev(lse)
    assert np.all(o[200:] == 0) and np.all(np.isneginf(l[200:]))
    ref_o, ref_l = oracle.window_fwd(f32_of(d["q"])[:200], f32_of(d["k"])[:200], f32_of(d["v"])[:200],
                                     cu, 64, 0.125)
    compare(o[:200], l[:200], ref_o, ref_l, "bf16", "window, shortened batch")

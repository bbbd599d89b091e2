"""Parity of the HIP backward (through the C ABI) with the CPU oracle.

* small ragged random shapes (every head_dim / block_size / group size the
  library supports, -1 / repeated / future / out-of-range ids): whole dq, dk,
  dv against the oracle's full fp64 backward;
* the 64K+32K GQA-4 workload with its dO (full size, the benchmark's launch
  configuration): every element of dq, dk and dv; and, as the fast tier, dq
  of more than 5% of the (token, kv head) rows and dk, dv of 264 key blocks
  -- among them the init block of every (sequence, kv head), which every
  token selects and whose rows span many workgroup ranges -- against the
  oracle's restricted backward, plus the column-sum identity
  sum_p dv_p = sum_r dout_r per kv head over every key;
* bitwise order invariance and run-to-run determinism, empty rows, keys no
  row attends to, tokens outside every sequence, zero tokens.

Tolerance: max-abs 5e-2 on every gradient element.
"""
import zlib

import numpy as np
import pytest

import nsa_selected_block_amd as nsa
import oracle
import workloads as W
from helpers import f32_of, from_dev, random_case, to_dev

pytestmark = pytest.mark.gpu

TOL_BWD = 5e-2


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def run_fb(dd, bs, scale, ws=None):
    """Forward, then backward with dd['do'], on the device."""
    import torch
    out, lse = nsa.attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], bs, scale,
                            workspace=ws)
    dq, dk, dv = nsa.attn_bwd(dd["q"], dd["k"], dd["v"], out, lse, dd["do"], dd["cu_seqlens"],
                              dd["block_idx"], bs, scale, workspace=ws)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def check(name, got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what} {name}: non-finite"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    mag = float(np.abs(ref).max()) if ref.size else 0.0
    print(f"{what} {name}: max-abs err {err:.3e} (max |ref| {mag:.3e}, tol {TOL_BWD})", flush=True)
    assert err <= TOL_BWD, f"{what} {name}: {err}"
    return err


def with_dout(d, rng):
    d = dict(d)
    x = rng.standard_normal(d["q"].shape, dtype=np.float32)
    d["do"] = x.astype(np.float16) if d["q"].dtype == np.float16 else W.f32_to_bf16_bits(x)
    return d


# (seqlens, Hkv, G, D, bs, topk, value scale)
SMALL = [
    ([1, 63, 64, 65, 200], 3, 1, 64, 32, 5, 1.0),
    ([0, 777, 0, 129], 2, 4, 128, 64, 17, 1.0),
    ([300, 1000], 1, 8, 128, 128, 6, 0.5),
    ([513, 900], 2, 2, 64, 64, 12, 1.0),
    ([1200], 2, 4, 128, 64, 16, 0.5),
    ([640, 64], 1, 16, 64, 128, 3, 1.0),
    ([250, 250, 250], 2, 2, 128, 32, 40, 1.0),
    ([0, 777, 0, 129], 2, 4, 128, 64, 17, 1.0, "f16"),
    ([513, 900], 2, 2, 64, 64, 12, 1.0, "f16"),
    ([300, 1000], 1, 8, 128, 128, 6, 0.5, "f16"),
    ([700, 130], 2, 4, 256, 64, 9, 1.0),
    ([300, 65, 0, 96], 1, 2, 256, 32, 7, 1.0, "f16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[7] if len(c) > 7 else 'bf16'}-G{c[2]}-d{c[3]}-bs{c[4]}-k{c[5]}"
                                             for c in SMALL])
def test_bwd_small_random(case):
    seqlens, Hkv, G, D, bs, topk, vs = case[:7]
    dtype = case[7] if len(case) > 7 else "bf16"
    print(f"bwd small {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    d = with_dout(random_case(rng, seqlens, Hkv, G, D, bs, topk, dtype, value_scale=vs), rng)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    scale = 1.0 / np.sqrt(D)
    _, _, dq, dk, dv = run_fb(dd, bs, scale)
    rq, rk, rv = oracle.bwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                            d["block_idx"], f32_of(d["do"]), bs, scale)
    check("dq", from_dev(dq), rq, str(case))
    check("dk", from_dev(dk), rk, str(case))
    check("dv", from_dev(dv), rv, str(case))


def test_bwd_structured_nsa_rule():
    """The workloads' own block rule (init + local + random blocks) on a small
    varlen batch: large buckets for the init block, small ones elsewhere."""
    cfg = W.Config("bwd-structured", (1500, 700), 8, 2, 128, 64, 16, "bf16", seed=77,
                   value_scale=0.5, with_grad=True, grad_seed=78, description="")
    d = W.make_inputs(cfg, use_cache=False)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    _, _, dq, dk, dv = run_fb(dd, cfg.block_size, cfg.scale)
    rq, rk, rv = oracle.bwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                            d["block_idx"], f32_of(d["do"]), cfg.block_size, cfg.scale)
    check("dq", from_dev(dq), rq, "structured")
    check("dk", from_dev(dk), rk, "structured")
    check("dv", from_dev(dv), rv, "structured")


_C4 = {}


def c4_results():
    """Inputs and the GPU's dq, dk, dv (host copies) of the 64K + 32K token,
    32 query / 8 kv head, d 128, block 64, topk 16 workload with dO."""
    import torch
    if not _C4:
        cfg = W.CONFIGS["c4"]
        print("bwd full size c4", flush=True)
        d = W.make_inputs(cfg)
        dd = {k: to_dev(a, dev()) for k, a in d.items()}
        _, _, dq, dk, dv = run_fb(dd, cfg.block_size, cfg.scale)
        _C4.update(cfg=cfg, d=d, dq=from_dev(dq), dk=from_dev(dk), dv=from_dev(dv))
        del dd, dq, dk, dv
        torch.cuda.empty_cache()
    return _C4


def test_bwd_full_size_dq_rows():
    """dq of more than 5% of the (token, kv head) rows -- every kv head of
    5,000 uniformly drawn tokens plus the first and last 40 tokens of each
    sequence -- and the column sums of dv over every key."""
    r = c4_results()
    cfg, d = r["cfg"], r["d"]
    T, Hkv, G, D, bs = cfg.total_tokens, cfg.num_kv_heads, cfg.group, cfg.head_dim, cfg.block_size
    q, k, v, do = (f32_of(d[n]) for n in ("q", "k", "v", "do"))
    cu, bi = d["cu_seqlens"], d["block_idx"]

    # every key: sum over keys of dv = sum over rows of dout (softmax rows sum to 1)
    lhs = r["dv"].astype(np.float64).sum(axis=0)                            # [Hkv, D]
    rhs = do.astype(np.float64).reshape(T, Hkv, G, D).sum(axis=(0, 2))      # [Hkv, D]
    err = float(np.abs(lhs - rhs).max())
    print(f"c4 column sums of dv: max-abs {err:.3e} (max |sum| {np.abs(rhs).max():.1f})", flush=True)
    assert err <= 0.5

    rng = np.random.default_rng(200)
    toks = []
    for s, L in enumerate(cfg.seqlens):
        c0 = int(cu[s])
        toks += list(range(c0, c0 + 40)) + list(range(c0 + L - 40, c0 + L))
    toks += list(rng.choice(T, 5000, replace=False))
    toks = np.unique(np.array(toks, dtype=np.int64))
    rows = (toks[:, None] * Hkv + np.arange(Hkv)[None, :]).reshape(-1)
    assert rows.size >= 0.05 * T * Hkv
    ref = oracle.bwd_dq_rows(q, k, v, cu, bi, do, bs, cfg.scale, rows)
    got = r["dq"].reshape(T, Hkv, G, D)[rows // Hkv, rows % Hkv]
    check("dq", got, ref, f"c4 sampled {rows.size} rows ({100.0 * rows.size / (T * Hkv):.1f}%)")


def test_bwd_full_size_dkv_blocks():
    """dk and dv of 264 key blocks: the init block of every (sequence, kv
    head) -- the largest buckets, every token of the sequence -- the last
    block of each, and 232 blocks drawn uniformly over heads, sequences and
    positions."""
    r = c4_results()
    cfg, d = r["cfg"], r["d"]
    bs = cfg.block_size
    q, k, v, do = (f32_of(d[n]) for n in ("q", "k", "v", "do"))
    cu, bi = d["cu_seqlens"], d["block_idx"]
    rng = np.random.default_rng(201)
    nbs = [L // bs for L in cfg.seqlens]
    blocks = [(h, s, 0) for h in range(cfg.num_kv_heads) for s in range(len(nbs))]
    blocks += [(h, s, nbs[s] - 1) for h in range(cfg.num_kv_heads) for s in range(len(nbs))]
    seen = set(blocks)
    while len(blocks) < 264:
        h = int(rng.integers(cfg.num_kv_heads))
        s = int(rng.integers(len(nbs)))
        j = int(rng.integers(1, nbs[s] - 1))
        if (h, s, j) not in seen:
            seen.add((h, s, j))
            blocks.append((h, s, j))
    print(f"oracle: dk, dv of {len(blocks)} key blocks", flush=True)
    rk, rv = oracle.bwd_dkv_blocks(q, k, v, cu, bi, do, bs, cfg.scale, blocks)
    idx = np.array([[int(cu[s]) + j * bs + p for p in range(bs)] for (h, s, j) in blocks])   # [n, bs]
    hh = np.array([h for (h, s, j) in blocks])[:, None]
    check("dk", r["dk"][idx, hh], rk, f"c4 {len(blocks)} key blocks")
    check("dv", r["dv"][idx, hh], rv, f"c4 {len(blocks)} key blocks")


@pytest.mark.parametrize("h", range(8), ids=[f"kv-head-{h}" for h in range(8)])
def test_bwd_full_size_whole(h):
    """Every element of dq, dk and dv at the 64K+32K GQA-4 workload with dO,
    one kv head per test (its G query heads, keys and values are a problem of
    their own): dq of every row of the head (the oracle's row entry point) and
    dk, dv of every key (its whole-output entry point, from the oracle
    forward's lse and D = dout . out of every row)."""
    r = c4_results()
    cfg, d = r["cfg"], r["d"]
    T, Hkv, G, D, bs = cfg.total_tokens, cfg.num_kv_heads, cfg.group, cfg.head_dim, cfg.block_size
    assert Hkv == 8
    qh = slice(h * G, (h + 1) * G)
    q = np.ascontiguousarray(f32_of(d["q"][:, qh]))
    do = np.ascontiguousarray(f32_of(d["do"][:, qh]))
    k = np.ascontiguousarray(f32_of(d["k"][:, h:h + 1]))
    v = np.ascontiguousarray(f32_of(d["v"][:, h:h + 1]))
    bi = np.ascontiguousarray(d["block_idx"][:, h:h + 1])
    cu = d["cu_seqlens"]
    print(f"oracle: kv head {h}, forward of every row (lse, D)", flush=True)
    out, lse = oracle.fwd(q, k, v, cu, bi, bs, cfg.scale)
    Drow = (out * do).sum(axis=2)
    del out
    print(f"oracle: kv head {h}, dk and dv of every key", flush=True)
    rk, rv = oracle.bwd_dkv_all(q, k, v, cu, bi, do, bs, cfg.scale, lse, Drow)
    check("dk", r["dk"][:, h:h + 1], rk, f"c4 kv head {h} every key")
    check("dv", r["dv"][:, h:h + 1], rv, f"c4 kv head {h} every key")
    del rk, rv
    print(f"oracle: kv head {h}, dq of every row", flush=True)
    rq = oracle.bwd_dq_rows(q, k, v, cu, bi, do, bs, cfg.scale, np.arange(T, dtype=np.int64))
    check("dq", r["dq"][:, qh], rq, f"c4 kv head {h} every row")


def test_bwd_order_invariance_and_determinism():
    rng = np.random.default_rng(61)
    d = with_dout(random_case(rng, [900, 400], 2, 4, 128, 64, 10, "bf16"), rng)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    r1 = [from_dev(x) for x in run_fb(dd, 64, 0.1)[2:]]
    r2 = [from_dev(x) for x in run_fb(dd, 64, 0.1)[2:]]
    assert all(np.array_equal(a, b) for a, b in zip(r1, r2))
    bi = d["block_idx"]
    perm = np.argsort(rng.random(bi.shape), axis=2)
    bi_p = np.take_along_axis(bi, perm, axis=2)
    bi_x = np.concatenate([bi_p, bi_p[:, :, :3], np.full_like(bi_p[:, :, :2], -1)], axis=2)
    dd["block_idx"] = to_dev(np.ascontiguousarray(bi_x), dev())
    r3 = [from_dev(x) for x in run_fb(dd, 64, 0.1)[2:]]
    assert all(np.array_equal(a, b) for a, b in zip(r1, r3))


def test_bwd_empty_rows_unselected_keys():
    rng = np.random.default_rng(71)
    d = with_dout(random_case(rng, [100, 0, 200], 1, 2, 64, 32, 3, "bf16"), rng)
    bi = d["block_idx"]
    bi[50:80] = -1         # no selection at all
    bi[150:160] = 99       # only future / out-of-range ids
    bi[:, :, :] = np.where(bi == 1, 2, bi)   # nobody selects block 1 of either sequence
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    _, _, dq, dk, dv = run_fb(dd, 32, 0.125)
    rq, rk, rv = oracle.bwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"], bi,
                            f32_of(d["do"]), 32, 0.125)
    dq, dk, dv = from_dev(dq), from_dev(dk), from_dev(dv)
    check("dq", dq, rq, "empty rows")
    check("dk", dk, rk, "empty rows")
    check("dv", dv, rv, "empty rows")
    assert np.all(dq[50:80] == 0)
    assert np.all(dk[32:64] == 0) and np.all(dv[32:64] == 0)      # block 1 of sequence 0
    assert np.all(dk[132:164] == 0) and np.all(dv[132:164] == 0)  # block 1 of sequence 2


def test_bwd_tokens_outside_sequences():
    """cu_seqlens ending before T: the trailing tokens get zero gradients; the
    rest match the oracle on the shortened batch."""
    import torch
    rng = np.random.default_rng(81)
    d = with_dout(random_case(rng, [300], 1, 2, 64, 64, 4, "bf16", junk=False), rng)
    d["block_idx"] = np.minimum(d["block_idx"], 3)
    cu_bad = d["cu_seqlens"].copy()
    cu_bad[-1] = 200
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    dd["cu_seqlens"] = to_dev(cu_bad, dev())
    # poison the outputs: every element must be written
    dq = torch.full_like(dd["q"], 7.0)
    dk = torch.full_like(dd["k"], 7.0)
    dv = torch.full_like(dd["v"], 7.0)
    ws = nsa.Workspace()
    out, lse = nsa.attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], 64, 0.125,
                            workspace=ws)
    nsa.attn_bwd(dd["q"], dd["k"], dd["v"], out, lse, dd["do"], dd["cu_seqlens"], dd["block_idx"],
                 64, 0.125, dq=dq, dk=dk, dv=dv, workspace=ws)
    assert nsa.check(ws) == 1
    dq, dk, dv = from_dev(dq), from_dev(dk), from_dev(dv)
    assert np.all(dq[200:] == 0) and np.all(dk[200:] == 0) and np.all(dv[200:] == 0)
    rq, rk, rv = oracle.bwd(f32_of(d["q"])[:200], f32_of(d["k"])[:200], f32_of(d["v"])[:200],
                            cu_bad, d["block_idx"][:200], f32_of(d["do"])[:200], 64, 0.125)
    check("dq", dq[:200], rq, "outside sequences")
    check("dk", dk[:200], rk, "outside sequences")
    check("dv", dv[:200], rv, "outside sequences")


def test_bwd_zero_tokens():
    import torch
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device=dev())
    cu = torch.zeros(2, dtype=torch.int32, device=dev())
    bi = torch.zeros((0, 2, 4), dtype=torch.int32, device=dev())
    lse = torch.zeros((0, 4), dtype=torch.float32, device=dev())
    dq, dk, dv = nsa.attn_bwd(z(0, 4, 64), z(0, 2, 64), z(0, 2, 64), z(0, 4, 64), lse, z(0, 4, 64),
                              cu, bi, 64, 0.125)
    torch.cuda.synchronize()
    assert dq.shape == (0, 4, 64) and dk.shape == (0, 2, 64) and dv.shape == (0, 2, 64)

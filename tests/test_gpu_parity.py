"""Parity of the HIP path (through the C ABI) with the CPU oracle.

* inverted index: bit-exact with the oracle's CSR on every workload, and
  bitwise identical from run to run;
* forward: element-wise max-abs against the oracle -- whole outputs on
  every workload (the tiny fp32 one, T=32K GQA-1, the 64K+32K GQA-4 one in
  the launch configuration the benchmark times and without the dense split,
  T=32K GQA-8 block 128 both ways) and on many small ragged random shapes;
  sampled rows and the softmax row sums as a faster tier at the two largest
  sizes;
* order invariance and run-to-run determinism (bitwise), empty rows, zero
  tokens, and the malformed-input report.
"""
import numpy as np
import pytest

import nsa_selected_block_amd as nsa
import oracle
import workloads as W
from helpers import compare, f32_of, from_dev, random_case, to_dev

pytestmark = pytest.mark.gpu

_CACHE = {}


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def cfg_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()  # hold one full-size workload at a time
        d = W.make_inputs(name)
        dd = {k: to_dev(a, dev()) for k, a in d.items()}
        _CACHE[name] = (d, dd)
    return _CACHE[name]


def run_fwd(dd, cfg_bs, scale, ws=None, dense=False):
    import torch
    out, lse = nsa.attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"],
                            cfg_bs, scale, workspace=ws, dense_split=dense)
    torch.cuda.synchronize()
    return out, lse


# ---------------------------------------------------------------------------
# index inversion
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c0", "c1", "c3", "c2"])
def test_index_bit_exact(name):
    import torch
    cfg = W.CONFIGS[name]
    print(f"index {name}", flush=True)
    d, dd = cfg_inputs(name)
    off, ent = nsa.build_index(dd["cu_seqlens"], dd["block_idx"], cfg.num_kv_heads, cfg.block_size)
    off2, ent2 = nsa.build_index(dd["cu_seqlens"], dd["block_idx"], cfg.num_kv_heads, cfg.block_size)
    torch.cuda.synchronize()
    off, ent, off2, ent2 = (x.cpu().numpy() for x in (off, ent, off2, ent2))
    ref_off, ref_ent = oracle.invert(d["cu_seqlens"], d["block_idx"], cfg.num_kv_heads,
                                     cfg.block_size)
    nnz = int(ref_off[-1])
    assert np.array_equal(off.astype(np.int64), ref_off)
    assert np.array_equal(ent[:nnz], ref_ent)
    assert np.array_equal(off, off2) and np.array_equal(ent[:nnz], ent2[:nnz])


def test_index_random_ragged():
    rng = np.random.default_rng(21)
    for seqlens, Hkv, bs, topk in [([1, 63, 64, 65, 200], 3, 32, 5), ([0, 777, 0, 129], 2, 64, 17),
                                   ([5000, 3], 1, 128, 40)]:
        d = random_case(rng, seqlens, Hkv, 1, 64, bs, topk, "f32")
        cu, bi = to_dev(d["cu_seqlens"], dev()), to_dev(d["block_idx"], dev())
        off, ent = nsa.build_index(cu, bi, Hkv, bs)
        ref_off, ref_ent = oracle.invert(d["cu_seqlens"], d["block_idx"], Hkv, bs)
        nnz = int(ref_off[-1])
        assert np.array_equal(off.cpu().numpy().astype(np.int64), ref_off)
        assert np.array_equal(ent.cpu().numpy()[:nnz], ref_ent)


def test_index_and_fwd_beyond_one_lds_window():
    """A sequence of more than 12,288 blocks of 64 (the buckets one LDS pass
    of the index build covers): the count and scatter walk the buckets in
    windows.  The index is bit-exact with the oracle's, and sampled rows of
    the forward (many of them late in the long sequence, whose blocks sit in
    the second window) match it, with and without the dense split."""
    import torch
    rng = np.random.default_rng(31)
    seqlens = [16384 * 64 + 777, 5000]
    Hkv, G, D, bs, topk = 1, 2, 64, 64, 6
    print(f"index and forward beyond one LDS window: {seqlens}", flush=True)
    d = random_case(rng, seqlens, Hkv, G, D, bs, topk, "bf16")
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    off, ent = nsa.build_index(dd["cu_seqlens"], dd["block_idx"], Hkv, bs)
    torch.cuda.synchronize()
    off, ent = off.cpu().numpy(), ent.cpu().numpy()
    ref_off, ref_ent = oracle.invert(d["cu_seqlens"], d["block_idx"], Hkv, bs)
    nnz = int(ref_off[-1])
    assert np.array_equal(off.astype(np.int64), ref_off)
    assert np.array_equal(ent[:nnz], ref_ent)
    T = int(d["cu_seqlens"][-1])
    rows = np.unique(np.concatenate([rng.integers(0, T * Hkv, 1500),
                                     rng.integers(800000 * Hkv, (16384 * 64 + 777) * Hkv, 1500),
                                     np.arange(T * Hkv - 200, T * Hkv)])).astype(np.int64)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                              d["block_idx"], bs, 1.0 / np.sqrt(D), rows=rows)
    sel = (rows // Hkv, rows % Hkv)
    for dense in (False, True):
        out, lse = run_fwd(dd, bs, 1.0 / np.sqrt(D), dense=dense)
        got_o = from_dev(out).reshape(T, Hkv, G, D)[sel]
        got_l = lse.cpu().numpy().reshape(T, Hkv, G)[sel]
        compare(got_o, got_l, ref_o, ref_l, "bf16", f"long sequence, dense split {dense}")
        del out, lse


# ---------------------------------------------------------------------------
# forward: whole outputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c0", "c1"])
def test_fwd_full(name):
    cfg = W.CONFIGS[name]
    print(f"fwd full {name}", flush=True)
    d, dd = cfg_inputs(name)
    out, lse = run_fwd(dd, cfg.block_size, cfg.scale)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                              d["block_idx"], cfg.block_size, cfg.scale)
    compare(from_dev(out), from_dev(lse), ref_o, ref_l, cfg.dtype, name)


def test_fwd_full_c1_dense_split():
    """Every element of the 32K MHA workload in the benchmark's configuration
    (dense split, the merge inside the dense kernel, four rows per wave)."""
    cfg = W.CONFIGS["c1"]
    print("fwd full c1 dense split", flush=True)
    d, dd = cfg_inputs("c1")
    out, lse = run_fwd(dd, cfg.block_size, cfg.scale, dense=True)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                              d["block_idx"], cfg.block_size, cfg.scale)
    compare(from_dev(out), from_dev(lse), ref_o, ref_l, cfg.dtype, "c1 dense split")


SMALL = [
    # seqlens, Hkv, G, D, bs, topk, dtype
    ([1000], 1, 2, 64, 64, 4, "f32"),
    ([130, 1, 0, 257, 64], 2, 3, 64, 32, 5, "f32"),
    ([333, 1025], 2, 1, 128, 128, 7, "f32"),
    ([1000, 700], 2, 4, 128, 64, 6, "bf16"),
    ([129, 1, 0, 511, 64, 65], 3, 1, 128, 32, 9, "bf16"),
    ([2047], 1, 8, 128, 128, 8, "bf16"),
    ([700, 300], 2, 16, 64, 64, 5, "bf16"),
    ([1500], 1, 5, 64, 32, 33, "bf16"),
    ([3000, 17], 2, 64, 128, 64, 3, "bf16"),
    ([4100], 1, 4, 128, 64, 64, "bf16"),
    ([1000, 700], 2, 4, 128, 64, 6, "f16"),
    ([129, 1, 0, 511, 64, 65], 3, 2, 64, 32, 9, "f16"),
    ([2047], 1, 8, 128, 128, 8, "f16"),
    ([900, 130], 2, 2, 256, 64, 7, "bf16"),
    ([513, 1, 64], 1, 4, 256, 32, 9, "f16"),
    ([1200], 1, 1, 256, 64, 16, "bf16"),
    # d = 256 with 128-key blocks (the main kernel's output tile in 4-row passes)
    ([1400, 300], 2, 2, 256, 128, 6, "bf16"),
    ([700, 129], 1, 4, 256, 128, 9, "f16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[6]}-G{c[2]}-d{c[3]}-bs{c[4]}-k{c[5]}" for c in SMALL])
def test_fwd_small_random(case):
    seqlens, Hkv, G, D, bs, topk, dtype = case
    print(f"fwd small {case}", flush=True)
    rng = np.random.default_rng(sum(seqlens) + 7 * topk + G)
    d = random_case(rng, seqlens, Hkv, G, D, bs, topk, dtype)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    scale = 1.0 / np.sqrt(D)
    out, lse = run_fwd(dd, bs, scale)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                              d["block_idx"], bs, scale)
    compare(from_dev(out), from_dev(lse), ref_o, ref_l, dtype, str(case))


STRUCTURED = [
    # seqlens, Hkv, G, D, bs, topk, extra law[, dtype]
    ((1000, 777, 64, 1), 2, 4, 128, 64, 8, "uniform"),
    ((2100, 130), 1, 8, 128, 128, 6, "zipf"),
    ((900,), 2, 1, 64, 32, 16, "uniform"),
    ((1500, 33), 1, 16, 64, 64, 5, "uniform"),
    ((1300, 400), 2, 4, 128, 64, 10, "uniform", "f16"),
    ((1000, 300), 2, 4, 256, 64, 8, "uniform"),
    ((800, 333), 2, 2, 256, 32, 7, "uniform"),
    ((1300, 260), 2, 4, 256, 128, 5, "zipf"),
    ((700, 450), 1, 8, 64, 64, 9, "zipf", "f16"),
    # rows narrower than a wave: the merges take 4 (G 1) or 2 (G 2) rows per wave
    ((1000, 300, 65), 2, 1, 128, 64, 12, "uniform"),
    ((900, 200), 2, 2, 128, 64, 16, "zipf", "f16"),
    # G not dividing 16: the dense partial goes through the separate merge
    ((700, 300), 2, 3, 64, 64, 6, "uniform"),
    ((500, 90), 1, 32, 64, 32, 4, "uniform"),
]


@pytest.mark.parametrize("dense", [True, False], ids=["dense-split", "gather-only"])
@pytest.mark.parametrize("case", STRUCTURED, ids=[f"G{c[2]}-d{c[3]}-bs{c[4]}-k{c[5]}-{c[6]}" for c in STRUCTURED])
def test_fwd_structured_dense_split(case, dense):
    """Rows built with the workloads' index rule (init + local + extra
    blocks), ragged lengths, and token blocks where one token drops a block,
    so the blocks kept by a whole token block are sometimes a strict subset."""
    seqlens, Hkv, G, D, bs, topk, law = case[:7]
    dtype = case[7] if len(case) > 7 else "bf16"
    print(f"fwd structured {case} dense={dense}", flush=True)
    cfg = W.Config("t", tuple(seqlens), Hkv * G, Hkv, D, bs, topk, "bf16", seed=5, extra=law)
    rng = np.random.default_rng(9)
    d = random_case(rng, list(seqlens), Hkv, G, D, bs, topk, dtype)
    bi = W.make_block_idx(cfg, rng)
    T = bi.shape[0]
    # perturb: in some token blocks one token loses its first slot (block 0)
    for t in rng.choice(T, size=max(1, T // 40), replace=False):
        bi[t, rng.integers(Hkv), 0] = -1
    d["block_idx"] = bi
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    scale = 1.0 / np.sqrt(D)
    out, lse = run_fwd(dd, bs, scale, dense=dense)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"], bi, bs, scale)
    compare(from_dev(out), from_dev(lse), ref_o, ref_l, dtype, f"{case} dense={dense}")
    # bitwise order invariance with the dense split in play
    perm = np.argsort(rng.random(bi.shape), axis=2)
    dd["block_idx"] = to_dev(np.ascontiguousarray(np.take_along_axis(bi, perm, axis=2)), dev())
    out2, lse2 = run_fwd(dd, bs, scale, dense=dense)
    assert np.array_equal(from_dev(out), from_dev(out2)) and np.array_equal(from_dev(lse), from_dev(lse2))


def test_fwd_dense_split_tokens_outside_sequences():
    """Dense split (the dense kernel merging its tokens) with tokens past the
    last sequence: those rows are 0 with lse -inf, the rest match the oracle."""
    Hkv, G, D, bs, topk = 2, 4, 64, 64, 6
    cfg = W.Config("t", (600, 200, 200), Hkv * G, Hkv, D, bs, topk, "bf16", seed=5, extra="uniform")
    rng = np.random.default_rng(21)
    d = random_case(rng, [600, 200, 200], Hkv, G, D, bs, topk, "bf16")
    d["block_idx"] = W.make_block_idx(cfg, rng)
    d["cu_seqlens"] = np.array([0, 600, 800], np.int32)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    out, lse = run_fwd(dd, bs, 0.125, dense=True)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"], d["block_idx"],
                              bs, 0.125)
    o, l = from_dev(out), from_dev(lse)
    assert np.all(o[800:] == 0) and np.all(l[800:] == -np.inf)
    # (the oracle's contract has cu_seqlens end at T: its rows past 800 are not defined)
    compare(o[:800], l[:800], ref_o[:800], ref_l[:800], "bf16", "dense split, tokens outside sequences")


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_fwd_dense_split_negative_and_zero_scale(scale):
    """The dense kernel folds the scale into its exponents (a negative one's
    sign into the query registers); the gather path multiplies: both against
    the oracle with a negative and a zero scale."""
    seqlens, Hkv, G, D, bs, topk = (1000, 200), 2, 4, 128, 64, 8
    cfg = W.Config("t", seqlens, Hkv * G, Hkv, D, bs, topk, "bf16", seed=5, extra="uniform")
    rng = np.random.default_rng(31)
    d = random_case(rng, list(seqlens), Hkv, G, D, bs, topk, "bf16")
    d["block_idx"] = W.make_block_idx(cfg, rng)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"], d["block_idx"],
                              bs, scale)
    for dense in (True, False):
        out, lse = run_fwd(dd, bs, scale, dense=dense)
        compare(from_dev(out), from_dev(lse), ref_o, ref_l, "bf16", f"scale {scale} dense={dense}")


# ---------------------------------------------------------------------------
# forward: whole outputs of the full-size workloads
# ---------------------------------------------------------------------------

_ORACLE = {}


def oracle_whole(name):
    """The oracle's out / lse of every row of a workload (one held at a time)."""
    if name not in _ORACLE:
        _ORACLE.clear()
        cfg = W.CONFIGS[name]
        d, _ = cfg_inputs(name)
        print(f"oracle, whole {name} ...", flush=True)
        _ORACLE[name] = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                                   d["block_idx"], cfg.block_size, cfg.scale)
    return _ORACLE[name]


@pytest.mark.parametrize("name,dense", [("c2", True), ("c2", False), ("c3", True), ("c3", False)],
                         ids=["c2-dense-split", "c2-gather-only", "c3-dense-split", "c3-gather-only"])
def test_fwd_full_size_whole(name, dense):
    """Every element of out and lse at the 64K+32K GQA-4 and the 32K GQA-8
    block-128 workloads, with and without the dense split, against the
    oracle's whole result."""
    cfg = W.CONFIGS[name]
    print(f"fwd whole {name} dense={dense}", flush=True)
    d, dd = cfg_inputs(name)
    out, lse = run_fwd(dd, cfg.block_size, cfg.scale, dense=dense)
    out_h, lse_h = from_dev(out), from_dev(lse)
    del out, lse
    ref_o, ref_l = oracle_whole(name)
    compare(out_h, lse_h, ref_o, ref_l, cfg.dtype, f"{name} dense={dense} every element")


# ---------------------------------------------------------------------------
# forward: full-size workloads, sampled rows + properties of every row
# ---------------------------------------------------------------------------

def sample_tokens(cfg, rng, n_random=600):
    toks = []
    start = 0
    for L in cfg.seqlens:
        toks += list(range(start, start + 70))                    # first blocks (dense)
        toks += list(range(start + 1000, start + 1100))           # end of the dense prefix
        toks += list(range(start + L - 70, start + L))            # last block
        start += L
    toks += list(rng.choice(cfg.total_tokens, n_random, replace=False))
    return np.unique(np.array(toks, dtype=np.int64))


@pytest.mark.parametrize("name,dense", [("c2", False), ("c2", True), ("c3", False), ("c3", True)])
def test_fwd_full_size_sampled(name, dense):
    cfg = W.CONFIGS[name]
    print(f"fwd sampled {name} dense={dense}", flush=True)
    d, dd = cfg_inputs(name)
    out, lse = run_fwd(dd, cfg.block_size, cfg.scale, dense=dense)
    out_h, lse_h = from_dev(out), from_dev(lse)
    assert np.isfinite(out_h).all() and np.isfinite(lse_h).all()
    rng = np.random.default_rng(100)
    toks = sample_tokens(cfg, rng)
    Hkv, G = cfg.num_kv_heads, cfg.group
    rows = (toks[:, None] * Hkv + np.arange(Hkv)[None, :]).reshape(-1)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"],
                              d["block_idx"], cfg.block_size, cfg.scale, rows=rows)
    got_o = out_h.reshape(cfg.total_tokens, Hkv, G, cfg.head_dim)[rows // Hkv, rows % Hkv]
    got_l = lse_h.reshape(cfg.total_tokens, Hkv, G)[rows // Hkv, rows % Hkv]
    compare(got_o, got_l, ref_o, ref_l, cfg.dtype, f"{name} dense={dense} sampled {rows.size} rows")
    # softmax rows sum to one under the GPU's own lse (recomputed scores)
    q, k = f32_of(d["q"]), f32_of(d["k"])
    bs = cfg.block_size
    cu = d["cu_seqlens"]
    for t in toks[::25]:
        s = int(np.searchsorted(cu, t, side="right") - 1)
        i = int(t - cu[s])
        for h in range(Hkv):
            ids = {int(j) for j in d["block_idx"][t, h] if 0 <= j <= i // bs}
            keys = np.array([int(cu[s]) + p for j in sorted(ids) for p in range(j * bs, min((j + 1) * bs, i + 1))])
            for g in range(G):
                sc = cfg.scale * (k[keys, h].astype(np.float64) @ q[t, h * G + g].astype(np.float64))
                total = np.exp(sc - lse_h[t, h * G + g]).sum()
                assert abs(total - 1.0) <= 2e-3, (t, h, g, total)


# ---------------------------------------------------------------------------
# invariances, determinism, edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_order_invariance_and_determinism(dtype):
    rng = np.random.default_rng(31)
    d = random_case(rng, [900, 400], 2, 4, 128, 64, 10, dtype)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    out1, lse1 = run_fwd(dd, 64, 0.1)
    out2, lse2 = run_fwd(dd, 64, 0.1)
    assert np.array_equal(from_dev(out1), from_dev(out2)) and np.array_equal(from_dev(lse1), from_dev(lse2))
    bi = d["block_idx"]
    perm = np.argsort(rng.random(bi.shape), axis=2)
    bi_p = np.take_along_axis(bi, perm, axis=2)
    # also add repeats and -1: same selection
    bi_x = np.concatenate([bi_p, bi_p[:, :, :3], np.full_like(bi_p[:, :, :2], -1)], axis=2)
    dd["block_idx"] = to_dev(np.ascontiguousarray(bi_x), dev())
    out3, lse3 = run_fwd(dd, 64, 0.1)
    assert np.array_equal(from_dev(out1), from_dev(out3)) and np.array_equal(from_dev(lse1), from_dev(lse3))


def test_empty_rows_and_sequences():
    rng = np.random.default_rng(41)
    d = random_case(rng, [100, 0, 200], 1, 2, 64, 32, 3, "bf16")
    bi = d["block_idx"]
    bi[50:80] = -1         # no selection at all
    bi[150:160] = 99       # only future / out-of-range ids
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    out, lse = run_fwd(dd, 32, 0.125)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"], bi,
                              32, 0.125)
    o, l = from_dev(out), from_dev(lse)
    compare(o, l, ref_o, ref_l, "bf16", "empty rows")
    assert np.all(o[50:80] == 0) and np.all(np.isneginf(l[50:80]))


def test_zero_tokens():
    import torch
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device=dev())
    cu = torch.zeros(2, dtype=torch.int32, device=dev())
    bi = torch.zeros((0, 2, 4), dtype=torch.int32, device=dev())
    out, lse = run_fwd(dict(q=z(0, 4, 64), k=z(0, 2, 64), v=z(0, 2, 64), cu_seqlens=cu, block_idx=bi),
                       64, 0.125)
    assert out.shape == (0, 4, 64) and lse.shape == (0, 4)


def test_check_reports_malformed_input():
    rng = np.random.default_rng(51)
    d = random_case(rng, [300], 1, 2, 64, 64, 4, "f32", junk=False)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    ws = nsa.Workspace()
    run_fwd(dd, 64, 0.125, ws)
    assert nsa.check(ws) == 0
    bi = d["block_idx"].copy()
    bi[10, 0, 1] = 1000   # beyond the sequence's blocks: ignored, reported
    bi[11, 0, 2] = -7
    dd["block_idx"] = to_dev(bi, dev())
    out, lse = run_fwd(dd, 64, 0.125, ws)
    assert nsa.check(ws) == 2
    ref_o, ref_l = oracle.fwd(d["q"], d["k"], d["v"], d["cu_seqlens"], bi, 64, 0.125)
    compare(from_dev(out), from_dev(lse), ref_o, ref_l, "f32", "malformed ids")
    cu_bad = d["cu_seqlens"].copy()
    cu_bad[-1] = 200      # does not end at T: tokens 200..299 belong to no sequence
    dd["cu_seqlens"] = to_dev(cu_bad, dev())
    # ids stay below the 4 blocks the shortened sequence has, so only the
    # cu_seqlens bit is expected
    dd["block_idx"] = to_dev(np.minimum(d["block_idx"], 3), dev())
    out, lse = run_fwd(dd, 64, 0.125, ws)
    assert nsa.check(ws) == 1
    o, l = from_dev(out), from_dev(lse)
    assert np.all(o[200:] == 0) and np.all(np.isneginf(l[200:]))

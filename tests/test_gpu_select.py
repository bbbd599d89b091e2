"""Parity of the HIP index producer (block lists from compressed attention)
with the CPU oracle, through the C ABI.

The lists are integers decided by floating point: the compressed keys are
the same bits on both sides (fp32 sums in position order, rounded to the
input format), but the GPU's compressed-attention probabilities are fp32
(MFMA products of 16-bit values, exact, accumulated in fp32; exp2 / log2 of
a few ulp; sums of at most 5 G terms per block), the oracle's double.  Their relative difference
stays below 1e-4 of the row's largest importance, so:
  - the forced prefix (init and local blocks) and the -1 padding are
    compared bit for bit;
  - the chosen blocks are compared as sets; where the sets differ, every
    block only one side chose must be a near-tie under the oracle's
    importance: within TIE = 2e-4 of the row's largest importance of the
    boundary between chosen and not chosen, and such rows must be rare.
The lists then drive the selected-attention forward, checked against the
oracle on the same lists."""
import zlib

import numpy as np
import pytest

import nsa_selected_block_amd as nsa
import oracle
import workloads as W
from helpers import compare, f32_of, from_dev, random_case, to_dev

pytestmark = pytest.mark.gpu

TIE = 2e-4


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def own_blocks(rows, Hkv, cu, bs):
    """b = i / bs of each row's token (rows r = t * Hkv + h)."""
    t = np.asarray(rows) // Hkv
    s = np.searchsorted(np.asarray(cu), t, side="right") - 1
    return (t - np.asarray(cu)[s]) // bs


def check_lists(got, ref, imp, bown, init, local, what, max_diff_frac=0.01):
    """got / ref: [rows, topk] lists, imp: the oracle's importance per row,
    bown: each row's own block b."""
    n_rows = got.shape[0]
    ndiff = 0
    for r in range(n_rows):
        g, o = got[r], ref[r]
        nf = int(np.sum(o >= 0))
        assert np.all(g[nf:] == -1) and np.all(g[:nf] >= 0), f"{what} row {r}: {g} vs {o}"
        # forced prefix: the ids the oracle lists before any importance choice
        b = int(bown[r])
        forced = [j for j in range(init) if j <= b]
        forced += [b - u for u in range(local) if b - u >= 0 and b - u not in forced]
        nfz = min(len(forced), nf)
        assert np.array_equal(g[:nfz], o[:nfz]), f"{what} row {r}: forced {g[:nfz]} vs {o[:nfz]}"
        gs, os_ = set(g[nfz:nf].tolist()), set(o[nfz:nf].tolist())
        assert len(gs) == nf - nfz and not (gs & set(forced)), f"{what} row {r}: repeats {g}"
        if gs == os_:
            continue
        ndiff += 1
        scale = float(np.max(imp[r][: b + 1])) if b >= 0 else 1.0
        only_g, only_o = gs - os_, os_ - gs
        # the oracle's cut lies between its weakest chosen and strongest unchosen block
        cut_lo = min(imp[r][j] for j in os_)
        for j in only_g:
            assert imp[r][j] >= cut_lo - TIE * scale, f"{what} row {r}: {j} far below the cut"
        cut_g = min(imp[r][x] for x in gs)
        for j in only_o:
            assert imp[r][j] <= cut_g + TIE * scale, f"{what} row {r}: {j} far above the cut"
    assert ndiff <= max(1, max_diff_frac * n_rows), f"{what}: {ndiff} of {n_rows} rows differ"
    return ndiff


# (seqlens, Hkv, G, d, dtype, topk, init, local)
SMALL = [
    ([1000, 77, 0, 640], 2, 4, 128, "bf16", 16, 1, 2),
    ([700], 1, 1, 64, "bf16", 8, 1, 2),
    ([1500, 31, 32], 1, 2, 128, "f16", 5, 1, 2),
    ([1200], 2, 8, 64, "bf16", 33, 2, 1),
    ([900, 400], 1, 16, 128, "bf16", 12, 0, 3),
    ([2100], 1, 4, 64, "f16", 16, 1, 0),
    # no forced ids: a full 16-slot list (four-register lists) and a 15-slot one
    ([1800, 300], 1, 4, 128, "bf16", 16, 0, 0),
    ([1100], 2, 2, 64, "bf16", 15, 0, 0),
    # the largest list
    ([2600], 1, 4, 64, "bf16", 64, 1, 2),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[4]}-G{c[2]}-d{c[3]}-k{c[5]}-i{c[6]}l{c[7]}" for c in SMALL])
def test_select_small_random(case):
    import torch
    seqlens, Hkv, G, D, dtype, topk, init, local = case
    print(f"select small {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    d = random_case(rng, seqlens, Hkv, G, D, 64, topk, dtype)
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "cu_seqlens")}
    scale = 1.0 / np.sqrt(D)
    got = nsa.select_blocks(dd["q"], dd["k"], dd["cu_seqlens"], 64, topk, scale, init_blocks=init,
                            local_blocks=local)
    got2 = nsa.select_blocks(dd["q"], dd["k"], dd["cu_seqlens"], 64, topk, scale, init_blocks=init,
                             local_blocks=local)
    torch.cuda.synchronize()
    got, got2 = got.cpu().numpy(), got2.cpu().numpy()
    assert np.array_equal(got, got2), "not reproducible"
    ref, imp = oracle.select(f32_of(d["q"]), f32_of(d["k"]), d["cu_seqlens"], scale, dtype, topk=topk,
                             init_blocks=init, local_blocks=local, with_importance=True)
    T = got.shape[0]
    cu = d["cu_seqlens"]
    valid = np.arange(T * Hkv) // Hkv < cu[-1]
    nd = check_lists(got.reshape(T * Hkv, topk)[valid], ref.reshape(T * Hkv, topk)[valid], imp[valid],
                     own_blocks(np.arange(T * Hkv)[valid], Hkv, cu, 64), init, local, str(case))
    print(f"{case}: {nd} of {T * Hkv} rows differ as near-ties", flush=True)


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_select_negative_and_zero_scale(scale):
    """A negative scale (its sign goes into the staged queries) and a zero
    one (uniform probabilities: block importances tie by window count)."""
    import torch
    seqlens, Hkv, G, D, topk = [1300, 200], 1, 4, 64, 12
    rng = np.random.default_rng(17 if scale else 18)
    d = random_case(rng, seqlens, Hkv, G, D, 64, topk, "bf16")
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "cu_seqlens")}
    got = nsa.select_blocks(dd["q"], dd["k"], dd["cu_seqlens"], 64, topk, scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ref, imp = oracle.select(f32_of(d["q"]), f32_of(d["k"]), d["cu_seqlens"], scale, "bf16", topk=topk,
                             with_importance=True)
    T = got.shape[0]
    nd = check_lists(got.reshape(T * Hkv, topk), ref.reshape(T * Hkv, topk), imp,
                     own_blocks(np.arange(T * Hkv), Hkv, d["cu_seqlens"], 64), 1, 2, f"scale {scale}")
    print(f"scale {scale}: {nd} rows differ as near-ties", flush=True)


def test_select_full_size_sampled_and_forward():
    """The 64K+32K GQA-4 workload's q and k (bf16, d 128): sampled rows
    against the oracle, then the lists as block_idx of the forward."""
    import torch
    cfg = W.CONFIGS["c2"]
    d = W.make_inputs(cfg)
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "v", "cu_seqlens")}
    got = nsa.select_blocks(dd["q"], dd["k"], dd["cu_seqlens"], 64, 16, cfg.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    T, Hkv = cfg.total_tokens, cfg.num_kv_heads
    toks = np.concatenate([np.arange(0, 40), np.arange(65536 - 20, 65536 + 40), T - 1 - np.arange(20),
                           rng.choice(T, 200, replace=False)])
    rows = np.unique((toks[:, None] * Hkv + rng.integers(0, Hkv, (toks.size, 1))).ravel())
    ref, imp = oracle.select(f32_of(d["q"]), f32_of(d["k"]), d["cu_seqlens"], cfg.scale, "bf16", topk=16,
                             rows=rows, with_importance=True)
    g = got.cpu().numpy().reshape(T * Hkv, 16)[rows]
    nd = check_lists(g, ref, imp, own_blocks(rows, Hkv, d["cu_seqlens"], 64), 1, 2, "c2 sampled",
                     max_diff_frac=0.02)
    print(f"c2 sampled: {nd} of {rows.size} rows differ as near-ties", flush=True)
    # the produced lists drive the forward
    out, lse = nsa.attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], got, 64, cfg.scale)
    torch.cuda.synchronize()
    bi = got.cpu().numpy()
    sample = rng.choice(T * Hkv, 300, replace=False)
    ref_o, ref_l = oracle.fwd(f32_of(d["q"]), f32_of(d["k"]), f32_of(d["v"]), d["cu_seqlens"], bi, 64,
                              cfg.scale, rows=sample)
    G = cfg.group
    o = from_dev(out).reshape(T * Hkv, G, -1)[sample]
    l = from_dev(lse).reshape(T * Hkv, G)[sample]
    compare(o, l, ref_o, ref_l, "bf16", "forward on produced lists")


def test_select_full_size_whole():
    """Every list of the 64K+32K GQA-4 workload's q and k (786,432 lists of
    16) against the oracle's: lists equal element for element pass as they
    are; every other one goes through the rule above (forced prefix and
    padding bit for bit, chosen sets equal or differing only in near-ties
    under the oracle's importance), and at most 2% of the lists may differ
    in their sets."""
    import torch
    cfg = W.CONFIGS["c2"]
    d = W.make_inputs(cfg)
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "cu_seqlens")}
    got = nsa.select_blocks(dd["q"], dd["k"], dd["cu_seqlens"], 64, 16, cfg.scale)
    torch.cuda.synchronize()
    T, Hkv = cfg.total_tokens, cfg.num_kv_heads
    g = got.cpu().numpy().reshape(T * Hkv, 16)
    del got, dd
    print("oracle: every list", flush=True)
    q, k = f32_of(d["q"]), f32_of(d["k"])
    ref = oracle.select(q, k, d["cu_seqlens"], cfg.scale, "bf16", topk=16).reshape(T * Hkv, 16)
    diff = np.nonzero((g != ref).any(axis=1))[0]
    print(f"c2 every list: {diff.size} of {T * Hkv} differ element for element", flush=True)
    assert diff.size <= 0.02 * T * Hkv
    if diff.size:
        ref_d, imp = oracle.select(q, k, d["cu_seqlens"], cfg.scale, "bf16", topk=16, rows=diff,
                                   with_importance=True)
        assert np.array_equal(ref_d, ref[diff])
        nd = check_lists(g[diff], ref_d, imp, own_blocks(diff, Hkv, d["cu_seqlens"], 64), 1, 2,
                         "c2 every list", max_diff_frac=1.0)
        print(f"c2 every list: {nd} of {T * Hkv} differ in their sets, all near-ties", flush=True)


def test_select_many_sequences():
    """1,100 short sequences and a long one: more sequences than the tile
    ranking takes (the lists' kernel then runs its tiles in tile order), so
    both dispatch orders are covered; every list against the oracle."""
    import torch
    rng = np.random.default_rng(21)
    seqlens = [int(x) for x in rng.integers(1, 90, 1100)] + [2500]
    Hkv, G, D, topk = 1, 4, 64, 8
    d = random_case(rng, seqlens, Hkv, G, D, 64, topk, "bf16")
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "cu_seqlens")}
    scale = 1.0 / np.sqrt(D)
    got = nsa.select_blocks(dd["q"], dd["k"], dd["cu_seqlens"], 64, topk, scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ref, imp = oracle.select(f32_of(d["q"]), f32_of(d["k"]), d["cu_seqlens"], scale, "bf16", topk=topk,
                             with_importance=True)
    T = got.shape[0]
    nd = check_lists(got.reshape(T * Hkv, topk), ref.reshape(T * Hkv, topk), imp,
                     own_blocks(np.arange(T * Hkv), Hkv, d["cu_seqlens"], 64), 1, 2, "many sequences")
    print(f"many sequences: {nd} of {T * Hkv} rows differ as near-ties", flush=True)


def test_select_outside_tokens():
    """Tokens past the last sequence get -1 lists."""
    import torch
    rng = np.random.default_rng(8)
    T = 1000
    q = to_dev(W.f32_to_bf16_bits(rng.standard_normal((T, 2, 64), dtype=np.float32)), dev())
    k = to_dev(W.f32_to_bf16_bits(rng.standard_normal((T, 1, 64), dtype=np.float32)), dev())
    cu = to_dev(np.array([0, 600, 800], np.int32), dev())
    # cu_seqlens ending before T: rows of the last 200 tokens are outside
    ws = nsa.Workspace()
    out = torch.full((T, 1, 6), 7, dtype=torch.int32, device=dev())
    nsa.select_blocks(q, k, cu, 64, 6, 0.125, out=out, workspace=ws)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[800:] == -1)
    assert np.all(o[:800, :, 0] == 0)


def test_select_long_sequence():
    """A 131,072-token sequence (2,048 blocks, 8,191 compressed windows) next
    to a short one: sampled rows -- the first tokens, the block boundaries
    near the end, random ones -- against the oracle, and no status bit."""
    import torch
    rng = np.random.default_rng(9)
    seqlens = [131072, 3000]
    d = random_case(rng, seqlens, 1, 2, 64, 64, 16, "bf16")
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "cu_seqlens")}
    ws = nsa.Workspace()
    got = nsa.select_blocks(dd["q"], dd["k"], dd["cu_seqlens"], 64, 16, 0.125, workspace=ws)
    torch.cuda.synchronize()
    assert nsa.check(ws) == 0
    T = int(d["cu_seqlens"][-1])
    toks = np.concatenate([np.arange(0, 40), np.arange(65536 - 70, 65536 + 70), np.arange(131072 - 70, 131072 + 70),
                           T - 1 - np.arange(10), rng.choice(T, 300, replace=False)])
    rows = np.unique(toks)  # one kv head: row = token
    ref, imp = oracle.select(f32_of(d["q"]), f32_of(d["k"]), d["cu_seqlens"], 0.125, "bf16", topk=16,
                             rows=rows, with_importance=True)
    g = got.cpu().numpy().reshape(T, 16)[rows]
    nd = check_lists(g, ref, imp, own_blocks(rows, 1, d["cu_seqlens"], 64), 1, 2, "131072-token sequence",
                     max_diff_frac=0.02)
    print(f"131072-token sequence: {nd} of {rows.size} rows differ as near-ties", flush=True)

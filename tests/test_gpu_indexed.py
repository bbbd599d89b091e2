"""The forward on a prebuilt index (nsa_sel_attn_fwd_indexed, through the C
ABI) against the plain forward: outputs and lse bitwise equal on ragged
random shapes with junk ids, with tokens outside every sequence, at head dim
256 and on the 64K+32K GQA-4 workload (whose plain forward the oracle checks
in the parity tests).  A corrupted index stays memory-safe, sets the status
bit, and leaves the rows it does not touch bitwise unchanged."""
import zlib

import numpy as np
import pytest

import nsa_selected_block_amd as nsa
import workloads as W
from helpers import random_case, to_dev

pytestmark = pytest.mark.gpu

BAD_PREBUILT_INDEX = 8


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def both(dd, Hkv, bs, scale, off=None, ent=None, ws=None):
    import torch
    if off is None:
        off, ent = nsa.build_index(dd["cu_seqlens"], dd["block_idx"], Hkv, bs)
    o1, l1 = nsa.attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], bs, scale)
    o2, l2 = nsa.attn_fwd_indexed(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], off, ent, bs,
                                  scale, workspace=ws)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


# (seqlens, Hkv, G, D, bs, topk, dtype)
CASES = [
    ([1000, 77, 0, 640], 2, 4, 128, 64, 16, "bf16"),
    ([700], 1, 1, 64, 32, 5, "f32"),
    ([513, 900], 2, 2, 64, 128, 12, "f16"),
    ([300, 65, 96], 1, 8, 256, 64, 9, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[6]}-G{c[2]}-d{c[3]}-bs{c[4]}-k{c[5]}" for c in CASES])
def test_indexed_equals_plain_forward(case):
    import torch
    seqlens, Hkv, G, D, bs, topk, dtype = case
    print(f"indexed {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    d = random_case(rng, seqlens, Hkv, G, D, bs, topk, dtype)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    ws = nsa.Workspace()
    o1, l1, o2, l2 = both(dd, Hkv, bs, 1.0 / np.sqrt(D), ws=ws)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert nsa.check(ws) & ~2 == 0  # (junk ids may set the bad-block-id bit)


def test_indexed_tokens_outside_sequences():
    import torch
    rng = np.random.default_rng(5)
    d = random_case(rng, [1000], 2, 2, 64, 64, 6, "bf16")
    d["cu_seqlens"] = np.array([0, 600, 800], np.int32)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    o1, l1, o2, l2 = both(dd, 2, 64, 0.125)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.all(l2[800:] == -float("inf"))


def test_indexed_full_size():
    """The 64K+32K GQA-4 workload: one inversion, two forwards."""
    import torch
    cfg = W.CONFIGS["c2"]
    d = W.make_inputs(cfg)
    dd = {k: to_dev(d[k], dev()) for k in ("q", "k", "v", "cu_seqlens", "block_idx")}
    o1, l1, o2, l2 = both(dd, cfg.num_kv_heads, cfg.block_size, cfg.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_indexed_corrupted_index():
    import torch
    rng = np.random.default_rng(11)
    seqlens, Hkv, G, D, bs, topk = [900, 300], 2, 4, 64, 64, 8
    d = random_case(rng, seqlens, Hkv, G, D, bs, topk, "bf16", junk=False)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    T = int(d["cu_seqlens"][-1])
    off, ent = nsa.build_index(dd["cu_seqlens"], dd["block_idx"], Hkv, bs)
    o_ref, l_ref = nsa.attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], bs, 0.125)
    off_h, ent_h = off.cpu().numpy(), ent.cpu().numpy().copy()
    nnz = int(off_h[-1])
    nbc = (len(off_h) - 1) // Hkv
    bucket = np.searchsorted(off_h, np.arange(nnz), side="right") - 1
    pos = rng.choice(nnz, 60, replace=False)
    # the rows whose entries are replaced
    hit = {(int(ent_h[x]) // topk, int(bucket[x]) // nbc) for x in pos}
    ent_h[pos[:20]] = rng.choice([-5, T * topk + 7, 2 ** 30, -(2 ** 31)], 20)
    for x in pos[20:]:  # an entry of another bucket: a kept (t, slot), but not of this block
        y = int(rng.integers(0, nnz))
        while bucket[y] == bucket[x]:
            y = int(rng.integers(0, nnz))
        ent_h[x] = ent_h[y]
        hit.add((int(ent_h[y]) // topk, int(bucket[x]) // nbc))  # (it may also be a row's own other slot)
    ws = nsa.Workspace()
    o, l = nsa.attn_fwd_indexed(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], off,
                                to_dev(ent_h, dev()), bs, 0.125, workspace=ws)
    torch.cuda.synchronize()
    assert nsa.check(ws) & BAD_PREBUILT_INDEX
    assert torch.isfinite(o.float()).all()
    keep = np.ones((T, Hkv), bool)
    for t, h in hit:
        keep[t, h] = False
    keep_q = np.repeat(keep, G, axis=1)  # [T, Hq]
    mask = torch.from_numpy(keep_q).to(dev())
    assert torch.equal(o[mask], o_ref[mask]) and torch.equal(l[mask], l_ref[mask])
    # offsets out of order and out of range: still memory-safe, rows of the
    # untouched buckets before the damage unchanged
    off_bad = off_h.copy()
    off_bad[len(off_bad) // 2] = 2 ** 30
    off_bad[len(off_bad) // 2 + 1] = -4
    ws2 = nsa.Workspace()
    o3, l3 = nsa.attn_fwd_indexed(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"],
                                  to_dev(off_bad, dev()), ent, bs, 0.125, workspace=ws2)
    torch.cuda.synchronize()
    assert nsa.check(ws2) & BAD_PREBUILT_INDEX
    assert torch.isfinite(o3.float()).all()


def test_indexed_unsorted_bucket():
    """A bucket whose entries are its kept (t, slot) pairs in descending
    order of t: the result is bitwise the plain forward's and no status bit
    is set.  The bucket holds its block's own (diagonal) tokens, whose keys
    need the causal mask: the main kernel's mask test takes each chunk's
    smallest token, so no row attends past its own token whatever the order."""
    import torch
    Hkv, G, D, bs, topk = 2, 4, 64, 64, 8
    seqlens = (900, 300)
    cfg = W.Config("t", seqlens, Hkv * G, Hkv, D, bs, topk, "bf16", seed=5, extra="uniform")
    rng = np.random.default_rng(17)
    d = random_case(rng, list(seqlens), Hkv, G, D, bs, topk, "bf16")
    d["block_idx"] = W.make_block_idx(cfg, rng)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    off, ent = nsa.build_index(dd["cu_seqlens"], dd["block_idx"], Hkv, bs)
    off_h, ent_h = off.cpu().numpy(), ent.cpu().numpy().copy()
    nbc = (len(off_h) - 1) // Hkv
    for h, j in ((1, 5), (0, 12)):   # blocks of sequence 0; tokens 64 j .. 64 j + 127 keep block j
        bkt = h * nbc + j
        a, b = int(off_h[bkt]), int(off_h[bkt + 1])
        toks = ent_h[a:b] // topk
        assert b - a > 70 and np.all(np.diff(toks) > 0) and toks[0] == j * bs
        ent_h[a:b] = ent_h[a:b][::-1].copy()
    ws = nsa.Workspace()
    o, l = nsa.attn_fwd_indexed(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], off,
                                to_dev(ent_h, dev()), bs, 0.125, workspace=ws)
    o_ref, l_ref = nsa.attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], dd["block_idx"], bs, 0.125)
    torch.cuda.synchronize()
    assert nsa.check(ws) == 0
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)

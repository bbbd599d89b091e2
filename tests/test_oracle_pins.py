"""Pins for the CPU oracle: facts fixed by the definition and the mathematics,
checked against implementations that share nothing with the oracle.

* hand-derived worked examples (tests/golden/hand_examples.json);
* a dense-mask brute force in numpy (a different algorithm: full T x T score
  matrix with the selection applied as a mask) on random tiny inputs,
  including -1, future and repeated ids anywhere in a row;
* the textbook special case: selecting every block 0..b(t) is dense causal
  attention (torch CPU scaled_dot_product_attention, float64);
* closed forms (q = 0, constant v, first token of a sequence);
* invariants (softmax rows sum to one, order / repeat / -1 / future-id
  invariance, varlen = separate sequences);
* the index inversion against a brute-force scan and the rule's closed forms;
* the backward against central finite differences of the forward and against
  torch autograd on the dense special case;
* the sliding-window branch against torch CPU SDPA under an explicit band
  mask (and scipy's logsumexp for lse), window 1 (each token sees itself) and
  a window longer than every sequence (dense causal).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import workloads as W


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------

def brute_force(q, k, v, cu, bi, bs, scale):
    """Dense masked softmax per (sequence, query head), float64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    topk = bi.shape[2]
    out = np.zeros((T, Hq, d))
    lse = np.full((T, Hq), -np.inf)
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        L = c1 - c0
        if L == 0:
            continue
        i = np.arange(L)
        nb = (L + bs - 1) // bs
        for h in range(Hkv):
            named = np.zeros((L, nb + 1), dtype=bool)
            for kk in range(topk):
                ids = bi[c0:c1, h, kk].astype(np.int64)
                ok = (ids >= 0) & (ids <= i // bs)
                named[i[ok], ids[ok]] = True
            allowed = named[:, i // bs] & (i[None, :] <= i[:, None])
            for g in range(G):
                qh = h * G + g
                S = scale * q[c0:c1, qh] @ k[c0:c1, h].T
                S = np.where(allowed, S, -np.inf)
                m = S.max(axis=1)
                has = np.isfinite(m)
                P = np.exp(S[has] - m[has, None])
                l = P.sum(axis=1)
                out[c0:c1][has, qh] = (P @ v[c0:c1, h]) / l[:, None]
                lse[c0:c1][has, qh] = m[has] + np.log(l)
    return out, lse


def full_selection(cu, Hkv, bs, topk_extra=0, rng=None):
    """block_idx naming every block 0..b(t) (ascending), padded with -1."""
    T = int(cu[-1])
    nbmax = max(((int(cu[s + 1]) - int(cu[s]) + bs - 1) // bs) for s in range(len(cu) - 1))
    topk = nbmax + topk_extra
    bi = np.full((T, Hkv, topk), -1, dtype=np.int32)
    for s in range(len(cu) - 1):
        for t in range(int(cu[s]), int(cu[s + 1])):
            b = (t - int(cu[s])) // bs
            bi[t, :, :b + 1] = np.arange(b + 1)
    return bi


def sdpa_dense(q, k, v, cu, scale):
    """Dense causal attention per sequence with torch CPU SDPA in float64."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, d))
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        qt = torch.from_numpy(np.asarray(q[c0:c1], np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(np.asarray(k[c0:c1], np.float64)).permute(1, 0, 2)
        vt = torch.from_numpy(np.asarray(v[c0:c1], np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(G, dim=0)[None]
        vt = vt.repeat_interleave(G, dim=0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                             scale=scale)
        out[c0:c1] = o[0].permute(1, 0, 2).numpy()
    return out


def rand_case(rng, seqlens, Hkv, G, d, bs, topk, junk=True):
    cu = W.cu_seqlens_of(seqlens)
    T = int(cu[-1])
    q = rng.standard_normal((T, Hkv * G, d)).astype(np.float32)
    k = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    nbmax = max((L + bs - 1) // bs for L in seqlens) if seqlens else 1
    lo = -2 if junk else 0
    hi = nbmax + 2 if junk else nbmax
    bi = rng.integers(lo, hi + 1, size=(T, Hkv, topk)).astype(np.int32)
    return q, k, v, cu, bi


# ---------------------------------------------------------------------------
# worked examples
# ---------------------------------------------------------------------------

def test_hand_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "hand_examples.json")) as f:
        ex = json.load(f)["examples"]
    assert len(ex) >= 4
    for e in ex:
        q, k, v = (np.array(e[n], dtype=np.float32) for n in ("q", "k", "v"))
        out, lse = oracle.fwd(q, k, v, np.array(e["cu_seqlens"]), np.array(e["block_idx"]),
                              e["block_size"], e["scale"])
        np.testing.assert_allclose(out, np.array(e["out"]), rtol=0, atol=2e-6, err_msg=e["name"])
        np.testing.assert_allclose(lse, np.array(e["lse"]), rtol=0, atol=2e-6, err_msg=e["name"])


# ---------------------------------------------------------------------------
# brute force on random tiny inputs
# ---------------------------------------------------------------------------

@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**31 - 1),
       seqlens=st.lists(st.integers(0, 90), min_size=1, max_size=3),
       Hkv=st.integers(1, 2), G=st.sampled_from([1, 2, 4]),
       d=st.sampled_from([1, 3, 8]), bs=st.sampled_from([1, 2, 4, 8, 16]),
       topk=st.integers(1, 6))
def test_bruteforce_random(seed, seqlens, Hkv, G, d, bs, topk):
    rng = np.random.default_rng(seed)
    q, k, v, cu, bi = rand_case(rng, seqlens, Hkv, G, d, bs, topk)
    scale = 0.7
    out, lse = oracle.fwd(q, k, v, cu, bi, bs, scale)
    ref_o, ref_l = brute_force(q, k, v, cu, bi, bs, scale)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-10)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(lse[fin], ref_l[fin], rtol=0, atol=1e-10)


def test_bruteforce_c0():
    d = W.make_inputs("c0")
    c = W.CONFIGS["c0"]
    out, lse = oracle.fwd(d["q"], d["k"], d["v"], d["cu_seqlens"], d["block_idx"],
                          c.block_size, c.scale)
    ref_o, ref_l = brute_force(d["q"], d["k"], d["v"], d["cu_seqlens"], d["block_idx"],
                               c.block_size, c.scale)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-9)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(5)
    q, k, v, cu, bi = rand_case(rng, [70, 33], 2, 2, 8, 8, 5)
    out, lse = oracle.fwd(q, k, v, cu, bi, 8, 0.5)
    rows = np.array([0, 5, 77, 140, 205], dtype=np.int64)  # t*Hkv + h
    o2, l2 = oracle.fwd(q, k, v, cu, bi, 8, 0.5, rows=rows)
    t, h = rows // 2, rows % 2
    assert np.array_equal(o2, out.reshape(103, 2, 2, 8)[t, h])
    assert np.array_equal(l2, lse.reshape(103, 2, 2)[t, h])


# ---------------------------------------------------------------------------
# dense special case (textbook routine)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seqlens,Hkv,G,d,bs", [
    ([100], 1, 1, 16, 8), ([64, 37, 5], 2, 2, 8, 4), ([129], 1, 4, 32, 16), ([1, 2, 3], 1, 3, 4, 1)])
def test_full_selection_is_dense_causal(seqlens, Hkv, G, d, bs):
    rng = np.random.default_rng(1)
    q, k, v, cu, _ = rand_case(rng, seqlens, Hkv, G, d, bs, 1)
    bi = full_selection(cu, Hkv, bs, topk_extra=1)
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.fwd(q, k, v, cu, bi, bs, scale)
    ref = sdpa_dense(q, k, v, cu, scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-10)
    # lse against a library log-sum-exp over the causal scores
    from scipy.special import logsumexp
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        for qh in range(Hkv * G):
            S = scale * q[c0:c1, qh].astype(np.float64) @ k[c0:c1, qh // G].T.astype(np.float64)
            S[np.triu_indices(c1 - c0, 1)] = -np.inf
            np.testing.assert_allclose(lse[c0:c1, qh], logsumexp(S, axis=1), rtol=0, atol=1e-10)


def test_dense_prefix_rows_of_c0():
    """Tokens 0..255 of c0 select every block 0..b, so they are dense causal."""
    d = W.make_inputs("c0")
    c = W.CONFIGS["c0"]
    out, _ = oracle.fwd(d["q"], d["k"], d["v"], d["cu_seqlens"], d["block_idx"],
                        c.block_size, c.scale)
    n = 256
    ref = sdpa_dense(d["q"][:n], d["k"][:n], d["v"][:n], np.array([0, n]), c.scale)
    np.testing.assert_allclose(out[:n], ref, rtol=0, atol=1e-10)
    # and token 256 (block 4) does not: it skips one of blocks 1..2
    ref_more = sdpa_dense(d["q"][:n + 1], d["k"][:n + 1], d["v"][:n + 1],
                          np.array([0, n + 1]), c.scale)
    assert np.abs(out[n] - ref_more[n]).max() > 1e-3


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_zero_query_gives_mean_and_log_count():
    rng = np.random.default_rng(2)
    q, k, v, cu, bi = rand_case(rng, [50, 77], 2, 2, 8, 8, 4)
    q[:] = 0
    out, lse = oracle.fwd(q, k, v, cu, bi, 8, 0.9)
    for t in range(q.shape[0]):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        i = t - int(cu[s])
        for h in range(2):
            ids = {j for j in bi[t, h] if 0 <= j <= i // 8}
            keys = [int(cu[s]) + p for p in range(i + 1) if p // 8 in ids]
            for g in range(2):
                if not keys:
                    assert np.isneginf(lse[t, h * 2 + g]) and not out[t, h * 2 + g].any()
                    continue
                assert abs(lse[t, h * 2 + g] - math.log(len(keys))) < 1e-12
                np.testing.assert_allclose(out[t, h * 2 + g], v[keys, h].astype(np.float64).mean(axis=0),
                                           rtol=0, atol=1e-12)


def test_constant_values_and_first_token():
    rng = np.random.default_rng(3)
    q, k, v, cu, bi = rand_case(rng, [40, 1, 23], 1, 2, 4, 4, 3, junk=False)
    bi[:, :, 0] = 0  # every token selects block 0 (so no row is empty)
    v_const = np.full_like(v, 2.5)
    out, _ = oracle.fwd(q, k, v_const, cu, bi, 4, 0.5)
    np.testing.assert_allclose(out, 2.5, rtol=0, atol=1e-12)
    out, lse = oracle.fwd(q, k, v, cu, bi, 4, 0.5)
    for s in range(3):
        c0 = int(cu[s])
        for qh in range(2):
            np.testing.assert_allclose(out[c0, qh], v[c0, 0], rtol=0, atol=1e-12)
            ref = 0.5 * float(q[c0, qh].astype(np.float64) @ k[c0, 0].astype(np.float64))
            assert abs(lse[c0, qh] - ref) < 1e-12


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_c0():
    d = W.make_inputs("c0")
    c = W.CONFIGS["c0"]
    q, k = d["q"].astype(np.float64), d["k"].astype(np.float64)
    _, lse = oracle.fwd(d["q"], d["k"], d["v"], d["cu_seqlens"], d["block_idx"],
                        c.block_size, c.scale)
    rng = np.random.default_rng(0)
    for t in rng.choice(1024, 64, replace=False):
        b = t // 64
        ids = {j for j in d["block_idx"][t, 0] if 0 <= j <= b}
        keys = [p for p in range(t + 1) if p // 64 in ids]
        for g in range(2):
            s = c.scale * (k[keys, 0] @ q[t, g])
            assert abs(np.exp(s - lse[t, g]).sum() - 1.0) < 1e-12


def test_order_repeat_and_junk_invariance():
    rng = np.random.default_rng(4)
    q, k, v, cu, bi = rand_case(rng, [90, 61], 2, 2, 8, 8, 6)
    out, lse = oracle.fwd(q, k, v, cu, bi, 8, 0.6)
    perm = np.stack([rng.permutation(6) for _ in range(bi.shape[0] * 2)]).reshape(-1, 2, 6)
    bi_p = np.take_along_axis(bi, perm, axis=2)
    o2, l2 = oracle.fwd(q, k, v, cu, bi_p, 8, 0.6)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    # append repeats, -1 and future ids: nothing changes
    extra = np.concatenate([bi, bi[:, :, :2], np.full_like(bi[:, :, :1], -1),
                            np.full_like(bi[:, :, :1], 10**6)], axis=2)
    o3, l3 = oracle.fwd(q, k, v, cu, extra, 8, 0.6)
    assert np.array_equal(out, o3) and np.array_equal(lse, l3)


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(6)
    seqlens = [45, 0, 80, 17]
    q, k, v, cu, bi = rand_case(rng, seqlens, 2, 2, 8, 8, 5)
    out, lse = oracle.fwd(q, k, v, cu, bi, 8, 0.5)
    for s in range(len(seqlens)):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        if c1 == c0:
            continue
        o, l = oracle.fwd(q[c0:c1], k[c0:c1], v[c0:c1], np.array([0, c1 - c0]), bi[c0:c1], 8, 0.5)
        assert np.array_equal(o, out[c0:c1]) and np.array_equal(l, lse[c0:c1])


def test_missing_block_moves_lse():
    """Dropping one selected block changes the result (the set is honoured)."""
    d = W.make_inputs("c0")
    c = W.CONFIGS["c0"]
    bi = d["block_idx"].copy()
    t = 900
    assert (bi[t, 0] >= 0).sum() == 4
    bi2 = bi.copy()
    bi2[t, 0, 3] = -1
    rows = np.array([t], dtype=np.int64)
    o1, l1 = oracle.fwd(d["q"], d["k"], d["v"], d["cu_seqlens"], bi, 64, c.scale, rows=rows)
    o2, l2 = oracle.fwd(d["q"], d["k"], d["v"], d["cu_seqlens"], bi2, 64, c.scale, rows=rows)
    assert np.all(l2 < l1)


# ---------------------------------------------------------------------------
# index inversion
# ---------------------------------------------------------------------------

def brute_invert(cu, bi, Hkv, bs, T):
    B = len(cu) - 1
    cap = T // bs + B
    nbs = [(int(cu[s + 1]) - int(cu[s]) + bs - 1) // bs for s in range(B)]
    blkoff = np.concatenate([[0], np.cumsum(nbs)]).astype(int)
    lists = {}
    topk = bi.shape[2]
    for h in range(Hkv):
        for s in range(B):
            for j in range(nbs[s]):
                bucket = []
                for t in range(int(cu[s]), int(cu[s + 1])):
                    b = (t - int(cu[s])) // bs
                    row = list(bi[t, h])
                    if j <= b and j in row:
                        bucket.append(t * topk + row.index(j))
                lists[h * cap + blkoff[s] + j] = bucket
    return lists, cap


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1),
       seqlens=st.lists(st.integers(0, 70), min_size=1, max_size=3),
       Hkv=st.integers(1, 3), bs=st.sampled_from([1, 3, 8, 16]), topk=st.integers(1, 6))
def test_invert_bruteforce(seed, seqlens, Hkv, bs, topk):
    rng = np.random.default_rng(seed)
    _, _, _, cu, bi = rand_case(rng, seqlens, Hkv, 1, 1, bs, topk)
    T = int(cu[-1])
    offsets, entries = oracle.invert(cu, bi, Hkv, bs, total_tokens=T)
    lists, cap = brute_invert(cu, bi, Hkv, bs, T)
    assert offsets.shape[0] == Hkv * cap + 1
    assert offsets[0] == 0 and np.all(np.diff(offsets) >= 0)
    for bkt in range(Hkv * cap):
        got = list(entries[offsets[bkt]:offsets[bkt + 1]])
        assert got == lists.get(bkt, []), bkt


@pytest.mark.parametrize("name", ["c0", "c1", "c3", "c2"])
def test_invert_closed_forms(name, golden_dir):
    with open(os.path.join(golden_dir, "config_index_stats.json")) as f:
        stats = json.load(f)["configs"][name]
    cfg = W.CONFIGS[name]
    d = W.make_inputs(name)
    cu, bi = d["cu_seqlens"], d["block_idx"]
    T, Hkv, bs, topk = cfg.total_tokens, cfg.num_kv_heads, cfg.block_size, cfg.topk
    offsets, entries = oracle.invert(cu, bi, Hkv, bs)
    assert offsets[-1] == stats["nnz"] == entries.shape[0]
    cap = T // bs + len(cfg.seqlens)
    t_of = entries // topk
    slot = entries % topk
    # every entry names a row slot holding the bucket's block
    blkoff = np.concatenate([[0], np.cumsum([L // bs for L in cfg.seqlens])])
    bucket_of_entry = np.repeat(np.arange(Hkv * cap), np.diff(offsets))
    h_e = bucket_of_entry // cap
    g_e = bucket_of_entry % cap
    s_e = np.searchsorted(blkoff, g_e, side="right") - 1
    j_e = g_e - blkoff[s_e]
    assert np.array_equal(bi[t_of, h_e, slot], j_e)
    # sequences never mix, lists ascending in t
    assert np.array_equal(np.searchsorted(cu, t_of, side="right") - 1, s_e)
    same = bucket_of_entry[1:] == bucket_of_entry[:-1]
    assert np.all(t_of[1:][same] > t_of[:-1][same])
    # block 0 holds every token; bucket j >= 1 holds all tokens of blocks j, j+1
    for h in (0, Hkv - 1):
        for s, L in enumerate(cfg.seqlens):
            c0 = int(cu[s])
            base = h * cap + blkoff[s]
            b0 = t_of[offsets[base]:offsets[base + 1]]
            assert np.array_equal(b0, np.arange(c0, c0 + L))
            for j in (1, 7, L // bs - 2, L // bs - 1):
                lst = set(t_of[offsets[base + j]:offsets[base + j + 1]].tolist())
                need = set(range(c0 + j * bs, c0 + min((j + 2) * bs, L)))
                assert need <= lst


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def test_bwd_finite_differences():
    rng = np.random.default_rng(7)
    q, k, v, cu, bi = rand_case(rng, [13, 9], 2, 2, 3, 4, 3)
    q, k, v = (a.astype(np.float64).astype(np.float32) for a in (q, k, v))
    do = rng.standard_normal(q.shape).astype(np.float32)
    scale = 0.8
    dq, dk, dv = oracle.bwd(q, k, v, cu, bi, do, 4, scale)

    # The oracle takes float32 inputs; for finite differences evaluate the
    # forward in float64 through the brute force (same definition, different code).
    def loss(qq, kk, vv):
        o, _ = brute_force(qq, kk, vv, cu, bi, 4, scale)
        return float((o * do.astype(np.float64)).sum())

    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        base = arr.astype(np.float64)
        num = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = base.copy(); p[idx] += eps
            m = base.copy(); m[idx] -= eps
            args = {"q": q.astype(np.float64), "k": k.astype(np.float64), "v": v.astype(np.float64)}
            args[name] = p
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = m
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=2e-7, err_msg=name)


def test_bwd_dense_matches_autograd():
    rng = np.random.default_rng(8)
    seqlens = [40, 25]
    q, k, v, cu, _ = rand_case(rng, seqlens, 2, 2, 8, 8, 1)
    bi = full_selection(cu, 2, 8)
    do = rng.standard_normal(q.shape).astype(np.float32)
    scale = 0.35
    dq, dk, dv = oracle.bwd(q, k, v, cu, bi, do, 8, scale)
    for s in range(2):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        qt = torch.tensor(q[c0:c1], dtype=torch.float64, requires_grad=True)
        kt = torch.tensor(k[c0:c1], dtype=torch.float64, requires_grad=True)
        vt = torch.tensor(v[c0:c1], dtype=torch.float64, requires_grad=True)
        o = torch.nn.functional.scaled_dot_product_attention(
            qt.permute(1, 0, 2)[None], kt.permute(1, 0, 2).repeat_interleave(2, 0)[None],
            vt.permute(1, 0, 2).repeat_interleave(2, 0)[None], is_causal=True, scale=scale)
        (o[0].permute(1, 0, 2) * torch.tensor(do[c0:c1], dtype=torch.float64)).sum().backward()
        np.testing.assert_allclose(dq[c0:c1], qt.grad.numpy(), rtol=0, atol=1e-10)
        np.testing.assert_allclose(dk[c0:c1], kt.grad.numpy(), rtol=0, atol=1e-10)
        np.testing.assert_allclose(dv[c0:c1], vt.grad.numpy(), rtol=0, atol=1e-10)


def test_bwd_dkv_all_matches_masked_autograd():
    """dk, dv of every key from the rows' lse and D (the whole-output entry
    point) against torch CPU autograd (float64) of attention under an explicit
    boolean mask built from the selection rule: key p visible to (t, h) iff
    its block is among t's ids in [0, b(t)] and p <= i.  Rows with repeated,
    -1 and future ids, ragged sequences and an empty sequence."""
    rng = np.random.default_rng(13)
    seqlens = [37, 0, 26]
    Hkv, G, d, bs, topk = 2, 2, 8, 8, 4
    q, k, v, cu, bi = rand_case(rng, seqlens, Hkv, G, d, bs, topk)
    T = int(cu[-1])
    bi[3, 0] = [0, 0, -1, 5]          # a repeat, "no block" and a future block
    do = rng.standard_normal(q.shape).astype(np.float32)
    scale = 0.45
    out, lse = oracle.fwd(q, k, v, cu, bi, bs, scale)
    D = (out * do.astype(np.float64)).sum(axis=2)
    dk, dv = oracle.bwd_dkv_all(q, k, v, cu, bi, do, bs, scale, lse, D)
    # reference: dense masked attention per sequence, kv head and query head
    rk = np.zeros(k.shape); rv = np.zeros(v.shape)
    for s in range(len(seqlens)):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        if c1 == c0:
            continue
        for h in range(Hkv):
            mask = np.zeros((c1 - c0, c1 - c0), dtype=bool)
            for i in range(c1 - c0):
                ids = {int(j) for j in bi[c0 + i, h] if 0 <= j <= i // bs}
                for j in ids:
                    mask[i, j * bs:min((j + 1) * bs, i + 1)] = True
            kt = torch.tensor(k[c0:c1, h], dtype=torch.float64, requires_grad=True)
            vt = torch.tensor(v[c0:c1, h], dtype=torch.float64, requires_grad=True)
            for g in range(G):
                qt = torch.tensor(q[c0:c1, h * G + g], dtype=torch.float64)
                sc = (qt @ kt.T) * scale
                sc = sc.masked_fill(~torch.tensor(mask), float("-inf"))
                pr = torch.softmax(sc, dim=1)
                pr = torch.nan_to_num(pr)  # rows with no visible key
                o = pr @ vt
                (o * torch.tensor(do[c0:c1, h * G + g], dtype=torch.float64)).sum().backward()
            rk[c0:c1, h] = kt.grad.numpy()
            rv[c0:c1, h] = vt.grad.numpy()
    np.testing.assert_allclose(dk, rk, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv, rv, rtol=0, atol=1e-10)


# ---------------------------------------------------------------------------
# generator facts the workloads rely on
# ---------------------------------------------------------------------------

def test_generator_rule_c0():
    d = W.make_inputs("c0")
    bi = d["block_idx"][:, 0]
    for t in range(1024):
        b = t // 64
        row = [j for j in bi[t] if j >= 0]
        assert len(row) == len(set(row)) == min(b + 1, 4)
        assert row[0] == 0 and set(range(max(0, b - 1), b + 1)) <= set(row)
        assert all(1 <= j <= b - 2 for j in row[3:])
        assert all(x == -1 for x in bi[t][len(row):])


def test_effective_flops_formula_matches_indices():
    for name in ("c0", "c3"):
        cfg = W.CONFIGS[name]
        d = W.make_inputs(name)
        bi = d["block_idx"]
        bs = cfg.block_size
        keys = 0
        for s, L in enumerate(cfg.seqlens):
            c0 = int(d["cu_seqlens"][s])
            i = np.arange(L)
            b = i // bs
            rows = bi[c0:c0 + L]
            valid = (rows >= 0) & (rows <= b[:, None, None])
            nsel = valid.sum(axis=2)
            keys += int(((nsel - 1) * bs + (i % bs + 1)[:, None]).sum())
        assert W.effective_flops(cfg) == 4 * cfg.head_dim * cfg.group * keys


def test_bwd_restricted_match_full():
    """The sampled backward entry points equal the full backward on their rows/blocks."""
    rng = np.random.default_rng(12)
    seqlens = [70, 45]
    q, k, v, cu, bi = rand_case(rng, seqlens, 2, 2, 8, 8, 5)
    do = rng.standard_normal(q.shape).astype(np.float32)
    dq, dk, dv = oracle.bwd(q, k, v, cu, bi, do, 8, 0.4)
    rows = np.array([0, 3, 17, 139, 229], dtype=np.int64)  # t*Hkv + h
    got = oracle.bwd_dq_rows(q, k, v, cu, bi, do, 8, 0.4, rows)
    assert np.allclose(got, dq.reshape(115, 2, 2, 8)[rows // 2, rows % 2], rtol=0, atol=1e-12)
    blocks = [(0, 0, 0), (1, 0, 3), (0, 1, 5), (1, 1, 0)]
    gk, gv = oracle.bwd_dkv_blocks(q, k, v, cu, bi, do, 8, 0.4, blocks)
    for i, (h, s, j) in enumerate(blocks):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        p0, p1 = c0 + j * 8, min(c0 + (j + 1) * 8, c1)
        assert np.allclose(gk[i, :p1 - p0], dk[p0:p1, h], rtol=0, atol=1e-12)
        assert np.allclose(gv[i, :p1 - p0], dv[p0:p1, h], rtol=0, atol=1e-12)
        assert not gk[i, p1 - p0:].any()


# ---------------------------------------------------------------------------
# sliding-window branch
# ---------------------------------------------------------------------------

def sdpa_banded(q, k, v, cu, scale, window):
    """Attention per sequence with torch CPU SDPA (float64) under an explicit
    boolean band mask: key p visible to query i iff i - window < p <= i."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, d))
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        L = c1 - c0
        if L == 0:
            continue
        i = torch.arange(L)[:, None]
        p = torch.arange(L)[None, :]
        mask = (p <= i) & (p > i - window)
        qt = torch.from_numpy(np.asarray(q[c0:c1], np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(np.asarray(k[c0:c1], np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        vt = torch.from_numpy(np.asarray(v[c0:c1], np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        out[c0:c1] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("seqlens,Hkv,G,d,window", [
    ([100, 1, 0, 37], 2, 2, 16, 8), ([300], 1, 4, 32, 64), ([65, 130], 3, 1, 8, 1),
    ([200, 90], 1, 3, 16, 500)])
def test_window_matches_banded_sdpa(seqlens, Hkv, G, d, window):
    rng = np.random.default_rng(3)
    q, k, v, cu, _ = rand_case(rng, seqlens, Hkv, G, d, 16, 1)
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.window_fwd(q, k, v, cu, window, scale)
    np.testing.assert_allclose(out, sdpa_banded(q, k, v, cu, scale, window), rtol=0, atol=1e-10)
    from scipy.special import logsumexp
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        L = c1 - c0
        i, p = np.arange(L)[:, None], np.arange(L)[None, :]
        band = (p <= i) & (p > i - window)
        for qh in range(Hkv * G):
            S = scale * q[c0:c1, qh].astype(np.float64) @ k[c0:c1, qh // G].T.astype(np.float64)
            S[~band] = -np.inf
            np.testing.assert_allclose(lse[c0:c1, qh], logsumexp(S, axis=1), rtol=0, atol=1e-10)


def test_window_closed_forms():
    """window 1: each token sees only itself (out = v_t, lse = scale q.k_t);
    window >= every length: dense causal attention."""
    rng = np.random.default_rng(4)
    q, k, v, cu, _ = rand_case(rng, [50, 7, 33], 2, 2, 8, 16, 1)
    G = 2
    out, lse = oracle.window_fwd(q, k, v, cu, 1, 0.3)
    kv_head = np.arange(4) // G
    np.testing.assert_allclose(out, v[:, kv_head].astype(np.float64), rtol=0, atol=1e-12)
    ref_l = 0.3 * np.einsum("thd,thd->th", q.astype(np.float64), k[:, kv_head].astype(np.float64))
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)
    out2, _ = oracle.window_fwd(q, k, v, cu, 10_000, 0.3)
    np.testing.assert_allclose(out2, sdpa_dense(q, k, v, cu, 0.3), rtol=0, atol=1e-10)


# ---------------------------------------------------------------------------
# index producer (compressed attention -> block lists)
# ---------------------------------------------------------------------------

def _select_bruteforce(q, k, cu, scale, dtype, ks, stride, bs, topk, init, local):
    """The same steps in a matrix formulation: the compressed keys as an
    explicit window-mean, the masked softmax as a dense [positions x windows]
    matrix, the block importance as a product with a 0/1 window-block overlap
    matrix, the list by a stable sort."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = -np.ones((T, Hkv, topk), dtype=np.int32)
    imps = {}
    for s in range(len(cu) - 1):
        c0, L = int(cu[s]), int(cu[s + 1] - cu[s])
        nc = (L - ks) // stride + 1 if L >= ks else 0
        nb = (L + bs - 1) // bs
        # window means: fp32, positions in order (the oracle's accumulation order)
        kc = np.zeros((nc, Hkv, d), dtype=np.float32)
        for a in range(ks):
            kc = (kc + k[c0 + np.arange(nc) * stride + a]).astype(np.float32)
        kc = (kc / np.float32(ks)).astype(np.float32)
        if dtype == "bf16":
            kc = W.bf16_bits_to_f32(W.f32_to_bf16_bits(kc))
        elif dtype == "f16":
            kc = kc.astype(np.float16).astype(np.float32)
        pos = np.arange(L)
        vis = (np.arange(nc)[None, :] * stride + ks - 1) <= pos[:, None]          # [L, nc]
        lo = np.arange(nc) * stride
        ov = ((lo[:, None] < (np.arange(nb)[None, :] + 1) * bs) &
              (lo[:, None] + ks > np.arange(nb)[None, :] * bs)).astype(np.float64)   # [nc, nb]
        for h in range(Hkv):
            imp = np.zeros((L, nb))
            for g in range(G):
                sc = scale * (q[c0:c0 + L, h * G + g].astype(np.float64) @ kc[:, h].astype(np.float64).T)
                sc = np.where(vis, sc, -np.inf)
                m = sc.max(axis=1, keepdims=True) if nc else np.zeros((L, 1))
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(sc - m)
                z = e.sum(axis=1, keepdims=True)
                p = np.divide(e, z, out=np.zeros_like(e), where=z > 0)
                imp += p @ ov
            for i in range(L):
                b = i // bs
                row, taken = [], set()
                for j in list(range(init)) + [b - u for u in range(local)]:
                    if 0 <= j <= b and j not in taken and len(row) < topk:
                        taken.add(j)
                        row.append(j)
                cand = [j for j in range(b + 1) if j not in taken]
                cand.sort(key=lambda j: (-imp[i, j], j))
                row += cand[:topk - len(row)]
                out[c0 + i, h, :len(row)] = row
            imps[(s, h)] = imp
    return out, imps


@pytest.mark.parametrize("seed,seqlens,Hkv,G,d,dtype,topk", [
    (0, [300], 1, 2, 32, "f32", 5),
    (1, [200, 17, 0, 150], 2, 4, 64, "bf16", 6),
    (2, [130, 260], 2, 1, 48, "f16", 16),
    (3, [400], 1, 8, 16, "bf16", 3),
])
def test_select_bruteforce(seed, seqlens, Hkv, G, d, dtype, topk):
    rng = np.random.default_rng(seed)
    cu = W.cu_seqlens_of(seqlens)
    T = int(cu[-1])
    q = rng.standard_normal((T, Hkv * G, d)).astype(np.float32)
    k = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    if dtype == "bf16":
        q, k = W.bf16_bits_to_f32(W.f32_to_bf16_bits(q)), W.bf16_bits_to_f32(W.f32_to_bf16_bits(k))
    elif dtype == "f16":
        q, k = q.astype(np.float16).astype(np.float32), k.astype(np.float16).astype(np.float32)
    scale = 1.0 / math.sqrt(d)
    bi, imp = oracle.select(q, k, cu, scale, dtype, topk=topk, with_importance=True)
    ref, ref_imp = _select_bruteforce(q, k, cu, scale, dtype, 32, 16, 64, topk, 1, 2)
    assert np.array_equal(bi, ref)
    imp = imp.reshape(T, Hkv, -1)
    for (s, h), r in ref_imp.items():
        c0, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for i in range(L):
            b = i // 64
            np.testing.assert_allclose(imp[c0 + i, h, :b + 1], r[i, :b + 1], rtol=1e-12, atol=1e-13)
            assert np.all(imp[c0 + i, h, b + 1:] == -1.0)


def test_select_zero_query_counts_windows():
    """q = 0: every visible window gets the same probability, so a block's
    importance is G times the share of visible windows that overlap it (a
    boundary window counts for both blocks), and the list takes the blocks
    with the most such windows, lowest ids first."""
    L, Hkv, G, d = 700, 2, 3, 16
    rng = np.random.default_rng(4)
    q = np.zeros((L, Hkv * G, d), np.float32)
    k = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    cu = np.array([0, L], np.int32)
    bi, imp = oracle.select(q, k, cu, 0.25, "f32", topk=8, with_importance=True)
    imp = imp.reshape(L, Hkv, -1)
    for i in (31, 32, 95, 250, 511, 699):
        nvis = (i - 31) // 16 + 1
        for j in range(i // 64 + 1):
            # windows c with 16c + 31 <= i overlapping [64j, 64j + 64): c in 4j-1 .. 4j+3
            cnt = sum(1 for c in range(max(0, 4 * j - 1), 4 * j + 4) if 16 * c + 31 <= i)
            assert imp[i, 0, j] == pytest.approx(G * cnt / nvis, rel=1e-12)
        b = i // 64
        want = [0] + [x for x in (b, b - 1) if x > 0]
        rest = sorted((x for x in range(1, b + 1) if x not in want),
                      key=lambda x: (-sum(1 for c in range(4 * x - 1, 4 * x + 4) if 16 * c + 31 <= i), x))
        want = (want + rest)[:8]
        assert list(bi[i, 1, :len(want)]) == want and np.all(bi[i, 1, len(want):] == -1)
    # before the first full window nothing is visible: importance 0
    assert np.all(imp[30, :, 0] == 0.0)


def test_select_disjoint_windows_importance_sums_to_group():
    """Windows inside single blocks (kernel size = stride = 16 with block 64):
    each query head's probabilities land once, so a row's importance sums to
    G as soon as one window is visible."""
    L, Hkv, G, d = 520, 1, 4, 8
    rng = np.random.default_rng(5)
    q = rng.standard_normal((L, G, d)).astype(np.float32)
    k = rng.standard_normal((L, 1, d)).astype(np.float32)
    _, imp = oracle.select(q, k, np.array([0, L], np.int32), 0.5, "f32", kernel_size=16,
                           kernel_stride=16, topk=4, with_importance=True)
    for i in (15, 16, 100, 519):
        v = imp[i, :i // 64 + 1]
        assert v.sum() == pytest.approx(G, rel=1e-12)


def test_select_windows_equal_blocks_is_softmax_topk():
    """Kernel size = stride = block size: each window is one block, so the
    importance is the group-summed softmax over the means of the complete
    past blocks, and the list past the forced ids is torch.topk of it."""
    L, Hkv, G, d, bs = 64 * 20, 2, 2, 32, 64
    rng = np.random.default_rng(6)
    q = rng.standard_normal((L, Hkv * G, d)).astype(np.float32)
    k = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    scale = 0.3
    bi = oracle.select(q, k, np.array([0, L], np.int32), scale, "f32", kernel_size=bs,
                       kernel_stride=bs, block_size=bs, topk=7, init_blocks=1, local_blocks=2)
    kmean = torch.from_numpy(k.reshape(L // bs, bs, Hkv, d)).double().mean(dim=1)   # [nb, Hkv, d]
    for i in (127, 128, 500, 1279):
        b = i // bs
        nvis = (i + 1) // bs            # complete blocks only
        for h in range(Hkv):
            imp = torch.zeros(b + 1, dtype=torch.float64)
            if nvis:
                for g in range(G):
                    s = scale * (torch.from_numpy(q[i, h * G + g]).double() @ kmean[:nvis, h].T)
                    imp[:nvis] += torch.softmax(s, dim=0)
            forced = [0] + [x for x in (b, b - 1) if x > 0]
            imp[forced] = -1.0
            n = min(7, b + 1) - len(forced)
            top = torch.topk(imp, n).indices.tolist() if n > 0 else []
            assert list(bi[i, h, :len(forced)]) == forced
            assert sorted(bi[i, h, len(forced):len(forced) + n].tolist()) == sorted(top)


def test_select_list_invariants():
    """Every list holds the forced ids first, no repeats, only ids in [0, b],
    min(topk, b + 1) ids in all, -1 after them."""
    seqlens = [1000, 333]
    cu = W.cu_seqlens_of(seqlens)
    T = int(cu[-1])
    rng = np.random.default_rng(7)
    q = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((T, 8, 32), dtype=np.float32)))
    k = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((T, 2, 32), dtype=np.float32)))
    bi = oracle.select(q, k, cu, 0.2, "bf16", topk=6)
    for t in range(T):
        s = 0 if t < cu[1] else 1
        b = (t - cu[s]) // 64
        for h in range(2):
            row = bi[t, h]
            n = min(6, b + 1)
            assert np.all(row[n:] == -1) and len(set(row[:n].tolist())) == n
            assert np.all((row[:n] >= 0) & (row[:n] <= b))
            forced = [0] + [x for x in (b, b - 1) if x > 0]
            assert list(row[:len(forced)]) == forced[:n]

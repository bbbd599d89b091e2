"""Benchmark: NSA selected-block attention on one MI355X.

Default: one step = one nsa_sel_attn_fwd call (index inversion -> main kernel
-> dense kernel -> merge; the 16-bit forward runs with the dense split, which
computes the blocks every token of a token block keeps with the dense kernel,
which then also merges its tokens' rows; --gather-only turns it off) over the varlen 64K + 32K token, 32 query / 8 kv
head (GQA-4), d=128, block 64, topk 16 bf16 workload, inputs resident in HBM.
With --config c4 (the same tensors plus dO) one step is a training step of
the operation: nsa_sel_attn_fwd then nsa_sel_attn_bwd.  With --branch window
one step is the sliding-window branch (nsa_sel_window_fwd, --window tokens)
on the same q/k/v.  Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config c2|c4|c1|c3]
                    [--branch selection|window] [--window 512]
                    [--no-cpu-baseline] [--cpu-seconds 15] [--gather-only]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected-attn fwd ms + effective TFLOP/s (% bf16 MFMA peak), 64K tok GQA-4"
METRIC_TRAIN = "selected-attn fwd+bwd ms + effective TFLOP/s (% bf16 MFMA peak), 64K tok GQA-4"
METRIC_SELECT = "index producer (compressed attention + top-k) ms + effective TFLOP/s (% bf16 MFMA peak), 64K tok GQA-4"
METRIC_WINDOW = "sliding-window attn fwd ms + effective TFLOP/s (% bf16 MFMA peak), 64K tok GQA-4"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "nsa_selected_block_amd", "csrc")
# sources each main kernel is compiled from (a change to any of them makes
# the recorded counters stale)
KERNEL_SRCS = {
    "fwd": ["attn_fwd.hip", "device_common.h", "internal.h"],
    "bwd": ["attn_bwd.hip", "device_common.h", "internal.h"],
}
COUNTERS = {
    "fwd": os.path.join(ROOT, "profiles", "main_kernel_c2_counters.json"),
    "bwd": os.path.join(ROOT, "profiles", "bwd_main_kernel_c4_counters.json"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_src_sha(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SRCS[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_keys_per_row(cfg, bi_rows, t_rows):
    """Causally visible selected keys of rows (t, h) (for the FLOP count)."""
    cu = np.array([0] + list(np.cumsum(cfg.seqlens)))
    s = np.searchsorted(cu, t_rows, side="right") - 1
    i = t_rows - cu[s]
    b = i // cfg.block_size
    valid = (bi_rows >= 0) & (bi_rows <= b[:, None])
    # rows never hold repeats in the generated workloads
    n = valid.sum(axis=1)
    diag = (bi_rows == b[:, None]).any(axis=1)
    return np.where(diag, (n - 1) * cfg.block_size + (i % cfg.block_size) + 1,
                    n * cfg.block_size)


def gather_units(cfg, block_idx, dense_split: bool):
    """(entries, non-empty buckets, causally visible keys of the entries) of
    the main kernel.  With the dense split, the ids every row of a (kv head,
    token block) keeps are computed by the dense kernel and never reach the
    gather path."""
    bs = cfg.block_size
    cu = np.array([0] + list(np.cumsum(cfg.seqlens)))
    t = np.arange(cfg.total_tokens)
    s = np.searchsorted(cu, t, side="right") - 1
    b = (t - cu[s]) // bs
    valid = (block_idx >= 0) & (block_idx <= b[:, None, None])
    # first occurrence only (set semantics of a row)
    srt = np.sort(np.where(valid, block_idx, -1), axis=2)
    first = np.concatenate([np.ones_like(srt[..., :1], bool), srt[..., 1:] != srt[..., :-1]], axis=2)
    keep_sorted = first & (srt >= 0)
    nbs = [(L + bs - 1) // bs for L in cfg.seqlens]
    blkoff = np.concatenate([[0], np.cumsum(nbs)])
    g_tok = blkoff[s] + b                                    # global token block of each token
    if dense_split:
        H, K = block_idx.shape[1], block_idx.shape[2]
        ng = int(blkoff[-1])
        # per (token block, kv head, id): number of tokens of the block keeping id
        ids = np.where(keep_sorted, srt, 0)
        key = (g_tok[:, None, None] * H + np.arange(H)[None, :, None]) * (int(np.max(nbs)) + 1) + ids
        cnt = np.bincount(key[keep_sorted], minlength=ng * H * (int(np.max(nbs)) + 1))
        ntok = np.bincount(g_tok, minlength=ng)
        dense = cnt[key] == ntok[g_tok][:, None, None]
        keep_sorted = keep_sorted & ~dense
    g = blkoff[s][:, None, None] + srt
    bkey = np.arange(cfg.num_kv_heads)[None, :, None] * int(blkoff[-1]) + g
    # keys of an entry: the whole block below the token's own, i mod bs + 1 in it
    # (the workloads' sequence lengths are multiples of the block size)
    i = (t - cu[s])[:, None, None]
    keys = np.where(srt < b[:, None, None], bs, i % bs + 1)
    return int(keep_sorted.sum()), int(np.unique(bkey[keep_sorted]).size), int(keys[keep_sorted].sum())


def nonempty_buckets(cfg, block_idx) -> int:
    """(kv head, block) pairs that at least one row keeps."""
    bs = cfg.block_size
    nbs = [(L + bs - 1) // bs for L in cfg.seqlens]
    blkoff = np.concatenate([[0], np.cumsum(nbs)])
    cu = np.array([0] + list(np.cumsum(cfg.seqlens)))
    t = np.arange(cfg.total_tokens)
    s = np.searchsorted(cu, t, side="right") - 1
    b = (t - cu[s]) // bs
    valid = (block_idx >= 0) & (block_idx <= b[:, None, None])
    g = blkoff[s][:, None, None] + block_idx
    key = np.arange(cfg.num_kv_heads)[None, :, None] * int(blkoff[-1]) + g
    return int(np.unique(key[valid]).size)


def algorithmic_bytes(cfg, kind: str, nnz: int, nbne: int) -> int:
    """HBM bytes a main-kernel launch must move in this design, per unit:
    forward, per kept (token, kv head, block) entry: the G gathered query
    rows (G*d*2) in, the G partial outputs (G*d*2) and lse (G*4) out, the
    entry (4); per non-empty bucket the K and V block (bs*d*2*2).
    Backward, per entry: q and dout rows in (2*G*d*2), lse and delta (2*G*4),
    the dq partial rows out (G*d*2), the entry (4); per bucket K, V in and
    dk, dv out (4*bs*d*2)."""
    G, d, bs = cfg.group, cfg.head_dim, cfg.block_size
    if kind == "fwd":
        return nnz * (G * (4 * d + 4) + 4) + nbne * bs * d * 4
    return nnz * (G * (6 * d + 8) + 4) + nbne * bs * d * 8


def counter_traffic(kind: str, cfg_name: str, dense_split: bool):
    path = COUNTERS[kind]
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        cnt = json.load(f)
    if cnt.get("kernel_src_sha") != kernel_src_sha(kind) or cnt.get("config") != cfg_name or \
            (kind == "fwd" and cnt.get("dense_split", False) != dense_split):
        log(f"{os.path.relpath(path, ROOT)} does not match this kernel source or configuration: traffic = null")
        return None, None
    return cnt["hbm_bytes_per_launch"], os.path.relpath(path, ROOT)


def window_keys(cfg, window: int) -> int:
    """Attended (token, key) pairs of the window branch, per kv head."""
    n = 0
    for L in cfg.seqlens:
        i = np.arange(L, dtype=np.int64)
        n += int(np.minimum(i + 1, window).sum())
    return n


def cpu_baseline_window(cfg, d, window: int, target_s: float):
    """The window oracle, as it is, on a bounded sample of (token, kv head) rows."""
    import oracle
    import workloads as W
    q, k, v = (W.as_f32(d[n], cfg.dtype) for n in ("q", "k", "v"))
    Hkv, G, D = cfg.num_kv_heads, cfg.group, cfg.head_dim
    rng = np.random.default_rng(1234)
    nrows_total = cfg.total_tokens * Hkv
    cu = np.array([0] + list(np.cumsum(cfg.seqlens)))

    def run(n):
        rows = np.sort(rng.choice(nrows_total, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.window_fwd(q, k, v, d["cu_seqlens"], window, cfg.scale, rows=rows)
        dt = time.perf_counter() - t0
        t = rows // Hkv
        i = t - cu[np.searchsorted(cu, t, side="right") - 1]
        return dt, 4.0 * D * G * float(np.minimum(i + 1, window).sum()), n

    dt, fl, n = run(2000)
    dt, fl, n = run(int(min(nrows_total, max(n, n * target_s / max(dt, 1e-3)))))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = min(threads, os.cpu_count() or threads)
    return {
        "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{n} of {nrows_total} (token, kv head) rows drawn uniformly (seed 1234), all {G} "
                  f"query heads each, fp64 C/OpenMP window oracle (4d FLOP per query head and key), "
                  f"{dt:.1f} s wall, {fl / 1e9:.1f} GFLOP",
        "seconds": dt,
    }


def cpu_baseline(cfg, d, target_s: float, train: bool):
    """The oracle, as it is, on a bounded sample of (token, kv head) rows."""
    import oracle
    import workloads as W
    q, k, v = (W.as_f32(d[n], cfg.dtype) for n in ("q", "k", "v"))
    do = W.as_f32(d["do"], cfg.dtype) if train else None
    Hkv, G, D = cfg.num_kv_heads, cfg.group, cfg.head_dim
    rng = np.random.default_rng(1234)
    nrows_total = cfg.total_tokens * Hkv

    def run(n):
        rows = np.sort(rng.choice(nrows_total, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        if train:
            oracle.bwd_dq_rows(q, k, v, d["cu_seqlens"], d["block_idx"], do, cfg.block_size,
                               cfg.scale, rows)
        else:
            oracle.fwd(q, k, v, d["cu_seqlens"], d["block_idx"], cfg.block_size, cfg.scale,
                       rows=rows)
        dt = time.perf_counter() - t0
        t_rows = rows // Hkv
        keys = visible_keys_per_row(cfg, d["block_idx"][t_rows, rows % Hkv], t_rows)
        # fwd: 4d per (query head, key); dq rows: the row's forward (4d), dP (2d), dq (2d)
        return dt, (8.0 if train else 4.0) * D * G * float(keys.sum()), n

    dt, fl, n = run(500 if train else 2000)
    n2 = int(min(nrows_total, max(n, n * target_s / max(dt, 1e-3))))
    dt, fl, n = run(n2)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = min(threads, os.cpu_count() or threads)
    what = ("dq of the rows (their forward, dP and dq: 8d FLOP per query head and key)"
            if train else "forward of the rows (4d FLOP per query head and key)")
    return {
        "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{n} of {nrows_total} (token, kv head) rows drawn uniformly (seed 1234), "
                  f"all {G} query heads each, fp64 C/OpenMP oracle, {what}, {dt:.1f} s wall, "
                  f"{fl / 1e9:.1f} GFLOP",
        "seconds": dt,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--gather-only", action="store_true",
                    help="no dense split: every kept block through the gather path")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--branch", default="selection", choices=["selection", "window", "select"],
                    help="selection: the selected-attention forward (the headline); window: the "
                         "sliding-window branch; select: the index producer (block lists)")
    ap.add_argument("--window", type=int, default=512)
    args = ap.parse_args()
    args.dense_split = not args.gather_only
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selected-attention path here runs on a "
              "single MI355X (no multi-GPU sharding is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import nsa_selected_block_amd as nsa
    import workloads as W

    cfg = W.CONFIGS[args.config]
    win = args.branch == "window"
    sel = args.branch == "select"
    train = cfg.with_grad and not win and not sel
    log(f"generating {cfg.name}: {cfg.description}")
    t0 = time.time()
    d = W.make_inputs(cfg)
    log(f"inputs ready in {time.time() - t0:.1f} s")
    dev = torch.device("cuda:0")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    cu, bi = to_dev(d["cu_seqlens"]), to_dev(d["block_idx"])
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = nsa.Workspace()
    if train:
        do = to_dev(d["do"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_b = nsa.Workspace()

    bi_out = torch.empty_like(bi)

    def step():
        if sel:
            nsa.select_blocks(q, k, cu, cfg.block_size, cfg.topk, cfg.scale, out=bi_out, workspace=ws)
            return
        if win:
            nsa.window_fwd(q, k, v, cu, args.window, cfg.scale, tile=cfg.block_size, out=out, lse=lse,
                           workspace=ws)
            return
        nsa.attn_fwd(q, k, v, cu, bi, cfg.block_size, cfg.scale, out=out, lse=lse, workspace=ws,
                     dense_split=args.dense_split)
        if train:
            nsa.attn_bwd(q, k, v, out, lse, do, cu, bi, cfg.block_size, cfg.scale,
                         dq=dq, dk=dk, dv=dv, workspace=ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # Every call of the timed region records HIP events on the stream its
    # kernels run on (torch's current stream), at its stage boundaries.
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nsa.profile_begin()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    prof = nsa.profile_end_all()
    fwd_ms, fwd_calls = prof["fwd"]
    bwd_ms, bwd_calls = prof["bwd"]
    win_ms, win_calls = prof["window"]
    total_ms = e0.elapsed_time(e1)
    ms = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {1e3 * wall / args.steps:.3f} ms/step)")
    if win:
        finish_window(args, cfg, d, ms, {kn: v_ / max(win_calls, 1) for kn, v_ in win_ms.items()})
        return
    if sel:
        sel_ms, sel_calls = prof["select"]
        finish_select(args, cfg, d, ms, {kn: v_ / max(sel_calls, 1) for kn, v_ in sel_ms.items()})
        return
    per_f = {kname: v_ / max(fwd_calls, 1) for kname, v_ in fwd_ms.items()}
    log("forward stage ms: " + ", ".join(f"{kname}={v_:.3f}" for kname, v_ in per_f.items()))
    per_b = None
    if train:
        per_b = {kname: v_ / max(bwd_calls, 1) for kname, v_ in bwd_ms.items()}
        log("backward stage ms: " + ", ".join(f"{kname}={v_:.3f}" for kname, v_ in per_b.items()))

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    flops_f = W.effective_flops(cfg)
    flops_b = flops_f * 10 // 4 if train else 0   # 10d per (query head, key): S, dP, dV, dK, dQ
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    value = (flops_f + flops_b) / (ms * 1e-3) / 1e12

    # dominant kernel: the main kernel of the forward, or of the backward in a training step
    kind = "bwd" if train else "fwd"
    main_ms = per_b["main"] if train else per_f["main"]
    kflops = flops_b if train else flops_f
    split = args.dense_split and bf16
    if split and not train:
        # the main kernel's own share: the entries outside the dense sets
        nnz, nbne, main_keys = gather_units(cfg, d["block_idx"], True)
        kflops = 4 * cfg.head_dim * cfg.group * main_keys
    else:
        nnz = W.rows_per_block_nnz(cfg)
        nbne = nonempty_buckets(cfg, d["block_idx"])
    alg = algorithmic_bytes(cfg, kind, nnz, nbne)
    traffic, src = counter_traffic(kind, cfg.name, split) if bf16 else (None, None)
    kname = ("k_bwd_main" if train else
             "k_main_h" if bf16 else "k_main_f32")
    roofline = {
        "kernel": kname, "bound": "hbm",
        "achieved": alg / (main_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": alg / (main_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": traffic,
        "algorithmic_bytes": alg, "kernel_ms": main_ms, "traffic_source": src,
        "units": {"entries": nnz, "nonempty_buckets": nbne},
    }
    roofline_mfma = {
        "kernel": kname, "bound": "mfma",
        "achieved": kflops / (main_ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
        "frac": kflops / (main_ms * 1e-3) / 1e12 / peak,
    }

    record = {
        "metric": METRIC_TRAIN if train else METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded; shapes, value law and block-index rule of the workload)",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "seqlens": list(cfg.seqlens), "num_q_heads": cfg.num_q_heads,
            "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
            "block_size": cfg.block_size, "topk": cfg.topk, "seed": cfg.seed,
            "effective_flop": flops_f + flops_b, "dense_split": split,
            "step": "forward + backward" if train else "forward",
        },
        "pct_mfma_peak": 100.0 * value / peak,
        "stage_ms": per_f if not train else {"fwd": per_f, "bwd": per_b},
        "roofline": roofline,
        "roofline_mfma": roofline_mfma,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a row sample (~{args.cpu_seconds:.0f} s)")
        record["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_seconds, train)
        log(f"cpu baseline: {record['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s")
    print(json.dumps(record), flush=True)


def finish_window(args, cfg, d, ms, per):
    """JSON line of the sliding-window branch (MFMA-bound: ~4d*window FLOP per
    row against 2*d*2 + 4 bytes of q/out/lse and K/V read once)."""
    log("window stage ms: " + ", ".join(f"{kn}={v_:.3f}" for kn, v_ in per.items()))
    G, D, Hkv = cfg.group, cfg.head_dim, cfg.num_kv_heads
    flops = 4 * D * G * Hkv * window_keys(cfg, args.window)
    peak = PEAK_BF16_TFLOPS
    kms = per["window"]
    T = cfg.total_tokens
    alg = T * cfg.num_q_heads * (2 * D * 2 + 4) + 2 * T * Hkv * D * 2
    record = {
        "metric": METRIC_WINDOW,
        "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes and value law of the workload)",
        "config": {"workload": f"{cfg.name} tensors, sliding window {args.window}",
                   "seqlens": list(cfg.seqlens), "num_q_heads": cfg.num_q_heads,
                   "num_kv_heads": Hkv, "head_dim": D, "tile": cfg.block_size,
                   "window": args.window, "effective_flop": flops, "step": "window forward"},
        "pct_mfma_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / peak,
        "stage_ms": per,
        "roofline": {"kernel": "k_dense_attn (window)", "bound": "mfma",
                     "achieved": flops / (kms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
                     "frac": flops / (kms * 1e-3) / 1e12 / peak, "traffic": None, "kernel_ms": kms},
        "roofline_hbm": {"kernel": "k_dense_attn (window)", "bound": "hbm",
                         "achieved": alg / (kms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": alg / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": alg},
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: window oracle on a row sample (~{args.cpu_seconds:.0f} s)")
        record["cpu_baseline"] = cpu_baseline_window(cfg, d, args.window, args.cpu_seconds)
    print(json.dumps(record), flush=True)


def visible_windows(cfg) -> int:
    """(token) x visible compressed windows (kernel 32, stride 16), summed."""
    n = 0
    for L in cfg.seqlens:
        i = np.arange(L, dtype=np.int64)
        nc = (L - 32) // 16 + 1 if L >= 32 else 0
        n += int(np.minimum(np.where(i >= 31, (i - 31) // 16 + 1, 0), nc).sum())
    return n


def cpu_baseline_select(cfg, d, target_s: float):
    """The index-producer oracle, as it is, on a bounded sample of rows."""
    import oracle
    import workloads as W
    q, k = (W.as_f32(d[n], cfg.dtype) for n in ("q", "k"))
    Hkv, G, D = cfg.num_kv_heads, cfg.group, cfg.head_dim
    rng = np.random.default_rng(1234)
    nrows_total = cfg.total_tokens * Hkv
    cu = np.array([0] + list(np.cumsum(cfg.seqlens)))

    def run(n):
        rows = np.sort(rng.choice(nrows_total, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.select(q, k, d["cu_seqlens"], cfg.scale, cfg.dtype, topk=cfg.topk, rows=rows)
        dt = time.perf_counter() - t0
        t = rows // Hkv
        s = np.searchsorted(cu, t, side="right") - 1
        i = t - cu[s]
        nc = np.array([(L - 32) // 16 + 1 if L >= 32 else 0 for L in cfg.seqlens])[s]
        nvis = np.minimum(np.where(i >= 31, (i - 31) // 16 + 1, 0), nc)
        return dt, 2.0 * D * G * float(nvis.sum()), n

    # the first calls also build the compressed keys of the whole workload:
    # size the sample from the growth between two row counts
    dt1, _, n1 = run(200)
    dt2, _, n2 = run(2000)
    per_row = max((dt2 - dt1) / (n2 - n1), 1e-7)
    dt, fl, n = run(int(min(nrows_total, max(n2, (target_s - dt1) / per_row))))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = min(threads, os.cpu_count() or threads)
    return {
        "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{n} of {nrows_total} (token, kv head) rows drawn uniformly (seed 1234), all {G} query "
                  f"heads each, fp64 C/OpenMP index-producer oracle (2d FLOP per query head and visible "
                  f"window; the compressed keys of the whole workload are built first, inside the timing), "
                  f"{dt:.1f} s wall, {fl / 1e9:.1f} GFLOP",
        "seconds": dt,
    }


def finish_select(args, cfg, d, ms, per):
    """JSON line of the index producer.  Effective work: the compressed-
    attention scores, 2d FLOP per (query head, visible window), counted once
    (the kernel evaluates them twice: log-sum-exp pass and binning pass)."""
    log("select stage ms: " + ", ".join(f"{kn}={v_:.3f}" for kn, v_ in per.items()))
    G, D, Hkv = cfg.group, cfg.head_dim, cfg.num_kv_heads
    flops = 2 * D * cfg.num_q_heads * visible_windows(cfg)
    peak = PEAK_BF16_TFLOPS
    kms = per["select"]
    T = cfg.total_tokens
    # HBM: q read once, the compressed keys written and read once, the lists written
    nc = sum((L - 32) // 16 + 1 for L in cfg.seqlens if L >= 32)
    alg = T * cfg.num_q_heads * D * 2 + 2 * nc * Hkv * D * 2 + T * Hkv * cfg.topk * 4
    record = {
        "metric": METRIC_SELECT,
        "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes and value law of the workload)",
        "config": {"workload": f"{cfg.name} tensors, compressed keys (kernel 32, stride 16), "
                               f"block {cfg.block_size}, topk {cfg.topk}, 1 init + 2 local blocks",
                   "seqlens": list(cfg.seqlens), "num_q_heads": cfg.num_q_heads,
                   "num_kv_heads": Hkv, "head_dim": D, "effective_flop": flops,
                   "step": "index producer"},
        "pct_mfma_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / peak,
        "stage_ms": per,
        "roofline": {"kernel": "k_select", "bound": "mfma",
                     "achieved": flops / (kms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
                     "frac": flops / (kms * 1e-3) / 1e12 / peak, "traffic": None, "kernel_ms": kms},
        "roofline_hbm": {"kernel": "k_select", "bound": "hbm",
                         "achieved": alg / (kms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": alg / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": alg},
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: index-producer oracle on a row sample (~{args.cpu_seconds:.0f} s)")
        record["cpu_baseline"] = cpu_baseline_select(cfg, d, args.cpu_seconds)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark: NSA selected-block attention forward (prefill) on one MI355X.

One step = one nsa_sel_attn_fwd call (index inversion -> main kernel ->
[dense kernel] -> merge) over the varlen 64K + 32K token, 32 query / 8 kv head (GQA-4),
d=128, block 64, topk 16 bf16 workload, inputs resident in HBM.  Prints one
JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config c2]
                    [--no-cpu-baseline] [--cpu-seconds 15]
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
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "nsa_selected_block_amd", "csrc", "attn_fwd.hip")
COUNTERS = os.path.join(ROOT, "profiles", "main_kernel_c2_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_src_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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


def cpu_baseline(cfg, d, target_s: float):
    """The oracle, as it is, on a bounded sample of (token, kv head) rows."""
    import oracle
    import workloads as W
    q, k, v = (W.as_f32(d[n], cfg.dtype) for n in ("q", "k", "v"))
    Hkv, G, D = cfg.num_kv_heads, cfg.group, cfg.head_dim
    rng = np.random.default_rng(1234)
    nrows_total = cfg.total_tokens * Hkv

    def run(n):
        rows = np.sort(rng.choice(nrows_total, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, d["cu_seqlens"], d["block_idx"], cfg.block_size, cfg.scale, rows=rows)
        dt = time.perf_counter() - t0
        t_rows = rows // Hkv
        keys = visible_keys_per_row(cfg, d["block_idx"][t_rows, rows % Hkv], t_rows)
        return dt, 4.0 * D * G * float(keys.sum()), n

    dt, fl, n = run(2000)
    n2 = int(min(nrows_total, max(2000, 2000 * target_s / max(dt, 1e-3))))
    dt, fl, n = run(n2)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = min(threads, os.cpu_count() or threads)
    return {
        "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{n} of {nrows_total} (token, kv head) rows drawn uniformly (seed 1234), "
                  f"all {G} query heads each, fp64 C/OpenMP oracle, {dt:.1f} s wall, "
                  f"{fl / 1e9:.1f} effective GFLOP",
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
    ap.add_argument("--dense-split", action="store_true",
                    help="compute blocks kept by whole token blocks with the dense kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selected-attention path here runs on a "
              "single MI355X (no multi-GPU sharding is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import nsa_selected_block_amd as nsa
    import workloads as W

    cfg = W.CONFIGS[args.config]
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

    def step():
        nsa.attn_fwd(q, k, v, cu, bi, cfg.block_size, cfg.scale, out=out, lse=lse, workspace=ws,
                     dense_split=args.dense_split)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

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
    stage_ms, calls = nsa.profile_end()
    total_ms = e0.elapsed_time(e1)
    ms = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {1e3 * wall / args.steps:.3f} ms/step)")
    per = {kname: v_ / max(calls, 1) for kname, v_ in stage_ms.items()}
    log("per stage ms: " + ", ".join(f"{kname}={v_:.3f}" for kname, v_ in per.items()))

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    flops = W.effective_flops(cfg)
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    value = flops / (ms * 1e-3) / 1e12
    main_tflops = flops / (per["main"] * 1e-3) / 1e12

    traffic = None
    hbm = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            cnt = json.load(f)
        if cnt.get("kernel_src_sha") == kernel_src_sha() and cnt.get("config") == cfg.name:
            traffic = cnt["hbm_bytes_per_launch"]
            hbm = {"bound": "hbm", "achieved": traffic / (per["main"] * 1e-3) / 1e9,
                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": traffic / (per["main"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                   "traffic": traffic, "source": os.path.relpath(COUNTERS, ROOT)}
        else:
            log("counter file is stale for this kernel source: traffic = null")

    record = {
        "metric": METRIC,
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
            "effective_flop": flops, "dense_split": args.dense_split,
        },
        "pct_mfma_peak": 100.0 * value / peak,
        "stage_ms": per,
        "roofline": {
            "kernel": "main (k_main_bf16)" if bf16 else "main (k_main_f32)",
            "bound": "mfma", "achieved": main_tflops, "peak": peak, "unit": "TFLOP/s",
            "frac": main_tflops / peak, "traffic": traffic,
        },
        "roofline_hbm": hbm,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a row sample (~{args.cpu_seconds:.0f} s)")
        record["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_seconds)
        log(f"cpu baseline: {record['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s")
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()

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
    "window": ["attn_fwd.hip", "device_common.h", "internal.h"],
    "select": ["select.hip", "device_common.h", "internal.h"],
}


# rocprofv3 counter summaries (bench.py --summarize-counters), per kind (fwd,
# bwd: the selection branch's forward and training step; window; select) and
# workload
def counters_path(kind: str, cfg_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"counters_{kind}_{cfg_name}.json")


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


def counter_traffic(kind: str, cfg_name: str, dense_split: bool, kname: str):
    """HBM bytes per launch of kernel `kname` from the committed counter
    summary of this workload, or (None, None) when there is none or it was
    taken from other kernel sources or another launch configuration."""
    path = counters_path(kind, cfg_name)
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        cnt = json.load(f)
    branch = {"window": "window", "select": "select"}.get(kind, "selection")
    if cnt.get(f"kernel_src_sha_{kind}") != kernel_src_sha(kind) or cnt.get("config") != cfg_name or \
            cnt.get("branch", "selection") != branch or \
            (kind == "fwd" and cnt.get("dense_split", False) != dense_split):
        log(f"{os.path.relpath(path, ROOT)} does not match this kernel source or configuration: traffic = null")
        return None, None
    keys = [k for k in cnt.get("kernels", {}) if k.startswith(kname + "<")]
    if len(keys) != 1 or "hbm_bytes" not in cnt["kernels"][keys[0]]:
        return None, None
    return cnt["kernels"][keys[0]]["hbm_bytes"], os.path.relpath(path, ROOT)


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
        n = min(n, nrows_total)
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


def cpu_baseline(cfg, d, target_s: float, train: bool, res=None, bi_dev=None):
    """The oracle, as it is, on a bounded sample of (token, kv head) rows,
    timed on the host's cores.  The same rows also give a parity check of the
    GPU results in `res` (out, lse; dq in a training step), and the oracle's
    inverted index is compared bit for bit with the GPU's."""
    import oracle
    import workloads as W
    q, k, v = (W.as_f32(d[n], cfg.dtype) for n in ("q", "k", "v"))
    do = W.as_f32(d["do"], cfg.dtype) if train else None
    Hkv, G, D = cfg.num_kv_heads, cfg.group, cfg.head_dim
    rng = np.random.default_rng(1234)
    nrows_total = cfg.total_tokens * Hkv

    def run(n):
        n = min(n, nrows_total)
        rows = np.sort(rng.choice(nrows_total, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        if train:
            r = oracle.bwd_dq_rows(q, k, v, d["cu_seqlens"], d["block_idx"], do, cfg.block_size,
                                   cfg.scale, rows)
        else:
            r = oracle.fwd(q, k, v, d["cu_seqlens"], d["block_idx"], cfg.block_size, cfg.scale,
                           rows=rows)
        dt = time.perf_counter() - t0
        t_rows = rows // Hkv
        keys = visible_keys_per_row(cfg, d["block_idx"][t_rows, rows % Hkv], t_rows)
        # fwd: 4d per (query head, key); dq rows: the row's forward (4d), dP (2d), dq (2d)
        return dt, (8.0 if train else 4.0) * D * G * float(keys.sum()), n, rows, r

    dt, fl, n, _, _ = run(500 if train else 2000)
    n2 = int(min(nrows_total, max(n, n * target_s / max(dt, 1e-3))))
    dt, fl, n, rows, ref = run(n2)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = min(threads, os.cpu_count() or threads)
    what = ("dq of the rows (their forward, dP and dq: 8d FLOP per query head and key)"
            if train else "forward of the rows (4d FLOP per query head and key)")
    rec = {
        "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{n} of {nrows_total} (token, kv head) rows drawn uniformly (seed 1234), "
                  f"all {G} query heads each, fp64 C/OpenMP oracle, {what}, {dt:.1f} s wall, "
                  f"{fl / 1e9:.1f} GFLOP",
        "seconds": dt,
    }
    if res is not None:
        T = cfg.total_tokens
        sel = (rows // Hkv, rows % Hkv)
        par = {"rows": int(rows.size)}
        if train:
            got = res["dq"].float().cpu().numpy().reshape(T, Hkv, G, D)[sel]
            par["max_abs_dq"] = float(np.abs(got - ref).max())
            par["tol"] = 5e-2
        else:
            ref_o, ref_l = ref
            got_o = res["out"].float().cpu().numpy().reshape(T, Hkv, G, D)[sel]
            got_l = res["lse"].cpu().numpy().reshape(T, Hkv, G)[sel]
            fin = np.isfinite(ref_l)
            par["max_abs_out"] = float(np.abs(got_o - ref_o).max())
            par["max_abs_lse"] = float(np.abs(got_l[fin] - ref_l[fin]).max()) if fin.any() else 0.0
            par["tol"] = [2e-2, 1e-3] if cfg.dtype == "bf16" else [1e-4, 1e-4]
        rec["parity"] = par
    if bi_dev is not None:
        import torch
        import nsa_selected_block_amd as nsa
        off, ent = nsa.build_index(torch.from_numpy(d["cu_seqlens"]).to(bi_dev.device), bi_dev,
                                   Hkv, cfg.block_size)
        ref_off, ref_ent = oracle.invert(d["cu_seqlens"], d["block_idx"], Hkv, cfg.block_size)
        nnz = int(ref_off[-1])
        rec["csr_bit_exact"] = bool(np.array_equal(off.cpu().numpy().astype(np.int64), ref_off) and
                                    np.array_equal(ent.cpu().numpy()[:nnz], ref_ent))
    return rec


_DEMANGLED = {}


def demangle(name: str) -> str:
    """Readable kernel name (c++filt where rocprofv3 wrote a mangled one)."""
    if not name.startswith("_Z"):
        return name
    if name not in _DEMANGLED:
        import subprocess
        try:
            out = subprocess.run(["c++filt", name], stdout=subprocess.PIPE, text=True, check=True).stdout.strip()
        except Exception:  # noqa: BLE001
            out = name
        if out == name:  # (this c++filt does not know the bf16 type code DF16b)
            out = _demangle_kernel(name)
        _DEMANGLED[name] = out
    return _DEMANGLED[name]


def _demangle_kernel(name: str) -> str:
    """name<args> of this library's kernels: nsa::[anonymous]::<name> with
    template arguments that are 16-bit types, ints and bools."""
    import re
    m = re.match(r"_ZN3nsa(?:12_GLOBAL__N_1)?(\d+)", name)
    if not m:
        return name
    i = m.end()
    n = int(m.group(1))
    base, rest = name[i:i + n], name[i + n:]
    if not rest.startswith("I"):
        return base
    args, j = [], 1
    while j < len(rest) and rest[j] != "E":
        if rest.startswith("DF16b", j):
            args.append("__bf16"); j += 5
        elif rest.startswith("DF16_", j):
            args.append("_Float16"); j += 5
        elif rest[j] == "L":
            k = rest.index("E", j)
            lit = rest[j + 1:k]
            args.append({"b0": "false", "b1": "true"}.get(lit, lit.lstrip("ij")))
            j = k + 1
        else:
            break
    return f"{base}<{', '.join(args)}>"


def summarize_counters(args):
    """Turns rocprofv3 --pmc outputs (counter_collection.csv files under the
    given directories) into the JSON record bench.py reads for `traffic`:
    per kernel, the mean of every counter over its dispatches; HBM bytes from
    FETCH_SIZE / WRITE_SIZE scaled by what the same counters read for the
    runtime's 1 GiB device copies (--copy-calibration) in the same runs; and,
    where the SQ counters were taken, MFMA-issued FLOP (512 per
    SQ_INSTS_VALU_MFMA_MOPS_BF16), MFMA busy fraction and LDS bank-conflict
    cycles per LDS instruction."""
    import csv
    import glob
    vals = {}   # kernel -> counter -> [values]
    for dd in args.summarize_counters:
        for path in glob.glob(os.path.join(dd, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    name = demangle(row["Kernel_Name"]).replace("nsa::(anonymous namespace)::", "")
                    name = name.replace("void ", "", 1).split("(")[0].strip()
                    vals.setdefault(name, {}).setdefault(row["Counter_Name"], []).append(
                        float(row["Counter_Value"]))
    mean = {k: {c: float(np.mean(v)) for c, v in cs.items()} for k, cs in vals.items()}
    copy = [k for k in vals if "copyBuffer" in k]
    fetch_scale = write_scale = None
    if copy:
        # the 1 GiB copies are the largest copy dispatches (the runtime's own
        # small copies of the inputs read a few KiB)
        c = vals[copy[0]]
        if "FETCH_SIZE" in c:
            fetch_scale = (1 << 20) / max(c["FETCH_SIZE"])     # KiB read by a 1 GiB copy -> bytes
        if "WRITE_SIZE" in c:
            write_scale = (1 << 20) / max(c["WRITE_SIZE"])
    per = {}
    for k, c in sorted(mean.items()):
        if "copyBuffer" in k:
            continue
        e = dict(c)
        if "FETCH_SIZE" in c and "WRITE_SIZE" in c and fetch_scale and write_scale:
            e["hbm_bytes"] = (c["FETCH_SIZE"] * fetch_scale + c["WRITE_SIZE"] * write_scale) * 1024.0
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            e["mfma_issued_flop"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c and c["GRBM_GUI_ACTIVE"] > 0:
            # GRBM_GUI_ACTIVE comes summed over the 8 XCDs; 1024 SIMDs
            e["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8.0 * 1024.0)
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_INSTS_LDS" in c and c["SQ_INSTS_LDS"] > 0:
            e["lds_conflict_cycles_per_instr"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_INSTS_LDS"]
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c and c["SQ_LDS_IDX_ACTIVE"] > 0:
            e["lds_conflict_frac"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
        per[k] = e
    rec = {"config": args.config, "branch": args.branch, "dense_split": not args.gather_only,
           "fetch_scale": fetch_scale,
           "write_scale": write_scale, "kernels": per, "sources": list(args.summarize_counters)}
    for kind in KERNEL_SRCS:
        rec[f"kernel_src_sha_{kind}"] = kernel_src_sha(kind)
    print(json.dumps(rec, indent=1))


def summarize_trace(args):
    """Markdown table of a rocprofv3 --kernel-trace --stats run: every
    kernel_stats.csv under the given directories, durations in microseconds,
    kernel names demangled."""
    import csv
    import glob
    for dd in args.summarize_trace:
        for path in sorted(glob.glob(os.path.join(dd, "**", "*kernel_stats.csv"), recursive=True)):
            print(f"`{os.path.relpath(path, dd)}`:\n")
            print("| kernel | calls | average us | min us | max us | % |")
            print("|---|---|---|---|---|---|")
            with open(path) as f:
                for row in csv.DictReader(f):
                    name = demangle(row["Name"]).replace("nsa::(anonymous namespace)::", "")
                    name = name.replace("void ", "", 1).split("(")[0].strip()
                    print(f"| {name} | {row['Calls']} | {float(row['AverageNs']) / 1e3:.1f} | "
                          f"{float(row['MinNs']) / 1e3:.1f} | {float(row['MaxNs']) / 1e3:.1f} | "
                          f"{float(row['Percentage']):.2f} |")
            print()


def membw(args):
    """Read bandwidth of the GPU over working sets from 16 MB to 4 GB (the
    probe library's kernel: 16-byte loads, default cache policy, repeated
    passes over the buffer, about 16 GB read per measurement).  A working set
    that the 256 MB memory-side cache holds reads at its rate, a larger one
    at the HBM rate."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "nsa_selected_block_amd", "probe", "libnsa_probe.so"))
    lib.nsa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.nsa_probe_read.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * 16
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    buf = torch.ones(4 << 30, dtype=torch.uint8, device=dev)
    rows = []
    for mb in (32, 64, 96, 128, 160, 192, 256, 384, 512, 1024, 4096):
        nbytes = mb << 20
        reps = max(1, (16 << 30) // nbytes)
        run = lambda: lib.nsa_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, reps, blocks,
                                         ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        for _ in range(2):
            if run() != 0:
                raise RuntimeError("probe launch failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(3):
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            times.append(e0.elapsed_time(e1))
        ms = min(times)
        gbs = nbytes * reps / (ms * 1e-3) / 1e9
        rows.append({"working_set_mb": mb, "passes": reps, "ms": ms, "read_gbps": gbs})
        log(f"working set {mb:5d} MB: {gbs:8.1f} GB/s ({reps} passes, {ms:.2f} ms)")
    # gathers of 1 KB pieces at random places of 4 GB, 13 in flight per wave
    # (the merges' read pattern: one partial output group per kept slot)
    lib.nsa_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.nsa_probe_gather.restype = ctypes.c_int
    grows = []
    for gblocks in (cus * 4, cus * 8, cus * 16, cus * 32):
        waves = gblocks * 4
        iters = max(1, (16 << 30) // (waves * 13 * 1024))
        run = lambda: lib.nsa_probe_gather(ctypes.c_void_p(buf.data_ptr()), 4 << 30, iters, gblocks,
                                           ctypes.c_void_p(gsink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        gsink = torch.empty(gblocks * 256, dtype=torch.int32, device=dev)
        for _ in range(2):
            if run() != 0:
                raise RuntimeError("probe launch failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(3):
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            times.append(e0.elapsed_time(e1))
        ms = min(times)
        gbs = waves * iters * 13 * 1024 / (ms * 1e-3) / 1e9
        grows.append({"workgroups": gblocks, "waves": waves, "iters": iters, "ms": ms, "read_gbps": gbs})
        log(f"1 KB gathers, {gblocks} workgroups: {gbs:8.1f} GB/s ({iters} x 13 pieces per wave, {ms:.2f} ms)")
    # the same gathers (8 workgroups per CU) over buffers of 0.25 to 16 GB: the
    # partials the merges read span about 10-13 GB at the 64K+32K workload
    del buf
    torch.cuda.empty_cache()
    srows = []
    gblocks = cus * 8
    waves = gblocks * 4
    iters = max(1, (16 << 30) // (waves * 13 * 1024))
    gsink = torch.empty(gblocks * 256, dtype=torch.int32, device=dev)
    for mb in (256, 1024, 4096, 8192, 16384):
        nbytes = mb << 20
        gbuf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        run = lambda: lib.nsa_probe_gather(ctypes.c_void_p(gbuf.data_ptr()), nbytes, iters, gblocks,
                                           ctypes.c_void_p(gsink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        for _ in range(2):
            if run() != 0:
                raise RuntimeError("probe launch failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(3):
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            times.append(e0.elapsed_time(e1))
        ms = min(times)
        gbs = waves * iters * 13 * 1024 / (ms * 1e-3) / 1e9
        srows.append({"buffer_mb": mb, "workgroups": gblocks, "iters": iters, "ms": ms, "read_gbps": gbs})
        log(f"1 KB gathers over {mb:5d} MB: {gbs:8.1f} GB/s ({ms:.2f} ms)")
        del gbuf
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "read bandwidth by working set (16-byte loads, default cache policy)",
                      "unit": "GB/s", "n_gpus": 1, "blocks": blocks, "rows": rows,
                      "gather_1kb": grows, "gather_1kb_by_buffer": srows}), flush=True)


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
    ap.add_argument("--branch", default="selection", choices=["selection", "window", "select", "membw"],
                    help="selection: the selected-attention forward (the headline); window: the "
                         "sliding-window branch; select: the index producer (block lists); membw: "
                         "read bandwidth by working-set size (memory-side cache against HBM)")
    ap.add_argument("--window", type=int, default=512)
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print the JSON summary of rocprofv3 --pmc outputs under DIR... and exit")
    ap.add_argument("--summarize-trace", nargs="+", metavar="DIR",
                    help="print the per-kernel table of rocprofv3 --kernel-trace --stats outputs "
                         "under DIR... and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    args.dense_split = not args.gather_only
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selected-attention path here runs on a "
              "single MI355X (no multi-GPU sharding is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.branch == "membw":
        membw(args)
        return
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

    def step(timer=None):
        ev = timer.next() if timer is not None else None
        if sel:
            nsa.select_blocks(q, k, cu, cfg.block_size, cfg.topk, cfg.scale, out=bi_out, workspace=ws,
                              stage_events=ev)
            return
        if win:
            nsa.window_fwd(q, k, v, cu, args.window, cfg.scale, tile=cfg.block_size, out=out, lse=lse,
                           workspace=ws, stage_events=ev)
            return
        nsa.attn_fwd(q, k, v, cu, bi, cfg.block_size, cfg.scale, out=out, lse=lse, workspace=ws,
                     dense_split=args.dense_split, stage_events=ev)
        if train:
            nsa.attn_bwd(q, k, v, out, lse, do, cu, bi, cfg.block_size, cfg.scale,
                         dq=dq, dk=dk, dv=dv, workspace=ws_b,
                         stage_events=timer_b.next() if timer is not None else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # Every call of the timed region records caller-owned HIP events on the
    # stream its kernels run on (torch's current stream), at its stage
    # boundaries.
    stream = torch.cuda.current_stream(dev)
    timer = nsa.StageTimer(args.steps, dev)
    timer_b = nsa.StageTimer(args.steps, dev) if train else None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step(timer)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    names = nsa.SEL_STAGES if sel else nsa.WIN_STAGES if win else nsa.FWD_STAGES
    fwd_ms, fwd_calls = timer.stage_ms(names), args.steps
    bwd_ms, bwd_calls = (timer_b.stage_ms(nsa.BWD_STAGES), args.steps) if train else ({}, 0)
    win_ms = sel_ms = fwd_ms
    win_calls = sel_calls = fwd_calls
    total_ms = e0.elapsed_time(e1)
    ms = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {1e3 * wall / args.steps:.3f} ms/step)")
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")
    if win:
        finish_window(args, cfg, d, ms, {kn: v_ / max(win_calls, 1) for kn, v_ in win_ms.items()})
        return
    if sel:
        finish_select(args, cfg, d, ms, {kn: v_ / max(sel_calls, 1) for kn, v_ in sel_ms.items()})
        return
    per_f = {kname: v_ / max(fwd_calls, 1) for kname, v_ in fwd_ms.items()}
    log("forward stage ms: " + ", ".join(f"{kname}={v_:.3f}" for kname, v_ in per_f.items()))
    per_b = None
    if train:
        per_b = {kname: v_ / max(bwd_calls, 1) for kname, v_ in bwd_ms.items()}
        log("backward stage ms: " + ", ".join(f"{kname}={v_:.3f}" for kname, v_ in per_b.items()))
    step_ms = step_times(timer, timer_b)

    clock = clock_under_load(lambda: step(None), args.steps, dev)

    flops_f = W.effective_flops(cfg)
    flops_b = flops_f * 10 // 4 if train else 0   # 10d per (query head, key): S, dP, dV, dK, dQ
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    value = (flops_f + flops_b) / (ms * 1e-3) / 1e12

    # FLOP of each forward stage: the main kernel's own entries (with the
    # dense split, the entries outside the dense sets), the dense kernel the rest
    split = args.dense_split and bf16
    nnz, nbne, main_keys = gather_units(cfg, d["block_idx"], split)
    main_flop = 4 * cfg.head_dim * cfg.group * main_keys
    stage_flop = {"main": main_flop, "dense": flops_f - main_flop if split else 0}
    if train:
        kind, kname, kstage, kms, kflops = "bwd", "k_bwd_main", "main", per_b["main"], flops_b
    else:
        # dominant forward kernel: the longer of the main and the dense kernel
        kstage = "dense" if split and per_f["dense"] > per_f["main"] else "main"
        kms, kflops, kind = per_f[kstage], stage_flop[kstage], "fwd"
        kname = {"main": "k_main_h" if bf16 else "k_main_f32", "dense": "k_dense_attn (merge inside)"}[kstage]
    alg = algorithmic_bytes(cfg, kind, nnz, nbne)
    traffic, src = counter_traffic(kind, cfg.name, split, kname.split(" ")[0]) if bf16 else (None, None)
    units = {"attended_key_pairs": (main_keys if kstage == "main" else None) if not train else None,
             "entries": nnz, "nonempty_buckets": nbne}
    roofline = {
        "kernel": kname, "bound": "mfma" if bf16 else "alu",
        "achieved": kflops / (kms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
        "frac": kflops / (kms * 1e-3) / 1e12 / peak, "traffic": traffic,
        "flop_per_launch": kflops,
        "unit_work": ("10d FLOP per attended (query head, key): S, dP, dV, dK, dQ" if train else
                      "4d FLOP per attended (query head, key): QK^T and PV"),
        "units": units, "kernel_ms": kms, "traffic_source": src,
    }
    # the same kernel against HBM: this design's bytes (per-entry query gather
    # and per-slot partials, K/V once per bucket) and the counters' bytes
    roofline_hbm = None
    if kstage == "main":
        roofline_hbm = {
            "kernel": kname, "bound": "hbm", "achieved": alg / (kms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": alg / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS, "design_bytes_per_launch": alg,
            "counter_bytes_per_launch": traffic,
            "counter_gbps": traffic / (kms * 1e-3) / 1e9 if traffic else None,
            "counter_frac": traffic / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS if traffic else None,
        }
    # the method's own bytes (q, k, v, block_idx in; out, lse out) over the
    # whole forward: what an ideal single pass would move
    elt = 2 if bf16 else 4
    T, Hq, Hkv, D = cfg.total_tokens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    method_bytes = T * Hq * D * elt * 2 + 2 * T * Hkv * D * elt + T * Hkv * cfg.topk * 4 + T * Hq * 4
    fwd_total = sum(per_f.values())
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
            "input_sha256": {n: W.sha256(d[n])[:16] for n in sorted(d)},
        },
        "pct_mfma_peak": 100.0 * value / peak,
        "ms_median": float(np.median(step_ms)), "ms_min": float(np.min(step_ms)),
        "ms_p90": float(np.percentile(step_ms, 90)),
        "stage_ms": per_f if not train else {"fwd": per_f, "bwd": per_b},
        "roofline": roofline,
        "roofline_hbm": roofline_hbm,
        "method_bytes": {"bytes": method_bytes, "forward_ms": fwd_total,
                         "gbps": method_bytes / (fwd_total * 1e-3) / 1e9,
                         "frac": method_bytes / (fwd_total * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "clock_mhz": clock,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a row sample (~{args.cpu_seconds:.0f} s)")
        res = {"out": out, "lse": lse}
        if train:
            res["dq"] = dq
        record["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_seconds, train, res, bi)
        log(f"cpu baseline: {record['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s; parity "
            f"{record['cpu_baseline']['parity']}")
    print(json.dumps(record), flush=True)


def step_times(timer, timer_b):
    """Per-step ms from each call's first and last stage event (forward, plus
    the backward in a training step)."""
    out = []
    for i in range(timer.used):
        evs = timer.events[i]
        evs[-1].synchronize()
        t = evs[0].elapsed_time(evs[-1])
        if timer_b is not None:
            eb = timer_b.events[i]
            eb[-1].synchronize()
            t = evs[0].elapsed_time(eb[-1])
        out.append(t)
    return np.array(out)


def clock_under_load(run_step, steps, dev):
    """GFX clock (MHz, mean over the XCDs) sampled with amdsmi while more
    steps run (outside the timed region); None where amdsmi is unavailable."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # noqa: BLE001 - diagnostics only
        log(f"clock: amdsmi unavailable ({e})")
        return None
    samples, stop = [], threading.Event()

    def read_mhz():
        # per-XCC current GFX clocks from the metrics table where present
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            xs = m.get("current_gfxclks")
            xs = [float(x) for x in xs if isinstance(x, (int, float)) and 0 < x < 10000] if \
                isinstance(xs, (list, tuple)) else []
            if xs:
                return float(np.mean(xs))
            x = m.get("current_gfxclk")
            if isinstance(x, (int, float)) and 0 < x < 10000:
                return float(x)
        except Exception:  # noqa: BLE001
            pass
        info = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
        return float(info.get("clk", info.get("cur_clk", 0)))

    def poll():
        while not stop.is_set():
            try:
                samples.append((time.perf_counter(), read_mhz()))
            except Exception:  # noqa: BLE001
                pass
            time.sleep(0.02)

    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    # the metrics table refreshes about once a second: load the GPU for 3 s
    # and keep the samples of the last 1.5 s
    while time.perf_counter() - t0 < 3.0:
        for _ in range(steps):
            run_step()
        torch.cuda.synchronize(dev)
    stop.set()
    th.join()
    samples = [v for (ts, v) in samples if ts - t0 >= 1.5]
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    if not samples:
        return None
    arr = np.array(samples)
    return {"median": float(np.median(arr)), "min": float(arr.min()), "max": float(arr.max()),
            "samples": int(arr.size)}


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
    traffic, src = counter_traffic("window", cfg.name, True, "k_dense_attn")
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
                     "frac": flops / (kms * 1e-3) / 1e12 / peak, "traffic": traffic, "kernel_ms": kms,
                     "traffic_source": src},
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
        n = min(n, nrows_total)
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
    traffic, src = counter_traffic("select", cfg.name, True, "k_select")
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
                     "frac": flops / (kms * 1e-3) / 1e12 / peak, "traffic": traffic, "kernel_ms": kms,
                     "traffic_source": src},
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

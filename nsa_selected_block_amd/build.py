"""Build ``libnsa_sel.so`` (the HIP kernels plus the C ABI) for gfx950, in-tree.

Each source is compiled to an object of its own (in parallel, under
``_build/`` at the repository root), then the objects are linked into the
shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "index.hip", "attn_fwd.hip", "attn_bwd.hip", "select.hip"]
LIB = os.path.join(HERE, "libnsa_sel.so")
# the benchmark's read-bandwidth probe: a library of its own
PROBE_SRC = os.path.join(HERE, "probe", "membw.hip")
PROBE_LIB = os.path.join(HERE, "probe", "libnsa_probe.so")
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _filter(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def _compile(src: str, extra) -> tuple:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj + ".tmp"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode == 0:
        os.replace(obj + ".tmp", obj)
    return src, obj, res.returncode, _filter(res.stdout), " ".join(cmd)


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source for gfx950 and link libnsa_sel.so; `extra` adds
    compiler flags (e.g. -D tuning macros)."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    for src, obj, rc, out, cmd in results:
        if verbose:
            print(cmd, flush=True)
            if out.strip():
                print(out, flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{out}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[r[1] for r in results], "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if verbose:
        print(" ".join(cmd), flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_filter(res.stdout)}")
    os.replace(tmp, LIB)
    cmd = [HIPCC, *FLAGS, "-shared", *extra, PROBE_SRC, "-o", PROBE_LIB + ".tmp"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if verbose:
        print(" ".join(cmd), flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on the probe ({res.returncode}):\n{_filter(res.stdout)}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, extra=[a for a in sys.argv[1:] if a.startswith("-D")])
    print(LIB)

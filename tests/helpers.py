"""Shared helpers for the GPU tests: moving generated inputs to the device,
reading results back, and the tolerance checks."""
import numpy as np

import workloads as W

# (max-abs out, max-abs lse); fp16 takes the bf16 bounds (the pages test both
# 16-bit types and state no tolerance; fp16 carries 3 more mantissa bits)
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-3), "f16": (2e-2, 1e-3)}


def to_dev(a: np.ndarray, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def f32_of(a: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.ascontiguousarray(a, np.float32)


def from_dev(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def compare(out, lse, ref_o, ref_l, dtype, what=""):
    """Max-abs parity of (out, lse) against the oracle; returns (err_o, err_l)."""
    tol_o, tol_l = TOL[dtype]
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf pattern differs"
    assert np.all(np.isneginf(lse[~fin])), what
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err_o = float(np.abs(out.astype(np.float64) - ref_o).max()) if out.size else 0.0
    err_l = float(np.abs(lse[fin].astype(np.float64) - ref_l[fin]).max()) if fin.any() else 0.0
    print(f"{what}: max|dO|={err_o:.3e} (tol {tol_o}) max|dLSE|={err_l:.3e} (tol {tol_l})",
          flush=True)
    assert err_o <= tol_o, f"{what}: out error {err_o}"
    assert err_l <= tol_l, f"{what}: lse error {err_l}"
    return err_o, err_l


def random_case(rng, seqlens, Hkv, G, D, bs, topk, dtype, junk=True, value_scale=1.0):
    """Random inputs with arbitrary block ids (-1, repeats, future and
    out-of-range ids included when junk is set)."""
    cu = W.cu_seqlens_of(seqlens)
    T = int(cu[-1])
    if dtype == "bf16":
        mk = lambda shp: W.f32_to_bf16_bits(value_scale * rng.standard_normal(shp, dtype=np.float32))
    elif dtype == "f16":
        mk = lambda shp: (value_scale * rng.standard_normal(shp, dtype=np.float32)).astype(np.float16)
    else:
        mk = lambda shp: (value_scale * rng.standard_normal(shp, dtype=np.float32)).astype(np.float32)
    q, k, v = mk((T, Hkv * G, D)), mk((T, Hkv, D)), mk((T, Hkv, D))
    nbmax = max([(L + bs - 1) // bs for L in seqlens] + [1])
    if junk:
        bi = rng.integers(-1, nbmax + 1, size=(T, Hkv, topk)).astype(np.int32)
    else:
        bi = rng.integers(0, nbmax, size=(T, Hkv, topk)).astype(np.int32)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, block_idx=bi)

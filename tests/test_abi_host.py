"""C-ABI checks that need no GPU: the library loads, exports every function
that include/nsa_sel.h declares, and rejects bad descriptors and arguments on
the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

import nsa_selected_block_amd as nsa
from nsa_selected_block_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"\b(nsa_sel_\w+)\s*\(", src)
    return sorted(set(names))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(nsa.lib, n), n


def test_desc_layout_matches_header():
    assert ctypes.sizeof(_abi.Desc) == 56
    assert _abi.Desc.total_tokens.offset == 16
    assert _abi.Desc.flags.offset == 44
    assert _abi.Desc.stage_events.offset == 48


def test_version_and_strings():
    assert nsa.version() == 2
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(nsa.status_string(s), str) and nsa.status_string(s)


def good():
    return nsa.make_desc(98304, 2, 32, 8, 128, 64, 16)


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 40, _abi.ERR_INVALID_ARG),
    ("num_seqs", 0, _abi.ERR_INVALID_ARG),
    ("total_tokens", -1, _abi.ERR_INVALID_ARG),
    ("num_q_heads", 30, _abi.ERR_INVALID_ARG),   # 30 % 8 != 0
    ("num_kv_heads", 0, _abi.ERR_INVALID_ARG),
    ("topk", 0, _abi.ERR_INVALID_ARG),
    ("flags", 2, _abi.ERR_INVALID_ARG),
    ("scale", float("nan"), _abi.ERR_INVALID_ARG),
    ("dtype", 4, _abi.ERR_UNSUPPORTED),
    ("dtype", 0, _abi.ERR_UNSUPPORTED),
    ("head_dim", 96, _abi.ERR_UNSUPPORTED),
    ("block_size", 16, _abi.ERR_UNSUPPORTED),
    ("topk", 65, _abi.ERR_UNSUPPORTED),
    ("num_q_heads", 8 * 128, _abi.ERR_UNSUPPORTED),  # G = 128
    ("total_tokens", (1 << 31) // (32 * 16), _abi.ERR_UNSUPPORTED),  # T * Hq * topk >= 2^31
])
def test_validate_rejects(field, value, status):
    d = good()
    assert nsa.validate(d) == 0
    setattr(d, field, value)
    assert nsa.validate(d) == status


def test_long_sequences_accepted():
    """More blocks per kv head than one LDS pass of the index build covers
    (12,288): the build walks the buckets in windows, so only the index-width
    limits apply."""
    d = nsa.make_desc(16384 * 64, 1, 1, 1, 64, 64, 16)
    assert nsa.validate(d) == 0
    d = nsa.make_desc(3 * 12288 * 64, 1, 2, 1, 64, 64, 8)
    assert nsa.validate(d) == 0


def test_head_dim_256_rules():
    """d = 256 takes 16-bit inputs, every block size in the forward and
    blocks of at most 64 keys in the backward."""
    d = good()
    d.head_dim = 256
    assert nsa.validate(d) == 0
    d.dtype = nsa.DTYPE_F16
    assert nsa.validate(d) == 0
    d.block_size = 32
    assert nsa.validate(d) == 0
    d.block_size = 128
    assert nsa.validate(d) == 0
    f = good()
    f.head_dim = 256
    f.dtype = nsa.DTYPE_F32
    assert nsa.validate(f) == _abi.ERR_UNSUPPORTED
    b = good()
    b.head_dim = 256
    n = ctypes.c_size_t()
    assert nsa.lib.nsa_sel_bwd_workspace_size(ctypes.byref(b), ctypes.byref(n)) == 0
    n128 = ctypes.c_size_t()
    assert nsa.lib.nsa_sel_bwd_workspace_size(ctypes.byref(good()), ctypes.byref(n128)) == 0
    assert n.value > n128.value
    b.block_size = 128
    assert nsa.lib.nsa_sel_bwd_workspace_size(ctypes.byref(b), ctypes.byref(n)) == _abi.ERR_UNSUPPORTED
    p = ctypes.c_void_p(0x2000)
    assert nsa.lib.nsa_sel_attn_bwd(ctypes.byref(b), *([p] * 11), ctypes.c_void_p(0x1000), 1 << 40,
                                    None) == _abi.ERR_UNSUPPORTED
    b.block_size = 64
    assert nsa.fwd_workspace_size(b) > nsa.fwd_workspace_size(good())


def test_validate_null():
    assert nsa.lib.nsa_sel_validate(None) == _abi.ERR_INVALID_ARG


def test_sizes():
    d = good()
    nb, ne = nsa.index_sizes(d)
    assert nb == 8 * (98304 // 64 + 2) and ne == 98304 * 8 * 16
    fw, iw = nsa.fwd_workspace_size(d), nsa.index_workspace_size(d)
    # partial outputs (bf16) and partial lse dominate the forward workspace
    assert fw >= ne * 4 * (128 * 2 + 4) and iw < fw
    d.total_tokens = 0
    assert nsa.fwd_workspace_size(d) > 0
    d2 = good()
    d2.dtype = nsa.DTYPE_F32
    assert nsa.fwd_workspace_size(d2) > fw


def test_entry_points_reject_before_enqueue():
    d = good()
    ws = ctypes.c_void_p(0x1000)  # never dereferenced: the host checks fail first
    p = ctypes.c_void_p(0x2000)
    rc = nsa.lib.nsa_sel_attn_fwd(ctypes.byref(d), None, p, p, p, p, p, p, ws, 1 << 40, None)
    assert rc == _abi.ERR_INVALID_ARG
    rc = nsa.lib.nsa_sel_attn_fwd(ctypes.byref(d), p, p, p, p, p, p, p, ws, 1024, None)
    assert rc == _abi.ERR_WORKSPACE
    rc = nsa.lib.nsa_sel_attn_fwd(ctypes.byref(d), p, p, p, p, p, p, p, None, 1 << 40, None)
    assert rc == _abi.ERR_WORKSPACE
    rc = nsa.lib.nsa_sel_build_index(ctypes.byref(d), p, p, None, p, ws, 1 << 40, None)
    assert rc == _abi.ERR_INVALID_ARG
    rc = nsa.lib.nsa_sel_build_index(ctypes.byref(d), p, p, p, p, ws, 16, None)
    assert rc == _abi.ERR_WORKSPACE
    bad = good()
    bad.head_dim = 80
    rc = nsa.lib.nsa_sel_attn_fwd(ctypes.byref(bad), p, p, p, p, p, p, p, ws, 1 << 40, None)
    assert rc == _abi.ERR_UNSUPPORTED
    st = ctypes.c_int()
    assert nsa.lib.nsa_sel_check(None, None, ctypes.byref(st)) == _abi.ERR_INVALID_ARG


def test_indexed_forward_host_checks():
    """nsa_sel_attn_fwd_indexed: null index arrays, the dense split flag, a
    short workspace and a bad descriptor are rejected before anything is
    enqueued; nsa_sel_workspace_size is the forward's workspace."""
    d = good()
    ws = ctypes.c_void_p(0x1000)
    p = ctypes.c_void_p(0x2000)
    f = nsa.lib.nsa_sel_attn_fwd_indexed
    assert f(ctypes.byref(d), p, p, p, p, p, None, p, p, p, ws, 1 << 40, None) == _abi.ERR_INVALID_ARG
    assert f(ctypes.byref(d), p, p, p, p, p, p, None, p, p, ws, 1 << 40, None) == _abi.ERR_INVALID_ARG
    assert f(ctypes.byref(d), p, p, p, p, p, p, p, p, None, ws, 1 << 40, None) == _abi.ERR_INVALID_ARG
    assert f(ctypes.byref(d), p, p, p, p, p, p, p, p, p, ws, 1024, None) == _abi.ERR_WORKSPACE
    ds = good()
    ds.flags = nsa.FLAG_DENSE_SPLIT
    assert f(ctypes.byref(ds), p, p, p, p, p, p, p, p, p, ws, 1 << 40, None) == _abi.ERR_UNSUPPORTED
    assert f(None, p, p, p, p, p, p, p, p, p, ws, 1 << 40, None) == _abi.ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert nsa.lib.nsa_sel_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == nsa.fwd_workspace_size(d)


def test_bwd_host_checks():
    d = good()
    bw = nsa.bwd_workspace_size(d)
    # per-slot dq partials (bf16) dominate the backward workspace
    assert bw >= 98304 * 8 * 16 * 4 * 128 * 2
    f = good()
    f.dtype = nsa.DTYPE_F32
    n = ctypes.c_size_t()
    assert nsa.lib.nsa_sel_bwd_workspace_size(ctypes.byref(f), ctypes.byref(n)) == _abi.ERR_UNSUPPORTED
    ws = ctypes.c_void_p(0x1000)
    p = ctypes.c_void_p(0x2000)
    args = [p] * 11  # q k v out lse dout cu_seqlens block_idx dq dk dv (never dereferenced)
    for i in range(11):
        a = list(args)
        a[i] = None
        rc = nsa.lib.nsa_sel_attn_bwd(ctypes.byref(d), *a, ws, 1 << 40, None)
        assert rc == _abi.ERR_INVALID_ARG, i
    assert nsa.lib.nsa_sel_attn_bwd(ctypes.byref(d), *args, ws, 1024, None) == _abi.ERR_WORKSPACE
    assert nsa.lib.nsa_sel_attn_bwd(ctypes.byref(d), *args, None, 1 << 40, None) == _abi.ERR_WORKSPACE
    assert nsa.lib.nsa_sel_attn_bwd(ctypes.byref(f), *args, ws, 1 << 40, None) == _abi.ERR_UNSUPPORTED
    fl = good()
    fl.flags = nsa.FLAG_DENSE_SPLIT
    assert nsa.lib.nsa_sel_attn_bwd(ctypes.byref(fl), *args, ws, 1 << 40, None) == _abi.ERR_INVALID_ARG


def test_output_buffers_checked_before_launch():
    """The forward wrappers accept only out / lse buffers the kernels may
    write in full: out of q's shape and dtype, lse float32 [T, Hq], both on
    q's device (CPU tensors stand in for device ones here)."""
    import torch
    q = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    _abi._check_out(torch.zeros_like(q), torch.zeros(10, 4), q)
    bad_out = [torch.zeros(9, 4, 64, dtype=torch.bfloat16), torch.zeros(10, 4, 32, dtype=torch.bfloat16),
               torch.zeros(10, 4, 64, dtype=torch.float16), torch.zeros(10, 4, 64, dtype=torch.bfloat16)[:, :2],
               torch.zeros(10, 256, dtype=torch.bfloat16)]
    for o in bad_out:
        with pytest.raises(ValueError):
            _abi._check_out(o, torch.zeros(10, 4), q)
    for l in (torch.zeros(10, 3), torch.zeros(9, 4), torch.zeros(10, 4, dtype=torch.float64), torch.zeros(40),
              torch.zeros(4, 10).t()):
        with pytest.raises(ValueError):
            _abi._check_out(torch.zeros_like(q), l, q)
    with pytest.raises(ValueError):
        _abi._check_out(torch.zeros_like(q), torch.zeros(10, 4, device="meta"), q)


def test_stage_events_field_is_ignored_by_host_entry_points():
    """The descriptor's caller-owned event array is only touched by compute
    calls; the host-only checks take a descriptor carrying one unchanged."""
    ev = (ctypes.c_void_p * _abi.STAGE_EVENTS)()
    d = nsa.make_desc(98304, 2, 32, 8, 128, 64, 16, stage_events=ev)
    assert d.stage_events == ctypes.addressof(ev)
    assert nsa.validate(d) == 0
    assert nsa.fwd_workspace_size(d) == nsa.fwd_workspace_size(good())


def test_product_path_has_no_oracle_dependency():
    """The package never imports or loads the oracle."""
    pkg = os.path.join(ROOT, "nsa_selected_block_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in src.lower(), fn


def test_noalloc_window_host_checks():
    """nsa_sel_window_fwd_noalloc rejects, before any HIP call, a problem
    whose window workspace exceeds its 64 KiB scratch and bad arguments."""
    p = ctypes.c_void_p(0x2000)
    f = nsa.lib.nsa_sel_window_fwd_noalloc
    big = nsa.make_desc(9000, 9000, 2, 1, 64, 64, 1)
    assert nsa.window_workspace_size(big) > 64 * 1024
    assert f(ctypes.byref(big), 16, p, p, p, p, p, p, None) == _abi.ERR_WORKSPACE
    d = nsa.make_desc(4096, 4, 8, 2, 128, 64, 1)
    assert nsa.window_workspace_size(d) <= 64 * 1024
    assert f(ctypes.byref(d), 0, p, p, p, p, p, p, None) == _abi.ERR_INVALID_ARG
    assert f(ctypes.byref(d), 16, None, p, p, p, p, p, None) == _abi.ERR_INVALID_ARG
    assert f(ctypes.byref(d), 16, p, p, p, None, p, p, None) == _abi.ERR_INVALID_ARG
    d.flags = nsa.FLAG_DENSE_SPLIT
    assert f(ctypes.byref(d), 16, p, p, p, p, p, p, None) == _abi.ERR_INVALID_ARG
    f32 = nsa.make_desc(4096, 4, 8, 2, 128, 64, 1, dtype=nsa.DTYPE_F32)
    assert f(ctypes.byref(f32), 16, p, p, p, p, p, p, None) == _abi.ERR_UNSUPPORTED
    assert f(None, 16, p, p, p, p, p, p, None) == _abi.ERR_INVALID_ARG

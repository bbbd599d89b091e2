"""The allocation-free sliding-window forward (nsa_sel_window_fwd_noalloc,
through the C ABI) against the workspace entry point nsa_sel_window_fwd:
bitwise equal out and lse on two calls in a row, the second with a smaller
input (fewer tokens and sequences, another head layout), so whatever the
first call left in the shared scratch must not leak into the second; a
problem larger than the scratch is rejected before anything runs."""
import numpy as np
import pytest

import nsa_selected_block_amd as nsa
from nsa_selected_block_amd import _abi
from helpers import random_case, to_dev

pytestmark = pytest.mark.gpu


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def both(seqlens, Hkv, G, D, window, tile, dtype, seed):
    import torch
    rng = np.random.default_rng(seed)
    d = random_case(rng, seqlens, Hkv, G, D, tile, 1, dtype)
    dd = {k: to_dev(a, dev()) for k, a in d.items()}
    scale = 1.0 / np.sqrt(D)
    o_ref, l_ref = nsa.window_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], window, scale, tile=tile)
    out = torch.full_like(dd["q"], 3.0)
    lse = torch.full((dd["q"].shape[0], dd["q"].shape[1]), 5.0, dtype=torch.float32, device=dev())
    nsa.window_fwd_noalloc(dd["q"], dd["k"], dd["v"], dd["cu_seqlens"], window, out, lse, scale, tile=tile)
    torch.cuda.synchronize()
    return out, lse, o_ref, l_ref


def test_noalloc_window_matches_workspace_entry_point():
    import torch
    print("no-alloc window: first call (5 sequences, 2700 tokens)", flush=True)
    o, l, o_ref, l_ref = both([700, 1, 0, 1500, 499], 2, 4, 128, 300, 64, "bf16", 3)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    print("no-alloc window: second, smaller call (2 sequences, 640 tokens)", flush=True)
    o, l, o_ref, l_ref = both([130, 510], 1, 2, 64, 100, 32, "f16", 4)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_window_rejects_beyond_scratch():
    """A batch whose window workspace exceeds the 64 KiB scratch: an error
    status, nothing launched (the outputs stay as they were)."""
    import torch
    seqlens = [1] * 9000
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)).to(dev())
    T = len(seqlens)
    q = torch.zeros(T, 2, 64, dtype=torch.bfloat16, device=dev())
    k = torch.zeros(T, 1, 64, dtype=torch.bfloat16, device=dev())
    out = torch.full_like(q, 3.0)
    lse = torch.full((T, 2), 5.0, dtype=torch.float32, device=dev())
    with pytest.raises(nsa.NsaSelError) as e:
        nsa.window_fwd_noalloc(q, k, k, cu, 16, out, lse)
    assert e.value.status == _abi.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 5.0)

"""MI355X-native NSA selected-block attention (prefill forward and backward), the
sliding-window branch and the index producer (block lists from compressed
attention).

Python face of the C ABI in ``include/nsa_sel.h``; the computation runs in
the HIP kernels of ``libnsa_sel.so`` (built in-tree by
``nsa_selected_block_amd.build``).
"""
from ._abi import (  # noqa: F401
    BWD_STAGES, WIN_STAGES, DTYPE_BF16, DTYPE_F16, DTYPE_F32, FLAG_DENSE_SPLIT, FWD_STAGES, Desc, NsaSelError, Workspace,
    attn_bwd, attn_fwd, attn_fwd_indexed, build_index, bwd_workspace_size, check,
    fwd_workspace_size, index_sizes, index_workspace_size, lib, make_desc, status_string,
    validate, version, LIB_PATH, window_fwd, window_fwd_noalloc, window_workspace_size,
    select_blocks, select_workspace_size, SEL_STAGES, STAGE_EVENTS, StageTimer,
)

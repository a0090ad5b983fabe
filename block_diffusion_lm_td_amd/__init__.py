"""Block-diffusion denoise step (TwoTower denoiser attention + confidence
commit, and the context-cache append after a block) on AMD MI355X: a thin
Python binding of libtd.so (include/td.h)."""
from ._td import (  # noqa: F401
    TD_BF16,
    TD_F32,
    TD_OK,
    TdAppendArgs,
    TdAttnArgs,
    TdCommitArgs,
    TdLmheadArgs,
    TdMambaArgs,
    Workspace,
    append_args,
    attn_args,
    commit_args,
    header_functions,
    lmhead_args,
    mamba_args,
    lib,
    status_str,
    td_block_attn,
    td_cache_append,
    td_commit,
    td_denoise_step,
    td_denoise_step_if,
    td_lmhead_commit,
    td_mamba_block_scan,
)

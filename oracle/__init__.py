"""fp64 CPU oracle of the block-diffusion denoise step (test infrastructure).

Only tests/, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may
import this package.  The product path never does.
"""
from .td_oracle import (  # noqa: F401
    block_attention,
    row_confidence,
    confidence_commit,
    commit_decision,
    denoise_step,
    denoise_loop,
    cache_append,
    lmhead_logits,
    lmhead_commit,
    mamba_block_scan,
    adaln_modulate,
)

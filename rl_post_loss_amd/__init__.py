"""rl_post_loss_amd: the GRPO loss hot path on AMD Instinct MI355X.

The compute lives in libgrpo.so (HIP kernels for gfx950 behind a C ABI,
declared in include/grpo.h).  This package is its thin torch binding.
"""

from ._abi import (  # noqa: F401
    GRPO_FAULT_BAD_ACTION,
    GRPO_FAULT_NO_TOKENS,
    GRPO_FAULT_NONFINITE,
    GrpoError,
    LIB_PATH,
    load_library,
)
from .loss import (  # noqa: F401
    GRPOResult,
    grpo_advantages,
    grpo_gdpo_advantages,
    grpo_loss,
    grpo_loss_bwd,
    grpo_loss_fwd_bwd,
    grpo_loss_fwd_bwd_noalloc,
    grpo_logp_loss,
    grpo_scale_grad,
    grpo_token_advantages,
    grpo_token_loss,
    set_timing_events,
    workspace,
)

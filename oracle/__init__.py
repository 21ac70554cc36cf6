"""fp64 CPU oracle for the GRPO loss hot path (test infrastructure only).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the HIP library never does.
"""

from .grpo_oracle import (  # noqa: F401
    ADV_ESTIMATORS,
    KL_ESTIMATORS,
    PG_LOSSES,
    REDUCTIONS,
    SEQUENCE_PG,
    TIS_TYPES,
    LossConfig,
    OracleInputError,
    OracleResult,
    clamp_advantages,
    discounted_returns,
    gdpo_advantages,
    global_masked_normalize,
    group_advantages,
    group_offsets,
    gspo_terms,
    grpo_advantages,
    grpo_loss_fwd_bwd,
    grpo_loss_rows,
    grpo_token_loss,
    is_weights,
    kl_terms,
    logits_rows,
    policy_terms,
    real_terms,
    reinforce_pp_baseline_raw,
    reinforce_pp_token_rewards,
    row_logsumexp,
    sequence_mask_keep,
    sequence_mean,
    sequence_terms,
    sequence_weights,
    softmax_grad_rows,
    token_advantages,
    token_terms,
)

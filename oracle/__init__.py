"""fp64 CPU oracle for the top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import, call or execute anything in this package; only the
tests, the smoke check and the bench's CPU-baseline leg use it.
"""
from .kd_oracle import (  # noqa: F401
    teacher_scaled_grid,
    teacher_distribution,
    oracle_from_logits,
    oracle_loss_grads,
    oracle_rows,
    oracle_dW_rows,
    oracle_entropy,
    oracle_entropy_rows,
    oracle_select_top_fraction,
    oracle_entropy_select_kl,
    oracle_validate_topk,
    oracle_teacher_topk,
    oracle_select_samples,
    oracle_position_signals,
    oracle_select_by_signal,
    oracle_select_above,
    oracle_validate_topk_order,
    oracle_teacher_cdf,
    oracle_teacher_sample,
)

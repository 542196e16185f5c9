"""fp64 CPU oracle for the fused, chunked top-K KL loss.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.
"""
from .kd_oracle import (  # noqa: F401
    dw_rows,
    entropy_filter_mask,
    kd_topk_kl,
    log_softmax_rows,
    loss_given_lse,
    row_lse,
    rows_loss_and_dh,
    scattered_teacher,
    slice_terms,
    teacher_distribution,
    teacher_entropy,
    topk_divergence,
)
from .teacher_topk import teacher_logits, teacher_topk_cache  # noqa: F401

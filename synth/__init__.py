"""Seeded synthetic inputs shared by the oracle tests and the GPU path."""
from .inputs import (  # noqa: F401
    BF16, CHUNK_SWEEP, F32, WORKLOADS, Inputs, bf16_bits_to_f32,
    exact_mask, f32_to_bf16_bits, make_case, teacher_topk, uniform_cache,
    workload, TeacherHead, teacher_head, teacher_head_integer,
    teacher_head_split,
)

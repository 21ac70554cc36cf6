"""Seeded synthetic input generators shared by the tests and the benchmark."""

from .synth import (  # noqa: F401
    TOKEN_WORKLOADS,
    WORKLOADS,
    LogitsWorkload,
    TokenWorkload,
    make_logits_inputs,
    make_gen_logps,
    make_token_inputs,
    poison_masked,
    shift_by_sequence,
)

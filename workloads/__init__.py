"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package draws inputs only; it holds none of the recurrence's
arithmetic and imports neither the oracle nor the HIP library.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    SEGMENT,
    round_to_bf16,
    prefill_inputs,
    config_prefill_inputs,
    decode_initial_state,
    decode_step_inputs,
    frontend_inputs,
    mtp_draft_inputs,
    qsa_inputs,
    qsa_select_inputs,
)

"""Seeded synthetic workloads for the cache-aware streaming Conformer chunk step.

This package only draws numbers: the workload configurations, seeded weights,
inputs and injected stream states. It holds none of the encoder's arithmetic, so the
oracle under ``oracle/`` and the HIP path can both consume it without sharing any
computation.
"""
from .configs import (A4, B8, B8S, BEAM_CONFIGS, C1, C2, C2Q, C3, C4, C4S, C5, CONFIGS, D1, D2, DEC_CONFIGS,  # noqa: F401
                      MEL_CONFIGS, BeamConfig, DecConfig, EncConfig, MelConfig, get_config)
from .gen import (  # noqa: F401
    bf16_round,
    make_weights,
    make_dec_weights,
    make_dec_inputs,
    make_audio,
    make_beam_inputs,
    dec_weight_names,
    make_inputs,
    make_state,
    make_token_head,
    state_position,
    weight_names,
)

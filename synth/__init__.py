"""Seeded synthetic inputs for the routed MoE FFN layer.

This package only *produces* inputs (activations, router weights or logits,
slot maps and expert weight bytes with their block scales).  It holds none of
the layer's own arithmetic: no routing, no dequantisation, no FFN.  Both the
HIP path and the CPU oracle consume what it returns.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Config,
    LayerInputs,
    config,
    expert_weights,
    make_inputs,
    make_logits,
    make_slot_map,
    make_x,
    stack_weights,
)

"""Seeded synthetic inputs for MoE expert-parallel dispatch and combine.

This package only draws inputs (activations, router choices, router weights,
expert outputs).  It holds none of the layout, dispatch, quantisation or
combine arithmetic, so both the CPU oracle and the GPU path can take their
inputs from it without sharing any of the method.
"""
from .gen import CONFIGS, Config, generate, expert_rows, bf16_from_f32, bf16_to_f32

__all__ = ["CONFIGS", "Config", "generate", "expert_rows", "bf16_from_f32", "bf16_to_f32"]

"""Seeded synthetic workloads (shapes, weights, prompts, random operands).

Shared by the GPU path and the CPU reference as *inputs only*; it contains no step of
the decoding method.
"""

from . import configs, inputs, weights  # noqa: F401

"""Seeded synthetic inputs for the sparsely-gated MoE layer forward.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds layer shapes, value distributions and the random-number
recipe, and nothing of the layer's own arithmetic: no gate, no top-k, no
dispatch, no expert FFN and no combine is computed here.
"""

from .configs import CONFIGS, MoEConfig, get_config, scaled  # noqa: F401
from .generate import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    zipf_gate_bias,
)
from .hier import HIER_CONFIGS, HierConfig, hier_scaled, make_hier_inputs  # noqa: F401
